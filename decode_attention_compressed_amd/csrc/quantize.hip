// kv_quantize_page and kv_gather: entries <-> physical pages through the block
// table (V4 page, section 3.1.1: one 256-token logical block, 256/m entries a
// page; section 3.1.3: page size = block size x compress ratio x bytes per
// element; sections 2.1/2.2: fp8 main KV, fp8 or fp4 indexer keys;
// vLLM-0.7.2 page, section 2.1: logical block -> physical page tables).
//
// fp8 pages need the amax of the whole page before any code can be written.
// Without a workspace one block owns a page: its fp32 rows are held in
// registers (or streamed twice), the max is reduced over the block and the
// codes are written.  With a workspace the page is cut into chunks of rows,
// one block each: an amax pass writes one partial per chunk, then an encode
// pass (same grid, so each chunk lands on the same XCD and re-reads its rows
// from that XCD's L2) takes the max of the page's partials and writes the
// chunk's codes.  A decode step that rewrites one open page per sequence thus
// spreads over pages x chunks blocks instead of one.
// fp4 scales are per 32 elements of a row, so four lanes own one block of 32
// and reduce its amax with two lane swaps; pages are cut into row chunks too.
#include "hca_common.h"
#include "hca_internal.h"

namespace hca {

constexpr int kQThreads = 256;

__device__ __forceinline__ bool page_ok(int phys, int num_pages) { return phys >= 0 && phys < num_pages; }

// fp8 pages: the page's fp32 rows are held in registers (up to kF8Regs float4
// per thread, all loads in flight at once), the amax is reduced over the block,
// and the codes are written from the registers.  Larger pages take two passes.
constexpr int kF8Threads = 1024;
constexpr int kF8Regs = 16;

__device__ __forceinline__ uint32_t encode4_fp8(const f32x4 v, float s) { return e4m3_encode4_div(v[0], v[1], v[2], v[3], s); }

__device__ __forceinline__ float block_max_1024(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kF8Threads / 64; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kF8Threads) void quantize_fp8_kernel(QuantArgs a) {
  const int b = blockIdx.y;
  const int epp = a.dst.epp, dim = a.dst.dim;
  const int n = clampi(a.ne[b], 0, a.max_ne);
  const int E0 = a.e0[b];
  const int npages = (n + epp - 1) / epp;
  uint8_t* codes = reinterpret_cast<uint8_t*>(a.dst.codes);
  float* scales = reinterpret_cast<float*>(a.dst.scales);
  __shared__ float red_s[kF8Threads / 64];
  const int tot4 = epp * dim / 4;
  for (int pg = blockIdx.x; pg < npages; pg += gridDim.x) {
    const int lb = E0 / epp + pg;
    HCA_DBG_CHECK(lb >= 0 && lb < a.bts, kDbgTable);
    if (lb < 0 || lb >= a.bts) continue;
    const int phys = a.bt[(int64_t)b * a.bts + lb];
    HCA_DBG_CHECK(page_ok(phys, a.dst.num_pages), kDbgPage);
    if (!page_ok(phys, a.dst.num_pages)) continue;  // uniform over the block
    const int rows = min(epp, n - pg * epp);
    const int nv4 = rows * dim / 4;  // valid float4 groups (dim % 4 == 0)
    const f32x4* src = reinterpret_cast<const f32x4*>(a.src + (int64_t)b * a.ss + (int64_t)pg * epp * dim);
    uint32_t* dst = reinterpret_cast<uint32_t*>(codes + (int64_t)phys * epp * dim);
    if (tot4 <= kF8Threads * kF8Regs) {
      f32x4 v[kF8Regs];
      float amax = 0.0f;
#pragma unroll
      for (int r = 0; r < kF8Regs; ++r) {
        const int i = threadIdx.x + r * kF8Threads;
        v[r] = i < nv4 ? src[i] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int r = 0; r < kF8Regs; ++r)
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[r][0]), fabsf(v[r][1])), fmaxf(fabsf(v[r][2]), fabsf(v[r][3]))));
      amax = block_max_1024(amax, red_s);
      const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
#pragma unroll
      for (int r = 0; r < kF8Regs; ++r) {
        const int i = threadIdx.x + r * kF8Threads;
        if (i < tot4) dst[i] = i < nv4 ? encode4_fp8(v[r], s) : 0u;
      }
      if (threadIdx.x == 0) scales[phys] = s;
    } else {
      // two passes, 8 loads in flight per thread; the second pass re-reads from L2
      constexpr int U = 8;
      float amax = 0.0f;
      for (int i0 = threadIdx.x; i0 < nv4; i0 += U * kF8Threads) {
        f32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * kF8Threads;
          v[u] = i < nv4 ? src[i] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
          amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[u][0]), fabsf(v[u][1])), fmaxf(fabsf(v[u][2]), fabsf(v[u][3]))));
      }
      amax = block_max_1024(amax, red_s);
      const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
      for (int i0 = threadIdx.x; i0 < tot4; i0 += U * kF8Threads) {
        f32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * kF8Threads;
          v[u] = i < nv4 ? src[i] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * kF8Threads;
          if (i < tot4) dst[i] = i < nv4 ? encode4_fp8(v[u], s) : 0u;
        }
      }
      if (threadIdx.x == 0) scales[phys] = s;
    }
  }
}

// ---- chunked fp8 path: rows [c*R, c*R + R) of page pg form chunk (pg, c)
constexpr int kChunkFloats = 8192;  // floats per chunk: 8 float4 per thread at 256 threads

struct ChunkGeom {
  int R, C;  // rows per chunk, chunks per page
};
__host__ __device__ __forceinline__ ChunkGeom chunk_geom(int epp, int dim) {
  int R = kChunkFloats / dim;
  R = R < 1 ? 1 : (R > epp ? epp : R);
  return ChunkGeom{R, (epp + R - 1) / R};
}

__device__ __forceinline__ float block_max_256(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

// Resolves chunk (pg, c) of sequence b; false if its page is outside the table
// or the pool (such pages are skipped by both passes alike).
struct ChunkLoc {
  int phys, row0, nrows;  // physical page, first row of the chunk in the page, valid rows in the chunk
};
__device__ __forceinline__ bool chunk_locate(const QuantArgs& a, int b, int n, int pg, int c, ChunkGeom g,
                                             ChunkLoc& loc) {
  const int epp = a.dst.epp;
  const int lb = a.e0[b] / epp + pg;
  HCA_DBG_CHECK(lb >= 0 && lb < a.bts, kDbgTable);
  if (lb < 0 || lb >= a.bts) return false;
  const int phys = a.bt[(int64_t)b * a.bts + lb];
  HCA_DBG_CHECK(page_ok(phys, a.dst.num_pages), kDbgPage);
  if (!page_ok(phys, a.dst.num_pages)) return false;
  const int rows = min(epp, n - pg * epp);
  loc.phys = phys;
  loc.row0 = c * g.R;
  loc.nrows = max(0, min(g.R, rows - loc.row0));
  return true;
}

__global__ __launch_bounds__(kQThreads) void amax_fp8_kernel(QuantArgs a, float* part, int pages_max) {
  const int b = blockIdx.y;
  const int epp = a.dst.epp, dim = a.dst.dim;
  const ChunkGeom g = chunk_geom(epp, dim);
  const int n = clampi(a.ne[b], 0, a.max_ne);
  const int npages = (n + epp - 1) / epp;
  __shared__ float red_s[kQThreads / 64];
  for (int u = blockIdx.x; u < npages * g.C; u += gridDim.x) {
    const int pg = u / g.C, c = u % g.C;
    ChunkLoc loc;
    if (!chunk_locate(a, b, n, pg, c, g, loc)) continue;  // uniform over the block
    const int nv4 = loc.nrows * dim / 4;
    const f32x4* src =
        reinterpret_cast<const f32x4*>(a.src + (int64_t)b * a.ss + ((int64_t)pg * epp + loc.row0) * dim);
    constexpr int U = kChunkFloats / 4 / kQThreads;
    float amax = 0.0f;
    for (int i0 = threadIdx.x; i0 < nv4; i0 += U * kQThreads) {
      f32x4 v[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int i = i0 + k * kQThreads;
        v[k] = i < nv4 ? src[i] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int k = 0; k < U; ++k)
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[k][0]), fabsf(v[k][1])), fmaxf(fabsf(v[k][2]), fabsf(v[k][3]))));
    }
    amax = block_max_256(amax, red_s);
    if (threadIdx.x == 0) part[((int64_t)b * pages_max + pg) * g.C + c] = amax;
  }
}

__global__ __launch_bounds__(kQThreads) void encode_fp8_kernel(QuantArgs a, const float* part, int pages_max) {
  const int b = blockIdx.y;
  const int epp = a.dst.epp, dim = a.dst.dim;
  const ChunkGeom g = chunk_geom(epp, dim);
  const int n = clampi(a.ne[b], 0, a.max_ne);
  const int npages = (n + epp - 1) / epp;
  uint8_t* codes = reinterpret_cast<uint8_t*>(a.dst.codes);
  float* scales = reinterpret_cast<float*>(a.dst.scales);
  for (int u = blockIdx.x; u < npages * g.C; u += gridDim.x) {
    const int pg = u / g.C, c = u % g.C;
    ChunkLoc loc;
    if (!chunk_locate(a, b, n, pg, c, g, loc)) continue;
    const float* pp = part + ((int64_t)b * pages_max + pg) * g.C;
    float amax = 0.0f;
    for (int i = 0; i < g.C; ++i) amax = fmaxf(amax, pp[i]);
    const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    const int nv4 = loc.nrows * dim / 4;
    const int rows_c = min(g.R, epp - loc.row0);  // slots of this chunk, valid or not
    const int tot4 = rows_c * dim / 4;
    const f32x4* src =
        reinterpret_cast<const f32x4*>(a.src + (int64_t)b * a.ss + ((int64_t)pg * epp + loc.row0) * dim);
    uint32_t* dst = reinterpret_cast<uint32_t*>(codes + ((int64_t)loc.phys * epp + loc.row0) * dim);
    constexpr int U = kChunkFloats / 4 / kQThreads;
    for (int i0 = threadIdx.x; i0 < tot4; i0 += U * kQThreads) {
      f32x4 v[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int i = i0 + k * kQThreads;
        v[k] = i < nv4 ? src[i] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int i = i0 + k * kQThreads;
        if (i < tot4) dst[i] = i < nv4 ? encode4_fp8(v[k], s) : 0u;
      }
    }
    if (c == 0 && threadIdx.x == 0) scales[loc.phys] = s;
  }
}

size_t quantize_ws_bytes(int B, int max_ne, const hca_paged_cache& dst) {
  if (dst.dtype != HCA_FP8_E4M3 || B <= 0 || max_ne <= 0) return 0;
  const int pages_max = (max_ne + dst.epp - 1) / dst.epp;
  const ChunkGeom g = chunk_geom(dst.epp, dst.dim);
  return ((size_t)B * pages_max * g.C * sizeof(float) + 255) & ~(size_t)255;
}

__global__ __launch_bounds__(kQThreads) void quantize_fp4_kernel(QuantArgs a) {
  // four lanes per 32-element block, 8 elements (two float4) each; a block
  // takes a chunk of rows with one (row, block, quarter) unit per thread
  const int b = blockIdx.y;
  const int epp = a.dst.epp, dim = a.dst.dim;
  const int n = clampi(a.ne[b], 0, a.max_ne);
  const int E0 = a.e0[b];
  const int npages = (n + epp - 1) / epp;
  const int nblk = dim / 32;
  const int R = max(1, min(epp, kQThreads / (nblk * 4)));  // rows per chunk
  const int C = (epp + R - 1) / R;
  uint8_t* codes = reinterpret_cast<uint8_t*>(a.dst.codes);
  uint8_t* scales = reinterpret_cast<uint8_t*>(a.dst.scales);
  for (int w = blockIdx.x; w < npages * C; w += gridDim.x) {
    const int pg = w / C, row0 = (w % C) * R;
    const int lb = E0 / epp + pg;
    HCA_DBG_CHECK(lb >= 0 && lb < a.bts, kDbgTable);
    if (lb < 0 || lb >= a.bts) continue;
    const int phys = a.bt[(int64_t)b * a.bts + lb];
    HCA_DBG_CHECK(page_ok(phys, a.dst.num_pages), kDbgPage);
    if (!page_ok(phys, a.dst.num_pages)) continue;
    const int rows = min(epp, n - pg * epp);
    const float* src = a.src + (int64_t)b * a.ss + (int64_t)pg * epp * dim;
    uint8_t* pc = codes + (int64_t)phys * epp * (dim / 2);
    uint8_t* ps = scales + (int64_t)phys * epp * nblk;
    const int units = min(R, epp - row0) * nblk * 4;  // (row, block, quarter)
    for (int u = threadIdx.x; u < units; u += kQThreads) {
      const int q = u & 3;
      const int blk = (u >> 2) % nblk;
      const int row = row0 + (u >> 2) / nblk;
      float v[8];
      float amax = 0.0f;
      if (row < rows) {
        const f32x4* p = reinterpret_cast<const f32x4*>(src + (int64_t)row * dim + blk * 32 + q * 8);
        const f32x4 v0 = p[0], v1 = p[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[i] = v0[i]; v[4 + i] = v1[i]; }
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
      }
      amax = quad_max(amax);
      const uint32_t sc = row < rows ? e4m3_encode(amax / 6.0f) : 0u;
      const float sdec = e4m3_decode(sc);
      uint32_t word = 0;
      if (sdec > 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) word |= e2m1_encode(v[i] / sdec) << (4 * i);
      }
      *reinterpret_cast<uint32_t*>(pc + (int64_t)row * (dim / 2) + blk * 16 + q * 4) = word;
      if (q == 0) ps[(int64_t)row * nblk + blk] = (uint8_t)sc;
    }
  }
}

__global__ __launch_bounds__(kQThreads) void quantize_bf16_kernel(QuantArgs a) {
  const int b = blockIdx.y;
  const int epp = a.dst.epp, dim = a.dst.dim;
  const int n = clampi(a.ne[b], 0, a.max_ne);
  const int E0 = a.e0[b];
  const int npages = (n + epp - 1) / epp;
  uint16_t* codes = reinterpret_cast<uint16_t*>(a.dst.codes);
  for (int pg = blockIdx.x; pg < npages; pg += gridDim.x) {
    const int lb = E0 / epp + pg;
    HCA_DBG_CHECK(lb >= 0 && lb < a.bts, kDbgTable);
    if (lb < 0 || lb >= a.bts) continue;
    const int phys = a.bt[(int64_t)b * a.bts + lb];
    HCA_DBG_CHECK(page_ok(phys, a.dst.num_pages), kDbgPage);
    if (!page_ok(phys, a.dst.num_pages)) continue;
    const int rows = min(epp, n - pg * epp);
    const int nv4 = rows * dim / 4;
    const f32x4* src = reinterpret_cast<const f32x4*>(a.src + (int64_t)b * a.ss + (int64_t)pg * epp * dim);
    u32x2* dst = reinterpret_cast<u32x2*>(codes + (int64_t)phys * epp * dim);
    const int tot4 = epp * dim / 4;
    for (int i = threadIdx.x; i < tot4; i += kQThreads) {
      u32x2 w = {0u, 0u};
      if (i < nv4) {
        const f32x4 v = src[i];
        w[0] = (uint32_t)bf16_encode(v[0]) | ((uint32_t)bf16_encode(v[1]) << 16);
        w[1] = (uint32_t)bf16_encode(v[2]) | ((uint32_t)bf16_encode(v[3]) << 16);
      }
      dst[i] = w;
    }
  }
}

hipError_t launch_quantize(const QuantArgs& a, float* ws, hipStream_t s) {
  const int epp = a.dst.epp;
  const int pages_max = (a.max_ne + epp - 1) / epp;
  if (a.B == 0 || pages_max == 0) return hipSuccess;
  switch (a.dst.dtype) {
    case HCA_FP8_E4M3: {
      const ChunkGeom g = chunk_geom(epp, a.dst.dim);
      if (ws == nullptr || g.C == 1) {  // a page that fits one chunk needs no split
        const int gx = pages_max > 8192 ? 8192 : pages_max;
        hipLaunchKernelGGL(quantize_fp8_kernel, dim3(gx, a.B), dim3(kF8Threads), 0, s, a);
      } else {
        const int64_t units = (int64_t)pages_max * g.C;
        const dim3 grid(units > 16384 ? 16384 : (int)units, a.B);
        hipLaunchKernelGGL(amax_fp8_kernel, grid, dim3(kQThreads), 0, s, a, ws, pages_max);
        hipLaunchKernelGGL(encode_fp8_kernel, grid, dim3(kQThreads), 0, s, a, (const float*)ws, pages_max);
      }
      break;
    }
    case HCA_FP4_E2M1: {
      const int nblk = a.dst.dim / 32;
      const int R = max(1, min(epp, kQThreads / (nblk * 4)));
      const int64_t units = (int64_t)pages_max * ((epp + R - 1) / R);
      hipLaunchKernelGGL(quantize_fp4_kernel, dim3(units > 16384 ? 16384 : (int)units, a.B), dim3(kQThreads), 0, s,
                         a);
      break;
    }
    default: {
      const int gx = pages_max > 8192 ? 8192 : pages_max;
      hipLaunchKernelGGL(quantize_bf16_kernel, dim3(gx, a.B), dim3(kQThreads), 0, s, a);
      break;
    }
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ gather
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  const int b = blockIdx.y;
  const int n = clampi(a.n_rows[b], 0, a.max_rows);
  const int epp = a.src.epp, dim = a.src.dim;
  const int row_bytes = a.src.dtype == HCA_FP8_E4M3 ? dim : (a.src.dtype == HCA_FP4_E2M1 ? dim / 2 : 2 * dim);
  const int w4 = row_bytes / 4;  // 32-bit words per row
  const uint8_t* codes = reinterpret_cast<const uint8_t*>(a.src.codes);
  uint8_t* dst = reinterpret_cast<uint8_t*>(a.dst_codes);
  for (int r = blockIdx.x; r < n; r += gridDim.x) {
    const int phys = a.bt[(int64_t)b * a.bts + r / epp];
    if (!page_ok(phys, a.src.num_pages)) continue;
    const int slot = r % epp;
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(codes + ((int64_t)phys * epp + slot) * row_bytes);
    uint32_t* dp = reinterpret_cast<uint32_t*>(dst + ((int64_t)b * a.max_rows + r) * row_bytes);
    for (int i = threadIdx.x; i < w4; i += 256) dp[i] = sp[i];
    if (threadIdx.x == 0 && a.src.dtype == HCA_FP8_E4M3)
      reinterpret_cast<float*>(a.dst_scales)[(int64_t)b * a.max_rows + r] = reinterpret_cast<const float*>(a.src.scales)[phys];
    if (a.src.dtype == HCA_FP4_E2M1 && threadIdx.x < dim / 32) {
      const uint8_t* ss = reinterpret_cast<const uint8_t*>(a.src.scales) + ((int64_t)phys * epp + slot) * (dim / 32);
      reinterpret_cast<uint8_t*>(a.dst_scales)[((int64_t)b * a.max_rows + r) * (dim / 32) + threadIdx.x] = ss[threadIdx.x];
    }
  }
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
  if (a.B == 0 || a.max_rows == 0) return hipSuccess;
  const int gx = a.max_rows > 16384 ? 16384 : a.max_rows;
  hipLaunchKernelGGL(gather_kernel, dim3(gx, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

#ifdef HCA_DEBUG
HCA_DBG_ACCESSOR(debug_bits_quantize)
#endif

}  // namespace hca
