// indexer_topk: indexer scoring and top-k for c4a layers (V4 page, section 2.2:
// a separate, smaller indexer KV decides which compressed entries the query
// looks in, instead of a brute-force search over the main KV).
//
// Score kernel (the HBM-bound stream of a c4a layer).  Each wave scores 16
// entries at a time with v_mfma_f32_16x16x32_bf16: A = the 16 indexer query
// heads (bf16, held in registers), B = 16 keys decoded to exact bf16 (E4M3 and
// E2M1 values are exact in bf16).  The contraction order inside an MFMA step is
// free, so each lane reads one contiguous run of its key (16-byte loads) and
// the query fragment uses the same dim order.  fp4 keys carry a scale per 32
// elements; a k-step covers exactly one such block, its MFMA writes a fresh
// accumulator and the block scale is applied in fp32 afterwards.  ReLU, the
// per-head weights and the head sum run on the accumulator lanes, and the
// order key of every score lands in a 4096-bin LDS histogram that is added to
// a per-sequence histogram in the workspace.
//
// Select kernel.  Every block re-derives the cut bin from the histogram, marks
// the scores above it in a bitmap and appends the cut bin's entries as
// candidates; the last block of a sequence (ticket counter) refines the cut
// with two 10-bit radix passes over the candidates, breaks exact ties by the
// lowest index, and compacts the bitmap into ascending indices.  It leaves the
// histogram, counters and bitmap zeroed for the next call.
#include "hca_common.h"
#include "hca_internal.h"

namespace hca {

constexpr int kScoreThreads = 256;
constexpr int kScoreChunk = 1024;  // entries per score block (256 per wave)
constexpr int kSelThreads = 256;
constexpr int kSelChunk = 8192;    // entries per select block (32 per thread)

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

IndexerWs indexer_ws_layout(int B, int max_seq_len, int m, int k) {
  (void)k;
  IndexerWs w;
  const int n_max = (max_seq_len + m - 1) / m;
  w.n_max = n_max;
  const int n_pad = ((n_max + kSelChunk - 1) / kSelChunk) * kSelChunk;
  size_t off = 0;
  w.scores = off; off = align256(off + (size_t)B * n_pad * sizeof(float));
  w.hist = off; off = align256(off + (size_t)B * kHistBins * sizeof(uint32_t));
  w.cand = off; off = align256(off + (size_t)B * n_pad * sizeof(uint2));
  w.bitmap = off; off = align256(off + (size_t)B * (n_pad / 32) * sizeof(uint32_t));
  w.counters = off; off = align256(off + (size_t)B * 4 * sizeof(uint32_t));
  w.total = off;
  return w;
}

// ------------------------------------------------------------------ scoring
template <int KDT>
struct KeyBytes;  // bytes of one stored key row
template <> struct KeyBytes<HCA_BF16> { static constexpr int per_dim_x2 = 4; };
template <> struct KeyBytes<HCA_FP8_E4M3> { static constexpr int per_dim_x2 = 2; };
template <> struct KeyBytes<HCA_FP4_E2M1> { static constexpr int per_dim_x2 = 1; };

__device__ __forceinline__ uint32_t pack_bf16_hi(float lo, float hi) {
  // exact values: the bf16 pattern is the top half of the fp32 pattern
  return (f2u(lo) >> 16) | (f2u(hi) & 0xFFFF0000u);
}

// 8 fp8 codes (two dwords) -> 8 exact bf16 values
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  u32x4 r;
  f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false);
  f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
  f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false);
  f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
  r[0] = pack_bf16_hi(a[0], a[1]);
  r[1] = pack_bf16_hi(b[0], b[1]);
  r[2] = pack_bf16_hi(c[0], c[1]);
  r[3] = pack_bf16_hi(d[0], d[1]);
  return __builtin_bit_cast(bf16x8, r);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// 8 fp4 codes (one dword, element 2c in the low nibble of byte c) -> 8 exact bf16
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
  return __builtin_bit_cast(bf16x8, r);
}

template <int KDT, int DI>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(IndexerArgs a) {
  constexpr int KS = DI / 32;  // MFMA k-steps
  const int b = blockIdx.y;
  const int L = clampi(a.lens[b], 0, a.max_len);
  const int N = (L + a.m - 1) / a.m;
  const int chunk0 = blockIdx.x * kScoreChunk;
  if (chunk0 >= N) return;
  const bool want_hist = a.k < N;
  __shared__ uint32_t hist_s[kHistBins];
  if (want_hist) {
    for (int i = threadIdx.x; i < kHistBins; i += kScoreThreads) hist_s[i] = 0;
    __syncthreads();
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int epp = a.keys.epp;

  // query fragments (heads >= HI are zero) and head weights of the 4 accumulator rows
  bf16x8 qa[KS];
  {
    const int h = col;
    const uint16_t* qrow = a.q + ((int64_t)b * a.HI + h) * DI;
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      // bf16 / fp8 keys: lane group g owns dims [g*DI/4, (g+1)*DI/4), step t the 8 at +8t
      // fp4 keys: step t is block t; lane group g owns dims 32t + 8g .. +8
      const int c0 = (KDT == HCA_FP4_E2M1) ? (32 * t + 8 * g) : (g * (DI / 4) + 8 * t);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (h < a.HI) v = *reinterpret_cast<const u32x4*>(qrow + c0);
      qa[t] = __builtin_bit_cast(bf16x8, v);
    }
  }
  float wgt[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g + i;
    wgt[i] = h < a.HI ? a.w[(int64_t)b * a.HI + h] : 0.0f;
  }

  const uint8_t* codes = reinterpret_cast<const uint8_t*>(a.keys.codes);
  const int row_bytes = DI * KeyBytes<KDT>::per_dim_x2 / 2;
  float* scores = reinterpret_cast<float*>(a.ws + a.lay.scores) + (size_t)b * ((a.lay.n_max + kSelChunk - 1) / kSelChunk) * kSelChunk;

  const int wave0 = chunk0 + wave * (kScoreChunk / 4);
  const int wave1 = min(N, wave0 + kScoreChunk / 4);
  for (int e_base = wave0; e_base < wave1; e_base += 16) {
    const int e = e_base + col;
    const bool valid = e < wave1;
    int phys = -1, slot = 0;
    if (valid) {
      phys = a.bt[(int64_t)b * a.bts + e / epp];
      slot = e % epp;
      if (phys >= a.keys.num_pages) phys = -1;
    }
    const bool live = phys >= 0;
    const uint8_t* row = codes + ((int64_t)(live ? phys : 0) * epp + slot) * row_bytes;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KDT == HCA_FP4_E2M1) {
      // per-block accumulators, block scales applied in fp32
      uint32_t sc_raw = 0;
      if (live) {
        const uint8_t* srow = reinterpret_cast<const uint8_t*>(a.keys.scales) + ((int64_t)phys * epp + slot) * KS;
        if constexpr (KS == 4) sc_raw = *reinterpret_cast<const uint32_t*>(srow);
        else {
#pragma unroll
          for (int t = 0; t < KS && t < 4; ++t) sc_raw |= (uint32_t)srow[t] << (8 * t);
        }
      }
      uint32_t kw[KS];
#pragma unroll
      for (int t = 0; t < KS; ++t) kw[t] = live ? *reinterpret_cast<const uint32_t*>(row + 16 * t + 4 * g) : 0u;
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[t], fp4x8_to_bf16(kw[t]), z, 0, 0, 0);
        // the accumulator column (entry) of this lane is `col`; its block-t scale:
        uint32_t sc;
        if constexpr (KS <= 4) sc = (sc_raw >> (8 * t)) & 0xFFu;
        else sc = live ? reinterpret_cast<const uint8_t*>(a.keys.scales)[((int64_t)phys * epp + slot) * KS + t] : 0u;
        const float sf = e4m3_decode(sc);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(sf, part[i], acc[i]);
      }
    } else {
      constexpr int LB = DI * KeyBytes<KDT>::per_dim_x2 / 8;  // bytes per lane
      const uint8_t* lrow = row + g * LB;
      bf16x8 kb[KS];
      if constexpr (KDT == HCA_FP8_E4M3) {
        // LB = DI/4 bytes: KS chunks of 8 codes
#pragma unroll
        for (int t = 0; t < KS; t += 2) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (live) {
            if (t + 1 < KS) v = *reinterpret_cast<const u32x4*>(lrow + 8 * t);
            else { u32x2 h2 = *reinterpret_cast<const u32x2*>(lrow + 8 * t); v[0] = h2[0]; v[1] = h2[1]; }
          }
          kb[t] = fp8x8_to_bf16(v[0], v[1]);
          if (t + 1 < KS) kb[t + 1] = fp8x8_to_bf16(v[2], v[3]);
        }
      } else {
        // bf16 keys: LB = DI/2 bytes, KS chunks of 8 values (16 bytes)
#pragma unroll
        for (int t = 0; t < KS; ++t) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (live) v = *reinterpret_cast<const u32x4*>(lrow + 16 * t);
          kb[t] = __builtin_bit_cast(bf16x8, v);
        }
      }
#pragma unroll
      for (int t = 0; t < KS; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[t], kb[t], acc, 0, 0, 0);
      if constexpr (KDT == HCA_FP8_E4M3) {
        const float ps = live ? reinterpret_cast<const float*>(a.keys.scales)[phys] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] *= ps;
      }
    }
    // lane holds heads 4g+i of entry `col`: ReLU, weight, sum over heads
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s = fmaf(wgt[i], fmaxf(acc[i], 0.0f), s);
    s += __shfl_xor(s, 16, 64);
    s += __shfl_xor(s, 32, 64);
    if (g == 0 && valid) {
      scores[e] = s;
      if (want_hist) atomicAdd(&hist_s[order_key(s) >> 20], 1u);
    }
  }
  if (want_hist) {
    __syncthreads();
    uint32_t* gh = reinterpret_cast<uint32_t*>(a.ws + a.lay.hist) + (size_t)b * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += kScoreThreads) {
      const uint32_t c = hist_s[i];
      if (c) atomicAdd(&gh[i], c);
    }
  }
}

// ------------------------------------------------------------------ select
// exclusive block scan of one uint per thread (kSelThreads threads)
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    const uint32_t t = tmp[w];
    if (w < wave) base += t;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return base + x - v;
}

// Find, scanning `bins` from the highest bin down, the bin where the running count
// reaches `need`; returns the bin and the count strictly above it.  nb = 1024 or 4096.
__device__ void find_cut(const uint32_t* bins, int nb, uint32_t need, uint32_t* tmp, int& cut, uint32_t& above) {
  const int per = nb / kSelThreads;
  const int hi = nb - per * threadIdx.x;  // this thread takes bins [hi-per, hi), top first
  uint32_t cnt = 0;
  for (int i = 1; i <= per; ++i) cnt += bins[hi - i];
  uint32_t total;
  const uint32_t before = block_excl_scan(cnt, tmp, total);
  __shared__ int cut_s;
  __shared__ uint32_t above_s;
  if (before < need && before + cnt >= need) {
    uint32_t run = before;
    for (int i = 1; i <= per; ++i) {
      const uint32_t c = bins[hi - i];
      if (run + c >= need) { cut_s = hi - i; above_s = run; break; }
      run += c;
    }
  }
  __syncthreads();
  cut = cut_s;
  above = above_s;
  __syncthreads();
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(IndexerArgs a) {
  const int b = blockIdx.y;
  const int L = clampi(a.lens[b], 0, a.max_len);
  const int N = (L + a.m - 1) / a.m;
  const int k = a.k;
  int32_t* out = a.out_idx + (int64_t)b * k;
  if (N <= k) {  // every entry is kept
    const int lo = blockIdx.x * kSelChunk, hi = min(N, lo + kSelChunk);
    for (int i = lo + threadIdx.x; i < hi; i += kSelThreads) out[i] = i;
    if (blockIdx.x == 0) {
      for (int i = N + threadIdx.x; i < k; i += kSelThreads) out[i] = -1;
      if (threadIdx.x == 0) a.out_n[b] = N;
    }
    return;
  }
  const int G = (N + kSelChunk - 1) / kSelChunk;
  if ((int)blockIdx.x >= G) return;
  const int n_pad = ((a.lay.n_max + kSelChunk - 1) / kSelChunk) * kSelChunk;
  const float* scores = reinterpret_cast<const float*>(a.ws + a.lay.scores) + (size_t)b * n_pad;
  uint32_t* hist = reinterpret_cast<uint32_t*>(a.ws + a.lay.hist) + (size_t)b * kHistBins;
  uint2* cand = reinterpret_cast<uint2*>(a.ws + a.lay.cand) + (size_t)b * n_pad;
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(a.ws + a.lay.bitmap) + (size_t)b * (n_pad / 32);
  uint32_t* ctr = reinterpret_cast<uint32_t*>(a.ws + a.lay.counters) + (size_t)b * 4;  // [0] candidates, [1] ticket

  __shared__ uint32_t tmp[kSelThreads / 64];
  __shared__ uint32_t h_s[1024];
  int cut;
  uint32_t above;
  find_cut(hist, kHistBins, (uint32_t)k, tmp, cut, above);

  // chunk pass: 32 consecutive entries per thread, one bitmap word each
  const int e0 = blockIdx.x * kSelChunk + threadIdx.x * 32;
  if (e0 < N) {
    uint32_t bits = 0;
    for (int i = 0; i < 32; ++i) {
      const int e = e0 + i;
      if (e >= N) break;
      const uint32_t key = order_key(scores[e]);
      const int bin = (int)(key >> 20);
      if (bin > cut) bits |= 1u << i;
      else if (bin == cut) {
        const uint32_t pos = atomicAdd(&ctr[0], 1u);
        cand[pos] = make_uint2(key, (uint32_t)e);
      }
    }
    bitmap[e0 >> 5] = bits;
  }
  __threadfence();
  __syncthreads();
  __shared__ int last_s;
  if (threadIdx.x == 0) last_s = (atomicAdd(&ctr[1], 1u) == (uint32_t)(G - 1));
  __syncthreads();
  if (!last_s) return;
  __threadfence();

  // ---- last block of this sequence: resolve the cut bin
  const uint32_t nc = __hip_atomic_load(&ctr[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t need = (uint32_t)k - above;  // 1 .. nc
  uint32_t T = 0xFFFFFFFFu;             // selected: key > T, or key == T and index <= X
  int X = -1;
  if (need < nc) {
    uint32_t prefix = (uint32_t)cut << 20, mask = 0xFFF00000u;
    for (int shift = 10; shift >= 0; shift -= 10) {
      for (int i = threadIdx.x; i < 1024; i += kSelThreads) h_s[i] = 0;
      __syncthreads();
      for (uint32_t i = threadIdx.x; i < nc; i += kSelThreads) {
        const uint32_t key = cand[i].x;
        if ((key & mask) == prefix) atomicAdd(&h_s[(key >> shift) & 1023u], 1u);
      }
      __syncthreads();
      int c2;
      uint32_t ab2;
      find_cut(h_s, 1024, need, tmp, c2, ab2);
      need -= ab2;
      prefix |= (uint32_t)c2 << shift;
      mask |= 1023u << shift;
      __syncthreads();
    }
    T = prefix;  // exact cut key; `need` entries with key == T are still to take
    // ties at T: keep the `need` lowest indices (binary search on the index bound)
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      const int mid = lo + (hi - lo) / 2;
      uint32_t c = 0;
      for (uint32_t i = threadIdx.x; i < nc; i += kSelThreads) {
        const uint2 cd = cand[i];
        c += (cd.x == T && (int)cd.y <= mid) ? 1u : 0u;
      }
      uint32_t tot;
      (void)block_excl_scan(c, tmp, tot);
      if (tot >= need) hi = mid; else lo = mid + 1;
    }
    X = lo;
  }
  for (uint32_t i = threadIdx.x; i < nc; i += kSelThreads) {
    const uint2 cd = cand[i];
    const bool take = (T == 0xFFFFFFFFu && X < 0) ? true : (cd.x > T || (cd.x == T && (int)cd.y <= X));
    if (take) atomicOr(&bitmap[cd.y >> 5], 1u << (cd.y & 31));
  }
  __threadfence();
  __syncthreads();

  // ---- ascending compaction of the bitmap; words are zeroed as they are read
  const int W = (N + 31) / 32;
  const int per = (W + kSelThreads - 1) / kSelThreads;
  const int w0 = min(W, threadIdx.x * per), w1 = min(W, w0 + per);
  uint32_t cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(__hip_atomic_load(&bitmap[w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  uint32_t total;
  uint32_t off = block_excl_scan(cnt, tmp, total);
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = __hip_atomic_load(&bitmap[w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bitmap[w] = 0u;
    while (bits) {
      const int bit = __ffs(bits) - 1;
      bits &= bits - 1;
      if (off < (uint32_t)k) out[off] = w * 32 + bit;
      ++off;
    }
  }
  for (int i = (int)total + threadIdx.x; i < k; i += kSelThreads) out[i] = -1;  // only if fewer (not expected)
  if (threadIdx.x == 0) a.out_n[b] = (int)min(total, (uint32_t)k);
  // ---- leave the workspace zeroed
  for (int i = threadIdx.x; i < kHistBins; i += kSelThreads) hist[i] = 0u;
  if (threadIdx.x == 0) { ctr[0] = 0u; ctr[1] = 0u; }
}

template <int KDT>
static hipError_t launch_score_dt(const IndexerArgs& a, dim3 grid, hipStream_t s) {
  switch (a.keys.dim) {
    case 32: hipLaunchKernelGGL((score_kernel<KDT, 32>), grid, dim3(kScoreThreads), 0, s, a); break;
    case 64: hipLaunchKernelGGL((score_kernel<KDT, 64>), grid, dim3(kScoreThreads), 0, s, a); break;
    case 128: hipLaunchKernelGGL((score_kernel<KDT, 128>), grid, dim3(kScoreThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((score_kernel<KDT, 256>), grid, dim3(kScoreThreads), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t s) {
  const int n_max = a.lay.n_max;
  if (a.B == 0) return hipSuccess;
  if (n_max > 0) {
    const dim3 grid((n_max + kScoreChunk - 1) / kScoreChunk, a.B);
    hipError_t e;
    switch (a.keys.dtype) {
      case HCA_FP8_E4M3: e = launch_score_dt<HCA_FP8_E4M3>(a, grid, s); break;
      case HCA_FP4_E2M1: e = launch_score_dt<HCA_FP4_E2M1>(a, grid, s); break;
      default: e = launch_score_dt<HCA_BF16>(a, grid, s); break;
    }
    if (e != hipSuccess) return e;
  }
  const int gsel = n_max > 0 ? (n_max + kSelChunk - 1) / kSelChunk : 1;
  const int gk = (a.k + kSelChunk - 1) / kSelChunk;
  hipLaunchKernelGGL(select_kernel, dim3(gsel > gk ? gsel : gk, a.B), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hca
