// paged_hybrid_decode: the decode query attends to the selected compressed
// entries plus the raw window, one shared K=V row each (V4 page, section 2.1:
// keys and values share one RoPE-rotated vector and the output is rotated back
// by inverse RoPE; section 2.3: every layer keeps a raw window; vLLM-0.7.2
// page, section 2.3: only window blocks are read).
//
// Work split: block = (split of the sequence's row list, sequence, 64-head
// group); wave w owns 16 query heads.  A 32-row tile is gathered through the
// block table with 16-byte loads (8 lanes cover 128 contiguous bytes of 8
// rows), decoded ONCE to f16 (fp8 code x page scale, or bf16) and stored in LDS
// row-major.  Both MFMA contractions are v_mfma_f32_16x16x32_f16:
//   S^T[rows x heads] = K[rows x d] . Q~^T          (Q~ in registers)
//   O[heads x d]     += P[heads x rows] . V[rows x d]
// The V operand (8 rows of one dim per lane) is read from the same row-major
// copy with ds_read_b64_tr_b16: within each 16-lane group, output lane i gets
// element i%4 of the 8-byte runs addressed by source lanes i/4, i/4+4, i/4+8,
// i/4+12, so source lane j addresses row R(j/4) at dims 4(j%4).. and lane i
// receives rows R(0..3) at dim i.
// The S^T accumulator of a lane is exactly its P operand for the PV step when
// the PV k-slot (g, j) is mapped to row 4g+j (j < 4) / 16+4g+j-4 (j >= 4), so
// P never leaves registers.  Online softmax keeps a running max per head and
// rescales the O accumulator only when the tile max exceeds it by more than 8
// (exp(8) still fits f16 for P), which makes the rescale rare.
// Partials (o, m, l) go to the workspace; a combine kernel merges the splits in
// split order (so the result does not depend on page placement) and applies
// inverse RoPE at position L-1.
#include "hca_common.h"
#include "hca_internal.h"

namespace hca {

constexpr int kAttnThreads = 256;
constexpr int kTileRows = 32;
constexpr int kHeadsPerBlock = 64;
constexpr float kRescaleSlack = 8.0f;
constexpr int kMaxRowsPerSplit = 256;
constexpr int kMaxSplits = kAttnMaxSplits;

static inline size_t align256a(size_t x) { return (x + 255) & ~(size_t)255; }

AttnPlan attn_plan(int B, int H, int d, int max_seq_len, int m, int window, int k, bool has_sel) {
  AttnPlan p;
  const int n_max = (max_seq_len + m - 1) / m;
  const int ent = has_sel ? (k < n_max ? k : n_max) : n_max;
  const int win = window < max_seq_len ? window : max_seq_len;
  p.rows_max = ent + win;
  p.head_blocks = (H + kHeadsPerBlock - 1) / kHeadsPerBlock;
  const int units = (B > 0 ? B : 1) * p.head_blocks;
  int S = (512 + units - 1) / units;
  const int tiles = (p.rows_max + kTileRows - 1) / kTileRows;
  if (S > tiles) S = tiles;
  if (S < 1) S = 1;
  int rps = (p.rows_max + S - 1) / S;
  rps = ((rps + kTileRows - 1) / kTileRows) * kTileRows;
  if (rps < 64) rps = 64;
  if (rps > kMaxRowsPerSplit) rps = kMaxRowsPerSplit;
  p.rows_per_split = rps;
  p.splits = p.rows_max > 0 ? (p.rows_max + rps - 1) / rps : 1;
  size_t off = 0;
  p.o_off = off; off = align256a(off + (size_t)B * p.splits * H * d * sizeof(float));
  p.ml_off = off; off = align256a(off + (size_t)B * p.splits * H * 2 * sizeof(float));
  p.total = off;
  return p;
}

// Address of one row of the sequence's row list (selected entries, then window
// tokens); 0 when the row is skipped (index outside [0, N) or unmapped page).
__device__ __forceinline__ uint64_t resolve_row(const AttnArgs& a, int b, int r, int n_sel, int N, int L, int n_win,
                                                float& scale) {
  const hca_paged_cache* pool;
  int phys, slot;
  scale = 0.0f;
  if (r < n_sel) {
    const int e = a.sel ? a.sel[(int64_t)b * a.k + r] : r;
    if (e < 0 || e >= N) return 0;
    pool = &a.kv;
    phys = a.bt[(int64_t)b * a.bts + e / a.kv.epp];
    slot = e % a.kv.epp;
  } else {
    const int t = L - n_win + (r - n_sel);
    pool = &a.win;
    phys = a.wbt[(int64_t)b * a.wbts + t / a.win.epp];
    slot = t % a.win.epp;
  }
  if (phys < 0 || phys >= pool->num_pages) return 0;
  const bool fp8 = pool->dtype == HCA_FP8_E4M3;
  const uint8_t* p = reinterpret_cast<const uint8_t*>(pool->codes) + ((int64_t)phys * pool->epp + slot) * pool->dim * (fp8 ? 1 : 2);
  scale = fp8 ? reinterpret_cast<const float*>(pool->scales)[phys] : 1.0f;
  return reinterpret_cast<uint64_t>(p);
}

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));

// the 4 rows x 16 dims one loader thread gathers per tile (raw bytes).  The
// gather is unconditional and branch-free: a skipped row, a thread with no
// chunk, or a tile past the end reads the pool's first row (masked when the
// tile is decoded), so the next tile's loads stay in flight across this
// tile's compute.
template <int KVDT>
struct RowRaw {
  static constexpr int NV = KVDT == HCA_FP8_E4M3 ? 1 : 2;  // 16-byte loads per row
  u32x4 w[4][NV];

  __device__ __forceinline__ void gather(const uint64_t* rowptr, int lr, bool tile_ok, int c16, const uint8_t* safe) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t t = rowptr[tile_ok ? lr + i : 0] & (tile_ok ? ~0ull : 0ull);
      const uint8_t* p = t ? reinterpret_cast<const uint8_t*>(t) + 16 * NV * c16 : safe;
#pragma unroll
      for (int v = 0; v < NV; ++v) w[i][v] = gload<u32x4>(p + 16 * v);
    }
  }
};

template <int D, int KVDT>
__global__ __launch_bounds__(kAttnThreads) void attn_split_kernel(AttnArgs a) {
  constexpr int KS = D / 32;          // k-steps of the S contraction
  constexpr int NT = D / 16;          // 16-dim tiles of O
  constexpr int KSTR = D + 16;        // LDS row stride (halves): 4 consecutive rows on disjoint banks
  constexpr int CHUNKS = D / 16;      // 16-dim chunks per row (load phase)
  __shared__ _Float16 k_s[kTileRows * KSTR];
  __shared__ float2 cs_s[D / 2];
  __shared__ uint64_t rowptr_s[kMaxRowsPerSplit];
  __shared__ float rowscale_s[kMaxRowsPerSplit];

  const int s = blockIdx.x, b = blockIdx.y, hb = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int L = clampi(a.lens[b], 0, a.max_len);
  const int N = (L + a.m - 1) / a.m;
  const int n_sel = a.sel ? clampi(a.sel_n[b], 0, a.k) : N;
  const int n_win = min(a.window, L);
  const int rows_b = n_sel + n_win;
  const int r0 = s * a.plan.rows_per_split;
  const int r1 = min(rows_b, r0 + a.plan.rows_per_split);
  const int H = a.H;
  const int head = hb * kHeadsPerBlock + wave * 16 + col;  // head of this lane's q / P / m / l
  float2* ml = reinterpret_cast<float2*>(a.ws + a.plan.ml_off);
  float* opart = reinterpret_cast<float*>(a.ws + a.plan.o_off);
  const size_t part = ((size_t)b * a.plan.splits + s) * H;

  if (r0 >= r1) {  // empty split
    if (g == 0 && head < H) ml[part + head] = make_float2(-INFINITY, 0.0f);
    return;
  }

  // row addresses of the whole split, and the RoPE table at the query position L-1
  for (int i = threadIdx.x; i < kMaxRowsPerSplit; i += kAttnThreads) {
    float sc = 0.0f;
    uint64_t rp = 0;
    if (r0 + i < r1) rp = resolve_row(a, b, r0 + i, n_sel, N, L, n_win, sc);
    rowptr_s[i] = rp;
    rowscale_s[i] = sc;
  }
  for (int i = threadIdx.x; i < D / 2; i += kAttnThreads) {
    float c, sn;
    rope_cs((double)(L - 1), rope_inv_freq(i, D, a.theta), c, sn);
    cs_s[i] = make_float2(c, sn);
  }
  __syncthreads();

  // rotated query fragments: lane holds Q~[head][32t + 8g + j], j < 8
  f16x8 qf[KS];
  {
    const bool hv = head < H;
    const uint16_t* qrow = a.q + ((int64_t)b * H + (hv ? head : 0)) * D;
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      const int c0 = 32 * t + 8 * g;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (hv) raw = *reinterpret_cast<const u32x4*>(qrow + c0);
      f16x8 v;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float x0 = u2f(raw[p] << 16), x1 = u2f(raw[p] & 0xFFFF0000u);
        const float2 cs = cs_s[c0 / 2 + p];
        v[2 * p] = (_Float16)(x0 * cs.x - x1 * cs.y);
        v[2 * p + 1] = (_Float16)(x0 * cs.y + x1 * cs.x);
      }
      qf[t] = v;
    }
  }

  f32x4 oacc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) oacc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;  // for head `head` (replicated over g)

  // load-phase mapping: quad q4 (rows 4q4..4q4+3 of the tile), 16-dim chunk c16
  const int q4 = threadIdx.x & 7;
  const int c16 = threadIdx.x >> 3;
  const bool loader = c16 < CHUNKS;

  const uint8_t* safe = reinterpret_cast<const uint8_t*>(a.kv.codes);
  const int c16e = loader ? c16 : 0;
  RowRaw<KVDT> raw;
  raw.gather(rowptr_s, 4 * q4, true, c16e, safe);

  for (int tr0 = r0; tr0 < r1; tr0 += kTileRows) {
    const int lr0 = tr0 - r0;
    // ---- decode this tile's 32 rows into both LDS copies
    if (loader) {
      f16x8 lo[4], hi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = rowptr_s[lr0 + 4 * q4 + i] != 0;  // skipped rows decode to zero
        const float sc = rowscale_s[lr0 + 4 * q4 + i];
        if constexpr (KVDT == HCA_BF16) {
          const u32x4 z = {0u, 0u, 0u, 0u};
          const u32x4 w0 = ok ? raw.w[i][0] : z, w1 = ok ? raw.w[i][1] : z;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            lo[i][2 * q] = (_Float16)u2f(w0[q] << 16);
            lo[i][2 * q + 1] = (_Float16)u2f(w0[q] & 0xFFFF0000u);
            hi[i][2 * q] = (_Float16)u2f(w1[q] << 16);
            hi[i][2 * q + 1] = (_Float16)u2f(w1[q] & 0xFFFF0000u);
          }
        } else {
          const u32x4 z = {0u, 0u, 0u, 0u};
          const u32x4 w = ok ? raw.w[i][0] : z;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x2 x = __builtin_amdgcn_cvt_pk_f32_fp8(w[q], false);
            const f32x2 y = __builtin_amdgcn_cvt_pk_f32_fp8(w[q], true);
            f16x8& dst = q < 2 ? lo[i] : hi[i];
            const int o = (q & 1) * 4;
            dst[o + 0] = (_Float16)(x[0] * sc);
            dst[o + 1] = (_Float16)(x[1] * sc);
            dst[o + 2] = (_Float16)(y[0] * sc);
            dst[o + 3] = (_Float16)(y[1] * sc);
          }
        }
        *reinterpret_cast<f16x8*>(&k_s[(4 * q4 + i) * KSTR + 16 * c16]) = lo[i];
        *reinterpret_cast<f16x8*>(&k_s[(4 * q4 + i) * KSTR + 16 * c16 + 8]) = hi[i];
      }
    }
    __syncthreads();
    // ---- next tile's gather is in flight while this tile is computed
    raw.gather(rowptr_s, lr0 + kTileRows + 4 * q4, tr0 + kTileRows < r1, c16e, safe);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of this tile's compute

    // ---- S^T = K . Q~^T for the two 16-row halves
    f32x4 sacc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sacc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        const f16x8 kf = *reinterpret_cast<const f16x8*>(&k_s[(16 * h + col) * KSTR + 32 * t + 8 * g]);
        sacc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[t], sacc[h], 0, 0, 0);
      }
    }
    // lane: rows 16h + 4g + i, head `head`
    float x[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lr = lr0 + 16 * h + 4 * g + i;
        const float v = (tr0 + 16 * h + 4 * g + i < r1 && rowptr_s[lr] != 0) ? sacc[h][i] * a.scale : -INFINITY;
        x[4 * h + i] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const bool need = tmax > m_run + kRescaleSlack;
    if (__any(need)) {
      const float m_new = need ? tmax : m_run;
      const float alpha = need ? expf(m_run - m_new) : 1.0f;  // exp(-inf) = 0 on the first tile
      l_run *= alpha;
      m_run = m_new;
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i, 64);  // lanes 0..15 hold heads 0..15
#pragma unroll
      for (int n = 0; n < NT; ++n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[n][i] *= al[i];
      }
    }
    f16x8 pf;
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = x[j] == -INFINITY ? 0.0f : expf(x[j] - m_run);
      psum += p;
      pf[j] = (_Float16)p;
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run += psum;

    // ---- O += P . V  (V operand: two transposing LDS reads of 4 rows each)
    const _Float16* vbase0 = &k_s[(4 * g + (col >> 2)) * KSTR + 4 * (col & 3)];
    const _Float16* vbase1 = vbase0 + 16 * KSTR;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const s4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(vbase0 + 16 * n));
      const s4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(vbase1 + 16 * n));
      const u32x4 vv = {__builtin_bit_cast(u32x2, v0)[0], __builtin_bit_cast(u32x2, v0)[1],
                        __builtin_bit_cast(u32x2, v1)[0], __builtin_bit_cast(u32x2, v1)[1]};
      oacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf, __builtin_bit_cast(f16x8, vv), oacc[n], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- partials: o (unnormalized, relative to m_run), m, l
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = hb * kHeadsPerBlock + wave * 16 + 4 * g + i;
    if (h < H) {
      float* dst = opart + (part + h) * D + col;
#pragma unroll
      for (int n = 0; n < NT; ++n) dst[16 * n] = oacc[n][i];
    }
  }
  if (g == 0 && head < H) ml[part + head] = make_float2(m_run, l_run);
}

// merge the splits of one (sequence, head) in split order, then inverse RoPE at L-1
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int H = a.H;
  const int L = clampi(a.lens[b], 0, a.max_len);
  const int N = (L + a.m - 1) / a.m;
  const int n_sel = a.sel ? clampi(a.sel_n[b], 0, a.k) : N;
  const int rows_b = n_sel + min(a.window, L);
  const int S = min(a.plan.splits, (rows_b + a.plan.rows_per_split - 1) / a.plan.rows_per_split);
  const float2* ml = reinterpret_cast<const float2*>(a.ws + a.plan.ml_off);
  const float* opart = reinterpret_cast<const float*>(a.ws + a.plan.o_off);
  __shared__ float w_s[kMaxSplits];
  __shared__ float red_s[256];
  // split weights exp(m_s - M): max and sum over splits, in split order
  float mloc = -INFINITY;
  for (int s = threadIdx.x; s < S; s += 256) mloc = fmaxf(mloc, ml[((size_t)b * a.plan.splits + s) * H + h].x);
  red_s[threadIdx.x] = mloc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red_s[threadIdx.x] = fmaxf(red_s[threadIdx.x], red_s[threadIdx.x + o]);
    __syncthreads();
  }
  const float M = red_s[0];
  __syncthreads();
  float* out = a.out + ((int64_t)b * H + h) * D;
  if (M == -INFINITY) {
    for (int c = threadIdx.x; c < D; c += 256) out[c] = 0.0f;
    if (threadIdx.x == 0 && a.lse) a.lse[(int64_t)b * H + h] = -INFINITY;
    return;
  }
  for (int s = threadIdx.x; s < S; s += 256) {
    const float2 v = ml[((size_t)b * a.plan.splits + s) * H + h];
    w_s[s] = v.y > 0.0f ? expf(v.x - M) : 0.0f;
  }
  __syncthreads();
  float tot = 0.0f;
  for (int s = 0; s < S; ++s) tot += w_s[s] * ml[((size_t)b * a.plan.splits + s) * H + h].y;
  const float inv_tot = 1.0f / tot;
  for (int pi = threadIdx.x; pi < D / 2; pi += 256) {
    float o0 = 0.0f, o1 = 0.0f;
    int s = 0;
    constexpr int U = 8;  // split partials loaded per round
    for (; s + U <= S; s += U) {
      float2 o[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        o[u] = *reinterpret_cast<const float2*>(opart + (((size_t)b * a.plan.splits + s + u) * H + h) * D + 2 * pi);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float w = w_s[s + u];
        o0 = fmaf(w, o[u].x, o0);
        o1 = fmaf(w, o[u].y, o1);
      }
    }
    for (; s < S; ++s) {
      const float w = w_s[s];
      if (w > 0.0f) {
        const float2 o = *reinterpret_cast<const float2*>(opart + (((size_t)b * a.plan.splits + s) * H + h) * D + 2 * pi);
        o0 = fmaf(w, o.x, o0);
        o1 = fmaf(w, o.y, o1);
      }
    }
    o0 *= inv_tot;
    o1 *= inv_tot;
    float c, sn;
    rope_cs((double)(L - 1), rope_inv_freq(pi, D, a.theta), c, sn);
    out[2 * pi] = o0 * c + o1 * sn;       // rotation by -angle
    out[2 * pi + 1] = -o0 * sn + o1 * c;
  }
  if (threadIdx.x == 0 && a.lse) a.lse[(int64_t)b * H + h] = M + logf(tot);
}

template <int D>
static hipError_t launch_attn_d(const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.plan.splits, a.B, a.plan.head_blocks);
  if (a.kv.dtype == HCA_FP8_E4M3)
    hipLaunchKernelGGL((attn_split_kernel<D, HCA_FP8_E4M3>), grid, dim3(kAttnThreads), 0, s, a);
  else
    hipLaunchKernelGGL((attn_split_kernel<D, HCA_BF16>), grid, dim3(kAttnThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel<D>, dim3(a.H, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  switch (a.kv.dim) {
    case 64: return launch_attn_d<64>(a, s);
    case 128: return launch_attn_d<128>(a, s);
    case 256: return launch_attn_d<256>(a, s);
    default: return launch_attn_d<512>(a, s);
  }
}

}  // namespace hca
