// kv_compress: softmax-weighted fold of m consecutive tokens into one shared
// K=V entry, rotated at the position of the group's first token
// (V4 page, section 2.1 compressor; section 3.1.2 rolling residual;
// section 3.2.1 RoPE before cache insertion).
//
// Overlapping windows (section 2.1 folds every 8 tokens into one c4a entry at
// a ratio of 1/4; section 3.1.2 keeps an 8-token state): with an overlap o,
// entry j also folds the o tokens before its group, read at negative rows
// relative to the run's first token (small groups only).
//
// HBM-bound stream: each thread owns 8 consecutive dims (one 16-byte bf16
// load per token) so a row of d dims is read by d/8 adjacent lanes in one
// coalesced sweep.  Small m: a row-group of d/8 threads folds whole entries on
// its own.  Large m: the 256 threads of a block share one entry, each
// row-group folding a strided subset of its tokens (a batch's loads all in
// flight before the first is summed), reduced through LDS.
//
// With a gain vector the folded entry is RMS-normalised before it is rotated
// (section 3.2.1 lists compressor, RMSNorm, RoPE and insertion as one fused
// step): the sum of squares of a row is reduced across the threads that hold
// it in a fixed order, so every thread of the row scales by the same factor
// and a fold gives the same bits wherever it runs.
#include "hca_common.h"
#include "hca_internal.h"
#include "indexer_internal.h"
#include "indexer_select.h"

namespace hca {


__device__ __forceinline__ void load_bf16x8(const uint16_t* p, float v[8]) {
  const u32x4 raw = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = u2f(raw[i] << 16);
    v[2 * i + 1] = u2f(raw[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ void rope_store8(float* dst, float* lds, const float acc[8], double pos, const double inv[4]) {
  float o[8];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float c, s;
    rope_cs(pos, inv[p], c, s);
    o[2 * p] = acc[2 * p] * c - acc[2 * p + 1] * s;
    o[2 * p + 1] = acc[2 * p] * s + acc[2 * p + 1] * c;
  }
  f32x4* d4 = reinterpret_cast<f32x4*>(dst);
  d4[0] = f32x4{o[0], o[1], o[2], o[3]};
  d4[1] = f32x4{o[4], o[5], o[6], o[7]};
  if (lds != nullptr) {
    f32x4* l4 = reinterpret_cast<f32x4*>(lds);
    l4[0] = f32x4{o[0], o[1], o[2], o[3]};
    l4[1] = f32x4{o[4], o[5], o[6], o[7]};
  }
}

// Entry j of a small-m fold, the 8 dims of this thread: softmax over the
// window's available slots, weighted sum (normalised, not yet rotated).  The
// window is the group's m tokens and, with an overlap o, the o tokens before
// it (rows -o .. -1 relative to the group); slots at positions below 0 or at
// or past the n tokens of the run are absent.
//
// Every load of a batch is issued before any of it is used, and the sums run
// in slot order.  The first batch's token rows and logits are loaded, then
// `mid()` runs (the insert issues its page loads there: they stay in flight
// while the fold computes, since its own loads were issued first), then the
// window of up to 2 * kSmallM slots is folded.
__device__ __forceinline__ void fold_batch(int ns, float mx, int k0, const u32x4 raw[], const float av[], float acc[8],
                                           float& tot) {
  constexpr int kFoldBatch = 8;
#pragma unroll
  for (int k = 0; k < kFoldBatch; ++k) {
    if (k0 + k < ns) {
      const float e = expf(av[k] - mx);
      tot += e;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(e, u2f(raw[k][q] << 16), acc[2 * q]);
        acc[2 * q + 1] = fmaf(e, u2f(raw[k][q] & 0xFFFF0000u), acc[2 * q + 1]);
      }
    }
  }
}

// The loads of one wave-form fold (its slots' logits and biases, and the
// first batch of its rows), kept apart from its arithmetic: all of them are
// issued before the first is used, and a caller's own work (mid) goes
// between the two.
struct FoldWaveIn {
  static constexpr int kBatch = 8;
  int t0, lo, ns;
  bool on;
  float zl, bl;
  u32x4 raw[kBatch];
};
__device__ __forceinline__ void small_fold_wave_load(const CompressArgs& a, const float* zb, const uint16_t* xb, int j,
                                                     int n, int p0, bool live, FoldWaveIn& f) {
  const int lane = threadIdx.x & 63;
  // uniform over the wave (its one row group): read from the first lane, so
  // that the slot tests below are scalar branches, not lane masks
  f.t0 = __builtin_amdgcn_readfirstlane(j * a.m - a.ov);
  f.lo = max(0, -(p0 + f.t0));
  f.ns = __builtin_amdgcn_readfirstlane(live ? min(a.m + a.ov, n - f.t0) - f.lo : 0);
  f.on = lane < f.ns;
  f.zl = f.on ? zb[f.t0 + f.lo + lane] : 0.0f;
  f.bl = f.on ? a.beta[f.lo + lane] : 0.0f;
  // the first batch's rows, loaded without per-slot tests: a slot past the
  // present ones re-reads the last present row (it is not added)
  if (f.ns > 0) {
#pragma unroll
    for (int k = 0; k < FoldWaveIn::kBatch; ++k)
      f.raw[k] = *reinterpret_cast<const u32x4*>(xb + (int64_t)(f.t0 + f.lo + min(k, f.ns - 1)) * a.d);
  } else {
#pragma unroll
    for (int k = 0; k < FoldWaveIn::kBatch; ++k) f.raw[k] = u32x4{0u, 0u, 0u, 0u};
  }
}
__device__ __forceinline__ void small_fold_wave_compute(const CompressArgs& a, const uint16_t* xb, FoldWaveIn& f,
                                                        float acc[8]) {
  constexpr int kFoldBatch = FoldWaveIn::kBatch;
  constexpr int kMaxSlots = 2 * kSmallM;
  const int ns = f.ns;
  const float av = f.on ? f.zl + f.bl : -INFINITY;
  // the slots' maximum: a max scan by DPP row shifts inside each 16-lane row,
  // then the last lanes of rows 0 and 1 (slots 0 .. 31)
  float mx = av;
#define HCA_DPP_MAX(CTRL) \
  mx = fmaxf(mx, u2f((uint32_t)__builtin_amdgcn_update_dpp((int)f2u(-INFINITY), (int)f2u(mx), CTRL, 0xF, 0xF, false)))
  HCA_DPP_MAX(0x111);  // row_shr:1
  HCA_DPP_MAX(0x112);  // row_shr:2
  HCA_DPP_MAX(0x114);  // row_shr:4
  HCA_DPP_MAX(0x118);  // row_shr:8
#undef HCA_DPP_MAX
  static_assert(kMaxSlots <= 32, "slots in lane rows 0 and 1");
  mx = fmaxf(u2f((uint32_t)__builtin_amdgcn_readlane((int)f2u(mx), 15)),
             u2f((uint32_t)__builtin_amdgcn_readlane((int)f2u(mx), 31)));
  const float e = f.on ? expf(av - mx) : 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
  float tot = 0.0f;
  for (int k0 = 0; k0 < ns; k0 += kFoldBatch) {
    if (k0 > 0) {
#pragma unroll
      for (int k = 0; k < kFoldBatch; ++k)
        f.raw[k] = k0 + k < ns ? *reinterpret_cast<const u32x4*>(xb + (int64_t)(f.t0 + f.lo + k0 + k) * a.d)
                               : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kFoldBatch; ++k) {
      if (k0 + k < ns) {
        const float ek = u2f((uint32_t)__builtin_amdgcn_readlane((int)f2u(e), k0 + k));  // slot k0 + k's weight
        tot += ek;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = fmaf(ek, u2f(f.raw[k][q] << 16), acc[2 * q]);
          acc[2 * q + 1] = fmaf(ek, u2f(f.raw[k][q] & 0xFFFF0000u), acc[2 * q + 1]);
        }
      }
    }
  }
  const float inv_tot = tot > 0.0f ? 1.0f / tot : 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] *= inv_tot;
}

// The same fold when a row group is exactly one wave (d = 512: 64 threads of
// 8 dims, and row groups start at wave boundaries), so every slot's weight is
// uniform over the wave: lane k loads slot k's logit and bias and computes its
// weight once, and the weights reach the other lanes by lane reads, in slot
// order.  The arithmetic is the row group fold's, value for value (the same
// maximum, the same expf of the same arguments, the same sums in the same
// order): the codes it leads to are identical.
template <typename Mid>
__device__ __forceinline__ void small_fold_wave(const CompressArgs& a, const float* zb, const uint16_t* xb, int j,
                                                int n, int p0, bool live, float acc[8], Mid&& mid) {
  FoldWaveIn f;
  small_fold_wave_load(a, zb, xb, j, n, p0, live, f);
  mid();
  small_fold_wave_compute(a, xb, f, acc);
}

template <typename Mid>
__device__ __forceinline__ void small_fold(const CompressArgs& a, const float* zb, const uint16_t* xb, int j, int n,
                                           int p0, bool live, float acc[8], Mid&& mid) {
  if (a.d == 512) {  // uniform
    small_fold_wave(a, zb, xb, j, n, p0, live, acc, mid);
    return;
  }
  constexpr int kFoldBatch = 8;
  constexpr int kMaxSlots = 2 * kSmallM;        // m + overlap, overlap <= m <= kSmallM
  const int t0 = j * a.m - a.ov;                // row of the window's first slot
  const int lo = max(0, -(p0 + t0));            // first slot at a position >= 0
  const int ns = live ? min(a.m + a.ov, n - t0) - lo : 0;  // slots present
  u32x4 raw[kFoldBatch];
  float zv[kFoldBatch], bv[kFoldBatch];
#pragma unroll
  for (int k = 0; k < kFoldBatch; ++k) {
    const bool on = k < ns;
    raw[k] = on ? *reinterpret_cast<const u32x4*>(xb + (int64_t)(t0 + lo + k) * a.d) : u32x4{0u, 0u, 0u, 0u};
    zv[k] = on ? zb[t0 + lo + k] : 0.0f;
    bv[k] = on ? a.beta[lo + k] : 0.0f;
  }
  mid();
  float av[kFoldBatch];
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < kFoldBatch; ++k) {
    av[k] = zv[k] + bv[k];
    if (k < ns) mx = fmaxf(mx, av[k]);
  }
#pragma unroll
  for (int k = kFoldBatch; k < kMaxSlots; ++k)
    if (k < ns) mx = fmaxf(mx, zb[t0 + lo + k] + a.beta[lo + k]);
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
  float tot = 0.0f;
  fold_batch(ns, mx, 0, raw, av, acc, tot);
#pragma unroll
  for (int k0 = kFoldBatch; k0 < kMaxSlots; k0 += kFoldBatch) {
    if (k0 < ns) {
#pragma unroll
      for (int k = 0; k < kFoldBatch; ++k) {
        const bool on = k0 + k < ns;
        raw[k] = on ? *reinterpret_cast<const u32x4*>(xb + (int64_t)(t0 + lo + k0 + k) * a.d) : u32x4{0u, 0u, 0u, 0u};
        av[k] = on ? zb[t0 + lo + k0 + k] + a.beta[lo + k0 + k] : 0.0f;
      }
      fold_batch(ns, mx, k0, raw, av, acc, tot);
    }
  }
  const float inv_tot = tot > 0.0f ? 1.0f / tot : 0.0f;  // no slot: a negative pos0
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] *= inv_tot;
}

// An xor butterfly over aligned groups of TD lanes (TD a power of two <= 64):
// every lane of a group gets the same sum (each step adds two equal partial
// sums in either order), by lane permutations on the VALU: DPP quad
// permutations for the partners l^1 and l^2; then, the quads holding equal
// values, the half-row mirror (l to 7 - l, a lane of the other quad) adds what
// l^4 would, and the row mirror what l^8 would; the permlane swaps give l^16
// and l^32.
__device__ __forceinline__ float lanes_sum_pow2(float v, int TD) {
#define HCA_DPP_ADD(CTRL) v += u2f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f2u(v), CTRL, 0xF, 0xF, false))
  if (TD > 1) HCA_DPP_ADD(0xB1);    // quad_perm [1, 0, 3, 2]
  if (TD > 2) HCA_DPP_ADD(0x4E);    // quad_perm [2, 3, 0, 1]
  if (TD > 4) HCA_DPP_ADD(0x141);   // row_half_mirror
  if (TD > 8) HCA_DPP_ADD(0x140);   // row_mirror
#undef HCA_DPP_ADD
  if (TD > 16) {
    const auto p16 = __builtin_amdgcn_permlane16_swap(f2u(v), f2u(v), false, false);
    v = u2f(p16[0]) + u2f(p16[1]);
  }
  if (TD > 32) {
    const auto p32 = __builtin_amdgcn_permlane32_swap(f2u(v), f2u(v), false, false);
    v = u2f(p32[0]) + u2f(p32[1]);
  }
  return v;
}

// Sum of v over the TD consecutive threads of row group gi (TD = threads per
// row, RP full groups in the block), the same value in every thread of the
// group.  Called by every thread of the block (it may synchronize it).
__device__ __forceinline__ float row_group_sum(float v, int TD, int RP, int gi, float* sq_s) {
  if ((TD & (TD - 1)) == 0 && TD <= 64) return lanes_sum_pow2(v, TD);
  if ((TD & (TD - 1)) == 0) {
    // an xor butterfly inside each wave, then the waves' sums in order
    v = lanes_sum_pow2(v, 64);
    if ((threadIdx.x & 63) == 0) sq_s[threadIdx.x >> 6] = v;
    __syncthreads();
    const int nw = TD >> 6;
    float t = 0.0f;
    for (int k = 0; k < nw; ++k) t += sq_s[gi * nw + k];
    __syncthreads();
    return t;
  }
  sq_s[threadIdx.x] = v;
  __syncthreads();
  float t = 0.0f;
  if (gi < RP)
    for (int k = 0; k < TD; ++k) t += sq_s[gi * TD + k];
  __syncthreads();
  return t;
}

// The fold of sequence b by one block of kCompressThreads threads, as block bx
// of gx blocks over the sequence's work.  With a non-null `lds_row` (a fold of
// a single entry) the entry is also left in that shared array.  The dynamic
// shared memory of the launch holds kCompressShm bytes.  PATHS selects the
// code compiled in: 1 small groups only, 2 large groups only, 3 both (a
// kernel holding only what its groups need keeps its register count down).
//
// n and p0 are sequence b's token count (clamped) and first position; `mid()`
// is called by every thread once per round of entries, after the round's
// first loads are issued (a no-op for a plain fold).
struct NoMid {
  __device__ void operator()() const {}
};

// A large-m fold may also keep every entry it folds in shared memory:
// lds_stride > 0 puts entry j at lds_row + (j - lds_j0) * lds_stride (the
// fused prefill's page); a null a.out then skips the global write.
template <int PATHS = 3, typename Mid = NoMid>
__device__ __forceinline__ void compress_block(const CompressArgs& a, int b, int bx, int gx, float* lds_row, int n,
                                               int p0, Mid&& mid, float* state_out = nullptr, int lds_j0 = 0,
                                               int lds_stride = 0) {
  const int TD = a.d >> 3;              // threads across the dims of a row
  const int RP = kCompressThreads / TD; // row groups
  const int li = threadIdx.x % TD;
  const int gi = threadIdx.x / TD;
  const bool active = gi < RP;
  const int m = a.m;
  const int N = (n + m - 1) / m;
  const uint16_t* xb = a.x + (int64_t)b * a.xs + li * 8;
  const float* zb = a.z + (int64_t)b * a.zs;
  float* ob = a.out + (int64_t)b * a.os + li * 8;

  const bool small = (PATHS & 1) && (!(PATHS & 2) || m <= kSmallM);
  // the gains are loaded first, so their latency hides behind the fold: a
  // small-m thread holds its 8 dims, a large-m thread its dim pairs
  // t = threadIdx.x + kCompressThreads * k (d <= 2048: at most 4)
  constexpr int kGainPairs = 4;
  float gam[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float2 gpair[kGainPairs];
#pragma unroll
  for (int k = 0; k < kGainPairs; ++k) gpair[k] = make_float2(0.0f, 0.0f);
  if (a.gamma != nullptr) {
    if (small) {
      if (active) {
        const f32x4* g4 = reinterpret_cast<const f32x4*>(a.gamma + li * 8);
        const f32x4 g0 = g4[0], g1 = g4[1];
#pragma unroll
        for (int c = 0; c < 4; ++c) { gam[c] = g0[c]; gam[4 + c] = g1[c]; }
      }
    } else {
#pragma unroll
      for (int k = 0; k < kGainPairs; ++k) {
        const int t = threadIdx.x + kCompressThreads * k;
        if (t < a.d / 2) gpair[k] = reinterpret_cast<const float2*>(a.gamma)[t];
      }
    }
  }

  double inv[4];
  rope_inv_freq4(li, a.rope_r, inv);

  if (small) {
    // every thread runs every round (mid() and the row sum of the
    // normalisation are block-wide)
    __shared__ float sq_s[kCompressThreads];
    for (int j0 = bx * RP; j0 < N; j0 += gx * RP) {
      const int j = j0 + gi;
      const bool live = active && j < N;
      float acc[8];
      small_fold(a, zb, xb, j, n, p0, live, acc, mid);
      if (a.gamma == nullptr) {
        if (live)
          rope_store8(ob + (int64_t)j * a.d, lds_row ? lds_row + li * 8 : nullptr, acc, (double)p0 + (double)(j * m),
                      inv);
        continue;
      }
      float ss = 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) ss = fmaf(acc[c], acc[c], ss);
      const float rs = 1.0f / sqrtf(row_group_sum(ss, TD, RP, gi, sq_s) / (float)a.d + a.eps);
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = acc[c] * rs * gam[c];
      if (live)
        rope_store8(ob + (int64_t)j * a.d, lds_row ? lds_row + li * 8 : nullptr, acc, (double)p0 + (double)(j * m), inv);
    }
    return;
  }

  // large m: a block folds one entry at a time; its row groups take strided
  // subsets of the group's tokens and are summed through LDS
  const int DS = a.d;                  // dims of a row (a multiple of 8, <= 2048)
  const int TS = DS >> 3;              // threads across the row
  const int RS = kCompressThreads / TS;
  const int ls = threadIdx.x % TS;
  const int gs = threadIdx.x / TS;
  __shared__ float w_s[256];
  __shared__ float red_s[kCompressThreads];
  extern __shared__ float acc_s[];     // [RS][DS]
  const uint16_t* xs = a.x + (int64_t)b * a.xs + ls * 8;
  for (int j = bx; j < N; j += gx) {
    const int t0 = j * m;
    const int r = min(m, n - t0);
    // the row group's first batch of token rows is in flight while the
    // softmax weights of the group's r slots are reduced (wave reductions,
    // then the four wave partials in a fixed order)
    constexpr int kBatch = 16;
    u32x4 raw[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int i = gs + k * RS;
      raw[k] = gs < RS && i < r ? *reinterpret_cast<const u32x4*>(xs + (int64_t)(t0 + i) * a.d)
                                : u32x4{0u, 0u, 0u, 0u};
    }
    const float zi = (int)threadIdx.x < r ? zb[t0 + threadIdx.x] : 0.0f;
    const float bi = (int)threadIdx.x < r ? a.beta[threadIdx.x] : 0.0f;
    mid();
    const float a_i = (int)threadIdx.x < r ? zi + bi : -INFINITY;
    const float wm = wave_max(a_i);
    if ((threadIdx.x & 63) == 0) red_s[threadIdx.x >> 6] = wm;
    __syncthreads();
    const float mx = fmaxf(fmaxf(red_s[0], red_s[1]), fmaxf(red_s[2], red_s[3]));
    const float e = threadIdx.x < r ? expf(a_i - mx) : 0.0f;
    w_s[threadIdx.x] = e;
    const float ws = wave_sum(e);
    if ((threadIdx.x & 63) == 0) red_s[4 + (threadIdx.x >> 6)] = ws;
    __syncthreads();
    const float tot = (red_s[4] + red_s[5]) + (red_s[6] + red_s[7]);
    if (gs < RS) {
      // the row group's tokens i = gs, gs + RS, ..., in batches whose loads
      // are all in flight before the first is summed (same order of sums)
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int i0 = gs; i0 < r; i0 += kBatch * RS) {
        if (i0 != gs) {
#pragma unroll
          for (int k = 0; k < kBatch; ++k) {
            const int i = i0 + k * RS;
            raw[k] = i < r ? *reinterpret_cast<const u32x4*>(xs + (int64_t)(t0 + i) * a.d)
                           : u32x4{0u, 0u, 0u, 0u};
          }
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int i = i0 + k * RS;
          if (i < r) {
            const float wi = w_s[i];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              acc[2 * q] = fmaf(wi, u2f(raw[k][q] << 16), acc[2 * q]);
              acc[2 * q + 1] = fmaf(wi, u2f(raw[k][q] & 0xFFFF0000u), acc[2 * q + 1]);
            }
          }
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) acc_s[gs * DS + ls * 8 + c] = acc[c];
    }
    __syncthreads();
    // one thread per dim pair of the slice: sum the row groups (the fold's
    // weighted sums, which a fold state keeps as they are), normalise, rotate.
    // A pair's normalised values are left in row group 0 of acc_s: each
    // thread reads and writes only its own pairs' columns.
    const float inv_tot = 1.0f / tot;
    const double pos = (double)p0 + (double)t0;
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < kGainPairs; ++k) {
      const int t = threadIdx.x + kCompressThreads * k;
      if (t >= DS / 2) break;
      float e0 = 0.0f, e1 = 0.0f;
      for (int g = 0; g < RS; ++g) {
        e0 += acc_s[g * DS + 2 * t];
        e1 += acc_s[g * DS + 2 * t + 1];
      }
      if (state_out != nullptr) {
        state_out[kFoldStateHead + 2 * t] = e0;
        state_out[kFoldStateHead + 2 * t + 1] = e1;
      }
      e0 *= inv_tot;
      e1 *= inv_tot;
      acc_s[2 * t] = e0;
      acc_s[2 * t + 1] = e1;
      ss = fmaf(e0, e0, ss);
      ss = fmaf(e1, e1, ss);
    }
    if (state_out != nullptr && threadIdx.x == 0) {
      state_out[0] = (float)r;
      state_out[1] = mx;
      state_out[2] = tot;
    }
    float rs = 1.0f;
    if (a.gamma != nullptr) {  // the entry's sum of squares
      ss = wave_sum(ss);
      if ((threadIdx.x & 63) == 0) red_s[threadIdx.x >> 6] = ss;
      __syncthreads();
      ss = (red_s[0] + red_s[1]) + (red_s[2] + red_s[3]);
      rs = 1.0f / sqrtf(ss / (float)a.d + a.eps);
    }
#pragma unroll
    for (int k = 0; k < kGainPairs; ++k) {
      const int t = threadIdx.x + kCompressThreads * k;
      if (t >= DS / 2) break;
      float e0 = acc_s[2 * t], e1 = acc_s[2 * t + 1];
      if (a.gamma != nullptr) {
        e0 *= rs * gpair[k].x;
        e1 *= rs * gpair[k].y;
      }
      float c, sn;
      rope_cs(pos, rope_inv_freq(t, a.rope_r), c, sn);
      const float o0 = e0 * c - e1 * sn, o1 = e0 * sn + e1 * c;
      if (a.out != nullptr) {
        float* o = a.out + (int64_t)b * a.os + (int64_t)j * a.d + 2 * t;
        o[0] = o0;
        o[1] = o1;
      }
      if (lds_row != nullptr) {
        float* l = lds_row + (int64_t)(j - lds_j0) * lds_stride;
        l[2 * t] = o0;
        l[2 * t + 1] = o1;
      }
    }
    __syncthreads();
  }
}

template <int PATHS>
__global__ __launch_bounds__(kCompressThreads) void compress_kernel(CompressArgs a) {
  const int b = blockIdx.y;
  compress_block<PATHS>(a, b, blockIdx.x, gridDim.x, nullptr, clampi(a.ntok[b], 0, a.max_ntok), a.pos0[b], NoMid{});
}


hipError_t launch_compress(CompressArgs a, hipStream_t s) {
  const int n_max = (a.max_ntok + a.m - 1) / a.m;
  if (a.B == 0 || n_max == 0) return hipSuccess;
  int gx;
  size_t shm = 0;
  a.rope_r = pow((double)a.theta, -2.0 / (double)a.d);
  if (a.m <= kSmallM) {
    const int RP = kCompressThreads / (a.d / 8);
    gx = (n_max + RP - 1) / RP;
    gx = gx > 2048 ? 2048 : gx;
  } else {
    gx = n_max > 4096 ? 4096 : n_max;
    shm = kCompressShm;
  }
  if (a.m <= kSmallM)
    hipLaunchKernelGGL(compress_kernel<1>, dim3(gx, a.B), dim3(kCompressThreads), shm, s, a);
  else
    hipLaunchKernelGGL(compress_kernel<2>, dim3(gx, a.B), dim3(kCompressThreads), shm, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------- fused prefill
// kv_prefill_pages: compressor + RMSNorm + RoPE + insertion of a whole run in
// one launch (V4 page, section 3.2.1 lists them as one fused step; sections
// 3.1.1 and 3.1.3: the page formats), one block per page: the block folds the
// page's entries exactly as kv_compress folds them (the same per-entry
// arithmetic in the same order), keeps them on chip, takes the page's amax and
// writes its codes and scale exactly as kv_quantize_page does.  The fp32
// entries never reach HBM.
//
// Small groups: a block of kPrefillThreads threads, row groups of d/8 threads
// folding one entry each per round, the rotated rows held in registers (at
// most kPrefillRounds rounds).  Large groups: a block of kCompressThreads
// threads folds the page's entries one after the other (compress_block's
// large path, so the same sums) into shared memory.
constexpr int kPrefillThreads = 1024;
constexpr int kPrefillRounds = 4;
constexpr int kPrefill512Threads = 512;  // 8 waves: two blocks share a CU
constexpr int kPrefill512Rounds = 8;

// four fp8 codes of x / s (an fp8 page's encoding), packed little-endian
__device__ __forceinline__ uint32_t enc4_e4m3(const f32x4 v, float s) { return e4m3_encode4_div(v[0], v[1], v[2], v[3], s); }

__device__ __forceinline__ void rope8(const float acc[8], double pos, const double inv[4], float o[8]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float c, s;
    rope_cs(pos, inv[p], c, s);
    o[2 * p] = acc[2 * p] * c - acc[2 * p + 1] * s;
    o[2 * p + 1] = acc[2 * p] * s + acc[2 * p + 1] * c;
  }
}

__device__ __forceinline__ float block_max_n(float v, float* red, int nwaves) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < nwaves; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

// the page of block (pg, b): its physical page and valid rows, or -1
__device__ __forceinline__ int prefill_page(const PrefillArgs& p, int b, int pg, int n, int p0, int& rows) {
  const int m = p.c.m, epp = p.dst.epp;
  const int N = (n + m - 1) / m;
  rows = min(epp, N - pg * epp);
  if (rows <= 0) return -1;
  const int lb = p0 / m / epp + pg;
  HCA_DBG_CHECK(lb >= 0 && lb < p.bts, kDbgTable);
  if (lb < 0 || lb >= p.bts) return -1;
  const int phys = p.bt[(int64_t)b * p.bts + lb];
  HCA_DBG_CHECK(phys >= 0 && phys < p.dst.num_pages, kDbgPage);
  return phys >= 0 && phys < p.dst.num_pages ? phys : -1;
}

// The same kernel specialized for 512-dim rows (the c4a pages): one row group
// per wave, the fold's wave form called directly, the rounds unrolled (their
// rows then sit in a register array with constant indices).  Eight waves and
// eight rounds per page rather than sixteen and four: at 125 registers two
// such blocks share a CU, so one block's folds (load-bound) overlap the
// other's page maximum and encode (a barrier, then VALU work).
__global__ __launch_bounds__(kPrefill512Threads) void prefill_small512_kernel(PrefillArgs p) {
  const CompressArgs& a = p.c;
  const int b = blockIdx.y, pg = blockIdx.x;
  const int n = clampi(a.ntok[b], 0, a.max_ntok);
  const int p0 = a.pos0[b];
  int rows;
  const int phys = prefill_page(p, b, pg, n, p0, rows);
  if (phys < 0) return;  // uniform over the block
  constexpr int d = 512, TD = 64, RP = kPrefill512Threads / TD;
  const int m = a.m, epp = p.dst.epp;
  const int li = threadIdx.x % TD, gi = __builtin_amdgcn_readfirstlane(threadIdx.x / TD);
  const uint16_t* xb = a.x + (int64_t)b * a.xs + li * 8;
  const float* zb = a.z + (int64_t)b * a.zs;
  float gam[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (a.gamma != nullptr) {
    const f32x4* g4 = reinterpret_cast<const f32x4*>(a.gamma + li * 8);
    const f32x4 g0 = g4[0], g1 = g4[1];
#pragma unroll
    for (int c = 0; c < 4; ++c) { gam[c] = g0[c]; gam[4 + c] = g1[c]; }
  }
  double inv[4];
  rope_inv_freq4(li, a.rope_r, inv);
  __shared__ float sq_s[kPrefill512Threads];
  __shared__ float red_s[kPrefill512Threads / 64];
  float v[kPrefill512Rounds][8];
  float amax = 0.0f;
#pragma unroll
  for (int r = 0; r < kPrefill512Rounds; ++r) {
#pragma unroll
    for (int c = 0; c < 8; ++c) v[r][c] = 0.0f;
    if (r * RP >= epp) continue;  // uniform
    const int row = r * RP + gi;
    const int j = pg * epp + row;
    const bool live = row < rows;
    float acc[8];
    small_fold_wave(a, zb, xb, j, n, p0, live, acc, NoMid{});
    if (a.gamma != nullptr) {
      float ss = 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) ss = fmaf(acc[c], acc[c], ss);
      const float rs = 1.0f / sqrtf(row_group_sum(ss, TD, RP, gi, sq_s) / (float)d + a.eps);
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = acc[c] * rs * gam[c];
    }
    if (live) {
      rope8(acc, (double)p0 + (double)(j * m), inv, v[r]);
#pragma unroll
      for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(v[r][c]));
    }
  }
  if (p.dst.dtype == HCA_FP8_E4M3) {
    amax = block_max_n(amax, red_s, kPrefill512Threads / 64);
    const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    uint8_t* codes = reinterpret_cast<uint8_t*>(p.dst.codes) + (int64_t)phys * epp * d;
#pragma unroll
    for (int r = 0; r < kPrefill512Rounds; ++r) {
      const int row = r * RP + gi;
      if (r * RP >= epp || row >= epp) continue;
      u32x2 w = {0u, 0u};
      if (row < rows) {
        w[0] = enc4_e4m3(f32x4{v[r][0], v[r][1], v[r][2], v[r][3]}, s);
        w[1] = enc4_e4m3(f32x4{v[r][4], v[r][5], v[r][6], v[r][7]}, s);
      }
      *reinterpret_cast<u32x2*>(codes + (int64_t)row * d + li * 8) = w;
    }
    if (threadIdx.x == 0) reinterpret_cast<float*>(p.dst.scales)[phys] = s;
  } else {  // bf16
    uint16_t* codes = reinterpret_cast<uint16_t*>(p.dst.codes) + (int64_t)phys * epp * d;
#pragma unroll
    for (int r = 0; r < kPrefill512Rounds; ++r) {
      const int row = r * RP + gi;
      if (r * RP >= epp || row >= epp) continue;
      u32x4 w = {0u, 0u, 0u, 0u};
      if (row < rows) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = (uint32_t)bf16_encode(v[r][2 * q]) | ((uint32_t)bf16_encode(v[r][2 * q + 1]) << 16);
      }
      *reinterpret_cast<u32x4*>(codes + (int64_t)row * d + li * 8) = w;
    }
  }
}

__global__ __launch_bounds__(kPrefillThreads) void prefill_small_kernel(PrefillArgs p) {
  const CompressArgs& a = p.c;
  const int b = blockIdx.y, pg = blockIdx.x;
  const int n = clampi(a.ntok[b], 0, a.max_ntok);
  const int p0 = a.pos0[b];
  int rows;
  const int phys = prefill_page(p, b, pg, n, p0, rows);
  if (phys < 0) return;  // uniform over the block
  const int m = a.m, d = a.d, epp = p.dst.epp;
  const int TD = d >> 3, RP = kPrefillThreads / TD;
  const int li = threadIdx.x % TD, gi = threadIdx.x / TD;
  const bool active = gi < RP;
  const uint16_t* xb = a.x + (int64_t)b * a.xs + li * 8;
  const float* zb = a.z + (int64_t)b * a.zs;
  float gam[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (a.gamma != nullptr && active) {
    const f32x4* g4 = reinterpret_cast<const f32x4*>(a.gamma + li * 8);
    const f32x4 g0 = g4[0], g1 = g4[1];
#pragma unroll
    for (int c = 0; c < 4; ++c) { gam[c] = g0[c]; gam[4 + c] = g1[c]; }
  }
  double inv[4];
  rope_inv_freq4(li, a.rope_r, inv);
  __shared__ float sq_s[kPrefillThreads];
  __shared__ float red_s[kPrefillThreads / 64];
  // the page's rotated rows stay in registers until the page scale is known:
  // one named vector per round (an array indexed by the round counter would be
  // placed in scratch memory, whose traffic exceeded the pages' own: the round
  // loop is too large to unroll)
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  f32x8 v0 = {}, v1 = {}, v2 = {}, v3 = {};
  static_assert(kPrefillRounds == 4, "one vector per round");
#define HCA_ROW_OF_ROUND(r) ((r) == 0 ? v0 : (r) == 1 ? v1 : (r) == 2 ? v2 : v3)
  float amax = 0.0f;
#pragma nounroll
  for (int r = 0; r < kPrefillRounds; ++r) {
    if (r * RP >= epp) break;  // uniform
    const int row = r * RP + gi;
    const int j = pg * epp + row;
    const bool live = active && row < rows;
    float acc[8];
    small_fold(a, zb, xb, j, n, p0, live, acc, NoMid{});
    if (a.gamma != nullptr) {
      float ss = 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) ss = fmaf(acc[c], acc[c], ss);
      const float rs = 1.0f / sqrtf(row_group_sum(ss, TD, RP, gi, sq_s) / (float)d + a.eps);
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = acc[c] * rs * gam[c];
    }
    if (live) {
      float o[8];
      rope8(acc, (double)p0 + (double)(j * m), inv, o);
#pragma unroll
      for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(o[c]));
      const f32x8 ov = {o[0], o[1], o[2], o[3], o[4], o[5], o[6], o[7]};
      switch (r) {  // uniform
        case 0: v0 = ov; break;
        case 1: v1 = ov; break;
        case 2: v2 = ov; break;
        default: v3 = ov; break;
      }
    }
  }
  // the page: codes of the valid rows, zeros past them, and the scale
  if (p.dst.dtype == HCA_FP8_E4M3) {
    amax = block_max_n(amax, red_s, kPrefillThreads / 64);
    const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    uint8_t* codes = reinterpret_cast<uint8_t*>(p.dst.codes) + (int64_t)phys * epp * d;
#pragma unroll
    for (int r = 0; r < kPrefillRounds; ++r) {
      const int row = r * RP + gi;
      if (r * RP >= epp || !active || row >= epp) continue;
      u32x2 w = {0u, 0u};
      if (row < rows) {
        const f32x8 vr = HCA_ROW_OF_ROUND(r);
        w[0] = enc4_e4m3(f32x4{vr[0], vr[1], vr[2], vr[3]}, s);
        w[1] = enc4_e4m3(f32x4{vr[4], vr[5], vr[6], vr[7]}, s);
      }
      *reinterpret_cast<u32x2*>(codes + (int64_t)row * d + li * 8) = w;
    }
    if (threadIdx.x == 0) reinterpret_cast<float*>(p.dst.scales)[phys] = s;
  } else {  // bf16
    uint16_t* codes = reinterpret_cast<uint16_t*>(p.dst.codes) + (int64_t)phys * epp * d;
#pragma unroll
    for (int r = 0; r < kPrefillRounds; ++r) {
      const int row = r * RP + gi;
      if (r * RP >= epp || !active || row >= epp) continue;
      u32x4 w = {0u, 0u, 0u, 0u};
      if (row < rows) {
        const f32x8 vr = HCA_ROW_OF_ROUND(r);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = (uint32_t)bf16_encode(vr[2 * q]) | ((uint32_t)bf16_encode(vr[2 * q + 1]) << 16);
      }
      *reinterpret_cast<u32x4*>(codes + (int64_t)row * d + li * 8) = w;
    }
  }
}

#undef HCA_ROW_OF_ROUND

__global__ __launch_bounds__(kCompressThreads) void prefill_large_kernel(PrefillArgs p) {
  const CompressArgs& a = p.c;
  const int b = blockIdx.y, pg = blockIdx.x;
  const int n = clampi(a.ntok[b], 0, a.max_ntok);
  const int p0 = a.pos0[b];
  int rows;
  const int phys = prefill_page(p, b, pg, n, p0, rows);
  if (phys < 0) return;  // uniform over the block
  const int m = a.m, d = a.d, epp = p.dst.epp;
  extern __shared__ float dyn_s[];  // compress_block's row-group sums, then the page's rows
  float* page_s = dyn_s + kCompressShm / sizeof(float);
  // the page's entries, folded as kv_compress folds them, into page_s
  const int j0 = pg * epp;
  const int n_page = min(n, (j0 + epp) * m);
  CompressArgs c = a;
  c.out = nullptr;
  compress_block<2>(c, b, j0, 1, page_s, n_page, p0, NoMid{}, nullptr, j0, d);
  const int nv = rows * d;
  if (p.dst.dtype == HCA_FP8_E4M3) {
    __shared__ float red_s[kCompressThreads / 64];
    float amax = 0.0f;
    for (int i = threadIdx.x; i < nv; i += kCompressThreads) amax = fmaxf(amax, fabsf(page_s[i]));
    amax = block_max_n(amax, red_s, kCompressThreads / 64);
    const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    uint32_t* codes = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(p.dst.codes) + (int64_t)phys * epp * d);
    const f32x4* v4 = reinterpret_cast<const f32x4*>(page_s);
    for (int i = threadIdx.x; i < epp * d / 4; i += kCompressThreads) codes[i] = i < nv / 4 ? enc4_e4m3(v4[i], s) : 0u;
    if (threadIdx.x == 0) reinterpret_cast<float*>(p.dst.scales)[phys] = s;
  } else {  // bf16
    uint32_t* codes = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(p.dst.codes) + (int64_t)phys * epp * d);
    for (int i = threadIdx.x; i < epp * d / 2; i += kCompressThreads)
      codes[i] = i < nv / 2 ? (uint32_t)bf16_encode(page_s[2 * i]) | ((uint32_t)bf16_encode(page_s[2 * i + 1]) << 16)
                            : 0u;
  }
}

bool prefill_supported(int m, int d, int epp, int dtype) {
  if (dtype != HCA_FP8_E4M3 && dtype != HCA_BF16) return false;
  if (m <= kSmallM && d == 512) return epp <= kPrefill512Rounds * (kPrefill512Threads / 64);
  if (m <= kSmallM) return epp <= kPrefillRounds * (kPrefillThreads / (d / 8));
  return (size_t)epp * d * sizeof(float) + kCompressShm <= (size_t)64 * 1024;
}

hipError_t launch_prefill(PrefillArgs p, hipStream_t s) {
  CompressArgs& a = p.c;
  const int n_max = (a.max_ntok + a.m - 1) / a.m;
  if (a.B == 0 || n_max == 0) return hipSuccess;
  a.rope_r = pow((double)a.theta, -2.0 / (double)a.d);
  const int pages = (n_max + p.dst.epp - 1) / p.dst.epp;
  if (a.m <= kSmallM) {
    if (a.d == 512)
      hipLaunchKernelGGL(prefill_small512_kernel, dim3(pages, a.B), dim3(kPrefill512Threads), 0, s, p);
    else
      hipLaunchKernelGGL(prefill_small_kernel, dim3(pages, a.B), dim3(kPrefillThreads), 0, s, p);
  } else {
    const size_t shm = kCompressShm + (size_t)p.dst.epp * a.d * sizeof(float);
    hipLaunchKernelGGL(prefill_large_kernel, dim3(pages, a.B), dim3(kCompressThreads), shm, s, p);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------- decode-step insert
// kv_compress_insert: a decode step's update of one pool in one launch, one
// block per sequence: the open group's fold (compress_block, so the entry is
// bit-identical to kv_compress's) into its row of the open page's staging,
// then the open page quantized (V4 page, section 3.2.1: RoPE, then insertion
// into the cache; sections 3.1.1 and 3.1.3: the page formats).  The new row is
// read back from shared memory, older rows from staging.
//   append = 0: the page is rewritten whole, as kv_quantize_page rewrites it.
//   append = 1: the page already holds the codes of the rows before the open
//   one, made with its current scale, so they stand as long as the scale does
//   and only the open row is encoded.  For a re-folded entry (m > 1) the scale
//   is recomputed from all rows (held in registers when the page fits).  For
//   a window insert (m = 1, a new row) it is not: an fp8 page scale is
//   fl32(amax/448), which is monotonic in amax, so the new scale is
//   max(old scale, new row's fl32(amax_row/448)) exactly.  The page is
//   rewritten whole when the scale changes, the page is new (row 0), or, for
//   m = 1, the old scale is 1.0 (which an all-zero page also has).
constexpr int kInsertMaxDim = 2048;


__device__ __forceinline__ float ins_block_max(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

__device__ __forceinline__ float amax4(const f32x4 v) {
  return fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
}

// One more token into a running fold state (groups of more than kSmallM
// tokens, whose re-fold reads the whole group): `prev` holds the state after
// tokens 0 .. n-2 of the open group, `next` receives it after token n-1, and
// the entry (weighted sums over the sum of weights, then the normalisation and
// rotation of every fold) goes to the staging row and row_s.  If `prev` is not
// the state after n-1 tokens (a group's first token, or a state the caller has
// not kept), the group is re-folded whole and `next` written from that fold.
// One row group does the row; every thread calls mid() once.
template <typename Mid>
__device__ __forceinline__ void state_fold(const CompressArgs& a, int b, int n, int p0, const float* prev, float* next,
                                           float* row_s, Mid&& mid) {
  const int TD = a.d >> 3;
  const int RP = kCompressThreads / TD;
  const int li = threadIdx.x % TD;
  const int gi = threadIdx.x / TD;
  const bool live = gi == 0;
  const int t = n - 1;  // the newest token
  // the newest token, its logit and the previous state are loaded first
  const u32x4 raw = live && t >= 0 ? *reinterpret_cast<const u32x4*>(a.x + (int64_t)b * a.xs + (int64_t)t * a.d + li * 8)
                                   : u32x4{0u, 0u, 0u, 0u};
  const float zt = t >= 0 ? a.z[(int64_t)b * a.zs + t] : 0.0f;
  const float bt = t >= 0 ? a.beta[t] : 0.0f;
  f32x4 A0 = {0.f, 0.f, 0.f, 0.f}, A1 = {0.f, 0.f, 0.f, 0.f};
  if (live) {
    A0 = reinterpret_cast<const f32x4*>(prev + kFoldStateHead + li * 8)[0];
    A1 = reinterpret_cast<const f32x4*>(prev + kFoldStateHead + li * 8)[1];
  }
  const float cnt = prev[0], M = prev[1], S = prev[2];
  float gam[8] = {1, 1, 1, 1, 1, 1, 1, 1};
  if (a.gamma != nullptr && live) {
    const f32x4 g0 = reinterpret_cast<const f32x4*>(a.gamma + li * 8)[0];
    const f32x4 g1 = reinterpret_cast<const f32x4*>(a.gamma + li * 8)[1];
#pragma unroll
    for (int c = 0; c < 4; ++c) { gam[c] = g0[c]; gam[4 + c] = g1[c]; }
  }
  if (!(n >= 2 && cnt == (float)(n - 1) && S > 0.0f)) {
    CompressArgs c = a;
    compress_block(c, b, 0, 1, row_s, n, p0, mid, next);
    return;
  }
  mid();
  double inv[4];
  rope_inv_freq4(li, a.rope_r, inv);
  const float at = zt + bt;
  const float M2 = fmaxf(M, at);
  const float co = expf(M - M2), cn = expf(at - M2);
  const float S2 = fmaf(S, co, cn);
  float A[8] = {A0[0], A0[1], A0[2], A0[3], A1[0], A1[1], A1[2], A1[3]};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    A[2 * q] = fmaf(A[2 * q], co, cn * u2f(raw[q] << 16));
    A[2 * q + 1] = fmaf(A[2 * q + 1], co, cn * u2f(raw[q] & 0xFFFF0000u));
  }
  if (live) {
    reinterpret_cast<f32x4*>(next + kFoldStateHead + li * 8)[0] = f32x4{A[0], A[1], A[2], A[3]};
    reinterpret_cast<f32x4*>(next + kFoldStateHead + li * 8)[1] = f32x4{A[4], A[5], A[6], A[7]};
  }
  if (threadIdx.x == 0) {
    next[0] = (float)n;
    next[1] = M2;
    next[2] = S2;
  }
  const float inv_tot = 1.0f / S2;
  float e[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) e[c] = A[c] * inv_tot;
  if (a.gamma != nullptr) {
    __shared__ float sq_s[kCompressThreads];
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) ss = fmaf(e[c], e[c], ss);
    const float rs = 1.0f / sqrtf(row_group_sum(live ? ss : 0.0f, TD, RP, gi, sq_s) / (float)a.d + a.eps);
#pragma unroll
    for (int c = 0; c < 8; ++c) e[c] *= rs * gam[c];
  }
  if (live) rope_store8(a.out + (int64_t)b * a.os + li * 8, row_s + li * 8, e, (double)p0, inv);
}

__device__ __forceinline__ void insert_block(const InsertArgs& a, int b, float* row_s, float* red_s) {
  const int m = a.c.m, d = a.c.d, epp = a.dst.epp;
  const bool fold = a.c.x != nullptr;  // else the open row is already in staging
  const int n = fold ? clampi(a.c.ntok[b], 0, a.c.max_ntok) : 1;
  if (n == 0) return;  // no open group: nothing to write
  const int E0 = a.e0[b];
  const int p0 = a.c.pos0[b];
  const int row = p0 / m - E0;  // the open entry's row in its page
  HCA_DBG_CHECK(row >= 0 && row < epp, kDbgRow);
  if (row < 0 || row >= epp) return;
  const int lb = E0 / epp;
  HCA_DBG_CHECK(lb >= 0 && lb < a.bts, kDbgTable);
  if (lb < 0 || lb >= a.bts) return;
  const int phys = a.bt[(int64_t)b * a.bts + lb];  // loaded now, used after the fold
  const bool page_ok = phys >= 0 && phys < a.dst.num_pages;
  HCA_DBG_CHECK(page_ok, kDbgPage);
  // an fp8 page's current scale, in flight during the fold
  const float s_prev = a.dst.dtype == HCA_FP8_E4M3 && page_ok ? reinterpret_cast<const float*>(a.dst.scales)[phys] : 1.0f;
  const float* st = a.stage + (int64_t)b * a.ss;  // the page's rows in staging
  const int d4 = d / 4;
  const f32x4* st4 = reinterpret_cast<const f32x4*>(st);
  const int old4 = row * d4, new4 = old4 + d4;  // float4 groups before / through the new row
  // the update state: a page header (how many of the open page's rows, and
  // the amax of those rows, which no longer change once their groups are
  // complete) read now, in flight during the fold; then, for groups of more
  // than kSmallM tokens, the two running fold states
  const bool refold8 = a.dst.dtype == HCA_FP8_E4M3 && a.append != 0 && m > 1;
  float* hdr = a.state != nullptr ? a.state + (int64_t)b * a.sts : nullptr;
  const float hc = refold8 && hdr != nullptr ? hdr[0] : -1.0f;
  const float ha = refold8 && hdr != nullptr ? hdr[1] : 0.0f;
  if (fold) {
    CompressArgs c = a.c;
    c.out = a.stage + (int64_t)row * d;
    c.os = a.ss;
    if (m > kSmallM && hdr != nullptr) {
      float* sb = hdr + kPageHead;
      const int sl = kFoldStateHead + d;
      state_fold(c, b, n, p0, sb + ((n - 1) & 1) * sl, sb + (n & 1) * sl, row_s, NoMid{});
    } else {
      compress_block(c, b, 0, 1, row_s, n, p0, NoMid{});
    }
  } else {
    for (int i = threadIdx.x; i < d4; i += kCompressThreads)
      reinterpret_cast<f32x4*>(row_s)[i] = st4[old4 + i];
  }
  __syncthreads();
  if (!page_ok) return;
  const f32x4* row4 = reinterpret_cast<const f32x4*>(row_s);

  if (a.dst.dtype == HCA_FP8_E4M3) {
    float* scales = reinterpret_cast<float*>(a.dst.scales);
    uint32_t* dst = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.dst.codes) + (int64_t)phys * epp * d);
    constexpr int U = 8;
    // the new row's max, taken by every wave over the whole row (no block
    // reduction, no barrier)
    float am = 0.0f;
    for (int i = threadIdx.x & 63; i < d4; i += 64) am = fmaxf(am, amax4(row4[i]));
    am = wave_max(am);
    bool full = a.append == 0 || row == 0;
    float s = 1.0f;
    if (!full && m == 1) {
      // a window insert: the new row's scale joins the page's by max
      if (!(s_prev > 0.0f) || s_prev == 1.0f || am / 448.0f > s_prev) full = true;
      else s = s_prev;
    } else if (!full) {
      // a re-folded open entry: the page max is the closed rows' (from the
      // header when it holds them, or all but the row that closed when this
      // group began) joined with the open row's
      float closed;
      if (hc == (float)row) {
        closed = ha;
      } else if (hc == (float)(row - 1)) {
        float v = 0.0f;
        for (int i = threadIdx.x; i < d4; i += kCompressThreads) v = fmaxf(v, amax4(st4[old4 - d4 + i]));
        closed = fmaxf(ha, ins_block_max(v, red_s));
      } else {
        float v = 0.0f;
        for (int i0 = threadIdx.x; i0 < old4; i0 += U * kCompressThreads) {
          f32x4 w[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int i = i0 + u * kCompressThreads;
            w[u] = i < old4 ? st4[i] : f32x4{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int u = 0; u < U; ++u) v = fmaxf(v, amax4(w[u]));
        }
        closed = ins_block_max(v, red_s);
      }
      if (hdr != nullptr && threadIdx.x == 0) {
        hdr[0] = (float)row;
        hdr[1] = closed;
      }
      const float amx = fmaxf(closed, am);
      s = amx > 0.0f ? amx / 448.0f : 1.0f;
      full = s != s_prev;  // the earlier rows' codes stand while the page scale does
    }
    if (full) {
      float amx = am;
      for (int i0 = threadIdx.x; i0 < old4; i0 += U * kCompressThreads) {
        f32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * kCompressThreads;
          v[u] = i < old4 ? st4[i] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) amx = fmaxf(amx, amax4(v[u]));
      }
      amx = ins_block_max(amx, red_s);
      s = amx > 0.0f ? amx / 448.0f : 1.0f;
      if (refold8 && hdr != nullptr && threadIdx.x == 0 && row == 0) {
        hdr[0] = 0.0f;  // a new page: no closed rows yet
        hdr[1] = 0.0f;
      }
      const int tot4 = epp * d4;
      for (int i0 = threadIdx.x; i0 < tot4; i0 += U * kCompressThreads) {
        f32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * kCompressThreads;
          v[u] = i < old4 ? st4[i] : (i < new4 ? row4[i - old4] : f32x4{0.f, 0.f, 0.f, 0.f});
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * kCompressThreads;
          if (i < tot4) dst[i] = i < new4 ? enc4_e4m3(v[u], s) : 0u;
        }
      }
      if (threadIdx.x == 0) scales[phys] = s;
    } else {
      for (int i = threadIdx.x; i < d4; i += kCompressThreads) dst[old4 + i] = enc4_e4m3(row4[i], s);
    }
  } else if (a.dst.dtype == HCA_FP4_E2M1) {
    // per-32 scales within a row: four lanes per block of 32, 8 elements each
    const int nblk = d / 32;
    uint8_t* pc = reinterpret_cast<uint8_t*>(a.dst.codes) + (int64_t)phys * epp * (d / 2);
    uint8_t* ps = reinterpret_cast<uint8_t*>(a.dst.scales) + (int64_t)phys * epp * nblk;
    const int r0 = a.append ? row : 0, r1 = a.append ? row + 1 : epp;
    const int units = (r1 - r0) * nblk * 4;
    for (int u0 = 0; u0 < units; u0 += kCompressThreads) {
      const int u = u0 + threadIdx.x;
      const bool live = u < units;
      const int q = u & 3;
      const int blk = (u >> 2) % nblk;
      const int r = r0 + (u >> 2) / nblk;
      float v[8];
      float amax = 0.0f;
      if (live && r <= row) {
        const float* src = r == row ? row_s + blk * 32 + q * 8 : st + (int64_t)r * d + blk * 32 + q * 8;
        const f32x4 v0 = reinterpret_cast<const f32x4*>(src)[0], v1 = reinterpret_cast<const f32x4*>(src)[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[i] = v0[i]; v[4 + i] = v1[i]; }
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
      }
      amax = quad_max(amax);
      if (!live) continue;
      const uint32_t sc = r <= row ? e4m3_encode(amax / 6.0f) : 0u;
      const float sdec = e4m3_decode(sc);
      uint32_t word = 0;
      if (sdec > 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) word |= e2m1_encode(v[i] / sdec) << (4 * i);
      }
      *reinterpret_cast<uint32_t*>(pc + (int64_t)r * (d / 2) + blk * 16 + q * 4) = word;
      if (q == 0) ps[(int64_t)r * nblk + blk] = (uint8_t)sc;
    }
  } else {
    u32x2* dst = reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.dst.codes) + (int64_t)phys * epp * d);
    const int i0 = a.append ? old4 : 0, i1 = a.append ? new4 : epp * d4;
    for (int i = i0 + threadIdx.x; i < i1; i += kCompressThreads) {
      u32x2 w = {0u, 0u};
      if (i < new4) {
        const f32x4 v = i < old4 ? st4[i] : row4[i - old4];
        w[0] = (uint32_t)bf16_encode(v[0]) | ((uint32_t)bf16_encode(v[1]) << 16);
        w[1] = (uint32_t)bf16_encode(v[2]) | ((uint32_t)bf16_encode(v[3]) << 16);
      }
      dst[i] = w;
    }
  }
}

__global__ __launch_bounds__(kCompressThreads) void insert_kernel(InsertJobs j) {
  __shared__ __attribute__((aligned(16))) float row_s[kInsertMaxDim];
  __shared__ float red_s[kCompressThreads / 64];
  insert_block(j.job[blockIdx.y], blockIdx.x, row_s, red_s);
}

hipError_t launch_insert(InsertJobs j, int B, hipStream_t s) {
  if (B == 0 || j.n == 0) return hipSuccess;
  for (int i = 0; i < j.n; ++i) {
    j.job[i].c.rope_r = pow((double)j.job[i].c.theta, -2.0 / (double)j.job[i].c.d);
  }
  hipLaunchKernelGGL(insert_kernel, dim3(B, j.n), dim3(kCompressThreads), kCompressShm, s, j);
  return hipGetLastError();
}

// ------------------------------------------------- select with the updates
// V4 page, section 3.2.2: the indexer runs beside the main-KV compression and
// the window insert.  Here the updates are extra blocks of the select's
// compaction launch: block i < n_jobs of row y runs update job i for sequence
// y, block n_jobs + x of row y compacts chunks 2x and 2x + 1 of sequence y.
// The blocks are independent (the jobs write no indexer data), and the
// compaction, like the updates, is a short chain of dependent loads with
// little traffic, so the updates run in its shadow.  The kernel's register
// count is the update path's (two blocks per CU); with two chunks per
// compaction block every block of the launch is resident at once.
static_assert(kCompressThreads == kSelThreads, "one block size for both kinds of block");

__global__ __launch_bounds__(kCompressThreads) void compact_insert_kernel(IndexerArgs a, InsertJobs j) {
  __shared__ SelLds sm;
  __shared__ uint32_t wbits_s[kCompactChunks * kSelChunk / 32];
  __shared__ __attribute__((aligned(16))) float row_s[kInsertMaxDim];
  __shared__ float red_s[kCompressThreads / 64];
  if ((int)blockIdx.x < j.n)
    insert_block(j.job[blockIdx.x], blockIdx.y, row_s, red_s);
  else
    select_compact_block(a, blockIdx.x - j.n, blockIdx.y, sm, wbits_s);
}

hipError_t launch_compact_insert(const IndexerArgs& a, const InsertJobs& jobs, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  InsertJobs j = jobs;
  for (int i = 0; i < j.n; ++i) j.job[i].c.rope_r = pow((double)j.job[i].c.theta, -2.0 / (double)j.job[i].c.d);
  hipLaunchKernelGGL(compact_insert_kernel, dim3(j.n + compact_blocks(a), a.B), dim3(kCompressThreads), kCompressShm,
                     s, a, j);
  return hipGetLastError();
}

#ifdef HCA_DEBUG
HCA_DBG_ACCESSOR(debug_bits_compress)
#endif

}  // namespace hca
