// The indexer's score pass as device code (V4 page, section 2.2: the indexer
// scores every compressed entry's key against the indexer query heads), shared
// by the indexer's own kernels and by the score launch that also runs a
// decode step's cache updates as extra blocks.
//
// Each wave scores 16 entries at a time with v_mfma_f32_16x16x32_bf16: A = the
// 16 indexer query heads (bf16, held in registers), B = 16 keys decoded to
// exact bf16 (E4M3 and E2M1 values are exact in bf16).  The contraction order
// inside an MFMA step is free, so each lane reads one contiguous run of its key
// and the query fragment uses the same dim order.  fp4 keys carry a scale per
// 32 elements; a k-step covers exactly one such block, its MFMA writes a fresh
// accumulator and the block scale is applied in fp32 afterwards.  ReLU, the
// per-head weights and the head sum run on the accumulator lanes, and the
// order key of every score lands in a 4096-bin LDS histogram that is added to
// one of several per-sequence histogram copies in the workspace (spread by
// block index, so the hot bins are not one queue).
#pragma once
#include "hca_common.h"
#include "indexer_internal.h"

namespace hca {

constexpr int kScoreThreads = 256;
constexpr int kSelChunk = 2048;    // entries per select block (8 per thread); score rows are padded to it

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
// (the block scale is applied after the product, in fp32: the conversion's
// scale operand does not reproduce the exact product for E4M3 scales)
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
  return __builtin_bit_cast(bf16x8, r);
}

// The bytes one lane reads for one 16-entry tile, and how they become the MFMA
// B operand.  Lane (col, g) serves entry `col` of the tile.
//   bf16 / fp8: lane group g owns the contiguous dims [g*DI/4, (g+1)*DI/4) of the
//               key (16-byte loads); k-step t uses the 8 dims at +8t.
//   fp4:        k-step t is scale block t; lane group g reads the 4 bytes holding
//               dims 32t + 8g .. +8 of it.
template <int KDT, int DI>
struct Tile {
  static constexpr int KS = DI / 32;
  static constexpr int NW = KDT == HCA_FP4_E2M1 ? KS : (KDT == HCA_FP8_E4M3 ? DI / 16 : DI / 8);
  uint32_t w[NW];
  uint32_t sc[(KS + 3) / 4];  // fp4 block-scale codes of the entry
  float ps;                   // fp8 page scale (0 for a missing row)

  // Branch-free: a dead lane (past N or an unmapped page) reads the pool's first
  // row and masks the value, so all loads stay in straight-line code and the
  // compiler can keep the next page's loads in flight while this one is used.
  __device__ __forceinline__ void load(const uint8_t* row, const uint8_t* srow, float page_scale, bool live, int g) {
    ps = live ? page_scale : 0.0f;
    if constexpr (KDT == HCA_FP4_E2M1) {
#pragma unroll
      for (int t = 0; t < KS; ++t) w[t] = *reinterpret_cast<const uint32_t*>(row + 16 * t + 4 * g);
      if constexpr (KS % 4 == 0) {
#pragma unroll
        for (int i = 0; i < KS / 4; ++i) sc[i] = *reinterpret_cast<const uint32_t*>(srow + 4 * i);
      } else {
        sc[0] = 0u;
#pragma unroll
        for (int t = 0; t < KS; ++t) sc[0] |= (uint32_t)srow[t] << (8 * t);
      }
#pragma unroll
      for (int i = 0; i < (KS + 3) / 4; ++i) sc[i] = live ? sc[i] : 0u;
    } else {
      const uint8_t* lrow = row + g * (NW * 4);
      if constexpr (NW >= 4) {
#pragma unroll
        for (int c = 0; c < NW / 4; ++c) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(lrow + 16 * c);
          w[4 * c] = v[0]; w[4 * c + 1] = v[1]; w[4 * c + 2] = v[2]; w[4 * c + 3] = v[3];
        }
      } else {
        const u32x2 v = *reinterpret_cast<const u32x2*>(lrow);
        w[0] = v[0]; w[1] = v[1];
      }
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = live ? w[i] : 0u;
  }

  // dot products of this lane's 4 heads (rows 4g..4g+3 of the accumulator) with entry col
  __device__ __forceinline__ f32x4 dots(const bf16x8* qa) const {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KDT == HCA_FP4_E2M1) {
      float sfs[4 * ((KS + 3) / 4)];  // exact E4M3 decode of the block scales
#pragma unroll
      for (int i = 0; i < (KS + 3) / 4; ++i) {
        sfs[4 * i + 0] = __builtin_amdgcn_cvt_f32_fp8((int)sc[i], 0);
        sfs[4 * i + 1] = __builtin_amdgcn_cvt_f32_fp8((int)sc[i], 1);
        sfs[4 * i + 2] = __builtin_amdgcn_cvt_f32_fp8((int)sc[i], 2);
        sfs[4 * i + 3] = __builtin_amdgcn_cvt_f32_fp8((int)sc[i], 3);
      }
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[t], fp4x8_to_bf16(w[t]), z, 0, 0, 0);
        const float sf = sfs[t];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(sf, part[i], acc[i]);
      }
    } else if constexpr (KDT == HCA_FP8_E4M3) {
#pragma unroll
      for (int t = 0; t < KS; ++t)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[t], fp8x8_to_bf16(w[2 * t], w[2 * t + 1]), acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= ps;
    } else {
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        const u32x4 v = {w[4 * t], w[4 * t + 1], w[4 * t + 2], w[4 * t + 3]};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[t], __builtin_bit_cast(bf16x8, v), acc, 0, 0, 0);
      }
    }
    return acc;
  }
};

struct ScoreCtx {
  float wgt[4];
  float* scores;
  uint32_t* hist_s;
  bool want_hist;
};

// ReLU, head weights, head sum; lanes 0..15 write the scores of the tile
__device__ __forceinline__ void finish_tile(const ScoreCtx& c, f32x4 acc, int e, bool valid, int g) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s = fmaf(c.wgt[i], fmaxf(acc[i], 0.0f), s);
  s = rows_sum4(s);
  if (g == 0 && valid) {
    c.scores[e] = s;
    if (c.want_hist) atomicAdd(&c.hist_s[order_key(s) >> 20], 1u);
  }
}

template <int KDT, int DI>
__device__ __forceinline__ void load_query(const IndexerArgs& a, int b, int col, int g, bf16x8* qa, float* wgt) {
  constexpr int KS = DI / 32;
  const int h = col;
  const uint16_t* qrow = a.q + ((int64_t)b * a.HI + (h < a.HI ? h : 0)) * DI;
#pragma unroll
  for (int t = 0; t < KS; ++t) {
    const int c0 = (KDT == HCA_FP4_E2M1) ? (32 * t + 8 * g) : (g * (DI / 4) + 8 * t);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (h < a.HI) v = *reinterpret_cast<const u32x4*>(qrow + c0);
    qa[t] = __builtin_bit_cast(bf16x8, v);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = 4 * g + i;
    wgt[i] = hh < a.HI ? a.w[(int64_t)b * a.HI + hh] : 0.0f;
  }
}

// The block's histogram is added to one of kHistCopies copies (by block index),
// so that the blocks of a sequence do not all queue on the same hot bins, and
// its sums over 256-bin ranges to the same copy of the coarse histogram (which
// tells the select which 256-bin slice holds its cut without scanning down to
// it).  Round r of the loop holds the bins of coarse bin r, so each wave adds
// its share of a coarse bin with one atomic, and only where it has counts;
// the wave sum is register-to-register (DPP row rotations inside each 16-lane
// row, then the two permlane swaps across rows).
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false);  // row_ror:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xF, 0xF, false);  // row_ror:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xF, 0xF, false);  // row_ror:1
  const auto x = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = x[0] + x[1];
  const auto y = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return y[0] + y[1];
}
__device__ __forceinline__ void hist_flush(const IndexerArgs& a, int b, int bx, const uint32_t* hist_s) {
  static_assert(kScoreThreads * kCoarseBins == kHistBins, "one coarse bin per round");
  __syncthreads();
  uint32_t* base = reinterpret_cast<uint32_t*>(a.ws + a.lay.hist) + (size_t)b * kHistWords;
  const int copy = bx % kHistCopies;
  uint32_t* gh = base + copy * kHistBins;
  uint32_t* gc = base + kHistCopies * kHistBins + copy * kCoarseBins;
  // all of the thread's bins are read before the first atomic (the compiler
  // does not move LDS reads across the atomics, so the rounds would each wait
  // for their own read)
  uint32_t cv[kCoarseBins];
#pragma unroll
  for (int r = 0; r < kCoarseBins; ++r) cv[r] = hist_s[(int)threadIdx.x + r * kScoreThreads];
#pragma unroll
  for (int r = 0; r < kCoarseBins; ++r) {
    const int i = (int)threadIdx.x + r * kScoreThreads;
    const uint32_t c = cv[r];
    if (c) atomicAdd(&gh[i], c);
    if (__ballot(c != 0u)) {
      const uint32_t s = wave_sum_u32(c);
      if ((threadIdx.x & 63) == 0) atomicAdd(&gc[r], s);
    }
  }
}

__device__ __forceinline__ float* score_row(const IndexerArgs& a, int b) {
  return reinterpret_cast<float*>(a.ws + a.lay.scores) +
         (size_t)b * ((a.lay.n_max + kSelChunk - 1) / kSelChunk) * kSelChunk;
}

// Fast path: 64 entries per page (m = 4).  A wave scores whole pages.  The
// page is uniform over the wave, so its table lookup is a scalar load and it
// gets a buffer resource of its own whose size is the page's valid bytes: a
// lane past the last valid entry, or a whole page that is unmapped, reads 0 in
// hardware, so the loads need no masks, no branches and only 32-bit offsets.
// A wave's pages go through a ring of kScoreBufs buffers (the loads of page
// i + kScoreBufs are issued right after page i is consumed), fully unrolled so
// that the waits count down in order.
constexpr int kPagesPerScoreBlock = 32;
constexpr int kPagesPerScoreWave = kPagesPerScoreBlock / 4;
constexpr int kScoreBufs = 3;  // pages a wave has in flight

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 4x4 transpose across the four 16-lane rows of a wave: with r[c] holding
// element (row, c) in every lane of row `row`, afterwards r[c] holds element
// (c, row).  Two v_permlane32_swap (off-diagonal 2x2 blocks of rows), then two
// v_permlane16_swap (within the blocks).
__device__ __forceinline__ void row_transpose4(uint32_t& r0, uint32_t& r1, uint32_t& r2, uint32_t& r3) {
  auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
  auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  r0 = c[0];
  r1 = c[1];
  r2 = d[0];
  r3 = d[1];
}

template <int KDT, int DI>
struct PageTiles {
  static constexpr int KS = DI / 32;
  static constexpr int ROW = KDT == HCA_FP4_E2M1 ? DI / 2 : (KDT == HCA_FP8_E4M3 ? DI : 2 * DI);
  static constexpr int NW = KDT == HCA_FP4_E2M1 ? KS : (KDT == HCA_FP8_E4M3 ? DI / 16 : DI / 8);
  uint32_t w[4][NW];
  uint32_t sc[4][(KS + 3) / 4];
  float ps;

  // fp4 pages are read with one 16-byte load per lane per 16 bytes of a row:
  // lane l takes entry l of the page (raw[] below); prepare() then moves the
  // bytes into the MFMA operand layout with row transposes.
  static constexpr int SW = (KS + 3) / 4;  // block-scale words per entry (fp4)
  uint32_t raw[KDT == HCA_FP4_E2M1 ? 4 * KS : 1];
  uint32_t rsc[KDT == HCA_FP4_E2M1 ? SW : 1];

  // `phys` is the page's table entry, read ahead of the sequence length
  __device__ __forceinline__ void load(const IndexerArgs& a, int phys, int p, bool p_ok, int N, int col, int g) {
    const bool live = p_ok && phys >= 0 && phys < a.keys.num_pages;
    HCA_DBG_CHECK(!p_ok || live, kDbgPage);
    const int rows = live ? min(64, N - 64 * p) : 0;
    const int pg = live ? phys : 0;
    const uint8_t* codes = reinterpret_cast<const uint8_t*>(a.keys.codes) + (int64_t)pg * 64 * ROW;
    const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(codes, (uint32_t)(rows * ROW));
    if constexpr (KDT == HCA_FP8_E4M3) ps = reinterpret_cast<const float*>(a.keys.scales)[pg];
    if constexpr (KDT == HCA_FP4_E2M1) {
      const int lane = 16 * g + col;
#pragma unroll
      for (int c = 0; c < KS; ++c) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, lane * ROW + 16 * c, 0, 0);
        raw[4 * c] = v[0]; raw[4 * c + 1] = v[1]; raw[4 * c + 2] = v[2]; raw[4 * c + 3] = v[3];
      }
      const uint8_t* scl = reinterpret_cast<const uint8_t*>(a.keys.scales) + (int64_t)pg * 64 * KS;
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(scl, (uint32_t)(rows * KS));
      if constexpr (KS % 4 == 0) {
#pragma unroll
        for (int i = 0; i < SW; ++i) rsc[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, lane * KS + 4 * i, 0, 0);
      } else if constexpr (KS == 2) {
        rsc[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, lane * KS, 0, 0);
      } else {
        rsc[0] = __builtin_amdgcn_raw_buffer_load_b8(rs, lane * KS, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int row_off = (16 * tt + col) * ROW;
      if constexpr (NW >= 4) {
#pragma unroll
        for (int c = 0; c < NW / 4; ++c) {
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, row_off + g * (NW * 4) + 16 * c, 0, 0);
          w[tt][4 * c] = v[0]; w[tt][4 * c + 1] = v[1]; w[tt][4 * c + 2] = v[2]; w[tt][4 * c + 3] = v[3];
        }
      } else {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rc, row_off + g * 8, 0, 0);
        w[tt][0] = v[0]; w[tt][1] = v[1];
      }
    }
  }

  // fp4: lane (col, g) of tile tt, k-step t needs dword 4t + g of entry 16tt + col,
  // which row tt holds in lane col: one row transpose per k-step (and per scale word)
  __device__ __forceinline__ void prepare() {
    if constexpr (KDT == HCA_FP4_E2M1) {
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        uint32_t r0 = raw[4 * t], r1 = raw[4 * t + 1], r2 = raw[4 * t + 2], r3 = raw[4 * t + 3];
        row_transpose4(r0, r1, r2, r3);
        w[0][t] = r0; w[1][t] = r1; w[2][t] = r2; w[3][t] = r3;
      }
#pragma unroll
      for (int i = 0; i < SW; ++i) {
        uint32_t r0 = rsc[i], r1 = rsc[i], r2 = rsc[i], r3 = rsc[i];
        row_transpose4(r0, r1, r2, r3);
        sc[0][i] = r0; sc[1][i] = r1; sc[2][i] = r2; sc[3][i] = r3;
      }
    }
  }

  __device__ __forceinline__ f32x4 dots(int tt, const bf16x8* qa) const {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KDT == HCA_FP4_E2M1) {
      float sfs[4 * ((KS + 3) / 4)];  // exact E4M3 decode of the block scales
#pragma unroll
      for (int i = 0; i < (KS + 3) / 4; ++i) {
        sfs[4 * i + 0] = __builtin_amdgcn_cvt_f32_fp8((int)sc[tt][i], 0);
        sfs[4 * i + 1] = __builtin_amdgcn_cvt_f32_fp8((int)sc[tt][i], 1);
        sfs[4 * i + 2] = __builtin_amdgcn_cvt_f32_fp8((int)sc[tt][i], 2);
        sfs[4 * i + 3] = __builtin_amdgcn_cvt_f32_fp8((int)sc[tt][i], 3);
      }
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[t], fp4x8_to_bf16(w[tt][t]), z, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(sfs[t], part[i], acc[i]);
      }
    } else if constexpr (KDT == HCA_FP8_E4M3) {
#pragma unroll
      for (int t = 0; t < KS; ++t)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[t], fp8x8_to_bf16(w[tt][2 * t], w[tt][2 * t + 1]), acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= ps;
    } else {
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        const u32x4 v = {w[tt][4 * t], w[tt][4 * t + 1], w[tt][4 * t + 2], w[tt][4 * t + 3]};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[t], __builtin_bit_cast(bf16x8, v), acc, 0, 0, 0);
      }
    }
    return acc;
  }
};

// The open indexer row of a decode step (fp4 keys, 128 dims, 64 entries per
// page), encoded by the wave that scores its page: lane l holds dims 2l and
// 2l + 1, so the 16 lanes of a 32-element block find its amax by xor shuffles;
// scale code E4M3(amax / 6), codes E2M1(x / decoded scale), all codes 0 for a
// zero scale, element 2l in the low nibble of byte l: the update kernel's
// encoding, operation for operation.  The row goes to the page (for the steps
// after this one) and, through LDS, into the registers of the lane that holds
// that entry of the loaded page.
struct OpenRow {
  int page = -1;       // page index of the open row in the sequence, -1: not this wave's
  int row = 0;         // its row in the page
  uint32_t byte = 0;   // this lane's code byte
  uint32_t sc = 0;     // the scale code of this lane's 32-element block
  __device__ __forceinline__ void prepare(const IndexerArgs& a, int b, int page0, int wave, int lane) {
    if (a.open.stage == nullptr) return;
    const int E0 = a.open.e0[b];
    const int r = a.open.pos0[b] / a.m - E0;
    const int lb = E0 >> 6;
    if (r < 0 || r >= 64 || E0 < 0 || lb >= a.bts) return;
    if (lb < page0 || lb >= page0 + kPagesPerScoreBlock || ((lb - page0) & 3) != wave) return;
    const float2 v = reinterpret_cast<const float2*>(a.open.stage + (int64_t)b * a.open.ss + (int64_t)r * 128)[lane];
    float amax = fmaxf(fabsf(v.x), fabsf(v.y));
    amax = row16_max(amax);
    sc = e4m3_encode(amax / 6.0f);
    const float sdec = e4m3_decode(sc);
    byte = sdec > 0.0f ? (e2m1_encode(v.x / sdec) | (e2m1_encode(v.y / sdec) << 4)) : 0u;
    const int phys = a.bt[(int64_t)b * a.bts + lb];
    HCA_DBG_CHECK(phys >= 0 && phys < a.keys.num_pages, kDbgPage);
    if (phys < 0 || phys >= a.keys.num_pages) return;  // an unmapped page: nothing written, nothing patched
    uint8_t* codes = reinterpret_cast<uint8_t*>(a.keys.codes) + ((int64_t)phys * 64 + r) * 64;
    uint8_t* scales = reinterpret_cast<uint8_t*>(a.keys.scales) + ((int64_t)phys * 64 + r) * 4;
    codes[lane] = (uint8_t)byte;
    if ((lane & 15) == 0) scales[lane >> 4] = (uint8_t)sc;
    page = lb;
    row = r;
  }
  // with the page's loads in: the open row's lane takes the new bytes
  __device__ __forceinline__ void patch(uint32_t* raw, uint32_t* rsc, int p, int lane) const {
    if (p != page) return;
    // the row's 16 code words and its scale word, gathered from the lanes
    uint32_t w[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t b0 = __shfl(byte, 4 * k, 64), b1 = __shfl(byte, 4 * k + 1, 64);
      const uint32_t b2 = __shfl(byte, 4 * k + 2, 64), b3 = __shfl(byte, 4 * k + 3, 64);
      w[k] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
    }
    const uint32_t s4 = __shfl(sc, 0, 64) | (__shfl(sc, 16, 64) << 8) | (__shfl(sc, 32, 64) << 16) |
                        (__shfl(sc, 48, 64) << 24);
    if (lane == row) {
#pragma unroll
      for (int k = 0; k < 16; ++k) raw[k] = w[k];
      rsc[0] = s4;
    }
  }
};

// One score block of the page path: block bx of sequence b, with the block's
// LDS histogram (kHistBins words).  Called by every thread of a block of
// kScoreThreads threads.
template <int KDT, int DI>
__device__ __forceinline__ void score_pages_block(const IndexerArgs& a, int bx, int b, uint32_t* hist_s) {
  const int page0 = bx * kPagesPerScoreBlock;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar page math
  const int col = lane & 15, g = lane >> 4;
  constexpr int PPW = kPagesPerScoreWave;
  auto page_of = [&](int i) { return page0 + wave + 4 * i; };
  // Nothing below waits for the sequence length before its loads are issued:
  // the length, the query and the table entries of the wave's pages go out
  // together (entries past the table's width are not read), so the page loads
  // follow one round trip after the start instead of two.
  const int len_raw = a.lens[b];
  const int32_t* btrow = a.bt + (int64_t)b * a.bts;
  int phys[PPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) phys[i] = btrow[min(page_of(i), a.bts - 1)];
  ScoreCtx c;
  bf16x8 qa[DI / 32];
  load_query<KDT, DI>(a, b, col, g, qa, c.wgt);
  // the histogram is cleared whatever k is; the barrier orders LDS only and
  // leaves the loads above in flight
  static_assert(kHistBins % (4 * kScoreThreads) == 0, "the clear writes 16 bytes per thread and round");
#pragma unroll
  for (int i = 4 * (int)threadIdx.x; i < kHistBins; i += 4 * kScoreThreads)
    *reinterpret_cast<u32x4*>(&hist_s[i]) = u32x4{0u, 0u, 0u, 0u};
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  // the open indexer row (fp4 keys of 128 dims): its wave encodes it from
  // staging, writes it to the page and scores it in place of the page's old
  // bytes for that row.  Written before the length check, so that a row whose
  // page lies inside the launch's pages is written even where it lies past
  // the sequence's entries (nothing scores it then)
  OpenRow orow;
  if constexpr (KDT == HCA_FP4_E2M1 && DI == 128) orow.prepare(a, b, page0, wave, lane);
  const int L = clampi(len_raw, 0, a.max_len);
  const int N = (L + a.m - 1) / a.m;
  const int NP = (N + 63) / 64;
  if (page0 >= NP) return;
  c.want_hist = a.k < N;
  c.hist_s = hist_s;
  c.scores = score_row(a, b);
  const int p_end = min(NP, page0 + kPagesPerScoreBlock);
  // a ring of kScoreBufs page buffers per wave: the first kScoreBufs pages are
  // loaded up front, page i + kScoreBufs as soon as page i is consumed
  PageTiles<KDT, DI> pt[kScoreBufs];
  auto consume = [&](PageTiles<KDT, DI>& t, int i) {
    if constexpr (KDT == HCA_FP4_E2M1 && DI == 128) orow.patch(t.raw, t.rsc, page_of(i), lane);
    t.prepare();
    const int p = page_of(i);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int e = 64 * p + 16 * tt + col;
      finish_tile(c, t.dots(tt, qa), e, p < p_end && e < N, g);
    }
  };
#pragma unroll
  for (int i = 0; i < kScoreBufs; ++i) pt[i].load(a, phys[i], page_of(i), page_of(i) < p_end, N, col, g);
  // every load of the first pages is issued before the first page is used
  // (left to itself the scheduler holds some back behind the first page)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    consume(pt[i % kScoreBufs], i);
    const int n = i + kScoreBufs;
    if (n < PPW) pt[i % kScoreBufs].load(a, phys[n], page_of(n), page_of(n) < p_end, N, col, g);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (c.want_hist) hist_flush(a, b, bx, hist_s);
}


}  // namespace hca
