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
// per-sequence histogram copies in the workspace.
//
// The score blocks add their LDS histograms to one of several copies in the
// workspace (spread by block index, so the hot bins are not one queue).
//
// Select.  The cut bin comes from the summed copies; every chunk block marks
// the scores above it in a bitmap and appends the cut bin's entries as
// candidates; then every compaction block refines the cut with two 10-bit
// radix passes over the candidates, breaks exact ties by the lowest index, and
// writes its chunk's kept indices in ascending order.  The histogram copies are left zeroed for the next call; every
// other part of the workspace is overwritten before it is read.
#include "hca_common.h"
#include "indexer_internal.h"

namespace hca {

constexpr int kScoreThreads = 256;
constexpr int kScoreChunk = 1024;  // entries per score block (256 per wave)
constexpr int kSelThreads = 256;
constexpr int kSelChunk = 2048;    // entries per select block (8 per thread)
constexpr int kMaxSelBlocks = 1024;  // select blocks per sequence (N <= 2M entries)
constexpr int kCandLds = 4096;      // candidates a compaction block stages in LDS

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

IndexerWs indexer_ws_layout(int B, int max_seq_len, int m, int k) {
  (void)k;
  IndexerWs w;
  const int n_max = (max_seq_len + m - 1) / m;
  w.n_max = n_max;
  const int n_pad = ((n_max + kSelChunk - 1) / kSelChunk) * kSelChunk;
  size_t off = 0;
  w.scores = off; off = align256(off + (size_t)B * n_pad * sizeof(float));
  w.hist = off; off = align256(off + (size_t)B * kHistCopies * kHistBins * sizeof(uint32_t));
  w.cand = off; off = align256(off + (size_t)B * n_pad * sizeof(uint2));
  w.bitmap = off; off = align256(off + (size_t)B * (n_pad / 32) * sizeof(uint32_t));
  w.counters = off; off = align256(off + (size_t)B * 4 * sizeof(uint32_t));
  w.cand_counts = off; off = align256(off + (size_t)B * 2 * (n_pad / kSelChunk) * sizeof(uint32_t));
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
// so that the blocks of a sequence do not all queue on the same hot bins.
__device__ __forceinline__ void hist_flush(const IndexerArgs& a, int b, const uint32_t* hist_s) {
  __syncthreads();
  uint32_t* gh = reinterpret_cast<uint32_t*>(a.ws + a.lay.hist) +
                 ((size_t)b * kHistCopies + blockIdx.x % kHistCopies) * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kScoreThreads) {
    const uint32_t c = hist_s[i];
    if (c) atomicAdd(&gh[i], c);
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
// Pages are double-buffered (the loads of page i+2 are issued right after page
// i is consumed), fully unrolled so that the waits count down in order.
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

template <int KDT, int DI>
__global__ __launch_bounds__(kScoreThreads) void score_pages_kernel(IndexerArgs a) {
  const int b = blockIdx.y;
  const int page0 = blockIdx.x * kPagesPerScoreBlock;
  __shared__ uint32_t hist_s[kHistBins];
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
  for (int i = threadIdx.x; i < kHistBins; i += kScoreThreads) hist_s[i] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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
  if (c.want_hist) hist_flush(a, b, hist_s);
}

// Generic path (any entries-per-page): per-lane table lookups, 16 entries a step.
template <int KDT, int DI>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(IndexerArgs a) {
  const int b = blockIdx.y;
  const int L = clampi(a.lens[b], 0, a.max_len);
  const int N = (L + a.m - 1) / a.m;
  const int chunk0 = blockIdx.x * kScoreChunk;
  if (chunk0 >= N) return;
  __shared__ uint32_t hist_s[kHistBins];
  ScoreCtx c;
  c.want_hist = a.k < N;
  c.hist_s = hist_s;
  c.scores = score_row(a, b);
  if (c.want_hist) {
    for (int i = threadIdx.x; i < kHistBins; i += kScoreThreads) hist_s[i] = 0;
    __syncthreads();
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int epp = a.keys.epp;
  bf16x8 qa[DI / 32];
  load_query<KDT, DI>(a, b, col, g, qa, c.wgt);
  constexpr int row_bytes = KDT == HCA_FP4_E2M1 ? DI / 2 : (KDT == HCA_FP8_E4M3 ? DI : 2 * DI);
  const uint8_t* codes = reinterpret_cast<const uint8_t*>(a.keys.codes);
  const uint8_t* scales = reinterpret_cast<const uint8_t*>(a.keys.scales);
  const int wave0 = chunk0 + wave * (kScoreChunk / 4);
  const int wave1 = min(N, wave0 + kScoreChunk / 4);
  for (int e_base = wave0; e_base < wave1; e_base += 16) {
    const int e = e_base + col;
    const bool valid = e < wave1;
    int phys = a.bt[(int64_t)b * a.bts + (valid ? e : wave0) / epp];
    const int slot = (valid ? e : wave0) % epp;
    const bool live = valid && phys >= 0 && phys < a.keys.num_pages;
    const float pscale = KDT == HCA_FP8_E4M3 ? reinterpret_cast<const float*>(a.keys.scales)[live ? phys : 0] : 0.0f;
    const int64_t r = live ? (int64_t)phys * epp + slot : 0;
    Tile<KDT, DI> t;
    t.load(codes + r * row_bytes, scales + r * (DI / 32), pscale, live, g);
    finish_tile(c, t.dots(qa), e, valid, g);
  }
  if (c.want_hist) hist_flush(a, b, hist_s);
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
  if (threadIdx.x == 0) { cut_s = 0; above_s = 0; }
  __syncthreads();
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

// Two launches after the score pass, so that kernel boundaries order the
// passes (no device-scope fences, which write back and invalidate the whole L2):
//   select_chunk   (G blocks per sequence) the cut bin from the summed
//                  histogram copies; entries whose 12-bit bin is above it go
//                  straight into the bitmap; cut-bin entries become (key,
//                  index) candidates in the block's region;
//   select_compact (one block per chunk) every block resolves the exact cut
//                  from all candidates (LDS radix passes, ties by index),
//                  takes its output offset from the kept counts of the
//                  chunks before it, and compacts its 64 bitmap words plus
//                  its winning candidates; re-zeroes the histogram copies.
// The chunk pass writes every bitmap word below N, so only the histogram has
// to start at zero.
struct SelView {
  int N, G, n_pad;
  const float* scores;
  uint32_t* hist;
  uint2* cand;
  uint32_t* bitmap;
  uint32_t* ctr;     // [0] cut bin, [1] count above the cut bin
  uint32_t* ccount;  // per chunk block: candidates
  uint32_t* above;   // per chunk block: entries above the cut bin
};
// Pointers only: nothing here waits for the sequence length, so the loads a
// kernel issues from them can be in flight while the length arrives
// (set_len then gives N and G).
__device__ __forceinline__ SelView sel_view(const IndexerArgs& a, int b) {
  SelView v;
  v.N = 0;
  v.G = 0;
  v.n_pad = ((a.lay.n_max + kSelChunk - 1) / kSelChunk) * kSelChunk;
  v.scores = reinterpret_cast<const float*>(a.ws + a.lay.scores) + (size_t)b * v.n_pad;
  v.hist = reinterpret_cast<uint32_t*>(a.ws + a.lay.hist) + (size_t)b * kHistCopies * kHistBins;
  v.cand = reinterpret_cast<uint2*>(a.ws + a.lay.cand) + (size_t)b * v.n_pad;
  v.bitmap = reinterpret_cast<uint32_t*>(a.ws + a.lay.bitmap) + (size_t)b * (v.n_pad / 32);
  v.ctr = reinterpret_cast<uint32_t*>(a.ws + a.lay.counters) + (size_t)b * 4;
  const int gp = v.n_pad / kSelChunk;
  v.ccount = reinterpret_cast<uint32_t*>(a.ws + a.lay.cand_counts) + (size_t)b * 2 * gp;
  v.above = v.ccount + gp;
  return v;
}
__device__ __forceinline__ void set_len(SelView& v, const IndexerArgs& a, int len_raw) {
  const int L = clampi(len_raw, 0, a.max_len);
  v.N = (L + a.m - 1) / a.m;
  v.G = (v.N + kSelChunk - 1) / kSelChunk;
}

// The cut bin (where the count from the top reaches `need`) and the count
// strictly above it, from the histogram copies: the bins are summed 256 at a
// time from the top, usually once, since the k highest scores sit in the top
// bins.  Every thread of the block gets the result.
// The top slice's per-thread sums (`first`) are loaded by the caller, ahead of
// the sequence length.
__device__ __forceinline__ uint32_t hist_slice_sum(const uint32_t* hist, int top) {
  const int bin = top - (int)threadIdx.x;  // descending with the thread index
  uint32_t c[kHistCopies];
#pragma unroll
  for (int r = 0; r < kHistCopies; ++r) c[r] = bin >= 0 ? hist[(size_t)r * kHistBins + bin] : 0u;
  uint32_t cnt = 0;
#pragma unroll
  for (int r = 0; r < kHistCopies; ++r) cnt += c[r];
  return cnt;
}
__device__ void find_cut_copies(const uint32_t* hist, uint32_t first, uint32_t need, uint32_t* tmp, int& cut,
                                uint32_t& above) {
  __shared__ int cut_s;
  __shared__ uint32_t above_s;
  uint32_t run = 0;  // entries in the bins already passed
  for (int top = kHistBins - 1; top >= 0; top -= kSelThreads) {
    const int bin = top - (int)threadIdx.x;
    const uint32_t cnt = top == kHistBins - 1 ? first : hist_slice_sum(hist, top);
    uint32_t total;
    const uint32_t before = run + block_excl_scan(cnt, tmp, total);
    if (run + total >= need) {  // the cut is in this slice
      if (before < need && before + cnt >= need) {
        cut_s = bin;
        above_s = before;
      }
      __syncthreads();
      cut = cut_s;
      above = above_s;
      __syncthreads();
      return;
    }
    run += total;
  }
  cut = 0;  // not reached: more than k entries were scored
  above = run;
}

__global__ __launch_bounds__(kSelThreads) void select_chunk_kernel(IndexerArgs a) {
  const int b = blockIdx.y;
  SelView v = sel_view(a, b);
  const int len_raw = a.lens[b];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // this block's scores and the histogram's top slice are loaded with the
  // length, unconditionally (a block past the last score chunk, which the grid
  // has when k exceeds the entries, reads chunk 0 and uses nothing)
  constexpr int kUnroll = kSelChunk / 256;  // one round of loads per wave
  const int c0 = blockIdx.x * kSelChunk;
  const int base0 = (c0 < v.n_pad ? c0 : 0) + wave * 64 * kUnroll;
  float sc[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) sc[u] = v.scores[base0 + 64 * u + lane];
  const uint32_t top_cnt = hist_slice_sum(v.hist, kHistBins - 1);
  __builtin_amdgcn_sched_barrier(0);
  set_len(v, a, len_raw);
  const int N = v.N, k = a.k;
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
  if ((int)blockIdx.x >= v.G) return;
  const int c1 = min(N, c0 + kSelChunk);  // scores at c1 and past it are not used
  __shared__ uint32_t tmp[kSelThreads / 64];
  int cut;
  uint32_t above;
  find_cut_copies(v.hist, top_cnt, (uint32_t)k, tmp, cut, above);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    v.ctr[0] = (uint32_t)cut;
    v.ctr[1] = above;
  }
  // a wave classifies 64 consecutive entries per step (coalesced); its ballot
  // is two bitmap words; cut-bin entries take positions from an LDS counter
  // (no returning global atomic stalls the wave)
  __shared__ uint32_t nc_s, na_s;
  if (threadIdx.x == 0) nc_s = na_s = 0;
  __syncthreads();
  uint32_t n_above = 0;  // kept-for-sure entries seen by this wave (lane 0)
  uint2* cand_blk = v.cand + (size_t)blockIdx.x * kSelChunk;
  {
    const int base = base0;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int e0 = base + 64 * u;
      if (e0 >= c1) break;
      const int e = e0 + lane;
      const bool in = e < c1;
      const uint32_t key = order_key(sc[u]);
      const int bin = (int)(key >> 20);
      const uint64_t selm = __ballot(in && bin > cut);
      const uint64_t cm = __ballot(in && bin == cut);
      if (lane == 0) v.bitmap[e0 >> 5] = (uint32_t)selm;
      n_above += (uint32_t)__popcll(selm);
      if (lane == 1 && e0 + 32 < N) v.bitmap[(e0 >> 5) + 1] = (uint32_t)(selm >> 32);
      if (cm) {
        uint32_t basepos = 0;
        if (lane == 0) basepos = atomicAdd(&nc_s, (uint32_t)__popcll(cm));
        basepos = __shfl(basepos, 0, 64);
        if (in && bin == cut) {
          const uint32_t rank = (uint32_t)__popcll(cm & ((1ull << lane) - 1ull));
          cand_blk[basepos + rank] = make_uint2(key, (uint32_t)e);
        }
      }
    }
  }
  if (lane == 0) atomicAdd(&na_s, n_above);
  __syncthreads();
  if (threadIdx.x == 0) {
    v.ccount[blockIdx.x] = nc_s;
    v.above[blockIdx.x] = na_s;
  }
}

// The exact cut from the candidates (cut-bin entries of every chunk block):
// they are staged in LDS (unless there are more than kCandLds; then every pass
// reads their regions), two 10-bit radix passes find the exact cut key T, and
// ties at T keep the lowest indices (index bound X).  Winners: key > T, or
// key == T and index <= X (all candidates when take_all).  Also counts the
// winners of every chunk into wc_s.  Runs in every compaction block (the
// candidates are few, so each block resolving them is cheaper than one more
// launch); block-wide, every thread gets the result.
struct SelLds {
  uint32_t tmp[kSelThreads / 64];
  uint32_t h_s[1024];
  uint32_t pre_s[kMaxSelBlocks + 1];
  uint32_t wc_s[kMaxSelBlocks];
  uint2 cl_s[kCandLds];
};

struct CutKey {
  uint32_t T;
  int X;
  bool take_all;
  bool in_lds;
  uint32_t nc;
};

// Per-thread chunk counts, contiguous: thread t holds chunks t*per .. t*per+per-1
// with per fixed by the padded chunk count, so they can be loaded before the
// sequence length is known (chunks at G and past it are dropped afterwards).
constexpr int kSelPer = kMaxSelBlocks / kSelThreads;
__device__ __forceinline__ int sel_per(const SelView& v) { return (v.n_pad / kSelChunk + kSelThreads - 1) / kSelThreads; }
__device__ __forceinline__ void load_chunk_counts(const SelView& v, const uint32_t* arr, uint32_t loc[kSelPer]) {
  const int per = sel_per(v), gp = v.n_pad / kSelChunk;
#pragma unroll
  for (int u = 0; u < kSelPer; ++u) {
    const int j = threadIdx.x * per + u;
    loc[u] = (u < per && j < gp) ? arr[j] : 0u;
  }
}

__device__ CutKey resolve_cut(const SelView& v, int k, SelLds& sm, int cut, uint32_t above,
                              const uint32_t ccount_pre[kSelPer]) {
  const int N = v.N, G = v.G;
  {
    uint32_t cv = 0;
    const int per = sel_per(v);
    uint32_t loc[kSelPer];
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
      const int j = threadIdx.x * per + u;
      loc[u] = (u < per && j < G) ? ccount_pre[u] : 0u;
      cv += loc[u];
    }
    uint32_t tot;
    uint32_t run = block_excl_scan(cv, sm.tmp, tot);
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
      const int j = threadIdx.x * per + u;
      if (u < per && j < G) sm.pre_s[j] = run;
      run += loc[u];
    }
    if (threadIdx.x == 0) sm.pre_s[G] = tot;
    __syncthreads();
  }
  CutKey r;
  r.nc = sm.pre_s[G];
  r.in_lds = r.nc <= (uint32_t)kCandLds;
  if (r.in_lds) {
    // flat candidate i lives in region j with pre_s[j] <= i < pre_s[j+1]
    constexpr int U = 8;
    for (uint32_t i0 = threadIdx.x; i0 < r.nc; i0 += U * kSelThreads) {
      uint2 cv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t i = i0 + u * kSelThreads;
        int lo = 0, hi = G - 1;  // last region with pre_s[j] <= i
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (sm.pre_s[mid] <= i) lo = mid; else hi = mid - 1;
        }
        cv[u] = i < r.nc ? v.cand[(size_t)lo * kSelChunk + (i - sm.pre_s[lo])] : make_uint2(0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t i = i0 + u * kSelThreads;
        if (i < r.nc) sm.cl_s[i] = cv[u];
      }
    }
    __syncthreads();
  }
  auto for_cands = [&](auto&& f) {
    if (r.in_lds) {
      for (uint32_t i = threadIdx.x; i < r.nc; i += kSelThreads) {
        const uint2 cd = sm.cl_s[i];
        f(cd.x, cd.y);
      }
    } else {
      for (int j = 0; j < G; ++j) {
        const uint2* cb = v.cand + (size_t)j * kSelChunk;
        const uint32_t n = sm.pre_s[j + 1] - sm.pre_s[j];
        for (uint32_t i = threadIdx.x; i < n; i += kSelThreads) {
          const uint2 cd = cb[i];
          f(cd.x, cd.y);
        }
      }
    }
  };
  uint32_t need = (uint32_t)k - above;  // 1 .. nc
  r.take_all = need >= r.nc;
  r.T = 0u;
  r.X = 0x7FFFFFFF;
  if (!r.take_all) {
    uint32_t prefix = (uint32_t)cut << 20, mask = 0xFFF00000u;
    for (int shift = 10; shift >= 0; shift -= 10) {
      for (int i = threadIdx.x; i < 1024; i += kSelThreads) sm.h_s[i] = 0;
      __syncthreads();
      for_cands([&](uint32_t key, uint32_t) {
        if ((key & mask) == prefix) atomicAdd(&sm.h_s[(key >> shift) & 1023u], 1u);
      });
      __syncthreads();
      int c2;
      uint32_t ab2;
      find_cut(sm.h_s, 1024, need, sm.tmp, c2, ab2);
      need -= ab2;
      prefix |= (uint32_t)c2 << shift;
      mask |= 1023u << shift;
    }
    r.T = prefix;  // exact cut key; `need` of the entries with key == T are taken
    const uint32_t ties = sm.h_s[r.T & 1023u];
    if (need < ties) {
      // keep the `need` lowest indices among the ties (binary search on the index bound)
      int lo = 0, hi = N - 1;
      while (lo < hi) {
        const int mid = lo + (hi - lo) / 2;
        uint32_t cnt = 0;
        for_cands([&](uint32_t key, uint32_t e) { cnt += (key == r.T && (int)e <= mid) ? 1u : 0u; });
        uint32_t tot;
        (void)block_excl_scan(cnt, sm.tmp, tot);
        if (tot >= need) hi = mid; else lo = mid + 1;
      }
      r.X = lo;
    }
  }
  for (int j = threadIdx.x; j < G; j += kSelThreads) sm.wc_s[j] = 0u;
  __syncthreads();
  for_cands([&](uint32_t key, uint32_t e) {
    if (r.take_all || key > r.T || (key == r.T && (int)e <= r.X)) atomicAdd(&sm.wc_s[e / kSelChunk], 1u);
  });
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kSelThreads) void select_compact_kernel(IndexerArgs a) {
  // block j writes the kept entries of chunk j: its output offset is the count
  // kept by chunks 0 .. j-1 (entries above the cut bin plus winning candidates)
  const int b = blockIdx.y, j = blockIdx.x;
  SelView v = sel_view(a, b);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Loaded with the length, none of them depending on it: the cut, the
  // per-chunk candidate and above-cut counts, and this chunk's bitmap words
  // (entries above the cut bin; words at N and past it are dropped below).
  const int w = j * (kSelChunk / 32) + lane;
  const uint32_t bits_pre = wave == 0 ? v.bitmap[w] : 0u;
  const int cut_pre = (int)v.ctr[0];
  const uint32_t above_pre = v.ctr[1];
  uint32_t cc_pre[kSelPer], ab_pre[kSelPer];
  load_chunk_counts(v, v.ccount, cc_pre);
  load_chunk_counts(v, v.above, ab_pre);
  set_len(v, a, a.lens[b]);
  const int N = v.N, G = v.G, k = a.k;
  if (N <= k || j >= G) return;
  int32_t* out = a.out_idx + (int64_t)b * k;
  __shared__ SelLds sm;
  __shared__ uint32_t wbits_s[kSelChunk / 32];
  const int W = (N + 31) / 32;
  if (wave == 0) wbits_s[lane] = w < W ? bits_pre : 0u;
  const CutKey ck = resolve_cut(v, k, sm, cut_pre, above_pre, cc_pre);
  // this chunk's winning candidates join its words
  {
    const uint32_t c0 = sm.pre_s[j], c1 = sm.pre_s[j + 1];
    const uint2* cb = v.cand + (size_t)j * kSelChunk;
    for (uint32_t i = c0 + threadIdx.x; i < c1; i += kSelThreads) {
      const uint2 cd = ck.in_lds ? sm.cl_s[i] : cb[i - c0];
      if (ck.take_all || cd.x > ck.T || (cd.x == ck.T && (int)cd.y <= ck.X))
        atomicOr(&wbits_s[(cd.y >> 5) - j * (kSelChunk / 32)], 1u << (cd.y & 31));
    }
  }
  uint32_t before = 0, all = 0;
  {
    const int per = sel_per(v);
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
      const int i = threadIdx.x * per + u;
      if (u < per && i < G) {
        const uint32_t c = ab_pre[u] + sm.wc_s[i];
        all += c;
        before += i < j ? c : 0u;
      }
    }
  }
  uint32_t tot_before, total;
  (void)block_excl_scan(before, sm.tmp, tot_before);
  (void)block_excl_scan(all, sm.tmp, total);  // its barriers also publish wbits_s
  // one word per lane of wave 0
  if (wave == 0) {
    const uint32_t bits0 = w < W ? wbits_s[lane] : 0u;
    const uint32_t pc = (uint32_t)__popc(bits0);
    uint32_t incl = pc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    uint32_t pos = tot_before + incl - pc;
    uint32_t bits = bits0;
    while (bits) {
      const int bit = __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < (uint32_t)k) out[pos] = w * 32 + bit;
      ++pos;
    }
  }
  if (j == G - 1) {
    for (int i = (int)total + threadIdx.x; i < k; i += kSelThreads) out[i] = -1;  // fewer than k: not expected
    if (threadIdx.x == 0) a.out_n[b] = (int)min(total, (uint32_t)k);
  }
  // leave the histogram copies zeroed for the next call: each block a slice
  {
    constexpr int kWords4 = kHistCopies * kHistBins / 4;
    const int per = (kWords4 + G - 1) / G;
    u32x4* h4 = reinterpret_cast<u32x4*>(v.hist);
    for (int i = j * per + threadIdx.x; i < min(kWords4, (j + 1) * per); i += kSelThreads) h4[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

template <int KDT, int DI>
static void launch_score_one(const IndexerArgs& a, hipStream_t s) {
  if (a.keys.epp == 64) {
    const int np = (a.lay.n_max + 63) / 64;
    const dim3 grid((np + kPagesPerScoreBlock - 1) / kPagesPerScoreBlock, a.B);
    hipLaunchKernelGGL((score_pages_kernel<KDT, DI>), grid, dim3(kScoreThreads), 0, s, a);
  } else {
    const dim3 grid((a.lay.n_max + kScoreChunk - 1) / kScoreChunk, a.B);
    hipLaunchKernelGGL((score_kernel<KDT, DI>), grid, dim3(kScoreThreads), 0, s, a);
  }
}

template <int KDT>
static hipError_t launch_score_dt(const IndexerArgs& a, hipStream_t s) {
  switch (a.keys.dim) {
    case 32: launch_score_one<KDT, 32>(a, s); break;
    case 64: launch_score_one<KDT, 64>(a, s); break;
    case 128: launch_score_one<KDT, 128>(a, s); break;
    default: launch_score_one<KDT, 256>(a, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_indexer_score(const IndexerArgs& a, hipStream_t s) {
  if (a.B == 0 || a.lay.n_max == 0) return hipSuccess;
  switch (a.keys.dtype) {
    case HCA_FP8_E4M3: return launch_score_dt<HCA_FP8_E4M3>(a, s);
    case HCA_FP4_E2M1: return launch_score_dt<HCA_FP4_E2M1>(a, s);
    default: return launch_score_dt<HCA_BF16>(a, s);
  }
}

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const hipError_t e = launch_indexer_score(a, s);
  if (e != hipSuccess) return e;
  const int n_max = a.lay.n_max;
  const int gsel = n_max > 0 ? (n_max + kSelChunk - 1) / kSelChunk : 1;
  const int gk = (a.k + kSelChunk - 1) / kSelChunk;
  hipLaunchKernelGGL(select_chunk_kernel, dim3(gsel > gk ? gsel : gk, a.B), dim3(kSelThreads), 0, s, a);
  hipLaunchKernelGGL(select_compact_kernel, dim3(gsel, a.B), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hca
