// paged_hybrid_decode: the decode query attends to the selected compressed
// entries plus the raw window, one shared K=V row each (V4 page, section 2.1:
// keys and values share one RoPE-rotated vector and the output is rotated back
// by inverse RoPE; section 2.3: every layer keeps a raw window; vLLM-0.7.2
// page, section 2.3: only window blocks are read).
//
// Work split: block = (split of the sequence's row list, sequence, 64-head
// group); wave w owns 16 query heads.  A split is at most kMaxTiles tiles of
// 32 rows, and the block issues the gathers of ALL its tiles before it waits
// for any of them (random 512-byte rows cost a full HBM round trip each, so
// the bytes in flight, not the arithmetic, set the pace); splits are sized so
// that all blocks are resident at once.  The rows are
// gathered through the block table with 16-byte loads (8 lanes cover 128
// contiguous bytes of 8 rows) and written to LDS row-major as f16.
//
// fp8 rows are converted without their page scale (every E4M3 value is exact
// in f16, so no overflow or rounding whatever the scale); the scale is applied
// per row in fp32: to the logit after the QK product, and to the probability
// before the PV product as scale/sigma (sigma = the split's largest scale,
// folded back into the partial output).  The rotated query is multiplied by a
// power of two per head so that its f16 copy is exact in range.
//
// Both MFMA contractions are v_mfma_f32_16x16x32_f16:
//   S^T[rows x heads] = K[rows x d] . Q~^T          (wave w: its 16 heads, all d)
//   O[heads x d]     += P[heads x rows] . V[rows x d]  (wave w: all 64 heads, d/4 dims)
// Each wave's P goes through LDS to the other three, so a V fragment read
// from LDS feeds four MFMAs instead of one.
// The V operand (8 rows of one dim per lane) is read from the same row-major
// copy with ds_read_b64_tr_b16: within each 16-lane group, output lane i gets
// element i%4 of the 8-byte runs addressed by source lanes i/4, i/4+4, i/4+8,
// i/4+12, so source lane j addresses row R(j/4) at dims 4(j%4).. and lane i
// receives rows R(0..3) at dim i.
// The S^T accumulator of a lane is exactly its P operand for the PV step when
// the PV k-slot (g, j) is mapped to row 4g+j (j < 4) / 16+4g+j-4 (j >= 4), so
// P is shared lane for lane.  The online softmax works in base 2 (log2(e) is
// folded into the logit factor, so P = 2^(x - m) is one v_exp_f32); it keeps a
// running max per head and rescales the O accumulator only when the tile max
// exceeds it by more than 8 (P <= 2^8 in f16), which makes the rescale rare.
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
constexpr int kMaxTiles = 8;  // tiles of one split, all in flight at once
constexpr int kMaxRowsPerSplit = kTileRows * kMaxTiles;
// A one-tile split keeps two blocks on a CU (<= 256 VGPRs); longer splits hold
// their tiles in registers and run one block per CU.  Splits are sized so that
// every block is resident at once: each then pays one HBM round trip.
constexpr int kCUs = 256;
constexpr int kMaxSplits = kAttnMaxSplits;

static inline size_t align256a(size_t x) { return (x + 255) & ~(size_t)255; }

AttnPlan attn_plan(int B, int H, int d, int max_seq_len, int m, int window, int k, bool has_sel) {
  AttnPlan p;
  const int n_max = (max_seq_len + m - 1) / m;
  const int ent = has_sel ? (k < n_max ? k : n_max) : n_max;
  const int win = window < max_seq_len ? window : max_seq_len;
  p.rows_max = ent + win;
  p.head_blocks = (H + kHeadsPerBlock - 1) / kHeadsPerBlock;
  // one tile per split if two blocks per CU cover the rows, else the fewest
  // tiles (1..6, or 8) that fit one block per CU
  const int64_t units = (int64_t)(B > 0 ? B : 1) * p.head_blocks;
  const int64_t tiles = (p.rows_max + kTileRows - 1) / kTileRows;
  int64_t tps = 1;
  if (tiles * units > 2 * kCUs) {
    tps = (tiles * units + kCUs - 1) / kCUs;
    tps = tps > 6 ? kMaxTiles : tps;
  }
  p.tiles = (int)tps;
  p.rows_per_split = kTileRows * p.tiles;
  const int64_t splits = p.rows_max > 0 ? (p.rows_max + p.rows_per_split - 1) / p.rows_per_split : 1;
  p.splits = (int)(splits > 2 * (int64_t)kMaxSplits ? 2 * (int64_t)kMaxSplits : splits);  // caller rejects > kMaxSplits
  size_t off = 0;
  p.o_off = off; off = align256a(off + (size_t)B * p.splits * H * d * sizeof(float));
  p.ml_off = off; off = align256a(off + (size_t)B * p.splits * H * 2 * sizeof(float));
  p.total = off;
  return p;
}

// LDS-only barrier: orders the block's LDS accesses without waiting for its
// outstanding global loads (a full __syncthreads also drains those).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Address of one row of the sequence's row list (selected entries, then window
// tokens); 0 when the row is skipped (index outside [0, N) or unmapped page).
// `sidx` is the row's page in its pool, for the page scale.
// `e_sel` is the row's selected entry index, loaded by the caller ahead of
// time (ignored without a selection); without a selection `phys_pre` is the
// page of entry r, also loaded ahead of time.
__device__ __forceinline__ uint64_t resolve_row(const AttnArgs& a, int b, int r, int e_sel, int phys_pre, int n_sel,
                                                int N, int L, int n_win, int row_bytes, bool& in_win, int& sidx) {
  int phys, slot, np, epp;
  uint64_t base;
  if (r < n_sel) {
    const int e = a.sel ? e_sel : r;
    if (e < 0 || e >= N) return 0;
    epp = a.kv.epp;
    phys = a.sel ? a.bt[(int64_t)b * a.bts + e / epp] : phys_pre;
    slot = e % epp;
    np = a.kv.num_pages;
    base = reinterpret_cast<uint64_t>(a.kv.codes);
    in_win = false;
  } else {
    const int t = L - n_win + (r - n_sel);
    epp = a.win.epp;
    phys = a.wbt[(int64_t)b * a.wbts + t / epp];
    slot = t % epp;
    np = a.win.num_pages;
    base = reinterpret_cast<uint64_t>(a.win.codes);
    in_win = true;
  }
  if (phys < 0 || phys >= np) return 0;
  sidx = phys;
  return base + ((uint64_t)phys * epp + slot) * row_bytes;
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// LDS tile layout.  For D >= 128 a row holds its D halves unpadded and the
// 16-byte chunk c of row r sits at chunk c ^ swz(r): the 16 rows a QK read
// touches and the 8 rows x 32 bytes a transposed PV read touches then fall on
// distinct banks.  D = 64 rows (8 chunks) are padded instead.
template <int D>
struct TileLayout {
  static constexpr bool kSwz = D >= 128;
  static constexpr int STR = kSwz ? D : D + 16;  // halves per row
  __device__ static __forceinline__ int swz(int r) { return kSwz ? (((r & 7) << 1) | ((r >> 3) & 1)) : 0; }
  // half index of chunk c (8 halves) of row r
  __device__ static __forceinline__ int chunk(int r, int c) { return r * STR + ((c ^ swz(r)) << 3); }
};
typedef short s4 __attribute__((ext_vector_type(4)));

// the 4 rows x 16 dims one loader thread gathers per tile (raw bytes).  The
// gather is unconditional and branch-free: a skipped row, a thread with no
// chunk, or a tile past the end reads the pool's first row (masked when the
// tile is decoded), so no wait is forced before the tile is used.
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

template <int D, int KVDT, int TILES>
__global__ __launch_bounds__(kAttnThreads, TILES == 1 ? 2 : 1) void attn_split_kernel(AttnArgs a) {
  constexpr int KS = D / 32;          // k-steps of the S contraction
  constexpr int NTW = D / 64;         // 16-dim tiles of O per wave (a quarter of the dims)
  using TL = TileLayout<D>;
  constexpr int CHUNKS = D / 16;      // 16-dim chunks per row (load phase)
  constexpr int RPS = kTileRows * TILES;
  constexpr bool kFp8 = KVDT == HCA_FP8_E4M3;
  __shared__ _Float16 k_s[kTileRows * TL::STR];
  __shared__ float2 cs_s[D / 2];
  __shared__ uint64_t rowptr_s[RPS];
  __shared__ __attribute__((aligned(16))) float ratio_s[RPS];  // page scale / sigma; -1 marks a skipped row
  __shared__ float red_s[kAttnThreads / 64];
  __shared__ f16x8 p_s[4][64];        // each wave's P operand, shared for the PV step
  __shared__ float al_s[4][16];       // rescale factor of each head this tile
  __shared__ int rs_s[4];             // did the head group rescale this tile

  const int s = blockIdx.x, b = blockIdx.y, hb = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  // loaded before the lengths are known: the selected entry of this thread's
  // row, or (no selection: row r is entry r) the page of that entry
  int e_sel = 0, phys_pre = 0;
  if (threadIdx.x < RPS) {
    const int r = s * a.plan.rows_per_split + (int)threadIdx.x;
    if (a.sel != nullptr)
      e_sel = gload<int>(a.sel + (int64_t)b * a.k + min(r, a.k - 1));
    else
      phys_pre = gload<int>(a.bt + (int64_t)b * a.bts + min(r / a.kv.epp, a.bts - 1));
  }
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

  // ---- query loads (bf16): in flight while the rows are resolved
  const bool hv = head < H;
  u32x4 qraw[KS];
  {
    const uint16_t* qrow = a.q + ((int64_t)b * H + (hv ? head : H - 1)) * D;
#pragma unroll
    for (int t = 0; t < KS; ++t) qraw[t] = gload<u32x4>(qrow + 32 * t + 8 * g);
  }

  // ---- row addresses of the split; page scales are loaded now, used later
  constexpr int row_bytes = kFp8 ? D : 2 * D;
  float pscale = 0.0f;
  bool row_ok = false;
  if (threadIdx.x < RPS) {
    const int r = r0 + threadIdx.x;
    uint64_t rp = 0;
    bool in_win = false;
    int sidx = 0;
    if (r < r1) rp = resolve_row(a, b, r, e_sel, phys_pre, n_sel, N, L, n_win, row_bytes, in_win, sidx);
    rowptr_s[threadIdx.x] = rp;
    row_ok = rp != 0;
    if constexpr (kFp8) {
      const float* sc = reinterpret_cast<const float*>(in_win ? a.win.scales : a.kv.scales);
      pscale = gload<float>(sc + (rp ? sidx : 0));
      if (rp == 0) pscale = 0.0f;
    } else {
      pscale = rp ? 1.0f : 0.0f;
    }
  }
  lds_barrier();

  // ---- every tile's gather, issued before anything waits for one
  const int q4 = threadIdx.x & 7;
  const int c16 = threadIdx.x >> 3;
  const bool loader = c16 < CHUNKS;
  const uint8_t* safe = reinterpret_cast<const uint8_t*>(a.kv.codes);
  const int c16e = loader ? c16 : 0;
  RowRaw<KVDT> raw[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) raw[t].gather(rowptr_s, kTileRows * t + 4 * q4, r0 + kTileRows * t < r1, c16e, safe);

  // ---- meanwhile: RoPE table at the query position L-1, sigma, row ratios
  for (int i = threadIdx.x; i < D / 2; i += kAttnThreads) {
    float c, sn;
    rope_cs((double)(L - 1), rope_inv_freq(i, D, a.theta), c, sn);
    cs_s[i] = make_float2(c, sn);
  }
  {
    const float wm = wave_max(pscale);
    if (lane == 0) red_s[wave] = wm;
  }
  lds_barrier();
  float sigma = fmaxf(fmaxf(red_s[0], red_s[1]), fmaxf(red_s[2], red_s[3]));
  sigma = sigma > 0.0f ? sigma : 1.0f;
  if (threadIdx.x < RPS) ratio_s[threadIdx.x] = row_ok ? pscale / sigma : -1.0f;

  // ---- rotated query fragments: lane holds Q~[head][32t + 8g + j] x qs, j < 8,
  // with qs a power of two that puts the head's largest |value| in [2^13, 2^14)
  f16x8 qf[KS];
  float hfac;  // base-2 logit = S x ratio x hfac
  {
    // pass 1: largest |component| of the rotated head; pass 2: rotate again, scale, round
    auto rot = [&](int t, int p, float& y0, float& y1) {
      const float x0 = u2f(qraw[t][p] << 16), x1 = u2f(qraw[t][p] & 0xFFFF0000u);
      const float2 cs = cs_s[(32 * t + 8 * g) / 2 + p];
      y0 = x0 * cs.x - x1 * cs.y;
      y1 = x0 * cs.y + x1 * cs.x;
    };
    float amax = 0.0f;
#pragma unroll
    for (int t = 0; t < KS; ++t) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float y0, y1;
        rot(t, p, y0, y1);
        amax = fmaxf(amax, fmaxf(fabsf(y0), fabsf(y1)));
      }
    }
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    int e = 0;
    if (amax > 0.0f) (void)frexpf(amax, &e);  // amax < 2^e
    const float qs = ldexpf(1.0f, min(14 - e, 126));
    hfac = a.scale * sigma / qs * 1.4426950408889634f;  // logits in base 2: p = 2^(x - m)
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      f16x8 v;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float y0, y1;
        rot(t, p, y0, y1);
        v[2 * p] = (_Float16)(y0 * qs);
        v[2 * p + 1] = (_Float16)(y1 * qs);
      }
      qf[t] = v;
    }
  }

  // O for all 64 heads (head group hg, rows 4g + i) over this wave's dims
  // 16 (wave * NTW + n) + col
  f32x4 oacc[4][NTW];
#pragma unroll
  for (int hg = 0; hg < 4; ++hg)
#pragma unroll
    for (int n = 0; n < NTW; ++n) oacc[hg][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;  // for head `head` (replicated over g)

#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    const int tr0 = r0 + kTileRows * t;
    if (tr0 >= r1) break;  // uniform over the block
    const int lr0 = kTileRows * t;
    // ---- write this tile's 32 rows to LDS as f16 (skipped rows as zeros)
    if (loader) {
      const f32x4 rok = *reinterpret_cast<const f32x4*>(&ratio_s[lr0 + 4 * q4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = rok[i] >= 0.0f;
        f16x8 lo, hi;
        const u32x4 z = {0u, 0u, 0u, 0u};
        if constexpr (KVDT == HCA_BF16) {
          const u32x4 w0 = ok ? raw[t].w[i][0] : z, w1 = ok ? raw[t].w[i][1] : z;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            lo[2 * q] = (_Float16)u2f(w0[q] << 16);
            lo[2 * q + 1] = (_Float16)u2f(w0[q] & 0xFFFF0000u);
            hi[2 * q] = (_Float16)u2f(w1[q] << 16);
            hi[2 * q + 1] = (_Float16)u2f(w1[q] & 0xFFFF0000u);
          }
        } else {
          const u32x4 w = ok ? raw[t].w[i][0] : z;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f16x2 x = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w[q], 1.0f, false);
            const f16x2 y = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w[q], 1.0f, true);
            f16x8& dst = q < 2 ? lo : hi;
            const int o = (q & 1) * 4;
            dst[o + 0] = x[0];
            dst[o + 1] = x[1];
            dst[o + 2] = y[0];
            dst[o + 3] = y[1];
          }
        }
        *reinterpret_cast<f16x8*>(&k_s[TL::chunk(4 * q4 + i, 2 * c16)]) = lo;
        *reinterpret_cast<f16x8*>(&k_s[TL::chunk(4 * q4 + i, 2 * c16 + 1)]) = hi;
      }
    }
    lds_barrier();

    // ---- S^T = K . Q~^T for the two 16-row halves: four independent MFMA
    // chains (half h, k-step parity); lane reads chunk 4kt + g of row 16h + col.
    // Fragments are read in batches of 8 before their MFMAs issue, so the LDS
    // latency is paid once per batch rather than once per MFMA.
    f32x4 sacc[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) sacc[h][0] = sacc[h][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int KB = KS < 4 ? KS : 4;  // k-steps per batch
#pragma unroll
    for (int kb = 0; kb < KS; kb += KB) {
      f16x8 kf[KB][2];
#pragma unroll
      for (int u = 0; u < KB; ++u) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          kf[u][h] = *reinterpret_cast<const f16x8*>(&k_s[TL::chunk(16 * h + col, 4 * (kb + u) + g)]);
      }
#pragma unroll
      for (int u = 0; u < KB; ++u) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          sacc[h][u & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[u][h], qf[kb + u], sacc[h][u & 1], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * KB, 0);  // the LDS reads first,
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * KB, 0);  // then the MFMAs
    }
    f32x4 sres[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) sres[h] = sacc[h][0] + sacc[h][1];
    // lane: rows 16h + 4g + i, head `head`
    float x[8], rr[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 rq = *reinterpret_cast<const f32x4*>(&ratio_s[lr0 + 16 * h + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = rq[i] >= 0.0f;  // also false past the end of the split
        rr[4 * h + i] = ok ? rq[i] : 0.0f;
        const float v = ok ? sres[h][i] * rq[i] * hfac : -INFINITY;
        x[4 * h + i] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const bool need = tmax > m_run + kRescaleSlack;
    float alpha = 1.0f;
    bool resc = false;
    if (__any(need)) {
      const float m_new = need ? tmax : m_run;
      alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;  // 2^-inf = 0 on the first tile
      resc = __any(m_run != -INFINITY);           // the accumulators hold something to rescale
      l_run *= alpha;
      m_run = m_new;
    }
    f16x8 pf;
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = x[j] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[j] - m_run);
      psum += p;
      pf[j] = (_Float16)(p * rr[j]);
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run += psum;

    // ---- share P and the rescale factors: each wave then accumulates O for
    // all 64 heads over its quarter of the dims, so one V fragment feeds four
    // MFMAs (one per head group)
    p_s[wave][lane] = pf;
    if (g == 0) al_s[wave][col] = alpha;
    if (lane == 0) rs_s[wave] = resc ? 1 : 0;
    lds_barrier();
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
      if (__builtin_amdgcn_readfirstlane(rs_s[hg])) {  // the same for every lane
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = al_s[hg][4 * g + i];
#pragma unroll
        for (int n = 0; n < NTW; ++n) {
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[hg][n][i] *= al[i];
        }
      }
    }
    f16x8 pa[4];
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) pa[hg] = p_s[hg][lane];

    // ---- O += P . V  (V operand: two transposing LDS reads of 4 rows each)
    // lane reads row R (and R + 16) at dims 16nn + 4(col & 3): chunk 2nn + (col & 3) / 2
    const int vr = 4 * g + (col >> 2);
    f16x8 vf[NTW];
#pragma unroll
    for (int n = 0; n < NTW; ++n) {
      const int nn = wave * NTW + n;
      const int vo = TL::chunk(vr, 2 * nn + ((col & 3) >> 1)) + 4 * (col & 1);
      const s4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(&k_s[vo]));
      const s4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s4*)(&k_s[vo + 16 * TL::STR]));
      const u32x4 vv = {__builtin_bit_cast(u32x2, v0)[0], __builtin_bit_cast(u32x2, v0)[1],
                        __builtin_bit_cast(u32x2, v1)[0], __builtin_bit_cast(u32x2, v1)[1]};
      vf[n] = __builtin_bit_cast(f16x8, vv);
    }
#pragma unroll
    for (int n = 0; n < NTW; ++n) {
#pragma unroll
      for (int hg = 0; hg < 4; ++hg)
        oacc[hg][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[hg], vf[n], oacc[hg][n], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * NTW + 4, 0);  // the LDS reads first,
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * NTW, 0);      // then the MFMAs
    lds_barrier();
  }

  // ---- partials: o (unnormalized, relative to m_run, sigma folded back), m, l
#pragma unroll
  for (int hg = 0; hg < 4; ++hg) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = hb * kHeadsPerBlock + hg * 16 + 4 * g + i;
      if (h < H) {
        float* dst = opart + (part + h) * D + 16 * wave * NTW + col;
#pragma unroll
        for (int n = 0; n < NTW; ++n) dst[16 * n] = oacc[hg][n][i] * sigma;
      }
    }
  }
  if (g == 0 && hv) ml[part + head] = make_float2(m_run * 0.6931471805599453f, l_run);  // m back to base e
}

// Merge the splits of one (sequence, head), then inverse RoPE at L-1.  The
// threads form SG split groups; a group's lanes cover the D dims with 16-byte
// loads and the group takes every SG-th split.  All partial loads of a round
// (up to kCombU splits per thread) are issued together with the (m, l) loads
// of the splits, so a round costs one memory round trip; the groups' sums meet
// in LDS in a fixed order.
constexpr int kCombThreads = 256;
constexpr int kCombU = 36;

template <int D>
__global__ __launch_bounds__(kCombThreads) void attn_combine_kernel(AttnArgs a) {
  constexpr int TPG = D / 4;                  // threads per split group (one float4 each)
  constexpr int SG = kCombThreads / TPG;      // split groups: 2 (D=512) .. 16 (D=64)
  const int h = blockIdx.x, b = blockIdx.y;
  const int H = a.H;
  const int grp = threadIdx.x / TPG, li = threadIdx.x % TPG;
  const int L = clampi(a.lens[b], 0, a.max_len);
  const int N = (L + a.m - 1) / a.m;
  const int n_sel = a.sel ? clampi(a.sel_n[b], 0, a.k) : N;
  const int rows_b = n_sel + min(a.window, L);
  const int S = min(a.plan.splits, (rows_b + a.plan.rows_per_split - 1) / a.plan.rows_per_split);
  const float2* ml = reinterpret_cast<const float2*>(a.ws + a.plan.ml_off) + (size_t)b * a.plan.splits * H + h;
  const f32x4* opart =
      reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.ws + a.plan.o_off) + ((size_t)b * a.plan.splits * H + h) * D) + li;
  const size_t ostride = (size_t)H * D / 4;  // f32x4 between consecutive splits
  __shared__ float w_s[kMaxSplits];
  __shared__ float red_s[kCombThreads / 64];
  __shared__ f32x4 acc_s[SG][TPG];

  // first round of partial loads, issued before anything else waits
  f32x4 o[kCombU];
#pragma unroll
  for (int u = 0; u < kCombU; ++u) {
    const int s = grp + SG * u;
    o[u] = opart[(size_t)(s < S ? s : 0) * ostride];
  }
  // split maxima -> M; weights w_s = exp(m_s - M) (0 for empty splits); tot = sum w_s l_s
  float mloc = -INFINITY;
  for (int s = threadIdx.x; s < S; s += kCombThreads) mloc = fmaxf(mloc, ml[(size_t)s * H].x);
  mloc = wave_max(mloc);
  if ((threadIdx.x & 63) == 0) red_s[threadIdx.x >> 6] = mloc;
  __syncthreads();
  const float M = fmaxf(fmaxf(red_s[0], red_s[1]), fmaxf(red_s[2], red_s[3]));
  __syncthreads();
  float* out = a.out + ((int64_t)b * H + h) * D;
  if (M == -INFINITY) {
    for (int c = threadIdx.x; c < D; c += kCombThreads) out[c] = 0.0f;
    if (threadIdx.x == 0 && a.lse) a.lse[(int64_t)b * H + h] = -INFINITY;
    return;
  }
  float tloc = 0.0f;
  for (int s = threadIdx.x; s < S; s += kCombThreads) {
    const float2 v = ml[(size_t)s * H];
    const float w = v.y > 0.0f ? expf(v.x - M) : 0.0f;
    w_s[s] = w;
    tloc += w * v.y;
  }
  tloc = wave_sum(tloc);
  if ((threadIdx.x & 63) == 0) red_s[threadIdx.x >> 6] = tloc;
  __syncthreads();
  const float tot = (red_s[0] + red_s[1]) + (red_s[2] + red_s[3]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = grp;; s0 += SG * kCombU) {
#pragma unroll
    for (int u = 0; u < kCombU; ++u) {
      const int s = s0 + SG * u;
      const float w = s < S ? w_s[s] : 0.0f;
      acc += w * o[u];
    }
    if (s0 + SG * kCombU >= S) break;
#pragma unroll
    for (int u = 0; u < kCombU; ++u) {  // next round (more than SG * kCombU splits)
      const int s = s0 + SG * (kCombU + u);
      o[u] = opart[(size_t)(s < S ? s : 0) * ostride];
    }
  }
  acc_s[grp][li] = acc;
  __syncthreads();
  const float inv_tot = 1.0f / tot;
  for (int pi = threadIdx.x; pi < D / 2; pi += kCombThreads) {
    float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int gq = 0; gq < SG; ++gq) {
      const float* ag = reinterpret_cast<const float*>(acc_s[gq]);
      o0 += ag[2 * pi];
      o1 += ag[2 * pi + 1];
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

template <int D, int KVDT>
static void launch_split(const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.plan.splits, a.B, a.plan.head_blocks);
  switch (a.plan.tiles) {
    case 1: hipLaunchKernelGGL((attn_split_kernel<D, KVDT, 1>), grid, dim3(kAttnThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((attn_split_kernel<D, KVDT, 2>), grid, dim3(kAttnThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL((attn_split_kernel<D, KVDT, 3>), grid, dim3(kAttnThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((attn_split_kernel<D, KVDT, 4>), grid, dim3(kAttnThreads), 0, s, a); break;
    case 5: hipLaunchKernelGGL((attn_split_kernel<D, KVDT, 5>), grid, dim3(kAttnThreads), 0, s, a); break;
    case 6: hipLaunchKernelGGL((attn_split_kernel<D, KVDT, 6>), grid, dim3(kAttnThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((attn_split_kernel<D, KVDT, kMaxTiles>), grid, dim3(kAttnThreads), 0, s, a); break;
  }
}

template <int D>
static hipError_t launch_attn_d(const AttnArgs& a, hipStream_t s) {
  if (a.kv.dtype == HCA_FP8_E4M3)
    launch_split<D, HCA_FP8_E4M3>(a, s);
  else
    launch_split<D, HCA_BF16>(a, s);
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
