// paged_hybrid_decode: the decode query attends to the selected compressed
// entries plus the raw window, one shared K=V row each (V4 page, section 2.1:
// keys and values share one RoPE-rotated vector and the output is rotated back
// by inverse RoPE; section 2.3: every layer keeps a raw window; vLLM-0.7.2
// page, section 2.3: only window blocks are read).
//
// Work split: block = (split of the sequence's row list, sequence, group of
// 16 query heads); the four waves of a block take the split's 32-row tiles in
// turn, each with its own online softmax, and merge their states through LDS
// at the end, so the main loop has no block-wide barrier.  A split is sized so
// that the grid fills the chip once: its partial output (16 heads x d fp32) is
// then written once per many rows instead of once per tile.  A wave issues
// its next tile's gather as soon as the current tile is in registers.
//
// fp8 rows are converted without their page scale (every E4M3 value is exact
// in f16, so no overflow or rounding whatever the scale); the scale is applied
// per row in fp32: to the logit after the QK product, and to the probability
// before the PV product as scale/sigma.  sigma is the largest page scale the
// wave has met so far; like the softmax max it only grows, and O is rescaled
// when it grows by more than kSigmaSlack, so P x scale/sigma stays within f16
// range and precision; it is folded back into the partial output.  The
// rotated query is multiplied by a power of two per head so that its f16 copy
// is exact in range.
//
// Both MFMA contractions are v_mfma_f32_16x16x32_f16:
//   S^T[rows x heads] = K[rows x d] . Q~^T          (K operand straight from the gather)
//   O[heads x d]     += P[heads x rows] . V[rows x d]  (V operand through LDS)
// The QK product takes its K operand from the registers the rows were gathered
// into: lane (row r, group g) loads 16 bytes at byte 64u + 16g of row r, and
// the k-slots of each k-step are mapped to those dims (the sum over d does not
// depend on the order of its terms); the query fragments use the same map.
// The same converted f16 values are written to the wave's LDS tile, from which
// the V operand (8 rows of one dim per lane) is read with ds_read_b64_tr_b16:
// within each 16-lane group, output lane i gets element i%4 of the 8-byte runs
// addressed by source lanes i/4, i/4+4, i/4+8, i/4+12, so source lane j
// addresses row R(j/4) at dims 4(j%4).. and lane i receives rows R(0..3) at dim i.
// The S^T accumulator of a lane is exactly its P operand for the PV step when
// the PV k-slot (g, j) is mapped to row 4g+j (j < 4) / 16+4g+j-4 (j >= 4), so
// P needs no exchange.  The online softmax works in base 2 (log2(e) is
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
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kTileRows = 32;
constexpr int kHeadsPerBlock = 16;
constexpr float kRescaleSlack = 8.0f;   // base-2 logit growth before O is rescaled
constexpr float kSigmaSlack = 16.0f;    // page-scale growth before O is rescaled
constexpr int kMaxSplitTiles = 32;  // tiles of one split (row addresses staged in LDS)
constexpr int kMaxSplitRows = kTileRows * kMaxSplitTiles;
// One block per CU (the waves hold a 16-head x d accumulator and two tiles of
// gathers each); the grid is sized to fill the chip once.
constexpr int kCUs = 256;
constexpr int kXcds = 8;
constexpr int kMaxSplits = kAttnMaxSplits;

static inline size_t align256a(size_t x) { return (x + 255) & ~(size_t)255; }

AttnPlan attn_plan(int B, int H, int d, int max_seq_len, int m, int window, int k, bool has_sel) {
  AttnPlan p;
  const int n_max = (max_seq_len + m - 1) / m;
  const int ent = has_sel ? (k < n_max ? k : n_max) : n_max;
  const int win = window < max_seq_len ? window : max_seq_len;
  p.tiles_max = (ent + win + kTileRows - 1) / kTileRows;
  p.head_blocks = (H + kHeadsPerBlock - 1) / kHeadsPerBlock;
  // as many items as give every CU one block, unless splits of kMaxSplitTiles
  // tiles need more
  const int64_t bb = B > 0 ? B : 1;
  const int64_t target = kCUs / p.head_blocks > 0 ? kCUs / p.head_blocks : 1;
  const int64_t need = (bb * p.tiles_max + kMaxSplitTiles - 1) / kMaxSplitTiles;
  // splits sized to fill `target` items; when the splits of kMaxSplitTiles
  // tiles are fewer than that, the grid still holds all of them
  const int64_t cap = (target > need ? target : need) + bb;
  p.spread = (int)target;
  p.items = (int)(cap > 1 << 25 ? 1 << 25 : cap);
  // the work list when every sequence has max_seq_len tokens (the device's
  // formula with those lengths): T tiles a split, S splits a sequence
  const int64_t tot = bb * p.tiles_max;
  int64_t tu = (tot + p.spread - 1) / p.spread;
  tu = tu < 1 ? 1 : (tu > kMaxSplitTiles ? kMaxSplitTiles : tu);
  p.t_uni = (int)tu;
  p.s_uni = (int)((p.tiles_max + tu - 1) / tu);
  p.s_uni = p.s_uni > 0 ? p.s_uni : 1;
  size_t off = 0;
  p.o_off = off; off = align256a(off + (size_t)p.items * H * d * sizeof(float));
  p.ml_off = off; off = align256a(off + (size_t)p.items * H * 4 * sizeof(float));
  p.total = off;
  return p;
}

// ---- the work list, derived by every wave from the lengths alone
// Tiles of sequence b as the plan counts them: an upper bound of its rows from
// its length (min(k, N) selected entries, or all N; then min(W, L) window rows).
__device__ __forceinline__ int plan_tiles(const AttnArgs& a, int L) {
  const int N = (L + a.m - 1) / a.m;
  const int n = a.sel ? min(a.k, N) : N;
  return (n + min(a.window, L) + kTileRows - 1) / kTileRows;
}

// Inclusive prefix sum over the wave, on the VALU: Hillis-Steele steps by DPP
// row shifts inside each row of 16 lanes (lanes shifted in from outside the
// row add 0), then the totals of the rows before, read from lanes 15, 31, 47.
// (A lane shuffle is an LDS round trip; a dozen of them in a row would be a
// microsecond before any work.)
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  return v + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
}
// the wave's sum, uniform (every lane gets it)
__device__ __forceinline__ int wave_sum_i(int v, int lane) { return __builtin_amdgcn_readlane(wave_incl_scan(v, lane), 63); }

struct Work {
  int b;  // sequence (-1: past the work list)
  int s;  // split of b (find by item), or b's first item (find by sequence)
  int T;  // tiles per split
  int S;  // splits of b
  int L;  // b's length, clamped
};

// The first 64 lengths, one per lane: loaded by a kernel before anything
// else, so that waiting for them (vector loads complete in issue order) waits
// for nothing issued after them.
__device__ __forceinline__ int attn_lens0(const AttnArgs& a) {
  const int lane = threadIdx.x & 63;
  const int v = a.lens[min(lane, a.B - 1)];  // unguarded (a.B >= 1): no branch around the load
  return lane < a.B ? v : 0;
}

// Every sequence's tiles are cut into splits of T tiles, with T = ceil(total /
// spread) clamped to [1, kMaxSplitTiles], so the splits number at most spread
// + B, or total / kMaxSplitTiles + B when T is clamped (a sequence of t tiles
// has ceil(t / T) <= t / T + 1 of them); items are numbered sequence by
// sequence.  by_item: the split that is item `key`; otherwise the splits of
// sequence `key`.  lens0 is attn_lens0(a).  Called by a whole wave, all lanes
// get the result; every wave of every block of a launch finds the same list.
__device__ Work attn_work(const AttnArgs& a, int key, bool by_item, int lens0) {
  const int lane = threadIdx.x & 63;
  int total = 0;
  const int L0 = clampi(lens0, 0, a.max_len);
  for (int c0 = 0; c0 < a.B; c0 += 64) {
    const int i = c0 + lane;
    const int L = c0 == 0 ? L0 : (i < a.B ? clampi(a.lens[i], 0, a.max_len) : 0);
    total += wave_sum_i(i < a.B ? plan_tiles(a, L) : 0, lane);
  }
  const int T = clampi((total + a.plan.spread - 1) / a.plan.spread, 1, kMaxSplitTiles);
  Work w{-1, 0, T, 0, 0};
  int off = 0;
  for (int c0 = 0; c0 < a.B; c0 += 64) {
    const int i = c0 + lane;
    const int L = c0 == 0 ? L0 : (i < a.B ? clampi(a.lens[i], 0, a.max_len) : 0);
    const int S = i < a.B ? (plan_tiles(a, L) + T - 1) / T : 0;
    const int incl = off + wave_incl_scan(S, lane);
    const int excl = incl - S;
    const bool hit = by_item ? (i < a.B && excl <= key && key < incl) : i == key;
    const uint64_t bal = __ballot(hit);
    if (bal != 0) {
      const int src = __builtin_ctzll(bal);  // uniform: read the hit lane's values with readlane
      w.b = c0 + src;
      w.S = __builtin_amdgcn_readlane(S, src);
      const int ex = __builtin_amdgcn_readlane(excl, src);
      w.s = by_item ? key - ex : ex;
      w.L = __builtin_amdgcn_readlane(L, src);
      break;
    }
    off = __builtin_amdgcn_readlane(incl, 63);
  }
  return w;
}

// Block -> (work item, head group): the head groups of one item run on one XCD
// (one L2: they read the same rows).  Workgroups go to the XCDs in turn, so
// block id i runs on XCD i % 8; the grid is padded to whole rounds.
__device__ __forceinline__ int attn_item_of_block(const AttnArgs& a) {
  const int id = blockIdx.x, HB = a.plan.head_blocks;
  const int item = (id / kXcds / HB) * kXcds + id % kXcds;
  return item < a.plan.items ? item : -1;
}
__device__ __forceinline__ int attn_hb_of_block(const AttnArgs& a) { return (blockIdx.x / kXcds) % a.plan.head_blocks; }

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
    HCA_DBG_CHECK(e >= 0 && e < N, kDbgEntry);
    if (e < 0 || e >= N) return 0;
    epp = a.kv.epp;  // a power of two, like the window's
    const int lg = __builtin_ctz(epp);
    phys = a.sel ? a.bt[(int64_t)b * a.bts + (e >> lg)] : phys_pre;
    slot = e & (epp - 1);
    np = a.kv.num_pages;
    base = reinterpret_cast<uint64_t>(a.kv.codes);
    in_win = false;
  } else {
    const int t = L - n_win + (r - n_sel);
    epp = a.win.epp;
    const int lg = __builtin_ctz(epp);
    phys = a.wbt[(int64_t)b * a.wbts + (t >> lg)];
    slot = t & (epp - 1);
    np = a.win.num_pages;
    base = reinterpret_cast<uint64_t>(a.win.codes);
    in_win = true;
  }
  HCA_DBG_CHECK(phys >= 0 && phys < np, kDbgPage);
  if (phys < 0 || phys >= np) return 0;
  sidx = phys;
  return base + ((uint64_t)phys * epp + slot) * row_bytes;
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));


// LDS tile layout.  For D >= 128 a row holds its D halves unpadded and the
// 16-byte chunk c of row r sits at chunk c ^ swz(r): the 16 rows one tile
// write touches and the 8 rows x 32 bytes a transposed PV read touches then
// fall on distinct banks.  D = 64 rows (8 chunks) are padded instead.
template <int D>
struct TileLayout {
  static constexpr bool kSwz = D >= 128;
  static constexpr int STR = kSwz ? D : D + 16;  // halves per row
  __device__ static __forceinline__ int swz(int r) { return kSwz ? (((r & 7) << 1) | ((r >> 3) & 1)) : 0; }
  // half index of chunk 16 hi + lo (8 halves each, lo < 16) of row r: the
  // swizzle moves a chunk only within its group of 16, so for a fixed lo the
  // group hi is a constant offset
  __device__ static __forceinline__ int at(int r, int lo, int hi) { return r * STR + ((lo ^ swz(r)) << 3) + (hi << 7); }
};
typedef short s4 __attribute__((ext_vector_type(4)));
typedef int i2v __attribute__((ext_vector_type(2)));

// One wave's gather of one tile: lane (col, g) loads rows col and 16 + col of
// the tile, NL 16-byte pieces of each at bytes off(u, g): lane group g takes
// runs of P consecutive pieces, so that the f16 chunks it writes to LDS differ
// from those of the other groups in the low four bits of the chunk index only.
// Branch-free: a skipped row or a row past the split reads the pool's first
// row instead (masked when the tile is used), so no wait is forced before the
// tile is used.
template <int D, int KVDT>
struct TileRaw {
  static constexpr int ROWB = KVDT == HCA_FP8_E4M3 ? D : 2 * D;  // bytes per row
  static constexpr int NL = ROWB / 64;
  static constexpr int P = D >= 128 ? (KVDT == HCA_FP8_E4M3 ? 2 : 4) : 1;
  u32x4 w[2][NL];

  __device__ static __forceinline__ int off(int u, int g) { return 64 * P * (u / P) + 16 * P * g + 16 * (u % P); }

  __device__ __forceinline__ void gather(const uint64_t* rowptr, int lr0, int col, int g, const uint8_t* safe) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint64_t t = rowptr[lr0 + 16 * h + col];
      const uint8_t* p = t ? reinterpret_cast<const uint8_t*>(t) : safe;
#pragma unroll
      for (int u = 0; u < NL; ++u) w[h][u] = gload<u32x4>(p + off(u, g));
    }
  }
};

// First dim of the 8 k-slots that lane group g holds in k-step t: an fp8 load
// gives a lane 16 consecutive dims (two k-steps), a bf16 load 8.
template <int D, int KVDT>
__device__ __forceinline__ int kslot_dim(int t, int g) {
  using Raw = TileRaw<D, KVDT>;
  return KVDT == HCA_FP8_E4M3 ? Raw::off(t >> 1, g) + 8 * (t & 1) : Raw::off(t, g) / 2;
}

// fp8 rows reach LDS through the load-to-LDS path (global_load_lds_dwordx4:
// lane l's 16 bytes land at the instruction's LDS base + 16 l), two tiles per
// wave in flight with no registers held.  A tile is 32 rows x D bytes; the
// 16-byte chunk c of row r sits at position c ^ f(r) within its group of G
// chunks, so that the 16 rows one K read touches and the 8 rows x 2 halves a
// transposing V read touches fall on distinct banks.
template <int D>
struct RawTile {
  static constexpr int CH = D / 16;              // chunks per row
  static constexpr int G = CH < 16 ? CH : 16;    // swizzle group
  static constexpr int BYTES = kTileRows * D;
  static constexpr int INSTR = kTileRows * CH / 64;  // load-to-LDS instructions per tile
  __device__ static __forceinline__ int f(int r) { return ((r & 15) ^ (((r >> 4) & 1) << 3)) & (G - 1); }
  // byte offset of chunk c of row r
  __device__ static __forceinline__ int at(int r, int c) {
    return 16 * (r * CH + ((c & ~(G - 1)) | ((c & (G - 1)) ^ f(r))));
  }
};

// s_waitcnt immediate for "at most n vector memory operations outstanding"
// (the LDS and export counters left free)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// 16 bytes per lane from global memory to LDS: lane l's bytes land at
// lds + 16 l (lds is the same for the whole wave).  Issued as inline assembly,
// so the compiler neither counts it nor makes LDS reads wait for it: the
// kernel waits for these loads itself (vmcnt), and the compiler's own waits
// for other loads stay correct, since loads it does not know of only make the
// outstanding count larger.
__device__ __forceinline__ void load_to_lds16(const void* src, void* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(base) : "memory", "m0");
}

template <int D, int KVDT>
__global__ __launch_bounds__(kAttnThreads, 1) void attn_split_kernel(AttnArgs a) {
  constexpr bool kFp8 = KVDT == HCA_FP8_E4M3;
  constexpr int KS = D / 32;  // k-steps of the S contraction
  constexpr int NB = D / 16;  // 16-dim column blocks of O
  using TL = TileLayout<D>;
  using Raw = TileRaw<D, KVDT>;
  using RT = RawTile<D>;
  constexpr int NL = Raw::NL;
  constexpr int kPer = kMaxSplitRows / kAttnThreads;  // rows each lane resolves
  constexpr int TILE_H = kTileRows * TL::STR;         // halves of one wave's f16 tile (bf16 rows)
  // fp8: two raw tiles per wave, one in each array; bf16: one f16 tile per
  // wave, waves 0-1 in the first array and 2-3 in the second.  The merge
  // reuses both.
  constexpr int kHalfBytes = kFp8 ? kAttnWaves * RT::BYTES : 2 * TILE_H * 2;
  __shared__ __attribute__((aligned(16))) uint8_t tile0_s[kHalfBytes];
  __shared__ __attribute__((aligned(16))) uint8_t tile1_s[kHalfBytes];
  __shared__ f16x8 q_s[KS][64];  // rotated query fragments of the block's heads
  __shared__ float qam_s[kAttnWaves][kHeadsPerBlock];  // per wave: the heads' largest rotated |q|
  __shared__ float2 cs_s[D / 2];
  __shared__ uint64_t rowptr_s[kMaxSplitRows];
  __shared__ __attribute__((aligned(16))) float ps_s[kMaxSplitRows];  // page scale; -1: skipped row
  __shared__ float2 ml_s[kAttnWaves][kHeadsPerBlock];
  __shared__ __attribute__((aligned(16))) float wt_s[kAttnWaves][kHeadsPerBlock];
  static_assert(sizeof(float) * 2 * kHeadsPerBlock * D <= kHalfBytes, "the merge reuses the tiles");

  const int item = attn_item_of_block(a);
  if (item < 0) return;
  const int lens0 = attn_lens0(a);
  const int hb = attn_hb_of_block(a);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, g = lane >> 4;
  // A wave owns the split's tiles wave, wave + 4, ... and resolves their rows
  // itself (lane l: row l % 32 of every other one of them), so nothing but the
  // RoPE table makes a wave wait for another before the merge.
  auto row_of = [&](int j) { return kTileRows * (wave + kAttnWaves * (2 * j + (lane >> 5))) + (lane & 31); };
  const int H = a.H;
  const int h0 = hb * kHeadsPerBlock;
  const int head = h0 + col;  // head of this lane's q / P / m / l
  // each wave loads and rotates a quarter of the query's k-steps (the block's
  // query is 16 x D bf16, read once per block rather than once per wave)
  constexpr int KSW = KS >= kAttnWaves ? KS / kAttnWaves : 1;
  const int tq0 = wave * KSW;
  const bool hv = head < H;
  // the first loads of a work item (sequence bb, split ss of tt tiles): the
  // selected entry of each row, or (no selection: row r is entry r) the page
  // of that entry, and the query (bf16) in the k-slot map
  int pre[kPer];
  u32x4 qraw[KSW];
  auto first_loads = [&](int bb, int ss, int tt) {
    const int rps = kTileRows * tt, rr0 = ss * rps;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = row_of(j);
      const int r = rr0 + min(i, rps - 1);  // loaded unguarded, masked after
      const int v = a.sel != nullptr ? gload<int>(a.sel + (int64_t)bb * a.k + min(r, a.k - 1))
                                     : gload<int>(a.bt + (int64_t)bb * a.bts + min(r >> __builtin_ctz(a.kv.epp), a.bts - 1));
      pre[j] = i < rps ? v : 0;
    }
    const uint16_t* qrow = a.q + ((int64_t)bb * H + (hv ? head : H - 1)) * D;
#pragma unroll
    for (int i = 0; i < KSW; ++i)
      qraw[i] = tq0 + i < KS ? gload<u32x4>(qrow + kslot_dim<D, KVDT>(tq0 + i, g)) : u32x4{0u, 0u, 0u, 0u};
  };
  // issued before the lengths are known, for the work list of equal lengths
  // (max_seq_len each); another list's item gets them again
  const int su = a.plan.s_uni, tu = a.plan.t_uni;
  first_loads(min(item / su, a.B - 1), item % su, tu);  // a guess past the batch loads from its last sequence
  const Work wk = attn_work(a, item, true, lens0);
  if (wk.b < 0) return;  // past the work list
  if (wk.b != item / su || wk.s != item % su || wk.T != tu) first_loads(wk.b, wk.s, wk.T);
  const int b = wk.b, s = wk.s;
  const int RPS = kTileRows * wk.T;  // <= kMaxSplitRows
  const int r0 = s * RPS;
  const int L = wk.L;
  const int N = (L + a.m - 1) / a.m;
  const int n_sel = a.sel ? clampi(a.sel_n[b], 0, a.k) : N;
  const int n_win = min(a.window, L);
  const int rows_b = n_sel + n_win;
  const int r1 = min(rows_b, r0 + RPS);
  f32x4* ml = reinterpret_cast<f32x4*>(a.ws + a.plan.ml_off);
  float* opart = reinterpret_cast<float*>(a.ws + a.plan.o_off);
  const size_t part = (size_t)item * H;

  if (r0 >= r1) {  // empty split
    if (threadIdx.x < kHeadsPerBlock && h0 + (int)threadIdx.x < H)
      ml[part + h0 + threadIdx.x] = f32x4{-INFINITY, 0.0f, 0.0f, 0.0f};
    return;
  }

  // ---- RoPE table at the query position L-1: the one block-wide wait
  for (int i = threadIdx.x; i < D / 2; i += kAttnThreads) {
    float c, sn;
    rope_cs((double)(L - 1), rope_inv_freq(i, a.rope_r), c, sn);
    cs_s[i] = make_float2(c, sn);
  }
  lds_barrier();

  // ---- rotated query fragments: lane holds Q~[head][kslot_dim(t, g) + j] x qs,
  // j < 8, with qs a power of two that puts the head's largest |value| in
  // [2^13, 2^14).  Each wave rotates its quarter of the k-steps, the head
  // maxima meet in LDS, the scaled fragments go to LDS; fp8 rows then keep
  // all of them in registers.
  float hfac;  // base-2 logit = S x page scale x hfac
  f16x8 qf[kFp8 ? KS : 1];
  {
    float y[KSW][8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < KSW; ++i) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float x0 = u2f(qraw[i][p] << 16), x1 = u2f(qraw[i][p] & 0xFFFF0000u);
        const float2 cs = cs_s[(kslot_dim<D, KVDT>(min(tq0 + i, KS - 1), g)) / 2 + p];
        y[i][2 * p] = x0 * cs.x - x1 * cs.y;
        y[i][2 * p + 1] = x0 * cs.y + x1 * cs.x;
        amax = fmaxf(amax, fmaxf(fabsf(y[i][2 * p]), fabsf(y[i][2 * p + 1])));
      }
    }
    amax = rows_max4(amax);
    if (g == 0) qam_s[wave][col] = amax;
    lds_barrier();
    amax = fmaxf(fmaxf(qam_s[0][col], qam_s[1][col]), fmaxf(qam_s[2][col], qam_s[3][col]));
    int e = 0;
    if (amax > 0.0f) (void)frexpf(amax, &e);  // amax < 2^e
    const float qs = ldexpf(1.0f, min(14 - e, 126));
    hfac = a.scale / qs * 1.4426950408889634f;  // logits in base 2: p = 2^(x - m)
#pragma unroll
    for (int i = 0; i < KSW; ++i) {
      f16x8 v;
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] = (_Float16)(y[i][c] * qs);
      if (tq0 + i < KS) q_s[tq0 + i][lane] = v;
    }
    lds_barrier();
    if constexpr (kFp8) {
#pragma unroll
      for (int t = 0; t < KS; ++t) qf[t] = q_s[t][lane];
    }
  }

  // ---- this wave's rows: addresses and page scales, for this wave only.
  // Every row slot of the wave's tiles is written, rows outside the split as
  // skipped, so the loads below need no guard.
  constexpr int row_bytes = Raw::ROWB;
  float ps[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = row_of(j);
    const int r = r0 + i;
    uint64_t rp = 0;
    bool in_win = false;
    int sidx = 0;
    if (i < RPS && r < r1) rp = resolve_row(a, b, r, pre[j], pre[j], n_sel, N, L, n_win, row_bytes, in_win, sidx);
    rowptr_s[i] = rp;
    if constexpr (kFp8) {
      const float* sc = reinterpret_cast<const float*>(in_win ? a.win.scales : a.kv.scales);
      ps[j] = rp ? gload<float>(sc + sidx) : -1.0f;
    } else {
      ps[j] = rp ? 1.0f : -1.0f;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");

  const int nt = (r1 - r0 + kTileRows - 1) / kTileRows;
  const uint8_t* safe = reinterpret_cast<const uint8_t*>(a.kv.codes);
  // fp8: load tile t of the split into one of this wave's two ring slots
  // (skipped rows read the pool's first row; their bytes are masked where they
  // matter)
  uint8_t* slot0 = tile0_s + wave * RT::BYTES;
  uint8_t* slot1 = tile1_s + wave * RT::BYTES;
  auto issue = [&](int t, uint8_t* dst) {
    const int lr0 = kTileRows * t;
#pragma unroll
    for (int j = 0; j < RT::INSTR; ++j) {
      const int pos = 64 * j + lane;  // chunk position this lane fills
      const int r = pos / RT::CH, p = pos % RT::CH;
      const int c = (p & ~(RT::G - 1)) | ((p & (RT::G - 1)) ^ RT::f(r));  // the data chunk stored there
      const uint64_t rp = rowptr_s[lr0 + r];
      const uint8_t* src = (rp ? reinterpret_cast<const uint8_t*>(rp) : safe) + 16 * c;
      load_to_lds16(src, dst + 1024 * j);
    }
  };
  Raw ra;  // bf16: register gather
  if constexpr (kFp8) {
    if (wave < nt) issue(wave, slot0);
    if (wave + kAttnWaves < nt) issue(wave + kAttnWaves, slot1);
  } else {
    ra.gather(rowptr_s, kTileRows * wave, col, g, safe);
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) ps_s[row_of(j)] = ps[j];
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");

  // O for the block's 16 heads (rows 4g + i) over all dims 16n + col, in units
  // of sigma: the largest page scale the wave has seen, up to kSigmaSlack
  f32x4 oacc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) oacc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;  // for head `head` (replicated over g)
  float sigma = 0.0f, inv_sigma = 0.0f;

  // ---- S^T = K . Q~^T for the tile's two 16-row halves.  fp8: K chunks from
  // the ring slot; bf16: from the gathered registers, converted to f16 and
  // also written to the wave's LDS tile for the PV step (skipped rows as zeros)
  // this wave's f16 tile (bf16 rows)
  _Float16* ks = reinterpret_cast<_Float16*>((wave < 2 ? tile0_s : tile1_s) + (wave & 1) * TILE_H * 2);
  auto qk = [&](const Raw& raw, int t, const uint8_t* tile, f32x4 sres[2]) {
    const int lr0 = kTileRows * t;
    f32x4 sacc[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) sacc[h][0] = sacc[h][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kFp8) {
#pragma unroll
      for (int u = 0; u < NL; ++u) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(tile + RT::at(16 * h + col, Raw::off(u, g) / 16));
          f16x8 v0, v1;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f16x2 x = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w[q], 1.0f, false);
            const f16x2 y = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w[q], 1.0f, true);
            f16x8& dst = q < 2 ? v0 : v1;
            const int o = (q & 1) * 4;
            dst[o + 0] = x[0];
            dst[o + 1] = x[1];
            dst[o + 2] = y[0];
            dst[o + 3] = y[1];
          }
          sacc[h][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v0, qf[2 * u], sacc[h][0], 0, 0, 0);
          sacc[h][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v1, qf[2 * u + 1], sacc[h][1], 0, 0, 0);
        }
      }
    } else {
      bool okr[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) okr[h] = ps_s[lr0 + 16 * h + col] >= 0.0f;
      const u32x4 z = {0u, 0u, 0u, 0u};
      constexpr int P = Raw::P;
#pragma unroll
      for (int u = 0; u < NL; ++u) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 w = okr[h] ? raw.w[h][u] : z;
          f16x8 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[2 * q] = (_Float16)u2f(w[q] << 16);
            v[2 * q + 1] = (_Float16)u2f(w[q] & 0xFFFF0000u);
          }
          const int cb = 4 * P * (u / P);
          *reinterpret_cast<f16x8*>(&ks[TL::at(16 * h + col, (cb & 15) + P * g + u % P, cb >> 4)]) = v;
          sacc[h][u & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v, q_s[u][lane], sacc[h][u & 1], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) sres[h] = sacc[h][0] + sacc[h][1];
  };

  // ---- online softmax and page-scale normalization, then O += P . V.  The V
  // operand (8 rows of one dim per lane): fp8, one transposing byte read from
  // the ring slot, skipped rows masked, then converted; bf16, two transposing
  // 16-bit reads of 4 rows from the wave's f16 tile.
  auto softmax = [&](int t, const f32x4 sres[2], f16x8& pf, uint32_t vmask[2]) {
    const int lr0 = kTileRows * t;
    // lane: rows 16h + 4g + i, head `head`
    float x[8], sc[8];
    float tmax = -INFINITY, tsig = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 rq = *reinterpret_cast<const f32x4*>(&ps_s[lr0 + 16 * h + 4 * g]);
      vmask[h] = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = rq[i] >= 0.0f;  // also false past the end of the split
        vmask[h] |= ok ? 0xFFu << (8 * i) : 0u;
        sc[4 * h + i] = ok ? rq[i] : 0.0f;
        const float v = ok ? sres[h][i] * rq[i] * hfac : -INFINITY;
        x[4 * h + i] = v;
        tmax = fmaxf(tmax, v);
        tsig = fmaxf(tsig, sc[4 * h + i]);
      }
    }
    tmax = rows_max4(tmax);
    tsig = rows_max4(tsig);  // the same in every lane
    const bool need = tmax > m_run + kRescaleSlack;
    const bool grow = tsig > sigma * kSigmaSlack;
    if (__any(need) || grow) {
      const float m_new = need ? tmax : m_run;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;  // 2^-inf = 0 on the first tile
      const float fs = grow ? sigma / tsig : 1.0f;
      if (__any(m_run != -INFINITY)) {  // the accumulators hold something to rescale
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i, 64) * fs;  // factor of head 4g + i
#pragma unroll
        for (int n = 0; n < NB; ++n) {
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[n][i] *= al[i];
        }
      }
      l_run *= alpha;
      m_run = m_new;
      if (grow) {
        sigma = tsig;
        inv_sigma = 1.0f / tsig;
      }
    }
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = x[j] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[j] - m_run);
      psum += p;
      pf[j] = (_Float16)(p * (sc[j] * inv_sigma));
    }
    psum = rows_sum4(psum);
    l_run += psum;
  };

  // ---- O += P . V
  auto pv_mma = [&](const uint8_t* tile, const f16x8& pf, const uint32_t vmask[2]) {

    constexpr int VB = NB < 8 ? NB : 8;  // column blocks per batch
    if constexpr (kFp8) {
      // source lane j of a 16-lane group addresses row R(j / 2) at byte 8 (j % 2)
      // of the column block; output lane i then holds rows R(0..7) at dim i
      const int k = col >> 1;
      const int vrow = k < 4 ? 4 * g + k : 16 + 4 * g + k - 4;
      const int half = 8 * (col & 1);
#pragma unroll
      for (int n0 = 0; n0 < NB; n0 += VB) {
        u32x2 raw8[VB];
#pragma unroll
        for (int u = 0; u < VB; ++u) {
          const i2v r8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) i2v*)(tile + RT::at(vrow, n0 + u) + half));
          raw8[u] = __builtin_bit_cast(u32x2, r8);
        }
#pragma unroll
        for (int u = 0; u < VB; ++u) {
          const uint32_t lo = raw8[u][0] & vmask[0], hi = raw8[u][1] & vmask[1];
          const f16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)lo, 1.0f, false);
          const f16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)lo, 1.0f, true);
          const f16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)hi, 1.0f, false);
          const f16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)hi, 1.0f, true);
          const f16x8 vf = {a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
          oacc[n0 + u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf, vf, oacc[n0 + u], 0, 0, 0);
        }
      }
    } else {
      // lane reads row R (and R + 16) at dims 16n + 4(col & 3): chunk 2n + (col & 3) / 2
      const int vr = 4 * g + (col >> 2);
      const int c01 = (col & 3) >> 1;
#pragma unroll
      for (int n0 = 0; n0 < NB; n0 += VB) {
        f16x8 vf[VB];
#pragma unroll
        for (int u = 0; u < VB; ++u) {
          const int n = n0 + u;
          const int vo = TL::at(vr, 2 * (n & 7) + c01, n >> 3) + 4 * (col & 1);
          const s4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(&ks[vo]));
          const s4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s4*)(&ks[vo + 16 * TL::STR]));
          const u32x4 vv = {__builtin_bit_cast(u32x2, v0)[0], __builtin_bit_cast(u32x2, v0)[1],
                            __builtin_bit_cast(u32x2, v1)[0], __builtin_bit_cast(u32x2, v1)[1]};
          vf[u] = __builtin_bit_cast(f16x8, vv);
        }
#pragma unroll
        for (int u = 0; u < VB; ++u) oacc[n0 + u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf, vf[u], oacc[n0 + u], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * VB, 0);  // the LDS reads first,
        __builtin_amdgcn_sched_group_barrier(0x008, VB, 0);      // then the MFMAs
      }
    }
  };

  // ---- the wave's tiles wave, wave + 4, ...  fp8: tile t is in ring slot sl
  // and tile t + 4 may still be loading behind it; a slot is refilled once its
  // reads are done.  bf16: the next tile's gather is issued as soon as the
  // current one's registers are converted.  LDS accesses of one wave complete
  // in issue order, so what qk writes is what pv reads, and pv's reads precede
  // the next qk's writes.
  if constexpr (kFp8) {
    // one ring slot: wait for its tile (the other slot's tile may still be
    // loading behind it), use it, then refill it
    auto step = [&](int t, uint8_t* slot) {
      if (t + kAttnWaves < nt)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(RT::INSTR));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      asm volatile("" ::: "memory");
      f32x4 sres[2];
      qk(ra, t, slot, sres);
      f16x8 pf;
      uint32_t vmask[2];
      softmax(t, sres, pf, vmask);
      pv_mma(slot, pf, vmask);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(63) & ~0x0F00);  // lgkmcnt(0): the slot's reads are done
      asm volatile("" ::: "memory");
      if (t + 2 * kAttnWaves < nt) issue(t + 2 * kAttnWaves, slot);
    };
    int sl = 0;
    for (int t = wave; t < nt; t += kAttnWaves, sl ^= 1) step(t, sl ? slot1 : slot0);
  } else {
    for (int t = wave; t < nt; t += kAttnWaves) {
      f32x4 sres[2];
      qk(ra, t, nullptr, sres);
      if (t + kAttnWaves < nt) ra.gather(rowptr_s, kTileRows * (t + kAttnWaves), col, g, safe);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
      f16x8 pf;
      uint32_t vmask[2];
      softmax(t, sres, pf, vmask);
      pv_mma(nullptr, pf, vmask);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
    }
  }

  // ---- merge the four waves' states: o (unnormalized, relative to the block
  // max), m, l.  The tiles' LDS holds each wave's O as [head quad][dim][4 heads].
  if constexpr (kFp8) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load into the tiles is in flight
  __syncthreads();  // every wave is done with its LDS tiles
  // wave w's O: [4 head quads][D][4] floats at (w < 2 ? first : second array) + (w & 1) x 64 D bytes
  auto o_of = [&](int w) { return reinterpret_cast<float*>((w < 2 ? tile0_s : tile1_s) + (w & 1) * 64 * D); };
  {
    float* o_s = o_of(wave);
#pragma unroll
    for (int n = 0; n < NB; ++n) *reinterpret_cast<f32x4*>(&o_s[(g * D + 16 * n + col) * 4]) = oacc[n] * sigma;
  }
  if (g == 0) ml_s[wave][col] = make_float2(m_run, l_run);
  __syncthreads();
  if (threadIdx.x < kHeadsPerBlock) {
    const int hh = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, ml_s[w][hh].x);
    float l = 0.0f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float wt = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml_s[w][hh].x - M);  // 0 for an empty wave
      wt_s[w][hh] = wt;
      l += wt * ml_s[w][hh].y;
    }
    // fp32 partials are unnormalized: their weight factor is 1
    if (h0 + hh < H)
      ml[part + h0 + hh] = M == -INFINITY ? f32x4{-INFINITY, 0.0f, 0.0f, 0.0f} : f32x4{M * 0.6931471805599453f, l, 1.0f, 0.0f};
  }
  __syncthreads();
  // thread -> (4 consecutive heads, one dim): consecutive threads store consecutive dims
  for (int e = threadIdx.x; e < D * (kHeadsPerBlock / 4); e += kAttnThreads) {
    const int hq = e / D, dim = e - hq * D;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const f32x4 o = *reinterpret_cast<const f32x4*>(&o_of(w)[(hq * D + dim) * 4]);
      const f32x4 wt = *reinterpret_cast<const f32x4*>(&wt_s[w][4 * hq]);
      acc += wt * o;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int h = h0 + 4 * hq + k;
      if (h < H) opart[(part + h) * D + dim] = acc[k];
    }
  }
}

// ---- fp8 rows of 512 dims: pairs of waves split each tile's dims.
// Block of 8 waves = 4 pairs (one block per CU, two waves per SIMD); pair p
// takes the split's tiles p, p + 4, ... as a wave of the 4-wave kernel does.
// Wave half hf of a pair loads, converts and multiplies only dims
// [256 hf, 256 hf + 256) of every row of the pair's tiles: its QK product is
// the partial S over those dims, the two partials are added through LDS (both
// waves then hold the same S and run the same softmax), and its PV product is
// O for those dims.  A wave's tile bytes are its own loads, so it waits for
// nothing of its partner's but the partial S.  Per wave and tile this is half
// the conversions and MFMAs of the 4-wave kernel, and half its accumulator
// and query registers, which leaves room for two waves per SIMD.
constexpr int kPairThreads = 512;
constexpr int kPairWaves = kPairThreads / 64;
constexpr int kPairs = kPairWaves / 2;
constexpr int kPairD = 512;

// One tile in LDS: half hf holds dims [256 hf, +256) of the 32 rows, 16
// chunks of 16 bytes per row, chunk cc of row r at position cc ^ f(r): the 16
// rows one K read touches and the 8 rows a transposing V read touches fall on
// distinct banks.  A half is filled by its wave's own loads.
struct PairTile {
  static constexpr int CHH = kPairD / 2 / 16;                // chunks per half row: 16
  static constexpr int HALF_BYTES = kTileRows * kPairD / 2;  // 8 KB
  static constexpr int BYTES = 2 * HALF_BYTES;
  static constexpr int INSTR = HALF_BYTES / 1024;            // load-to-LDS instructions per half: 8
  __device__ static __forceinline__ int f(int r) { return (r & 15) ^ (((r >> 4) & 1) << 3); }
  __device__ static __forceinline__ int at(int hf, int r, int cc) {
    return hf * HALF_BYTES + 16 * (r * CHH + (cc ^ f(r)));
  }
};

// k-step t (of 16, 32 dims each) of the QK product, lane group g: 8 dims from
// this first dim.  Steps 0-7 are half 0's, 8-15 half 1's; within a half,
// steps 2u and 2u + 1 are the two 8-dim halves of chunk 4u + g.
__device__ __forceinline__ int pair_kdim(int t, int g) {
  return 256 * (t >> 3) + 16 * (4 * ((t & 7) >> 1) + g) + 8 * (t & 1);
}

// The two waves of a pair meet through LDS counters instead of block
// barriers, so a pair never waits for another pair's loads.  flag[w][0] counts
// the steps whose partial S wave w has written, flag[w][1] the steps whose
// partner partial wave w has read.  A wave's LDS operations complete in order
// and the release waits for them (lgkmcnt), so a counter never runs ahead of
// the data it announces.  The spin is bounded (a few ms): if a partner never
// arrives the kernel still ends.
__device__ __forceinline__ void pair_signal(int* flag, int v) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  if ((threadIdx.x & 63) == 0) __hip_atomic_store(flag, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void pair_wait(const int* flag, int v) {
  for (int it = 0; it < (1 << 16); ++it) {
    if (__builtin_amdgcn_readfirstlane(__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) >= v) break;
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__global__ __launch_bounds__(kPairThreads, 1) void attn_pair_kernel(AttnArgs a) {
  constexpr int D = kPairD;
  constexpr int KS = D / 32;     // k-steps of the whole S contraction
  constexpr int KSH = KS / 2;    // k-steps of a half
  constexpr int NBH = D / 2 / 16;  // 16-dim column blocks of a half's O
  using PT = PairTile;
  constexpr int kPer = kMaxSplitRows / kPairThreads;  // rows each lane resolves: 2
  __shared__ __attribute__((aligned(16))) uint8_t tile0_s[kPairs * PT::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t tile1_s[kPairs * PT::BYTES];
  // rotated query fragments; once every wave holds its half in registers, the
  // same memory carries the partial S of each wave to its partner
  __shared__ __attribute__((aligned(16))) f16x8 q_s[KS][64];
  __shared__ float qam_s[kPairWaves][kHeadsPerBlock];
  __shared__ float2 cs_s[D / 2];
  __shared__ uint64_t rowptr_s[kMaxSplitRows];
  __shared__ __attribute__((aligned(16))) float ps_s[kMaxSplitRows];  // page scale; -1: skipped row
  __shared__ float2 ml_s[kPairs][kHeadsPerBlock];
  __shared__ float sg_s[kPairs];
  __shared__ int psync_s[kPairWaves][2];
  static_assert(sizeof(q_s) == (size_t)kPairWaves * 2 * 64 * sizeof(f32x4), "partial S exchange area");
  static_assert(sizeof(float) * kHeadsPerBlock * D / 2 == 2 * PT::HALF_BYTES, "a wave's O fills its halves of its pair's slots");

  const int item = attn_item_of_block(a);
  if (item < 0) return;
  const int lens0 = attn_lens0(a);
  const int hb = attn_hb_of_block(a);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pair = wave >> 1, hf = wave & 1;
  const int col = lane & 15, g = lane >> 4;
  // rows of the pair's tiles, split over its two waves: lane l of wave
  // (pair, hf) resolves row l % 32 of the pair's tiles 4j + 2hf + l / 32
  auto row_of = [&](int j) { return kTileRows * (pair + kPairs * (4 * j + 2 * hf + (lane >> 5))) + (lane & 31); };
  const int H = a.H;
  const int h0 = hb * kHeadsPerBlock;
  const int head = h0 + col;
  // query: each wave loads and rotates 2 of the 16 k-steps
  constexpr int KSW = KS / kPairWaves;
  const int tq0 = wave * KSW;
  const bool hv = head < H;
  // the first loads of a work item (sequence bb, split ss of tt tiles): the
  // selected entry or the page of each row, and the query
  int pre[kPer];
  u32x4 qraw[KSW];
  auto first_loads = [&](int bb, int ss, int tt) {
    const int rps = kTileRows * tt, rr0 = ss * rps;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = row_of(j);
      const int r = rr0 + min(i, rps - 1);  // loaded unguarded, masked after
      const int v = a.sel != nullptr ? gload<int>(a.sel + (int64_t)bb * a.k + min(r, a.k - 1))
                                     : gload<int>(a.bt + (int64_t)bb * a.bts + min(r >> __builtin_ctz(a.kv.epp), a.bts - 1));
      pre[j] = i < rps ? v : 0;
    }
    const uint16_t* qrow = a.q + ((int64_t)bb * H + (hv ? head : H - 1)) * D;
#pragma unroll
    for (int i = 0; i < KSW; ++i) qraw[i] = gload<u32x4>(qrow + pair_kdim(tq0 + i, g));
  };
  // issued before the lengths are known, for the work list of equal lengths
  // (max_seq_len each); another list's item gets them again
  const int su = a.plan.s_uni, tu = a.plan.t_uni;
  first_loads(min(item / su, a.B - 1), item % su, tu);  // a guess past the batch loads from its last sequence
  const Work wk = attn_work(a, item, true, lens0);
  if (wk.b < 0) return;  // past the work list
  if (wk.b != item / su || wk.s != item % su || wk.T != tu) first_loads(wk.b, wk.s, wk.T);
  const int b = wk.b, s = wk.s;
  const int RPS = kTileRows * wk.T;  // <= kMaxSplitRows
  const int r0 = s * RPS;
  const int L = wk.L;
  const int N = (L + a.m - 1) / a.m;
  const int n_sel = a.sel ? clampi(a.sel_n[b], 0, a.k) : N;
  const int n_win = min(a.window, L);
  const int rows_b = n_sel + n_win;
  const int r1 = min(rows_b, r0 + RPS);
  f32x4* ml = reinterpret_cast<f32x4*>(a.ws + a.plan.ml_off);
  _Float16* opart = reinterpret_cast<_Float16*>(a.ws + a.plan.o_off);
  const size_t part = (size_t)item * H;

  if (r0 >= r1) {  // empty split (the whole block returns)
    if (threadIdx.x < kHeadsPerBlock && h0 + (int)threadIdx.x < H)
      ml[part + h0 + threadIdx.x] = f32x4{-INFINITY, 0.0f, 0.0f, 0.0f};
    return;
  }

  // ---- RoPE table at the query position L-1
  for (int i = threadIdx.x; i < D / 2; i += kPairThreads) {
    float c, sn;
    rope_cs((double)(L - 1), rope_inv_freq(i, a.rope_r), c, sn);
    cs_s[i] = make_float2(c, sn);
  }
  lds_barrier();

  // ---- rotated query fragments, scaled per head by a power of two that puts
  // the head's largest |value| in [2^13, 2^14) (exact in f16); each wave then
  // keeps its half's 8 k-steps in registers
  float hfac;
  f16x8 qf[KSH];
  {
    float y[KSW][8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < KSW; ++i) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float x0 = u2f(qraw[i][p] << 16), x1 = u2f(qraw[i][p] & 0xFFFF0000u);
        const float2 cs = cs_s[pair_kdim(tq0 + i, g) / 2 + p];
        y[i][2 * p] = x0 * cs.x - x1 * cs.y;
        y[i][2 * p + 1] = x0 * cs.y + x1 * cs.x;
        amax = fmaxf(amax, fmaxf(fabsf(y[i][2 * p]), fabsf(y[i][2 * p + 1])));
      }
    }
    amax = rows_max4(amax);
    if (g == 0) qam_s[wave][col] = amax;
    lds_barrier();
    amax = 0.0f;
#pragma unroll
    for (int w = 0; w < kPairWaves; ++w) amax = fmaxf(amax, qam_s[w][col]);
    int e = 0;
    if (amax > 0.0f) (void)frexpf(amax, &e);  // amax < 2^e
    const float qs = ldexpf(1.0f, min(14 - e, 126));
    hfac = a.scale / qs * 1.4426950408889634f;  // logits in base 2: p = 2^(x - m)
#pragma unroll
    for (int i = 0; i < KSW; ++i) {
      f16x8 v;
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] = (_Float16)(y[i][c] * qs);
      q_s[tq0 + i][lane] = v;
    }
    lds_barrier();
#pragma unroll
    for (int t = 0; t < KSH; ++t) qf[t] = q_s[KSH * hf + t][lane];
  }

  // ---- rows: addresses and page scales
  float ps[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = row_of(j);
    const int r = r0 + i;
    uint64_t rp = 0;
    bool in_win = false;
    int sidx = 0;
    if (i < RPS && r < r1) rp = resolve_row(a, b, r, pre[j], pre[j], n_sel, N, L, n_win, D, in_win, sidx);
    if (i < RPS) rowptr_s[i] = rp;
    const float* sc = reinterpret_cast<const float*>(in_win ? a.win.scales : a.kv.scales);
    ps[j] = rp ? gload<float>(sc + sidx) : -1.0f;
  }
  // the partner's row addresses are needed for this wave's loads, and every
  // wave is done reading the query fragments before they are overwritten by
  // partial S (LDS only: the scale loads stay in flight)
  lds_barrier();

  const int nt = (r1 - r0 + kTileRows - 1) / kTileRows;
  const uint8_t* safe = reinterpret_cast<const uint8_t*>(a.kv.codes);
  uint8_t* slot0 = tile0_s + pair * PT::BYTES;
  uint8_t* slot1 = tile1_s + pair * PT::BYTES;
  // this wave's half of tile t into a slot (skipped rows read the pool's
  // first row; their bytes are masked where they matter)
  // (the row addresses are read from LDS first, all of them: the loads are
  // inline assembly that the compiler does not move LDS reads across)
  auto issue = [&](int t, uint8_t* dst) {
    const int lr0 = kTileRows * t;
    uint64_t rp[PT::INSTR];
#pragma unroll
    for (int j = 0; j < PT::INSTR; ++j) rp[j] = rowptr_s[lr0 + (64 * j + lane) / PT::CHH];
#pragma unroll
    for (int j = 0; j < PT::INSTR; ++j) {
      const int pos = 64 * j + lane;  // chunk position this lane fills in the half
      const int r = pos / PT::CHH, p = pos % PT::CHH;
      const int cc = p ^ PT::f(r);  // the data chunk stored there
      const uint8_t* src = (rp[j] ? reinterpret_cast<const uint8_t*>(rp[j]) : safe) + (D / 2) * hf + 16 * cc;
      load_to_lds16(src, dst + PT::HALF_BYTES * hf + 1024 * j);
    }
  };
  if (pair < nt) issue(pair, slot0);  // the pair's second tile goes out once its first has landed
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (row_of(j) < RPS) ps_s[row_of(j)] = ps[j];
  if (lane < 2) psync_s[wave][lane] = 0;
  lds_barrier();  // every row's page scale is visible to both waves of its pair

  f32x4 oacc[NBH];  // O for the 16 heads (rows 4g + i) over dims 256 hf + 16n + col, in units of sigma
#pragma unroll
  for (int n = 0; n < NBH; ++n) oacc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;  // the same in both waves of a pair
  float sigma = 0.0f, inv_sigma = 0.0f;
  f32x4* xs = reinterpret_cast<f32x4*>(&q_s[0][0]);  // [wave][h][lane]: partial S

  // ---- this wave's partial S^T = K[:, half] . Q~[:, half]^T for the tile's two 16-row halves
  auto qk_half = [&](const uint8_t* tile, f32x4 sres[2]) {
    f32x4 sacc[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) sacc[h][0] = sacc[h][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < KSH / 2; ++u) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(tile + PT::at(hf, 16 * h + col, 4 * u + g));
        f16x8 v0, v1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f16x2 x = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w[q], 1.0f, false);
          const f16x2 y = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w[q], 1.0f, true);
          f16x8& dst = q < 2 ? v0 : v1;
          const int o = (q & 1) * 4;
          dst[o + 0] = x[0];
          dst[o + 1] = x[1];
          dst[o + 2] = y[0];
          dst[o + 3] = y[1];
        }
        sacc[h][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v0, qf[2 * u], sacc[h][0], 0, 0, 0);
        sacc[h][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v1, qf[2 * u + 1], sacc[h][1], 0, 0, 0);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) sres[h] = sacc[h][0] + sacc[h][1];
  };

  // ---- online softmax and page-scale normalization (as in the 4-wave kernel)
  auto softmax = [&](int t, const f32x4 sres[2], f16x8& pf, uint32_t vmask[2]) {
    const int lr0 = kTileRows * t;
    float x[8], sc[8];
    float tmax = -INFINITY, tsig = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 rq = *reinterpret_cast<const f32x4*>(&ps_s[lr0 + 16 * h + 4 * g]);
      vmask[h] = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = rq[i] >= 0.0f;  // also false past the end of the split
        vmask[h] |= ok ? 0xFFu << (8 * i) : 0u;
        sc[4 * h + i] = ok ? rq[i] : 0.0f;
        const float v = ok ? sres[h][i] * rq[i] * hfac : -INFINITY;
        x[4 * h + i] = v;
        tmax = fmaxf(tmax, v);
        tsig = fmaxf(tsig, sc[4 * h + i]);
      }
    }
    tmax = rows_max4(tmax);
    tsig = rows_max4(tsig);
    const bool need = tmax > m_run + kRescaleSlack;
    const bool grow = tsig > sigma * kSigmaSlack;
    if (__any(need) || grow) {
      const float m_new = need ? tmax : m_run;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
      const float fs = grow ? sigma / tsig : 1.0f;
      if (__any(m_run != -INFINITY)) {
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i, 64) * fs;  // factor of head 4g + i
#pragma unroll
        for (int n = 0; n < NBH; ++n) {
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[n][i] *= al[i];
        }
      }
      l_run *= alpha;
      m_run = m_new;
      if (grow) {
        sigma = tsig;
        inv_sigma = 1.0f / tsig;
      }
    }
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = x[j] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[j] - m_run);
      psum += p;
      pf[j] = (_Float16)(p * (sc[j] * inv_sigma));
    }
    l_run += rows_sum4(psum);
  };

  // ---- O[:, half] += P . V[:, half]
  auto pv_half = [&](const uint8_t* tile, const f16x8& pf, const uint32_t vmask[2]) {
    const int k = col >> 1;
    const int vrow = k < 4 ? 4 * g + k : 16 + 4 * g + k - 4;
    const int half8 = 8 * (col & 1);
    u32x2 raw8[NBH];
#pragma unroll
    for (int n = 0; n < NBH; ++n) {
      const i2v r8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) i2v*)(tile + PT::at(hf, vrow, n) + half8));
      raw8[n] = __builtin_bit_cast(u32x2, r8);
    }
#pragma unroll
    for (int n = 0; n < NBH; ++n) {
      const uint32_t lo = raw8[n][0] & vmask[0], hi = raw8[n][1] & vmask[1];
      const f16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)lo, 1.0f, false);
      const f16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)lo, 1.0f, true);
      const f16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)hi, 1.0f, false);
      const f16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)hi, 1.0f, true);
      const f16x8 vf = {a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
      oacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf, vf, oacc[n], 0, 0, 0);
    }
  };

  // ---- the pair's tiles pair, pair + 4, ...: both waves of a pair run the
  // same steps and meet only each other (pair_signal / pair_wait).  Tile t is
  // in ring slot st & 1 and tile t + 4 may still be loading behind it; a slot
  // is refilled with tile t + 8 once this wave's reads of its half are done.
  const int nsteps = nt > pair ? (nt - pair + kPairs - 1) / kPairs : 0;
  for (int st = 0; st < nsteps; ++st) {
    const int t = pair + kPairs * st;
    uint8_t* slot = (st & 1) ? slot1 : slot0;
    f32x4 sres[2];
    if (st == 0) {
      // the first tile alone was in flight: a smaller first burst lands sooner
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      asm volatile("" ::: "memory");
      if (t + kPairs < nt) issue(t + kPairs, slot1);
    } else if (t + kPairs < nt) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(PT::INSTR));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    asm volatile("" ::: "memory");
    qk_half(slot, sres);
    if (st > 0) pair_wait(&psync_s[wave ^ 1][1], st);  // the partner has read this wave's last partial
#pragma unroll
    for (int h = 0; h < 2; ++h) xs[(wave * 2 + h) * 64 + lane] = sres[h];
    pair_signal(&psync_s[wave][0], st + 1);
    pair_wait(&psync_s[wave ^ 1][0], st + 1);  // the partner's partial S of this tile is in LDS
    // the full S: half 0's partial plus half 1's, the same sum in both waves
    f32x4 o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) o[h] = xs[((wave ^ 1) * 2 + h) * 64 + lane];
    pair_signal(&psync_s[wave][1], st + 1);  // (the release waits for these reads)
#pragma unroll
    for (int h = 0; h < 2; ++h) sres[h] = hf == 0 ? sres[h] + o[h] : o[h] + sres[h];
    f16x8 pf;
    uint32_t vmask[2];
    softmax(t, sres, pf, vmask);
    pv_half(slot, pf, vmask);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(63) & ~0x0F00);  // lgkmcnt(0): the slot's reads are done
    asm volatile("" ::: "memory");
    if (t + 2 * kPairs < nt) issue(t + 2 * kPairs, slot);
  }

  // ---- merge the four pairs' states.  A wave's O goes into the LDS that only
  // its own loads fill (half hf of both of its pair's ring slots: head quads
  // 0-1, then 2-3), so it is written as soon as the wave's last tile is read,
  // while other pairs may still be working; one barrier, then every wave
  // finds the weights of all 4 pairs x 16 heads (one per lane) and the sum
  // takes them by lane reads.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load of this wave's into the slots is in flight
  auto o_at = [&](int p, int hfx, int hq, int dh) {  // f32x4 of head quad hq, dim 256 hfx + dh, pair p
    return reinterpret_cast<f32x4*>((hq < 2 ? tile0_s : tile1_s) + p * PT::BYTES + PT::HALF_BYTES * hfx +
                                    16 * ((hq & 1) * (D / 2) + dh));
  };
#pragma unroll
  for (int n = 0; n < NBH; ++n) *o_at(pair, hf, g, 16 * n + col) = oacc[n] * sigma;
  if (hf == 0 && g == 0) ml_s[pair][col] = make_float2(m_run, l_run);
  if (threadIdx.x == (unsigned)(2 * pair * 64)) sg_s[pair] = sigma;
  __syncthreads();
  // lane 16 p + h: the weight of pair p's O for head h0 + h.  The f16 partial
  // is O / c with c = l * sg: every row's value is a code (|code| <= 448) times
  // its page scale, which is at most kSigmaSlack * sg (sigma grows lazily), so
  // |O / c| <= 448 * kSigmaSlack, well inside f16, whatever the data's
  // magnitude.
  float wl;
  {
    const int hh = lane & 15, pl = lane >> 4;
    float M = -INFINITY, sg = 0.0f;
#pragma unroll
    for (int p = 0; p < kPairs; ++p) {
      M = fmaxf(M, ml_s[p][hh].x);
      sg = fmaxf(sg, sg_s[p]);
    }
    float l = 0.0f, wt[kPairs];
#pragma unroll
    for (int p = 0; p < kPairs; ++p) {
      wt[p] = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml_s[p][hh].x - M);  // 0 for an idle pair
      l += wt[p] * ml_s[p][hh].y;
    }
    const float c = l * sg;
    const float inv = c > 0.0f ? 1.0f / c : 0.0f;
    wl = (pl == 0 ? wt[0] : pl == 1 ? wt[1] : pl == 2 ? wt[2] : wt[3]) * inv;
    if (wave == 0 && lane < kHeadsPerBlock && h0 + hh < H)
      ml[part + h0 + hh] = M == -INFINITY ? f32x4{-INFINITY, 0.0f, 0.0f, 0.0f} : f32x4{M * 0.6931471805599453f, l, c, 0.0f};
  }
  static_assert(D == kPairThreads, "one dim per thread in the sum");
  {
    const int dim = threadIdx.x, hfx = dim / (D / 2), dh = dim % (D / 2);
#pragma unroll
    for (int hq = 0; hq < kHeadsPerBlock / 4; ++hq) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < kPairs; ++p) {
        const f32x4 o = *o_at(p, hfx, hq, dh);
        f32x4 wt;
#pragma unroll
        for (int k = 0; k < 4; ++k) wt[k] = u2f((uint32_t)__builtin_amdgcn_readlane((int)f2u(wl), 16 * p + 4 * hq + k));
        acc += wt * o;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int h = h0 + 4 * hq + k;
        if (h < H) opart[(part + h) * D + dim] = (_Float16)acc[k];
      }
    }
  }
}

// Merge the splits of one (sequence, head), then inverse RoPE at L-1.  The
// threads form SG split groups; a group's lanes cover the D dims with 16-byte
// loads and the group takes every SG-th split.  All partial loads of a round
// (up to kCombU splits per thread) are issued together with the (m, l) loads
// of the splits, before the sequence length is read, so a round costs one
// memory round trip; the groups' sums meet in LDS in a fixed order.
constexpr int kCombThreads = 256;
constexpr int kCombU = 16;

// The partials are fp32 (kHalf false: O unnormalized, weight factor c = 1) or
// f16 (O / c, with c from the split's (m, l, c) entry); either way a thread
// reads 16 bytes of a split's row: VEC dims.
template <int D, bool kHalf>
__global__ __launch_bounds__(kCombThreads) void attn_combine_kernel(AttnArgs a) {
  constexpr int VEC = kHalf ? 8 : 4;          // dims per 16-byte load
  constexpr int TPG = D / VEC;                // threads per split group
  constexpr int SG = kCombThreads / TPG;      // split groups: 2 (D=512, fp32) .. 16 (D=64)
  constexpr int kPairs = (D / 2 + kCombThreads - 1) / kCombThreads;  // RoPE pairs per thread
  const int h = blockIdx.x, b = blockIdx.y;
  const int H = a.H;
  const int grp = threadIdx.x / TPG, li = threadIdx.x % TPG;
  const f32x4* ml = reinterpret_cast<const f32x4*>(a.ws + a.plan.ml_off) + h;
  const u32x4* opart = reinterpret_cast<const u32x4*>(a.ws + a.plan.o_off + (size_t)h * D * (kHalf ? 2 : 4)) + li;
  const size_t ostride = (size_t)H * D / VEC;  // 16-byte units between consecutive items
  __shared__ float w_s[kMaxSplits];
  __shared__ float red_s[kCombThreads / 64];
  __shared__ __attribute__((aligned(16))) float acc_s[SG][D];
  // this sequence's splits are items off .. off + Sp - 1.  The first round of
  // partial loads and the first kCombThreads (m, l) pairs are issued before the
  // lengths are known, for the work list of equal lengths (max_seq_len each),
  // and again if the lengths give another list ((m, l) first: loads complete
  // in issue order, and the split maximum needs only these; unguarded, the
  // split index clamped into the sequence's, item 0 if it has none: guarded
  // loads are branches, across which the loads' waits are no longer counted
  // exactly)
  const int lens0 = attn_lens0(a);
  int off = b * a.plan.s_uni, Sp = a.plan.s_uni;
  auto item_of = [&](int s) { return Sp > 0 ? off + min(s, Sp - 1) : 0; };
  f32x4 ml0;
  u32x4 o[kCombU];
  auto first_loads = [&]() {
    const f32x4 v = ml[(size_t)item_of(threadIdx.x) * H];
    ml0 = (int)threadIdx.x < Sp ? v : f32x4{-INFINITY, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < kCombU; ++u) o[u] = opart[(size_t)item_of(grp + SG * u) * ostride];
  };
  first_loads();
  const Work wk = attn_work(a, b, false, lens0);
  if (wk.s != off || wk.S != Sp) {
    off = wk.s;
    Sp = wk.S;
    first_loads();
  }
  const int L = wk.L;
  const int N = (L + a.m - 1) / a.m;
  const int n_sel = a.sel ? clampi(a.sel_n[b], 0, a.k) : N;
  const int rows_b = n_sel + min(a.window, L);
  const int RPS = kTileRows * wk.T;
  const int S = min(Sp, (rows_b + RPS - 1) / RPS);
  // the inverse rotation at L-1, while the loads are in flight
  float2 cs[kPairs];
#pragma unroll
  for (int k = 0; k < kPairs; ++k) {
    const int pi = threadIdx.x + kCombThreads * k;
    float c = 1.0f, sn = 0.0f;
    if (pi < D / 2) rope_cs((double)(L - 1), rope_inv_freq(pi, a.rope_r), c, sn);
    cs[k] = make_float2(c, sn);
  }
  // split maxima -> M; weights exp(m_s - M) (0 for empty splits); tot = sum
  // exp(m_s - M) l_s; a partial counts with exp(m_s - M) c_s (w_s)
  float mloc = (int)threadIdx.x < S ? ml0.x : -INFINITY;
  for (int s = threadIdx.x + kCombThreads; s < S; s += kCombThreads) mloc = fmaxf(mloc, ml[(size_t)(off + s) * H].x);
  mloc = wave_max(mloc);
  if ((threadIdx.x & 63) == 0) red_s[threadIdx.x >> 6] = mloc;
  __syncthreads();
  const float M = fmaxf(fmaxf(red_s[0], red_s[1]), fmaxf(red_s[2], red_s[3]));
  __syncthreads();
  const int64_t row = (int64_t)b * H + h;
  float* out = a.out ? a.out + row * D : nullptr;
  if (M == -INFINITY) {
    if (out)
      for (int c = threadIdx.x; c < D; c += kCombThreads) out[c] = 0.0f;
    if (a.out8)
      for (int c = threadIdx.x; c < D; c += kCombThreads) a.out8[row * D + c] = 0;
    if (threadIdx.x == 0) {
      if (a.lse) a.lse[row] = -INFINITY;
      if (a.out8) a.out8_scale[row] = 1.0f;
    }
    return;
  }
  float tloc = 0.0f;
  if ((int)threadIdx.x < S) {  // the first round from the registers (a select between them and a load
    const float w = ml0.y > 0.0f ? expf(ml0.x - M) : 0.0f;  // put ml0 on the stack)
    w_s[threadIdx.x] = w * ml0.z;
    tloc += w * ml0.y;
  }
  for (int s = threadIdx.x + kCombThreads; s < S; s += kCombThreads) {
    const f32x4 v = ml[(size_t)(off + s) * H];
    const float w = v.y > 0.0f ? expf(v.x - M) : 0.0f;
    w_s[s] = w * v.z;
    tloc += w * v.y;
  }
  tloc = wave_sum(tloc);
  if ((threadIdx.x & 63) == 0) red_s[threadIdx.x >> 6] = tloc;
  __syncthreads();
  const float tot = (red_s[0] + red_s[1]) + (red_s[2] + red_s[3]);
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.0f;
  for (int s0 = grp;; s0 += SG * kCombU) {
#pragma unroll
    for (int u = 0; u < kCombU; ++u) {
      const int s = s0 + SG * u;
      // splits at S and past it hold no partial of this sequence (whatever
      // the workspace holds there, it is not added, not even times 0)
      if (s < S) {
        const float w = w_s[s];
        if constexpr (kHalf) {
          const f16x8 x = __builtin_bit_cast(f16x8, o[u]);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += w * (float)x[i];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] += w * u2f(o[u][i]);
        }
      }
    }
    if (s0 + SG * kCombU >= S) break;
#pragma unroll
    for (int u = 0; u < kCombU; ++u) {  // next round (more than SG * kCombU splits)
      const int s = s0 + SG * (kCombU + u);
      o[u] = opart[(size_t)item_of(s) * ostride];
    }
  }
#pragma unroll
  for (int i = 0; i < VEC; i += 4)
    *reinterpret_cast<f32x4*>(&acc_s[grp][VEC * li + i]) = f32x4{acc[i], acc[i + 1], acc[i + 2], acc[i + 3]};
  __syncthreads();
  const float inv_tot = 1.0f / tot;
  float2 ov[kPairs];
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < kPairs; ++k) {
    const int pi = threadIdx.x + kCombThreads * k;
    ov[k] = make_float2(0.0f, 0.0f);
    if (pi >= D / 2) break;
    float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int gq = 0; gq < SG; ++gq) {
      const float* ag = acc_s[gq];
      o0 += ag[2 * pi];
      o1 += ag[2 * pi + 1];
    }
    o0 *= inv_tot;
    o1 *= inv_tot;
    ov[k] = make_float2(o0 * cs[k].x + o1 * cs[k].y, -o0 * cs[k].y + o1 * cs[k].x);  // rotation by -angle
    if (out) {
      out[2 * pi] = ov[k].x;
      out[2 * pi + 1] = ov[k].y;
    }
    amax = fmaxf(amax, fmaxf(fabsf(ov[k].x), fabsf(ov[k].y)));
  }
  if (threadIdx.x == 0 && a.lse) a.lse[row] = M + logf(tot);
  if (a.out8) {
    // fp8 form of the row for the next projection: one scale per (token, head)
    // row, amax / 448 (1 for an all-zero row), codes E4M3(x / scale)
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) red_s[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red_s[0], red_s[1]), fmaxf(red_s[2], red_s[3]));
    const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
    uint16_t* o8 = reinterpret_cast<uint16_t*>(a.out8 + row * D);
#pragma unroll
    for (int k = 0; k < kPairs; ++k) {
      const int pi = threadIdx.x + kCombThreads * k;
      if (pi >= D / 2) break;
      o8[pi] = (uint16_t)e4m3_encode2_hw<false>(ov[k].x / sc, ov[k].y / sc, 0u);
    }
    if (threadIdx.x == 0) a.out8_scale[row] = sc;
  }
}

template <int D, int KVDT>
static hipError_t launch_split(const AttnArgs& a, hipStream_t s) {
  const int64_t blocks = ((int64_t)a.plan.items + kXcds - 1) / kXcds * kXcds * a.plan.head_blocks;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if constexpr (D == kPairD && KVDT == HCA_FP8_E4M3)
    hipLaunchKernelGGL(attn_pair_kernel, dim3((unsigned)blocks), dim3(kPairThreads), 0, s, a);
  else
    hipLaunchKernelGGL((attn_split_kernel<D, KVDT>), dim3((unsigned)blocks), dim3(kAttnThreads), 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_attn_d(const AttnArgs& a, hipStream_t s) {
  const hipError_t e = a.kv.dtype == HCA_FP8_E4M3 ? launch_split<D, HCA_FP8_E4M3>(a, s) : launch_split<D, HCA_BF16>(a, s);
  if (e != hipSuccess) return e;
  // the split kernel for 512-dim fp8 rows writes f16 partials
  if (D == kPairD && a.kv.dtype == HCA_FP8_E4M3)
    hipLaunchKernelGGL((attn_combine_kernel<D, true>), dim3(a.H, a.B), dim3(kCombThreads), 0, s, a);
  else
    hipLaunchKernelGGL((attn_combine_kernel<D, false>), dim3(a.H, a.B), dim3(kCombThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& args, hipStream_t s, bool split_only) {
  if (args.B == 0) return hipSuccess;
  AttnArgs a = args;
  a.rope_r = pow((double)a.theta, -2.0 / (double)a.kv.dim);
  if (split_only) {
    const bool f8 = a.kv.dtype == HCA_FP8_E4M3;
    switch (a.kv.dim) {
      case 64: return f8 ? launch_split<64, HCA_FP8_E4M3>(a, s) : launch_split<64, HCA_BF16>(a, s);
      case 128: return f8 ? launch_split<128, HCA_FP8_E4M3>(a, s) : launch_split<128, HCA_BF16>(a, s);
      case 256: return f8 ? launch_split<256, HCA_FP8_E4M3>(a, s) : launch_split<256, HCA_BF16>(a, s);
      default: return f8 ? launch_split<512, HCA_FP8_E4M3>(a, s) : launch_split<512, HCA_BF16>(a, s);
    }
  }
  switch (a.kv.dim) {
    case 64: return launch_attn_d<64>(a, s);
    case 128: return launch_attn_d<128>(a, s);
    case 256: return launch_attn_d<256>(a, s);
    default: return launch_attn_d<512>(a, s);
  }
}

#ifdef HCA_DEBUG
HCA_DBG_ACCESSOR(debug_bits_attention)
#endif

}  // namespace hca
