// indexer_topk: indexer scoring and top-k for c4a layers (V4 page, section 2.2:
// a separate, smaller indexer KV decides which compressed entries the query
// looks in, instead of a brute-force search over the main KV).
//
// Score kernel (the HBM-bound stream of a c4a layer): the device code is in
// indexer_score.h, shared with the score launch that also runs a decode
// step's cache updates.
//
// Select.  The cut bin comes from the summed copies; every chunk block marks
// the scores above it in a bitmap and appends the cut bin's entries as
// candidates; then every compaction block refines the cut with two 10-bit
// radix passes over the candidates, breaks exact ties by the lowest index, and
// writes its chunk's kept indices in ascending order.  The histogram copies are left zeroed for the next call; every
// other part of the workspace is overwritten before it is read.
#include "hca_common.h"
#include "indexer_internal.h"
#include "indexer_score.h"
#include "indexer_select.h"

namespace hca {

constexpr int kScoreChunk = 1024;  // entries per score block (256 per wave)

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

IndexerWs indexer_ws_layout(int B, int max_seq_len, int m, int k) {
  (void)k;
  IndexerWs w;
  const int n_max = (max_seq_len + m - 1) / m;
  w.n_max = n_max;
  const int n_pad = ((n_max + kSelChunk - 1) / kSelChunk) * kSelChunk;
  size_t off = 0;
  w.scores = off; off = align256(off + (size_t)B * n_pad * sizeof(float));
  w.hist = off; off = align256(off + (size_t)B * kHistWords * sizeof(uint32_t));
  w.cand = off; off = align256(off + (size_t)B * n_pad * sizeof(uint2));
  w.bitmap = off; off = align256(off + (size_t)B * (n_pad / 32) * sizeof(uint32_t));
  w.counters = off; off = align256(off + (size_t)B * 4 * sizeof(uint32_t));
  w.cand_counts = off; off = align256(off + (size_t)B * 2 * (n_pad / kSelChunk) * sizeof(uint32_t));
  w.total = off;
  return w;
}

template <int KDT, int DI>
__global__ __launch_bounds__(kScoreThreads) void score_pages_kernel(IndexerArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t hist_s[kHistBins];
  score_pages_block<KDT, DI>(a, blockIdx.x, blockIdx.y, hist_s);
}

// Generic path (any entries-per-page): per-lane table lookups, 16 entries a step.
template <int KDT, int DI>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(IndexerArgs a) {
  const int b = blockIdx.y;
  const int L = clampi(a.lens[b], 0, a.max_len);
  const int N = (L + a.m - 1) / a.m;
  const int chunk0 = blockIdx.x * kScoreChunk;
  if (chunk0 >= N) return;
  __shared__ __attribute__((aligned(16))) uint32_t hist_s[kHistBins];
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
    HCA_DBG_CHECK(!valid || live, kDbgPage);
    const float pscale = KDT == HCA_FP8_E4M3 ? reinterpret_cast<const float*>(a.keys.scales)[live ? phys : 0] : 0.0f;
    const int64_t r = live ? (int64_t)phys * epp + slot : 0;
    Tile<KDT, DI> t;
    t.load(codes + r * row_bytes, scales + r * (DI / 32), pscale, live, g);
    finish_tile(c, t.dots(qa), e, valid, g);
  }
  if (c.want_hist) hist_flush(a, b, blockIdx.x, hist_s);
}

__global__ __launch_bounds__(kSelThreads) void select_chunk_kernel(IndexerArgs a) {
  const int b = blockIdx.y;
  SelView v = sel_view(a, b);
  const int len_raw = a.lens[b];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // this block's scores and the coarse histogram are loaded with the
  // length, unconditionally (a block past the last score chunk, which the grid
  // has when k exceeds the entries, reads chunk 0 and uses nothing)
  constexpr int kUnroll = kSelChunk / 256;  // one round of loads per wave
  const int c0 = blockIdx.x * kSelChunk;
  const int base0 = (c0 < v.n_pad ? c0 : 0) + wave * 64 * kUnroll;
  float sc[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) sc[u] = v.scores[base0 + 64 * u + lane];
  // copy t / 16, coarse bin t % 16 of the coarse histogram
  static_assert(kSelThreads == kHistCopies * kCoarseBins, "one coarse count per thread");
  const uint32_t coarse = v.hist[kHistCopies * kHistBins + threadIdx.x];
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
  // the coarse bin that holds the cut, and the entries above it: its 256-bin
  // slice is then the only one summed
  __shared__ uint32_t coarse_s[kCoarseBins];
  if (threadIdx.x < kCoarseBins) coarse_s[threadIdx.x] = 0u;
  __syncthreads();
  if (coarse) atomicAdd(&coarse_s[threadIdx.x % kCoarseBins], coarse);
  __syncthreads();
  int cb = kCoarseBins - 1;
  uint32_t run = 0;
  for (; cb > 0; --cb) {
    const uint32_t x = coarse_s[cb];
    if (run + x >= (uint32_t)k) break;
    run += x;
  }
  const int top0 = 256 * cb + 255;
  const uint32_t first = hist_slice_sum(v.hist, top0);
  int cut;
  uint32_t above;
  find_cut_copies(v.hist, top0, first, run, (uint32_t)k, tmp, cut, above);
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

__global__ __launch_bounds__(kSelThreads) void select_compact_kernel(IndexerArgs a) {
  __shared__ SelLds sm;
  __shared__ uint32_t wbits_s[kCompactChunks * kSelChunk / 32];
  select_compact_block(a, blockIdx.x, blockIdx.y, sm, wbits_s);
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
  return launch_select(a, s);
}

hipError_t launch_select_chunk(const IndexerArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const int gk = (a.k + kSelChunk - 1) / kSelChunk;
  const int g = select_chunks(a);
  hipLaunchKernelGGL(select_chunk_kernel, dim3(g > gk ? g : gk, a.B), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select(const IndexerArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const hipError_t e = launch_select_chunk(a, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_compact_kernel, dim3(compact_blocks(a), a.B), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

#ifdef HCA_DEBUG
HCA_DBG_ACCESSOR(debug_bits_indexer)
#endif

}  // namespace hca
