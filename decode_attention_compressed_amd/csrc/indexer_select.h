// The indexer's select passes as device code (the k highest scores, ties to
// the lower index, in ascending index order), shared by the indexer's own
// kernels and by the compaction launch that also runs a decode step's cache
// updates as extra blocks.
#pragma once
#include "hca_common.h"
#include "indexer_internal.h"
#include "indexer_score.h"

namespace hca {

constexpr int kSelThreads = 256;
constexpr int kMaxSelBlocks = 1024;  // select blocks per sequence (N <= 2M entries)
constexpr int kCandLds = 4096;      // candidates a compaction block stages in LDS

// score chunks of kSelChunk entries per sequence (at least one)
inline int select_chunks(const IndexerArgs& a) {
  return a.lay.n_max > 0 ? (a.lay.n_max + kSelChunk - 1) / kSelChunk : 1;
}

// ------------------------------------------------------------------ select
// inclusive scan over the 64 lanes of a wave, register to register: DPP row
// shifts scan each 16-lane row, then every lane adds the totals of the rows
// below its own (read from the rows' last lanes)
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// exclusive block scan of one uint per thread (kSelThreads threads)
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
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
  v.hist = reinterpret_cast<uint32_t*>(a.ws + a.lay.hist) + (size_t)b * kHistWords;
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
// time from slice top0 down, starting with `run` entries above it; the caller
// starts at the slice the coarse histogram names, so this is one slice.
// Every thread of the block gets the result.  The first slice's per-thread
// sums (`first`) come from the caller.
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
__device__ void find_cut_copies(const uint32_t* hist, int top0, uint32_t first, uint32_t run, uint32_t need,
                                uint32_t* tmp, int& cut, uint32_t& above) {
  __shared__ int cut_s;
  __shared__ uint32_t above_s;
  // run: entries in the bins already passed
  for (int top = top0; top >= 0; top -= kSelThreads) {
    const int bin = top - (int)threadIdx.x;
    const uint32_t cnt = top == top0 ? first : hist_slice_sum(hist, top);
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
  uint32_t tot3[3][kSelThreads / 64];
  uint32_t spec_over;  // a chunk has more candidates than its speculative slots
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

// Speculative candidates: the two threads t of chunk t / 2 load one half each
// of the first kSpecSlots slots of its candidate region, before the counts are
// known; when there are at most kSelThreads / 2 chunks and
// none has more than kSpecSlots candidates, these are all of them and no
// second round trip gathers them.
constexpr int kSpecSlots = 32;
constexpr int kSpecU = kSpecSlots / 2 / 2;  // 16-byte loads per thread (two candidates each)
__device__ __forceinline__ void load_spec(const SelView& v, uint4 spec[kSpecU]) {
  const int gp = v.n_pad / kSelChunk;
  const int j = min((int)threadIdx.x >> 1, gp - 1);
  const uint4* p = reinterpret_cast<const uint4*>(v.cand + (size_t)j * kSelChunk + (threadIdx.x & 1) * (kSpecSlots / 2));
#pragma unroll
  for (int u = 0; u < kSpecU; ++u) spec[u] = p[u];
}

__device__ CutKey resolve_cut(const SelView& v, int k, SelLds& sm, int cut, uint32_t above,
                              const uint32_t ccount_pre[kSelPer], const uint4 spec[kSpecU]) {
  const int N = v.N, G = v.G;
  if (threadIdx.x == 0) sm.spec_over = 0u;  // set below, after the scan's barriers
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
      if (loc[u] > (uint32_t)kSpecSlots) sm.spec_over = 1u;
    }
    if (threadIdx.x == 0) sm.pre_s[G] = tot;
    __syncthreads();
  }
  CutKey r;
  r.nc = sm.pre_s[G];
  r.in_lds = r.nc <= (uint32_t)kCandLds;
  if (r.in_lds && G <= kSelThreads / 2 && sm.spec_over == 0u) {
    // every candidate is in the speculative slots: chunk t / 2's go to LDS
    const int j = threadIdx.x >> 1;
    if (j < G) {
      const uint32_t p0 = sm.pre_s[j], n = sm.pre_s[j + 1] - p0;
      const uint32_t s0 = (threadIdx.x & 1) * (kSpecSlots / 2);
#pragma unroll
      for (int u = 0; u < kSpecU; ++u) {
        const uint32_t s = s0 + 2 * u;
        if (s < n) sm.cl_s[p0 + s] = make_uint2(spec[u].x, spec[u].y);
        if (s + 1 < n) sm.cl_s[p0 + s + 1] = make_uint2(spec[u].z, spec[u].w);
      }
    }
    __syncthreads();
  } else if (r.in_lds) {
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

// One compaction block: chunk j of sequence b, with the block's LDS.  Called
// by every thread of a block of kSelThreads threads.
// Chunks one compaction block writes (each by one of its waves).
constexpr int kCompactChunks = 2;
static_assert(kCompactChunks == 2, "the second wave's offset is the first chunk's count");
inline int compact_blocks(const IndexerArgs& a) { return (select_chunks(a) + kCompactChunks - 1) / kCompactChunks; }

// One compaction block: chunks kCompactChunks x .. of sequence b, with the
// block's LDS (wbits_s: kCompactChunks x 64 words).  Called by every thread of
// a block of kSelThreads threads.
__device__ __forceinline__ void select_compact_block(const IndexerArgs& a, int x, int b, SelLds& sm,
                                                     uint32_t* wbits_s) {
  // chunk j0 + c is written by wave c: its output offset is the count kept by
  // chunks 0 .. j0 + c - 1 (entries above the cut bin plus winning candidates)
  SelView v = sel_view(a, b);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j0 = kCompactChunks * x;
  // Loaded with the length, none of them depending on it: the cut, the
  // per-chunk candidate and above-cut counts, and the chunks' bitmap words
  // (entries above the cut bin; words at N and past it are dropped below).
  // The grid has no block past the padded chunks, so the words are in range.
  const int gp = v.n_pad / kSelChunk;
  const int w = (j0 + wave) * (kSelChunk / 32) + lane;
  const uint32_t bits_pre = wave < kCompactChunks && j0 + wave < gp ? v.bitmap[w] : 0u;
  const int cut_pre = (int)v.ctr[0];
  const uint32_t above_pre = v.ctr[1];
  uint32_t cc_pre[kSelPer], ab_pre[kSelPer];
  load_chunk_counts(v, v.ccount, cc_pre);
  load_chunk_counts(v, v.above, ab_pre);
  uint4 spec[kSpecU];
  load_spec(v, spec);
  set_len(v, a, a.lens[b]);
  const int N = v.N, G = v.G, k = a.k;
  if (N <= k || j0 >= G) return;
  const int j1 = min(G, j0 + kCompactChunks);  // chunks j0 .. j1-1
  int32_t* out = a.out_idx + (int64_t)b * k;
  const int W = (N + 31) / 32;
  if (wave < kCompactChunks) wbits_s[wave * 64 + lane] = j0 + wave < j1 && w < W ? bits_pre : 0u;
  const CutKey ck = resolve_cut(v, k, sm, cut_pre, above_pre, cc_pre, spec);
  // the chunks' winning candidates join their words
  {
    const uint32_t c0 = sm.pre_s[j0], c1 = sm.pre_s[j1];
    for (uint32_t i = c0 + threadIdx.x; i < c1; i += kSelThreads) {
      uint2 cd;
      if (ck.in_lds) {
        cd = sm.cl_s[i];
      } else {  // candidate i lives in the region of the chunk whose range holds it
        int jj = j0;
        while (jj + 1 < j1 && sm.pre_s[jj + 1] <= i) ++jj;
        cd = v.cand[(size_t)jj * kSelChunk + (i - sm.pre_s[jj])];
      }
      if (ck.take_all || cd.x > ck.T || (cd.x == ck.T && (int)cd.y <= ck.X))
        atomicOr(&wbits_s[(cd.y >> 5) - j0 * (kSelChunk / 32)], 1u << (cd.y & 31));
    }
  }
  // kept counts: before chunk j0, in chunk j0, in all chunks
  uint32_t before = 0, first = 0, all = 0;
  {
    const int per = sel_per(v);
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
      const int i = threadIdx.x * per + u;
      if (u < per && i < G) {
        const uint32_t c = ab_pre[u] + sm.wc_s[i];
        all += c;
        before += i < j0 ? c : 0u;
        first += i == j0 ? c : 0u;
      }
    }
  }
  // block totals of the three (one barrier, which also publishes wbits_s)
  uint32_t tot_before, tot_first, total;
  {
    const uint32_t sb = wave_incl_scan(before), sf = wave_incl_scan(first), sa = wave_incl_scan(all);
    if (lane == 63) {
      sm.tot3[0][wave] = sb;
      sm.tot3[1][wave] = sf;
      sm.tot3[2][wave] = sa;
    }
    __syncthreads();
    tot_before = tot_first = total = 0u;
#pragma unroll
    for (int w = 0; w < kSelThreads / 64; ++w) {
      tot_before += sm.tot3[0][w];
      tot_first += sm.tot3[1][w];
      total += sm.tot3[2][w];
    }
  }
  // wave c compacts chunk j0 + c, one word per lane
  if (wave < kCompactChunks && j0 + wave < j1) {
    const uint32_t bits0 = w < W ? wbits_s[wave * 64 + lane] : 0u;
    const uint32_t pc = (uint32_t)__popc(bits0);
    const uint32_t incl = wave_incl_scan(pc);
    uint32_t pos = tot_before + (wave == 1 ? tot_first : 0u) + incl - pc;
    uint32_t bits = bits0;
    while (bits) {
      const int bit = __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < (uint32_t)k) out[pos] = w * 32 + bit;
      ++pos;
    }
  }
  if (j1 == G) {
    for (int i = (int)total + threadIdx.x; i < k; i += kSelThreads) out[i] = -1;  // fewer than k: not expected
    if (threadIdx.x == 0) a.out_n[b] = (int)min(total, (uint32_t)k);
  }
  // leave the histogram copies zeroed for the next call: each block a slice
  {
    constexpr int kWords4 = kHistWords / 4;
    const int nb = (G + kCompactChunks - 1) / kCompactChunks;
    const int per = (kWords4 + nb - 1) / nb;
    u32x4* h4 = reinterpret_cast<u32x4*>(v.hist);
    for (int i = x * per + threadIdx.x; i < min(kWords4, (x + 1) * per); i += kSelThreads) h4[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

}  // namespace hca
