// Arguments, workspace layout and launchers of the indexer kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hca.h"

namespace hca {

// indexer workspace layout (all offsets 256-byte aligned)
struct IndexerWs {
  size_t scores, hist, cand, bitmap, counters, cand_counts, total;
  int n_max;  // max entries per sequence
};
IndexerWs indexer_ws_layout(int B, int max_seq_len, int m, int k);
constexpr int kHistBins = 4096;  // top 12 bits of the score key
constexpr int kHistCopies = 16;  // per-sequence histogram copies the score blocks spread over
constexpr int kCoarseBins = 16;  // coarse bins of 256 fine bins each, kept beside the fine ones
// words per sequence: kHistCopies fine histograms, then kHistCopies coarse ones
constexpr int kHistWords = kHistCopies * (kHistBins + kCoarseBins);
static_assert(kHistBins == 256 * kCoarseBins && kHistWords % 4 == 0, "coarse bins of 256, zeroed as 16-byte words");

// A decode step's open indexer row, written by the score pass itself: the key
// of the open entry, row p0/m - e0 of page table[e0/64] of the keys, from f32
// staging [B][64][128] (fp4 keys of 128 dims, 64 entries per page; the other
// rows of the page keep their codes).  stage null: none.
struct IndexerOpen {
  const float* stage; int64_t ss;
  const int32_t* pos0; const int32_t* e0;
};
struct IndexerArgs {
  const uint16_t* q; const float* w; int HI;
  hca_paged_cache keys;
  const int32_t* bt; int bts;
  const int32_t* lens;
  int B, max_len, m, k;
  int32_t* out_idx; int32_t* out_n;
  unsigned char* ws; IndexerWs lay;
  IndexerOpen open;
};
hipError_t launch_indexer(const IndexerArgs& a, hipStream_t s);
hipError_t launch_indexer_score(const IndexerArgs& a, hipStream_t s);
// the select launches that follow a score pass (cut and bitmap, then the
// ascending compaction), and the first of them alone
hipError_t launch_select(const IndexerArgs& a, hipStream_t s);
hipError_t launch_select_chunk(const IndexerArgs& a, hipStream_t s);
struct InsertJobs;
// the compaction launch of the select with a decode step's cache updates as
// extra blocks of the same launch (after launch_select_chunk); the jobs must
// not write the indexer keys
hipError_t launch_compact_insert(const IndexerArgs& a, const InsertJobs& j, hipStream_t s);

}  // namespace hca
