// Internal launchers shared by the kernel sources and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hca.h"
#include "indexer_internal.h"

namespace hca {

struct CompressArgs {
  const uint16_t* x; int64_t xs;
  const float* z; int64_t zs;
  const float* beta;
  const int32_t* pos0; const int32_t* ntok;
  int B, max_ntok, d, m;
  int ov;  // overlap: tokens of the previous group in each window (rows -ov .. -1), m <= kSmallM when > 0
  float theta;
  double rope_r;  // theta^(-2/d) in fp64 (set by the launcher)
  const float* gamma; float eps;  // RMS normalisation of each entry before its rotation (gamma null: none)
  float* out; int64_t os;
};
hipError_t launch_compress(CompressArgs a, hipStream_t s);
constexpr int kCompressThreads = 256;
constexpr int kSmallM = 16;  // groups up to this size are folded by one row group of threads
constexpr size_t kCompressShm = (size_t)kCompressThreads * 8 * sizeof(float);  // a large-m fold's row-group sums

// the fused prefill of one pool: fold, normalise, rotate and quantize a run's
// pages in one launch, a block per page (the run starts a page)
struct PrefillArgs {
  CompressArgs c;
  const int32_t* bt;
  int bts;
  hca_paged_cache dst;
};
bool prefill_supported(int m, int d, int epp, int dtype);
hipError_t launch_prefill(PrefillArgs p, hipStream_t s);

// decode-step update of pools: fold each open group into its staging row and
// quantize the open page, all in one launch (a job per pool)
struct InsertArgs {
  CompressArgs c;           // the open group (c.x null: the row is already in staging); c.out, c.os set per sequence
  float* stage; int64_t ss; // [B][epp][d] f32 staging of the open page
  const int32_t* e0;        // [B] first entry of the open page
  const int32_t* bt; int bts;
  hca_paged_cache dst;
  int append;
  float* state; int64_t sts;  // [B][kPageHead (+ 2 (kFoldStateHead + d) for m > kSmallM)] update states, or null
};
// an update state: the open page's header, [0] how many of its rows and [1]
// their amax (fp8 pages of re-folded entries), [2], [3] unused; then, for
// groups of more than kSmallM tokens, two running fold states:
// [0] tokens folded, [1] running max of the logits, [2] running sum of
// exp(logit - max), [3] unused, then the d running sums of exp(logit - max) * token
constexpr int kPageHead = 4;
constexpr int kFoldStateHead = 4;
constexpr int kMaxInsertJobs = 4;
struct InsertJobs {
  InsertArgs job[kMaxInsertJobs];
  int n;
};
hipError_t launch_insert(InsertJobs j, int B, hipStream_t s);

struct QuantArgs {
  const float* src; int64_t ss;
  const int32_t* e0; const int32_t* ne;
  int B, max_ne;
  const int32_t* bt; int bts;
  hca_paged_cache dst;
};
// ws: NULL (one block per page) or quantize_ws_bytes(...) bytes of chunk partials
size_t quantize_ws_bytes(int B, int max_ne, const hca_paged_cache& dst);
hipError_t launch_quantize(const QuantArgs& a, float* ws, hipStream_t s);

struct GatherArgs {
  hca_paged_cache src;
  const int32_t* bt; int bts;
  const int32_t* n_rows;
  int B, max_rows;
  void* dst_codes; void* dst_scales;
};
hipError_t launch_gather(const GatherArgs& a, hipStream_t s);

// the indexer's arguments and launchers (their own header: the indexer
// source depends on nothing else here)

// attention launch plan.  The work list itself (which sequence and split a
// block takes) is derived on the device from the lengths; the host bounds it:
// every sequence's 32-row tiles are cut into splits of T tiles, T sized so that
// the splits of all sequences fill `spread` work items (at most kMaxSplitTiles
// tiles a split, which may take more), so at most `items` items exist.  The
// workspace holds a partial (m, l) and o[d] per (item, head).
struct AttnPlan {
  int tiles_max;    // upper bound of 32-row tiles of any sequence
  int head_blocks;  // ceil(H / 16)
  int spread;       // items the splits are sized to fill
  int items;        // work items the grid holds: max(spread, B x tiles_max / kMaxSplitTiles) + B
  int t_uni, s_uni; // tiles a split and splits a sequence when every sequence has max_seq_len tokens
  size_t o_off, ml_off, total;
};
constexpr int kAttnMaxSplits = 4096;  // splits per sequence the combine kernel handles
AttnPlan attn_plan(int B, int H, int d, int max_seq_len, int m, int window, int k, bool has_sel);

struct AttnArgs {
  const uint16_t* q; int H;
  hca_paged_cache kv; const int32_t* bt; int bts;
  hca_paged_cache win; const int32_t* wbt; int wbts;
  const int32_t* lens; int B, max_len, m, window;
  const int32_t* sel; const int32_t* sel_n; int k;
  float scale, theta;
  double rope_r;  // theta^(-2/d) in fp64 (set by the launcher)
  float* out; float* lse;
  uint8_t* out8; float* out8_scale;  // fp8 form of the output (null: none)
  unsigned char* ws; AttnPlan plan;
};
// split_only: the split kernel alone (partials in the workspace, no output), for timing
hipError_t launch_attention(const AttnArgs& a, hipStream_t s, bool split_only = false);

#ifdef HCA_DEBUG
// each module's debug word (kDbg* bits; 0x80000000 when it cannot be read),
// cleared when `clear`
uint32_t debug_bits_attention(bool clear);
uint32_t debug_bits_compress(bool clear);
uint32_t debug_bits_indexer(bool clear);
uint32_t debug_bits_quantize(bool clear);
#endif

}  // namespace hca
