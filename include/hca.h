/*
 * hca.h -- decode attention over hybrid compressed KV caches, C ABI.
 *
 * The method (from "DeepSeek-V4 Serving ... vLLM", wmrh.cn news 47220, and
 * "vLLM 0.7.2 ... DeepSeek-V4", lpnh.cn news 995630):
 *   - a compressor folds every m consecutive token vectors (m = 4: c4a layers,
 *     m = 128: c128a layers) into one shared K=V entry (V4 page, section 2.1);
 *   - entries are stored in fp8 pages (indexer keys in fp8 or fp4) behind a block
 *     table whose logical block is 256 raw tokens (V4 page, sections 2.1, 2.2,
 *     3.1.1, 3.1.3; vLLM-0.7.2 page, section 2.1);
 *   - for c4a layers an indexer scores the entries and keeps the top k
 *     (V4 page, section 2.2);
 *   - the decode query attends to the selected entries plus a raw sliding window
 *     of recent tokens, with RoPE on the key use of the shared vector and inverse
 *     RoPE on the output (V4 page, sections 2.1 and 2.3).
 *
 * Conventions shared by every entry point
 *   Memory     every pointer argument is DEVICE memory owned by the caller (for
 *              example a torch tensor's data pointer), unless it is documented
 *              as a host value.  The library allocates nothing, keeps no state
 *              between calls, never synchronizes, and enqueues all work on
 *              `stream` (a hipStream_t; NULL is the null stream).
 *   Layout     all arrays are dense row-major C arrays of the shapes given;
 *              "bf16" arrays hold bfloat16 bit patterns in uint16_t.
 *   Block      logical block i of a sequence covers raw positions
 *   tables     [256 i, 256 i + 256) and, in a pool with epp = 256/m entries per
 *              page, entries [i*epp, (i+1)*epp).  table[b * stride + i] is the
 *              physical page of block i of sequence b, or -1 if unmapped.  One
 *              table may serve every compressed pool of every layer; the window
 *              pool (m = 1, 256 tokens a page) has its own table.  Pages may be
 *              shared by several sequences (prefix aliasing); shared pages are
 *              read-only while shared.
 *   Errors     arguments are validated on the host before anything is
 *              launched; a failed validation returns the status and launches
 *              nothing.  Launch failures return HCA_ERR_HIP.  Device-side values
 *              (lengths, table entries, indices) are not validated; kernels
 *              clamp lengths to the host bound they are given and skip page ids
 *              outside [0, num_pages) and indices outside the valid range, so a
 *              bad value gives a wrong result, never an out-of-bounds access.
 *   Threads    all functions are reentrant; calls that write the same memory
 *              must be ordered by the caller (same stream or events).
 */
#ifndef HCA_H
#define HCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HCA_OK = 0,
  HCA_ERR_INVALID = 1,     /* an argument is out of range or a pointer is NULL */
  HCA_ERR_UNSUPPORTED = 2, /* valid, but not a shape/type this build handles    */
  HCA_ERR_WORKSPACE = 3,   /* the workspace is NULL or too small                */
  HCA_ERR_HIP = 4          /* a HIP launch or runtime call failed               */
} hca_status;

/* Storage formats (OCP definitions):
 *   HCA_BF16      bfloat16, round to nearest even from fp32, no scale;
 *   HCA_FP8_E4M3  E4M3 "FN" (bias 7, max 448, no inf), one fp32 scale per
 *                 physical page: s = fl32(amax/448) over the page's valid
 *                 elements (1 when amax = 0), code = E4M3(fl32(x/s)), round to
 *                 nearest even, saturating at +-448;
 *   HCA_FP4_E2M1  E2M1 (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6), two per byte
 *                 (element 2c in the low nibble of byte c), one E4M3 scale per
 *                 32 consecutive elements of a row: sc = E4M3(fl32(amax32/6)),
 *                 code = E2M1(fl32(x/sc)), all codes 0 when sc decodes to 0. */
typedef enum { HCA_BF16 = 0, HCA_FP8_E4M3 = 1, HCA_FP4_E2M1 = 2 } hca_dtype;

/* One paged pool (one KV kind of one layer).
 *   codes   HCA_FP8_E4M3: uint8  [num_pages][epp][dim]
 *           HCA_FP4_E2M1: uint8  [num_pages][epp][dim/2]
 *           HCA_BF16:     uint16 [num_pages][epp][dim]
 *   scales  HCA_FP8_E4M3: float  [num_pages]
 *           HCA_FP4_E2M1: uint8  [num_pages][epp][dim/32]   (E4M3 codes)
 *           HCA_BF16:     unused (may be NULL)
 *   epp     entries (rows) per page: 256/m; 256 for a window pool. */
typedef struct {
  void* codes;
  void* scales;
  int32_t num_pages;
  int32_t epp;
  int32_t dim;
  int32_t dtype; /* hca_dtype */
} hca_paged_cache;

/* Human-readable name of a status (static string). */
const char* hca_status_string(hca_status s);

/* Library version, e.g. "hca 0.1.0 gfx950" ("... debug" for the debug build). */
const char* hca_version(void);

/*
 * hca_debug_status -- the debug build's record of indices that the inputs
 * should not hold (a checked build of the same kernels, compiled with
 * -DHCA_DEBUG into libhca_debug.so; no section of the pages: it checks the
 * paging contract of the entry points below).  Where a kernel meets a page id
 * outside its pool, a block-table slot past the table's width, a selected
 * entry outside its sequence's entries or a row outside its page, the release
 * build skips that row or page (documented per entry point); the debug build
 * does the same and also sets a bit in a device word.  This call waits for the
 * device (hipDeviceSynchronize), reads the bits of every module into *bits
 * (1 page id, 2 table slot, 4 selected entry, 8 row) and clears them.
 *   returns    HCA_OK when no bit is set, HCA_ERR_INVALID when some are,
 *              HCA_ERR_HIP when the device or the read fails, HCA_ERR_INVALID
 *              for a NULL bits; HCA_ERR_UNSUPPORTED (and *bits = 0) in the
 *              release build, which records nothing.
 */
hca_status hca_debug_status(uint32_t* bits);

/*
 * kv_compress -- the compressor (V4 page, section 2.1: a learned weighted sum
 * with positional bias folds every m tokens into one entry; section 3.1.2: the
 * not-yet-folded tokens are a rolling residual; section 3.2.1: RoPE is applied
 * before the entry is inserted into the cache).
 *
 * For sequence b, tokens t = 0 .. ntok[b]-1 are the raw vectors of positions
 * pos0[b] + t (pos0[b] a multiple of m).  Entry j (j < ceil(ntok[b]/m)) folds
 * the slots i < m + overlap of its window, t = j*m - overlap + i, that lie at
 * positions >= 0 and below pos0[b] + ntok[b]:
 *     w_i = softmax_i(gate_logit[t] + pos_bias[i])   (over those slots)
 *     c   = sum_i w_i x[t]
 *     c   = c * norm_gamma / sqrt(mean_c(c^2) + norm_eps)   (only if norm_gamma)
 *     out[b][j] = RoPE(c, pos0[b] + j*m)
 * A partial group (r < m) is normalized over its r slots, which is the state of
 * the rolling residual; re-running the call on a decode step's open group
 * (pos0 = m*floor((L-1)/m), ntok = L - pos0) re-emits the open entry.  With
 * m = 1 this is the window insert RoPE(x_t, t).  RoPE rotates adjacent pairs
 * (2i, 2i+1) by angle p * rope_theta^(-2i/d); the angle is reduced in fp64.
 * With overlap = 0 a window is the entry's own m tokens; c4a's window (section
 * 2.1 folds every 8 tokens into one entry at a ratio of 1/4, section 3.1.2
 * keeps an 8-token state) is m = 4, overlap = 4: tokens [4j-4, 4j+4).  The
 * overlap's tokens are read at rows t = -overlap .. -1 before the run's first
 * row (x and gate_logit), so for pos0[b] > 0 the caller keeps the previous
 * group's last tokens there (as a ring of overlap + m rows does, or a buffer
 * of the whole context); rows at positions below 0 are never read.
 * The optional RMS normalisation is the RMSNorm that section 3.2.1 fuses
 * between the compressor and RoPE; it acts on the folded (possibly partial)
 * entry, before the rotation.
 *
 *   x          bf16  x[b * x_stride_b + t * d + c]
 *   gate_logit float gate_logit[b * z_stride_b + t]
 *   pos_bias   float [m + overlap]
 *   pos0, ntok int32 [B] (device); ntok[b] is clamped to [0, max_ntok]
 *   max_ntok   host bound on ntok (sizes the grid)
 *   d          even, 2 <= d, d % 8 == 0;  m in {1, 2, 4, ..., 256}
 *   overlap    0 .. m (HCA_ERR_INVALID otherwise); > 0 needs m <= 16
 *              (HCA_ERR_UNSUPPORTED)
 *   norm_gamma float [d] (16-byte aligned) or NULL (no normalisation);
 *   norm_eps   finite, > 0 when norm_gamma is given (ignored otherwise)
 *   out        float out[b * out_stride_b + j * d + c]
 */
hca_status kv_compress(const uint16_t* x, int64_t x_stride_b, const float* gate_logit,
                       int64_t z_stride_b, const float* pos_bias, const int32_t* pos0,
                       const int32_t* ntok, int32_t B, int32_t max_ntok, int32_t d, int32_t m,
                       int32_t overlap, float rope_theta, const float* norm_gamma, float norm_eps,
                       float* out, int64_t out_stride_b, void* stream);

/*
 * kv_quantize_page -- quantize entries into their pages (V4 page, sections
 * 3.1.1 and 3.1.3: one 256-token logical block, page size = block size x
 * compress ratio x bytes per element; fp8 main KV, fp8/fp4 indexer keys).
 *
 * For sequence b, rows i = 0 .. ne[b]-1 of src are entries e0[b] + i
 * (e0[b] a multiple of dst.epp).  Every page touched is rewritten whole: its
 * valid rows are the rows of this call that fall in it; slots past them are
 * zeroed; the fp8 page scale is taken over the valid rows only.  Pages written
 * by different sequences in one call must be distinct.
 *
 *   src        float src[b * src_stride_b + i * dst.dim + c]
 *   e0, ne     int32 [B] (device); ne[b] clamped to [0, max_ne]
 *   block_table int32 [B][bt_stride]
 *   ws         NULL, or kv_quantize_page_workspace(B, max_ne, dst) bytes of
 *              device scratch (no initial contents needed).  With a
 *              workspace an fp8 page is split over several blocks (an amax
 *              pass then an encode pass), which is what a decode step that
 *              rewrites one open page per sequence needs; without one, each
 *              page is done by a single block.  The codes are the same either
 *              way.  Calls that overlap in time must use different workspaces.
 *              The size is 0 for fp4 and bf16 pools (ws is then ignored).
 */
size_t kv_quantize_page_workspace(int32_t B, int32_t max_ne, hca_paged_cache dst);
hca_status kv_quantize_page(const float* src, int64_t src_stride_b, const int32_t* e0,
                            const int32_t* ne, int32_t B, int32_t max_ne,
                            const int32_t* block_table, int32_t bt_stride, hca_paged_cache dst,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * kv_prefill_pages -- the prefill of one pool in one launch: the compressor,
 * its RMSNorm, RoPE and the insertion into the cache fused (V4 page, section
 * 3.2.1 lists compressor, RMSNorm, RoPE and cache insertion as one fused
 * step; sections 3.1.1 and 3.1.3: the page formats).  The result is that of
 * kv_compress(...) followed by kv_quantize_page(e0 = pos0[b] / m, ne =
 * ceil(ntok[b] / m)) on its output: the same bytes in every page written,
 * without the fp32 entries passing through memory.  Each page is folded,
 * normalised, rotated and quantized by one block of the launch.
 *
 *   x, gate_logit, pos_bias, pos0, ntok, max_ntok, m, overlap, rope_theta,
 *   norm_gamma, norm_eps: as kv_compress (d = dst.dim); pos0[b] must be a
 *              multiple of 256 (the run starts a page; another value writes
 *              the wrong pages, never out of bounds)
 *   block_table int32 [B][bt_stride]: the page of logical block
 *              pos0[b] / 256 + i holds the run's entries [i * epp, i * epp + epp)
 *   dst        the pool; dst.epp == 256 / m; dtype HCA_FP8_E4M3 or HCA_BF16;
 *              a page must fit one block: for m <= 16, dst.epp * d <= 32768
 *              (d = 512: m >= 4; d = 128: any m), for m > 16,
 *              dst.epp * d <= 14336 (HCA_ERR_UNSUPPORTED otherwise, nothing
 *              launched: use kv_compress + kv_quantize_page)
 */
hca_status kv_prefill_pages(const uint16_t* x, int64_t x_stride_b, const float* gate_logit, int64_t z_stride_b,
                            const float* pos_bias, const int32_t* pos0, const int32_t* ntok, int32_t B,
                            int32_t max_ntok, int32_t m, int32_t overlap, float rope_theta, const float* norm_gamma,
                            float norm_eps, const int32_t* block_table, int32_t bt_stride, hca_paged_cache dst,
                            void* stream);

/*
 * kv_compress_insert -- a decode step's update of one pool in one launch: the
 * open group is folded as kv_compress folds it (V4 page, section 2.1; section
 * 3.1.2: the open group is the rolling residual; section 3.2.1: RoPE, then
 * insertion into the cache) into its row of the open page's f32 staging, and
 * the open page is quantized as kv_quantize_page quantizes it (sections 3.1.1
 * and 3.1.3).  Without a fold state, the staging row and the page bytes are
 * identical to those of kv_compress(max_ntok = m) followed by kv_quantize_page
 * on that page; with one (below), the page bytes are those of kv_quantize_page
 * on the staging rows.
 *
 * For sequence b the open group has ntok[b] tokens (clamped to [0, m]; 0
 * writes nothing) starting at position pos0[b] (a multiple of m); its entry
 * j = pos0[b]/m is row j - e0[b] of the page that starts at entry e0[b] (a
 * multiple of dst.epp), which must be in [0, dst.epp) (else nothing is
 * written); rows 0 .. j-e0[b]-1 of stage are the page's earlier entries.
 *
 *   x, gate_logit, pos_bias, overlap, norm_gamma, norm_eps: as kv_compress,
 *              with T = m tokens per sequence after the overlap's rows (a
 *              ring of overlap + m rows, x pointing at row overlap); m = 1 is
 *              the window insert of one token (dst.epp = 256)
 *   stage      float stage[b * stage_stride_b + r * dst.dim + c], r < dst.epp;
 *              row j - e0[b] is written
 *   block_table int32 [B][bt_stride]: page of logical block e0[b] / dst.epp
 *   dst        the pool; dst.epp == 256 / m, dst.dim <= 2048
 *   append     0: the page is rewritten whole from staging;
 *              1: the caller guarantees that the page already holds the codes
 *              of rows 0 .. j-e0[b]-1, made from the same staging rows (as a
 *              previous call leaves them), and, for m = 1, that row j-e0[b] is
 *              new or unchanged (a window insert).  Only what changes is then
 *              written: the earlier rows' codes stand while the fp8 page scale
 *              does.  For m > 1 (the open entry is re-folded every step) the
 *              scale is taken over all rows; for m = 1 it is max(old scale,
 *              the new row's), which is exact because fl32(amax/448) is
 *              monotonic in amax.  The result equals that of append = 0.
 *   fold_state float [B][S] (16-byte aligned, S % 4 == 0) or NULL: the
 *              pool's update state per sequence, S >= 4, and S >= 4 + 2 *
 *              (4 + dst.dim) when m > 16.  Zero-filled is a valid state; the
 *              caller keeps it with its ring and page (re-zero it when either
 *              is rewritten otherwise).  Floats 0..3, for fp8 pages in append
 *              mode with m > 1: how many of the open page's rows, and their
 *              amax (rows before the open one no longer change), so a call
 *              reads no earlier staging row while the page scale holds; a
 *              header that holds the rows before the open one but the last
 *              is completed from that row, any other is rebuilt from staging.
 *              Then, for m > 16 (a re-fold reads the whole open group), two
 *              running fold states of 4 + dim floats (token count, max logit,
 *              sum of exp(logit - max), unused, exp-weighted token sums): a
 *              call with ntok = n reads slot (n-1) % 2 and writes slot n % 2,
 *              folding only the newest token (a repeated call gives the same
 *              result); where the slot does not hold the state after n-1
 *              tokens (a new group, a zero-filled state), the group is
 *              re-folded whole and the state rewritten.  With fold states the
 *              entry is the same fold up to rounding (the running sums rescale
 *              as the maximum grows), so it need not match kv_compress bit for
 *              bit.  Page bytes are the same with or without a state.
 * Calls that write the same page or staging must be ordered by the caller.
 */
hca_status kv_compress_insert(const uint16_t* x, int64_t x_stride_b, const float* gate_logit, int64_t z_stride_b,
                              const float* pos_bias, const int32_t* pos0, const int32_t* ntok, int32_t B, int32_t m,
                              int32_t overlap, float rope_theta, const float* norm_gamma, float norm_eps, float* stage,
                              int64_t stage_stride_b, const int32_t* e0, const int32_t* block_table,
                              int32_t bt_stride, hca_paged_cache dst, int32_t append, float* fold_state,
                              int64_t fold_state_stride_b, void* stream);

/*
 * kv_compress_insert_jobs -- several kv_compress_insert calls over the same B
 * sequences in one launch (a layer's window insert, its open entry and its
 * open indexer page), so the decode update of a layer costs one launch.
 * Each job has the arguments of kv_compress_insert; a job whose x is NULL
 * folds nothing: its open row j - e0[b] is already in stage (gate_logit,
 * pos_bias, ntok, overlap, rope_theta and the norm arguments are then unused) and the page is quantized as
 * described above.  Jobs must write different pages and staging rows.
 *   n_jobs     0 .. 4 (HCA_ERR_UNSUPPORTED above); every job is validated
 *              before anything is launched.
 */
typedef struct {
  const uint16_t* x; /* NULL: nothing to fold */
  int64_t x_stride_b;
  const float* gate_logit;
  int64_t z_stride_b;
  const float* pos_bias;
  const int32_t* pos0;
  const int32_t* ntok;
  int32_t m;
  int32_t overlap;
  float rope_theta;
  const float* norm_gamma; /* NULL: no normalisation */
  float norm_eps;
  float* stage;
  int64_t stage_stride_b;
  const int32_t* e0;
  const int32_t* block_table;
  int32_t bt_stride;
  hca_paged_cache dst;
  int32_t append;
  float* fold_state; /* NULL: the open group is re-folded whole */
  int64_t fold_state_stride_b;
} hca_insert_job;
hca_status kv_compress_insert_jobs(const hca_insert_job* jobs, int32_t n_jobs, int32_t B, void* stream);

/*
 * indexer_topk -- indexer scoring and top-k selection for c4a layers (V4 page,
 * section 2.2: a separate, smaller indexer KV tells the query which compressed
 * entries to look in).
 *
 * N_b = ceil(seq_lens[b] / m) entries.  For entry j the decoded key k_j
 * (dim = idx_keys.dim) is scored by
 *     s_j = sum_h head_w[b][h] * max(0, q_idx[b][h] . k_j),   h < HI
 * (fp32 accumulation of exact bf16 products).  The k largest scores are kept
 * (ties: lower index first) and written in ascending index order to
 * out_idx[b][0 .. n-1], n = min(k, N_b); the rest of the row is -1 and
 * out_n[b] = n.
 *
 *   q_idx      bf16 [B][HI][idx_keys.dim];  head_w float [B][HI]
 *   HI         1 .. 16;  idx_keys.dim in {32, 64, 128, 256};  epp = 256/m
 *   seq_lens   int32 [B] (device), clamped to [0, max_seq_len]
 *   k          1 .. 8192; at most 2^21 entries per sequence (ceil(max_seq_len/m))
 *   ws         workspace of indexer_topk_workspace(...) bytes.  It must be
 *              zero-filled before its first use; every successful call leaves
 *              the part that must start at zero (a score histogram) zeroed
 *              again, so it can be reused as is (re-zero it after a failed
 *              call).  Calls that overlap in time must use different
 *              workspaces.
 */
size_t indexer_topk_workspace(int32_t B, int32_t max_seq_len, int32_t m, int32_t k);
hca_status indexer_topk(const uint16_t* q_idx, const float* head_w, int32_t HI,
                        hca_paged_cache idx_keys, const int32_t* block_table, int32_t bt_stride,
                        const int32_t* seq_lens, int32_t B, int32_t max_seq_len, int32_t m,
                        int32_t k, int32_t* out_idx, int32_t* out_n, void* ws, size_t ws_bytes,
                        void* stream);

/*
 * indexer_topk_with_updates -- indexer_topk with a decode step's cache updates
 * run beside its score pass (V4 page, section 3.2.2: the indexer overlaps the
 * main-KV compression and the window insert).  The result is that of
 * kv_compress_insert_jobs(jobs, n_jobs, B) followed by indexer_topk(...): the
 * same bytes in every output and page.  Jobs that write other pools run as
 * extra blocks of the select's last launch.  A job that writes the indexer
 * keys runs before the score pass: the open indexer row of a decode step (no
 * fold, append, fp4 keys of dim 128 with 64 entries per page, the indexer's
 * block table) inside it, encoded by the score blocks of its page; any other
 * as a launch of its own.  The open row is written whenever it lies within
 * the first ceil(max_seq_len / m) entries, the pages the score launch covers
 * (it is scored only when it also lies within the sequence's
 * ceil(seq_lens[b] / m) entries); an open row past that bound, from
 * positions that disagree with max_seq_len, may be left unwritten, where the
 * two-call form would write it.  Jobs are validated as for kv_compress_insert_jobs,
 * the indexer arguments as for indexer_topk; nothing is launched on any
 * error.
 */
hca_status indexer_topk_with_updates(const uint16_t* q_idx, const float* head_w, int32_t HI,
                                     hca_paged_cache idx_keys, const int32_t* block_table, int32_t bt_stride,
                                     const int32_t* seq_lens, int32_t B, int32_t max_seq_len, int32_t m,
                                     int32_t k, int32_t* out_idx, int32_t* out_n, void* ws, size_t ws_bytes,
                                     const hca_insert_job* jobs, int32_t n_jobs, void* stream);

/*
 * paged_hybrid_decode -- attention of the decode query over the selected
 * compressed entries plus the raw window (V4 page, section 2.1: shared K=V,
 * RoPE on the key use, inverse RoPE on the output; c128a attends to all of its
 * entries; section 2.3: every layer keeps a raw window, usually 128 tokens;
 * vLLM-0.7.2 page, section 2.3: only window blocks are read).
 *
 * For sequence b with L = seq_lens[b], the rows are
 *   - the entries sel_idx[b][0 .. sel_n[b]-1] (indices outside [0, ceil(L/m))
 *     are skipped), or all ceil(L/m) entries when sel_idx is NULL, read from
 *     `kv` through block_table; then
 *   - the window tokens t in [max(0, L - window), L), read from `win` through
 *     win_block_table.
 * Stored rows are already rotated.  With q~_h = RoPE(q[b][h], L-1):
 *     p = softmax(softmax_scale * q~_h . rows),  o = sum p * rows
 *     out[b][h] = RoPE^-1(o, L-1),  lse[b][h] = log sum exp(logits)
 * A sequence with no rows gets out = 0 and lse = -inf.
 * The output can also be delivered in fp8, as section 3.2.1 fuses inverse RoPE
 * with the fp8 quantization that feeds the fp8 o_lora GEMM: one scale per
 * (b, h) row, out_scale[b][h] = amax/448 over the row's d values (1 for an
 * all-zero row), out_fp8[b][h][c] = E4M3(out[b][h][c] / out_scale[b][h]),
 * round to nearest even, saturating at +-448 (the fp8 pages' rule).
 *
 *   q          bf16 [B][H][kv.dim], unrotated;  H in 1 .. 128
 *   kv.dim     in {64, 128, 256, 512}; win.dim == kv.dim; win.epp == 256
 *   kv, win    dtype HCA_FP8_E4M3 or HCA_BF16, the same for both pools
 *   sel_idx    int32 [B][k] or NULL;  sel_n int32 [B] (required with sel_idx)
 *   window     0 .. 256 (0: no window; win and win_block_table may be NULL)
 *   out        float [B][H][kv.dim] or NULL;  lse float [B][H] or NULL
 *   out_fp8    uint8 [B][H][kv.dim] (2-byte aligned) or NULL, with
 *   out_scale  float [B][H]; at least one of out and out_fp8 is required
 *   ws         workspace of paged_hybrid_decode_workspace(B, H, d, max_seq_len,
 *              m, window, k) bytes, with k = 0 when sel_idx will be NULL; its
 *              contents on entry do not matter.
 */
size_t paged_hybrid_decode_workspace(int32_t B, int32_t H, int32_t d, int32_t max_seq_len,
                                     int32_t m, int32_t window, int32_t k);
hca_status paged_hybrid_decode(const uint16_t* q, int32_t H, hca_paged_cache kv,
                               const int32_t* block_table, int32_t bt_stride, hca_paged_cache win,
                               const int32_t* win_block_table, int32_t wbt_stride,
                               const int32_t* seq_lens, int32_t B, int32_t max_seq_len, int32_t m,
                               int32_t window, const int32_t* sel_idx, const int32_t* sel_n,
                               int32_t k, float softmax_scale, float rope_theta, float* out,
                               float* lse, uint8_t* out_fp8, float* out_scale, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * paged_hybrid_decode_noalloc -- paged_hybrid_decode without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments, results and errors as paged_hybrid_decode, with the same
 * kernels; the scratch its kernels need (per-split partial outputs) is a
 * static array of paged_hybrid_decode_noalloc_max_bytes() bytes (32 MiB) in
 * the library's code object, one per GPU, held until the process ends.  The
 * call allocates nothing.  A shape whose scratch,
 * paged_hybrid_decode_workspace(B, H, d, max_seq_len, m, window, k), exceeds
 * that size returns HCA_ERR_WORKSPACE and launches nothing.  Every call on a
 * GPU shares that GPU's scratch: calls that may overlap in time on one GPU
 * (different streams, other threads) race and must be ordered by the caller.
 * The scratch needs no initial contents.
 */
size_t paged_hybrid_decode_noalloc_max_bytes(void);
hca_status paged_hybrid_decode_noalloc(const uint16_t* q, int32_t H, hca_paged_cache kv,
                                       const int32_t* block_table, int32_t bt_stride, hca_paged_cache win,
                                       const int32_t* win_block_table, int32_t wbt_stride,
                                       const int32_t* seq_lens, int32_t B, int32_t max_seq_len, int32_t m,
                                       int32_t window, const int32_t* sel_idx, const int32_t* sel_n,
                                       int32_t k, float softmax_scale, float rope_theta, float* out,
                                       float* lse, uint8_t* out_fp8, float* out_scale, void* stream);

/*
 * kv_gather -- paged -> contiguous copy of rows 0 .. n_rows[b]-1 of every
 * sequence (vLLM-0.7.2 page, section 2.1: logical blocks map to physical
 * pages).  A layout check: the bytes must not depend on where pages live.
 *
 *   dst_codes  row r of sequence b at dst_codes + (b * max_rows + r) * row_bytes,
 *              row_bytes = dim (fp8), dim/2 (fp4), 2*dim (bf16)
 *   dst_scales fp8: float [B][max_rows] (the row's page scale);
 *              fp4: uint8 [B][max_rows][dim/32]; bf16: unused (may be NULL)
 *   n_rows     int32 [B] (device), clamped to [0, max_rows]; rows past n_rows[b]
 *              are left untouched
 */
hca_status kv_gather(hca_paged_cache src, const int32_t* block_table, int32_t bt_stride,
                     const int32_t* n_rows, int32_t B, int32_t max_rows, void* dst_codes,
                     void* dst_scales, void* stream);

/*
 * Page-pool packing (V4 page, section 3.1.3: the page of a KV kind is block
 * size x compress ratio x bytes per element, and the pools of all KV kinds
 * are packed into a few buckets by page size, each a pool of fixed-size
 * pages; section 3.1.1: one 256-token logical block; vLLM-0.7.2 page, section
 * 2.1: block tables name physical pages, and sequences with a common prefix
 * name the same ones).  Host-side bookkeeping over one device arena that the
 * caller allocates; nothing here touches the device.
 *
 * A kind is (m, dim, dtype): m = 1 for the raw window, 4 or 128 for the
 * compressed entries, and the indexer keys' (4, d_I, fp8 or fp4).
 *   hca_page_bytes   code bytes of one page, 256/m rows of dim elements
 *                    (fp8 1 byte, fp4 half a byte, bf16 2 bytes), and its
 *                    scale bytes (fp8: one float per page; fp4: one E4M3 byte
 *                    per 32 elements of a row; bf16: none).
 *   hca_pool_plan    kinds with equal (code, scale) bytes share a bucket:
 *                    kind_bucket[n_kinds], *n_buckets.
 *   hca_pool_create  capacity[b] pages for each bucket; *arena_bytes is the
 *                    device arena the pools need (256-byte aligned regions:
 *                    per bucket its pages' codes, then their scales).  The
 *                    pool object is the caller's until hca_pool_destroy.
 *   hca_pool_view    the hca_paged_cache of a kind inside an arena (256-byte
 *                    aligned): the kernels take it as they take any pool;
 *                    kinds of one bucket share its pages' memory and ids.
 *   hca_pool_alloc   n pages of a bucket, each with one reference (all or
 *                    nothing; HCA_ERR_UNSUPPORTED when the bucket has fewer
 *                    free pages).  Pages are taken from the free pages first,
 *                    then from the released pages that kept a key, oldest
 *                    released first (their keys are dropped).
 *   hca_pool_share   one more reference to held pages (a shared prefix).
 *   hca_pool_release drop one reference per listed page (a page may be
 *                    listed as often as it is held); at zero a page is free,
 *                    or cached if it was published.
 *   hca_pool_publish a held page's contents are the block named by `key`
 *                    (say, a hash of the prefix through that block); a key
 *                    names one page at a time.
 *   hca_pool_lookup  the page published under `key` with one more reference
 *                    (brought back if it was cached), or -1.
 *   hca_pool_stats   free, cached and held pages of a bucket, and the arena
 *                    offsets of its codes and scales.
 * Invalid arguments return HCA_ERR_INVALID and change nothing.  Calls on one
 * pool must not overlap in time.
 */
typedef struct {
  int32_t m;
  int32_t dim;
  int32_t dtype; /* hca_dtype */
} hca_kv_kind;
typedef struct hca_page_pool hca_page_pool;
hca_status hca_page_bytes(hca_kv_kind kind, size_t* code_bytes, size_t* scale_bytes);
hca_status hca_pool_plan(const hca_kv_kind* kinds, int32_t n_kinds, int32_t* kind_bucket, int32_t* n_buckets);
hca_status hca_pool_create(const hca_kv_kind* kinds, int32_t n_kinds, const int32_t* capacity,
                           size_t* arena_bytes, hca_page_pool** out);
void hca_pool_destroy(hca_page_pool* pool);
hca_status hca_pool_view(const hca_page_pool* pool, int32_t kind, void* arena, hca_paged_cache* out);
int32_t hca_pool_bucket(const hca_page_pool* pool, int32_t kind);
hca_status hca_pool_alloc(hca_page_pool* pool, int32_t bucket, int32_t n, int32_t* pages);
hca_status hca_pool_share(hca_page_pool* pool, int32_t bucket, const int32_t* pages, int32_t n);
hca_status hca_pool_release(hca_page_pool* pool, int32_t bucket, const int32_t* pages, int32_t n);
hca_status hca_pool_publish(hca_page_pool* pool, int32_t bucket, int32_t page, uint64_t key);
hca_status hca_pool_lookup(hca_page_pool* pool, int32_t bucket, uint64_t key, int32_t* page);
hca_status hca_pool_stats(const hca_page_pool* pool, int32_t bucket, int64_t* free_pages, int64_t* cached_pages,
                          int64_t* held_pages, size_t* codes_offset, size_t* scales_offset);

#ifdef __cplusplus
}
#endif

#endif /* HCA_H */
