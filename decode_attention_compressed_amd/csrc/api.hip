// C ABI of libhca: host-side argument validation, then kernel launches.
// Nothing here allocates, synchronizes or keeps state between calls.
#include <math.h>
#include <string.h>

#include <mutex>

#include "hca.h"
#include "hca_common.h"
#include "hca_internal.h"
#include "hca_testing.h"

using namespace hca;

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool valid_m(int m) { return m >= 1 && m <= 256 && (256 % m) == 0; }
// overlapping windows: 0 <= overlap <= m, and only for groups the small-group fold takes
hca_status overlap_ok(int m, int overlap) {
  if (overlap < 0 || overlap > m) return HCA_ERR_INVALID;
  if (overlap > 0 && m > kSmallM) return HCA_ERR_UNSUPPORTED;
  return HCA_OK;
}
// RMS normalisation arguments: none, or a 16-byte aligned gain vector with a finite eps > 0
bool norm_ok(const float* gamma, float eps) {
  return gamma == nullptr || (aligned(gamma, 16) && eps > 0.0f && isfinite(eps));
}

// a pool descriptor that the kernels can index safely
bool cache_ok(const hca_paged_cache& c) {
  if (!c.codes || c.num_pages < 1 || c.epp < 1 || c.dim < 8 || (c.dim % 8) != 0) return false;
  if (256 % c.epp != 0) return false;
  if (c.dtype != HCA_BF16 && c.dtype != HCA_FP8_E4M3 && c.dtype != HCA_FP4_E2M1) return false;
  if (c.dtype != HCA_BF16 && !c.scales) return false;
  if (c.dtype == HCA_FP4_E2M1 && (c.dim % 32) != 0) return false;
  if (!aligned(c.codes, 16)) return false;
  return true;
}

hca_status from_hip(hipError_t e) { return e == hipSuccess ? HCA_OK : HCA_ERR_HIP; }

}  // namespace

extern "C" {

const char* hca_status_string(hca_status s) {
  switch (s) {
    case HCA_OK: return "ok";
    case HCA_ERR_INVALID: return "invalid argument";
    case HCA_ERR_UNSUPPORTED: return "unsupported shape or type";
    case HCA_ERR_WORKSPACE: return "workspace missing or too small";
    case HCA_ERR_HIP: return "HIP launch or runtime error";
  }
  return "unknown status";
}

const char* hca_version(void) {
#ifdef HCA_DEBUG
  return "hca 0.1.0 gfx950 debug";
#else
  return "hca 0.1.0 gfx950";
#endif
}

hca_status hca_debug_status(uint32_t* bits) {
#ifdef HCA_DEBUG
  if (bits == nullptr) return HCA_ERR_INVALID;
  if (hipDeviceSynchronize() != hipSuccess) return HCA_ERR_HIP;
  const uint32_t v = debug_bits_attention(true) | debug_bits_compress(true) | debug_bits_indexer(true) |
                     debug_bits_quantize(true);
  if (v & 0x80000000u) return HCA_ERR_HIP;
  *bits = v;
  return v != 0 ? HCA_ERR_INVALID : HCA_OK;
#else
  if (bits != nullptr) *bits = 0;
  return HCA_ERR_UNSUPPORTED;
#endif
}

hca_status kv_compress(const uint16_t* x, int64_t x_stride_b, const float* gate_logit, int64_t z_stride_b,
                       const float* pos_bias, const int32_t* pos0, const int32_t* ntok, int32_t B, int32_t max_ntok,
                       int32_t d, int32_t m, int32_t overlap, float rope_theta, const float* norm_gamma,
                       float norm_eps, float* out, int64_t out_stride_b, void* stream) {
  if (B < 0 || max_ntok < 0) return HCA_ERR_INVALID;
  if (!valid_m(m) || d < 8 || (d % 8) != 0) return HCA_ERR_INVALID;
  if (d > 2048) return HCA_ERR_UNSUPPORTED;
  const hca_status ov = overlap_ok(m, overlap);
  if (ov != HCA_OK) return ov;
  if (!(rope_theta > 0.0f) || !isfinite(rope_theta)) return HCA_ERR_INVALID;
  if (!norm_ok(norm_gamma, norm_eps)) return HCA_ERR_INVALID;
  if (B == 0 || max_ntok == 0) return HCA_OK;
  if (!x || !gate_logit || !pos_bias || !pos0 || !ntok || !out) return HCA_ERR_INVALID;
  if (!aligned(x, 16) || !aligned(out, 16)) return HCA_ERR_INVALID;
  const int64_t n_out = (max_ntok + m - 1) / m;
  if (x_stride_b % 8 != 0 || out_stride_b % 4 != 0) return HCA_ERR_INVALID;
  if (B > 1 && (x_stride_b < (int64_t)max_ntok * d || z_stride_b < max_ntok || out_stride_b < n_out * d))
    return HCA_ERR_INVALID;
  CompressArgs a{x, x_stride_b, gate_logit, z_stride_b, pos_bias, pos0, ntok, B, max_ntok, d, m, overlap,
                 rope_theta, 0.0, norm_gamma, norm_eps, out, out_stride_b};
  return from_hip(launch_compress(a, (hipStream_t)stream));
}

}  // extern "C"

namespace {
// one job of a fused insert: validated on the host, nothing launched on failure
hca_status make_insert(const hca_insert_job& j, int32_t B, InsertArgs& out) {
  if (j.bt_stride < 1 || (j.append != 0 && j.append != 1)) return HCA_ERR_INVALID;
  if (!valid_m(j.m) || !cache_ok(j.dst) || j.dst.epp != 256 / j.m) return HCA_ERR_INVALID;
  const int d = j.dst.dim;
  if (d > 2048) return HCA_ERR_UNSUPPORTED;
  const bool fold = j.x != nullptr;
  if (fold && (!(j.rope_theta > 0.0f) || !isfinite(j.rope_theta))) return HCA_ERR_INVALID;
  if (fold && !norm_ok(j.norm_gamma, j.norm_eps)) return HCA_ERR_INVALID;
  if (fold && overlap_ok(j.m, j.overlap) != HCA_OK) return overlap_ok(j.m, j.overlap);
  if (!j.pos0 || !j.stage || !j.e0 || !j.block_table) return HCA_ERR_INVALID;
  if (fold && (!j.gate_logit || !j.pos_bias || !j.ntok || !aligned(j.x, 16) || j.x_stride_b % 8 != 0))
    return HCA_ERR_INVALID;
  if (!aligned(j.stage, 16) || j.stage_stride_b % 4 != 0) return HCA_ERR_INVALID;
  if (B > 1 && j.stage_stride_b < (int64_t)j.dst.epp * d) return HCA_ERR_INVALID;
  if (fold && B > 1 && (j.x_stride_b < (int64_t)j.m * d || j.z_stride_b < j.m)) return HCA_ERR_INVALID;
  const bool state = fold && j.fold_state != nullptr;
  const int64_t state_floats = kPageHead + (j.m > kSmallM ? 2 * (int64_t)(kFoldStateHead + d) : 0);
  if (state && (!aligned(j.fold_state, 16) || j.fold_state_stride_b % 4 != 0)) return HCA_ERR_INVALID;
  if (state && B > 1 && j.fold_state_stride_b < state_floats) return HCA_ERR_INVALID;
  out = InsertArgs{CompressArgs{j.x, j.x_stride_b, j.gate_logit, j.z_stride_b, j.pos_bias, j.pos0, j.ntok, B, j.m, d,
                                j.m, fold ? j.overlap : 0, j.rope_theta, 0.0, j.norm_gamma, j.norm_eps, nullptr, 0},
                   j.stage, j.stage_stride_b, j.e0, j.block_table, j.bt_stride, j.dst, j.append,
                   state ? j.fold_state : nullptr, j.fold_state_stride_b};
  return HCA_OK;
}
}  // namespace

extern "C" {

hca_status kv_compress_insert(const uint16_t* x, int64_t x_stride_b, const float* gate_logit, int64_t z_stride_b,
                              const float* pos_bias, const int32_t* pos0, const int32_t* ntok, int32_t B, int32_t m,
                              int32_t overlap, float rope_theta, const float* norm_gamma, float norm_eps, float* stage,
                              int64_t stage_stride_b, const int32_t* e0, const int32_t* block_table, int32_t bt_stride,
                              hca_paged_cache dst, int32_t append, float* fold_state, int64_t fold_state_stride_b,
                              void* stream) {
  if (B < 0) return HCA_ERR_INVALID;
  if (!x) return HCA_ERR_INVALID;  // this entry point always folds
  const hca_insert_job j{x,        x_stride_b,     gate_logit, z_stride_b,  pos_bias,   pos0,
                         ntok,     m,              overlap,    rope_theta,  norm_gamma, norm_eps,
                         stage,    stage_stride_b, e0,         block_table, bt_stride,  dst,
                         append,   fold_state,     fold_state_stride_b};
  InsertJobs jobs{};
  const hca_status st = make_insert(j, B, jobs.job[0]);
  if (st != HCA_OK || B == 0) return st;
  jobs.n = 1;
  return from_hip(launch_insert(jobs, B, (hipStream_t)stream));
}

hca_status kv_compress_insert_jobs(const hca_insert_job* jobs, int32_t n_jobs, int32_t B, void* stream) {
  if (B < 0 || n_jobs < 0 || (n_jobs > 0 && !jobs)) return HCA_ERR_INVALID;
  if (n_jobs > kMaxInsertJobs) return HCA_ERR_UNSUPPORTED;
  InsertJobs all{};
  for (int i = 0; i < n_jobs; ++i) {
    const hca_status st = make_insert(jobs[i], B, all.job[i]);
    if (st != HCA_OK) return st;
  }
  if (B == 0 || n_jobs == 0) return HCA_OK;
  all.n = n_jobs;
  return from_hip(launch_insert(all, B, (hipStream_t)stream));
}

hca_status kv_prefill_pages(const uint16_t* x, int64_t x_stride_b, const float* gate_logit, int64_t z_stride_b,
                            const float* pos_bias, const int32_t* pos0, const int32_t* ntok, int32_t B,
                            int32_t max_ntok, int32_t m, int32_t overlap, float rope_theta, const float* norm_gamma,
                            float norm_eps, const int32_t* block_table, int32_t bt_stride, hca_paged_cache dst,
                            void* stream) {
  if (B < 0 || max_ntok < 0 || bt_stride < 1) return HCA_ERR_INVALID;
  if (!valid_m(m) || !cache_ok(dst) || dst.epp != 256 / m) return HCA_ERR_INVALID;
  const int d = dst.dim;
  if (d > 2048) return HCA_ERR_UNSUPPORTED;
  const hca_status ov = overlap_ok(m, overlap);
  if (ov != HCA_OK) return ov;
  if (!(rope_theta > 0.0f) || !isfinite(rope_theta)) return HCA_ERR_INVALID;
  if (!norm_ok(norm_gamma, norm_eps)) return HCA_ERR_INVALID;
  if (!prefill_supported(m, d, dst.epp, dst.dtype)) return HCA_ERR_UNSUPPORTED;
  if (B == 0 || max_ntok == 0) return HCA_OK;
  if (!x || !gate_logit || !pos_bias || !pos0 || !ntok || !block_table) return HCA_ERR_INVALID;
  if (!aligned(x, 16) || x_stride_b % 8 != 0) return HCA_ERR_INVALID;
  if (B > 1 && (x_stride_b < (int64_t)max_ntok * d || z_stride_b < max_ntok)) return HCA_ERR_INVALID;
  PrefillArgs p{CompressArgs{x, x_stride_b, gate_logit, z_stride_b, pos_bias, pos0, ntok, B, max_ntok, d, m, overlap,
                             rope_theta, 0.0, norm_gamma, norm_eps, nullptr, 0},
                block_table, bt_stride, dst};
  return from_hip(launch_prefill(p, (hipStream_t)stream));
}

size_t kv_quantize_page_workspace(int32_t B, int32_t max_ne, hca_paged_cache dst) {
  if (B < 0 || max_ne < 0 || !cache_ok(dst)) return 0;
  return quantize_ws_bytes(B, max_ne, dst);
}

hca_status kv_quantize_page(const float* src, int64_t src_stride_b, const int32_t* e0, const int32_t* ne, int32_t B,
                            int32_t max_ne, const int32_t* block_table, int32_t bt_stride, hca_paged_cache dst,
                            void* ws, size_t ws_bytes, void* stream) {
  if (B < 0 || max_ne < 0 || bt_stride < 1) return HCA_ERR_INVALID;
  if (!cache_ok(dst)) return HCA_ERR_INVALID;
  if (B == 0 || max_ne == 0) return HCA_OK;
  if (!src || !e0 || !ne || !block_table) return HCA_ERR_INVALID;
  if (!aligned(src, 16) || src_stride_b % 4 != 0) return HCA_ERR_INVALID;
  if (B > 1 && src_stride_b < (int64_t)max_ne * dst.dim) return HCA_ERR_INVALID;
  float* part = nullptr;
  const size_t need = quantize_ws_bytes(B, max_ne, dst);
  if (ws != nullptr && need > 0) {
    if (ws_bytes < need || !aligned(ws, 16)) return HCA_ERR_INVALID;
    part = static_cast<float*>(ws);
  }
  QuantArgs a{src, src_stride_b, e0, ne, B, max_ne, block_table, bt_stride, dst};
  return from_hip(launch_quantize(a, part, (hipStream_t)stream));
}

size_t indexer_topk_workspace(int32_t B, int32_t max_seq_len, int32_t m, int32_t k) {
  if (B < 0 || max_seq_len < 0 || !valid_m(m) || k < 1) return 0;
  return indexer_ws_layout(B, max_seq_len, m, k).total;
}

static hca_status indexer_prepare(const uint16_t* q_idx, const float* head_w, int32_t HI, hca_paged_cache idx_keys,
                                  const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens, int32_t B,
                                  int32_t max_seq_len, int32_t m, int32_t k, int32_t* out_idx, int32_t* out_n,
                                  bool need_out, void* ws, size_t ws_bytes, IndexerArgs& a) {
  if (B < 0 || max_seq_len < 0 || !valid_m(m) || k < 1 || bt_stride < 1) return HCA_ERR_INVALID;
  if (k > 8192) return HCA_ERR_UNSUPPORTED;
  if (HI < 1) return HCA_ERR_INVALID;
  if (HI > 16) return HCA_ERR_UNSUPPORTED;
  if (!cache_ok(idx_keys) || idx_keys.epp != 256 / m) return HCA_ERR_INVALID;
  const int di = idx_keys.dim;
  if (di != 32 && di != 64 && di != 128 && di != 256) return HCA_ERR_UNSUPPORTED;
  if ((int64_t)bt_stride * 256 < max_seq_len) return HCA_ERR_INVALID;
  if (B == 0) return HCA_OK;
  if (!q_idx || !head_w || !block_table || !seq_lens) return HCA_ERR_INVALID;
  if (need_out && (!out_idx || !out_n)) return HCA_ERR_INVALID;
  if (!aligned(q_idx, 16)) return HCA_ERR_INVALID;
  const IndexerWs lay = indexer_ws_layout(B, max_seq_len, m, k);
  if (lay.n_max > (1 << 21)) return HCA_ERR_UNSUPPORTED;  // more than 2M entries per sequence
  if (!ws || ws_bytes < lay.total || !aligned(ws, 256)) return HCA_ERR_WORKSPACE;
  a = IndexerArgs{q_idx, head_w, HI, idx_keys, block_table, bt_stride, seq_lens, B, max_seq_len, m, k, out_idx, out_n,
                  reinterpret_cast<unsigned char*>(ws), lay};
  return HCA_OK;
}

hca_status indexer_topk(const uint16_t* q_idx, const float* head_w, int32_t HI, hca_paged_cache idx_keys,
                        const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens, int32_t B,
                        int32_t max_seq_len, int32_t m, int32_t k, int32_t* out_idx, int32_t* out_n, void* ws,
                        size_t ws_bytes, void* stream) {
  IndexerArgs a{};
  const hca_status st = indexer_prepare(q_idx, head_w, HI, idx_keys, block_table, bt_stride, seq_lens, B, max_seq_len,
                                        m, k, out_idx, out_n, true, ws, ws_bytes, a);
  if (st != HCA_OK || B == 0) return st;
  return from_hip(launch_indexer(a, (hipStream_t)stream));
}

hca_status indexer_topk_with_updates(const uint16_t* q_idx, const float* head_w, int32_t HI,
                                     hca_paged_cache idx_keys, const int32_t* block_table, int32_t bt_stride,
                                     const int32_t* seq_lens, int32_t B, int32_t max_seq_len, int32_t m, int32_t k,
                                     int32_t* out_idx, int32_t* out_n, void* ws, size_t ws_bytes,
                                     const hca_insert_job* jobs, int32_t n_jobs, void* stream) {
  IndexerArgs a{};
  const hca_status st = indexer_prepare(q_idx, head_w, HI, idx_keys, block_table, bt_stride, seq_lens, B, max_seq_len,
                                        m, k, out_idx, out_n, true, ws, ws_bytes, a);
  if (st != HCA_OK) return st;
  if (n_jobs < 0 || (n_jobs > 0 && !jobs)) return HCA_ERR_INVALID;
  if (n_jobs > kMaxInsertJobs) return HCA_ERR_UNSUPPORTED;
  // jobs that write the keys go before the score pass: the open indexer row
  // (fp4 keys of 128 dims, one staged row appended, same block table) inside
  // it, any other as a launch of its own; the rest beside the compaction
  InsertJobs pre{}, side{};
  IndexerOpen open{};
  for (int i = 0; i < n_jobs; ++i) {
    const hca_insert_job& j = jobs[i];
    InsertArgs ins{};
    const hca_status sj = make_insert(j, B, ins);
    if (sj != HCA_OK) return sj;
    if (j.dst.codes != idx_keys.codes) {
      side.job[side.n++] = ins;
    } else if (open.stage == nullptr && j.x == nullptr && j.append == 1 && j.m == m &&
               idx_keys.dtype == HCA_FP4_E2M1 && idx_keys.dim == 128 && idx_keys.epp == 64 &&
               j.dst.dtype == idx_keys.dtype && j.dst.dim == idx_keys.dim && j.dst.epp == idx_keys.epp &&
               j.dst.scales == idx_keys.scales && j.dst.num_pages == idx_keys.num_pages &&
               j.block_table == block_table && j.bt_stride == bt_stride) {
      open = IndexerOpen{j.stage, j.stage_stride_b, j.pos0, j.e0};
    } else {
      pre.job[pre.n++] = ins;
    }
  }
  if (B == 0) return HCA_OK;
  a.open = open;
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = pre.n > 0 ? launch_insert(pre, B, s) : hipSuccess;
  if (e == hipSuccess) e = launch_indexer_score(a, s);
  if (e == hipSuccess) e = launch_select_chunk(a, s);
  if (e == hipSuccess) e = launch_compact_insert(a, side, s);
  return from_hip(e);
}

hca_status hca_indexer_score(const uint16_t* q_idx, const float* head_w, int32_t HI, hca_paged_cache idx_keys,
                             const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens, int32_t B,
                             int32_t max_seq_len, int32_t m, int32_t k, void* ws, size_t ws_bytes, void* stream) {
  IndexerArgs a{};
  const hca_status st = indexer_prepare(q_idx, head_w, HI, idx_keys, block_table, bt_stride, seq_lens, B, max_seq_len,
                                        m, k, nullptr, nullptr, false, ws, ws_bytes, a);
  if (st != HCA_OK || B == 0) return st;
  return from_hip(launch_indexer_score(a, (hipStream_t)stream));
}

size_t paged_hybrid_decode_workspace(int32_t B, int32_t H, int32_t d, int32_t max_seq_len, int32_t m, int32_t window,
                                     int32_t k) {
  if (B < 0 || H < 1 || d < 1 || max_seq_len < 0 || !valid_m(m) || window < 0 || k < 0) return 0;
  return attn_plan(B, H, d, max_seq_len, m, window, k, k > 0).total;
}

}  // extern "C"

namespace {
// paged_hybrid_decode's host validation and launch arguments (the workspace
// pointer left null); HCA_OK when a launch may follow (B > 0)
hca_status attn_prepare(const uint16_t* q, int32_t H, hca_paged_cache kv, const int32_t* block_table,
                        int32_t bt_stride, hca_paged_cache win, const int32_t* win_block_table, int32_t wbt_stride,
                        const int32_t* seq_lens, int32_t B, int32_t max_seq_len, int32_t m, int32_t window,
                        const int32_t* sel_idx, const int32_t* sel_n, int32_t k, float softmax_scale,
                        float rope_theta, float* out, float* lse, uint8_t* out_fp8, float* out_scale, AttnArgs& a,
                        bool& empty) {
  empty = false;
  if (B < 0 || max_seq_len < 0 || !valid_m(m) || bt_stride < 1) return HCA_ERR_INVALID;
  if (H < 1) return HCA_ERR_INVALID;
  if (H > 128) return HCA_ERR_UNSUPPORTED;
  if (!cache_ok(kv) || kv.epp != 256 / m) return HCA_ERR_INVALID;
  if (kv.dtype == HCA_FP4_E2M1) return HCA_ERR_UNSUPPORTED;
  const int d = kv.dim;
  if (d != 64 && d != 128 && d != 256 && d != 512) return HCA_ERR_UNSUPPORTED;
  if (window < 0 || window > 256) return HCA_ERR_INVALID;
  if (window > 0) {
    if (!cache_ok(win) || win.epp != 256 || win.dim != d || !win_block_table || wbt_stride < 1) return HCA_ERR_INVALID;
    if (win.dtype != kv.dtype) return HCA_ERR_UNSUPPORTED;  // one row format per launch
    if ((int64_t)wbt_stride * 256 < max_seq_len) return HCA_ERR_INVALID;
  }
  if ((int64_t)bt_stride * 256 < max_seq_len) return HCA_ERR_INVALID;
  if (sel_idx && (!sel_n || k < 1)) return HCA_ERR_INVALID;
  if (!isfinite(softmax_scale) || !(rope_theta > 0.0f) || !isfinite(rope_theta)) return HCA_ERR_INVALID;
  if (B == 0) {
    empty = true;
    return HCA_OK;
  }
  if (!q || !block_table || !seq_lens || (!out && !out_fp8)) return HCA_ERR_INVALID;
  if (out_fp8 && (!out_scale || !aligned(out_fp8, 2))) return HCA_ERR_INVALID;
  if (!aligned(q, 16)) return HCA_ERR_INVALID;
  const AttnPlan plan = attn_plan(B, H, d, max_seq_len, m, window, sel_idx ? k : 0, sel_idx != nullptr);
  if (plan.items - B + 1 > kAttnMaxSplits) return HCA_ERR_UNSUPPORTED;  // splits of one sequence
  hca_paged_cache w = win;
  if (window == 0) { w = kv; w.epp = 256; }  // never read
  a = AttnArgs{q, H, kv, block_table, bt_stride, w, window > 0 ? win_block_table : block_table,
               window > 0 ? wbt_stride : bt_stride, seq_lens, B, max_seq_len, m, window, sel_idx, sel_n,
               sel_idx ? k : 0, softmax_scale, rope_theta, 0.0, out, lse, out_fp8, out_fp8 ? out_scale : nullptr,
               nullptr, plan};
  return HCA_OK;
}

// The allocation-free variant's scratch: one array per device, in the code
// object, held until the process ends.  Host code never uses its name as an
// address: the device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the device address of the current device's scratch (looked up on its first use)
hca_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return HCA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return HCA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return HCA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HCA_OK;
}
}  // namespace

extern "C" {

hca_status paged_hybrid_decode(const uint16_t* q, int32_t H, hca_paged_cache kv, const int32_t* block_table,
                               int32_t bt_stride, hca_paged_cache win, const int32_t* win_block_table,
                               int32_t wbt_stride, const int32_t* seq_lens, int32_t B, int32_t max_seq_len, int32_t m,
                               int32_t window, const int32_t* sel_idx, const int32_t* sel_n, int32_t k,
                               float softmax_scale, float rope_theta, float* out, float* lse, uint8_t* out_fp8,
                               float* out_scale, void* ws, size_t ws_bytes, void* stream) {
  AttnArgs a{};
  bool empty = false;
  const hca_status st = attn_prepare(q, H, kv, block_table, bt_stride, win, win_block_table, wbt_stride, seq_lens, B,
                                     max_seq_len, m, window, sel_idx, sel_n, k, softmax_scale, rope_theta, out, lse,
                                     out_fp8, out_scale, a, empty);
  if (st != HCA_OK || empty) return st;
  if (!ws || ws_bytes < a.plan.total || !aligned(ws, 256)) return HCA_ERR_WORKSPACE;
  a.ws = reinterpret_cast<unsigned char*>(ws);
  return from_hip(launch_attention(a, (hipStream_t)stream));
}

hca_status hca_attention_split(const uint16_t* q, int32_t H, hca_paged_cache kv, const int32_t* block_table,
                               int32_t bt_stride, hca_paged_cache win, const int32_t* win_block_table,
                               int32_t wbt_stride, const int32_t* seq_lens, int32_t B, int32_t max_seq_len, int32_t m,
                               int32_t window, const int32_t* sel_idx, const int32_t* sel_n, int32_t k,
                               float softmax_scale, float rope_theta, void* ws, size_t ws_bytes, void* stream) {
  AttnArgs a{};
  bool empty = false;
  float dummy_out = 0.0f;  // never written: the combine is not launched
  const hca_status st = attn_prepare(q, H, kv, block_table, bt_stride, win, win_block_table, wbt_stride, seq_lens, B,
                                     max_seq_len, m, window, sel_idx, sel_n, k, softmax_scale, rope_theta, &dummy_out,
                                     nullptr, nullptr, nullptr, a, empty);
  if (st != HCA_OK || empty) return st;
  if (!ws || ws_bytes < a.plan.total || !aligned(ws, 256)) return HCA_ERR_WORKSPACE;
  a.ws = reinterpret_cast<unsigned char*>(ws);
  a.out = nullptr;
  return from_hip(launch_attention(a, (hipStream_t)stream, true));
}

size_t paged_hybrid_decode_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

hca_status paged_hybrid_decode_noalloc(const uint16_t* q, int32_t H, hca_paged_cache kv, const int32_t* block_table,
                                       int32_t bt_stride, hca_paged_cache win, const int32_t* win_block_table,
                                       int32_t wbt_stride, const int32_t* seq_lens, int32_t B, int32_t max_seq_len,
                                       int32_t m, int32_t window, const int32_t* sel_idx, const int32_t* sel_n,
                                       int32_t k, float softmax_scale, float rope_theta, float* out, float* lse,
                                       uint8_t* out_fp8, float* out_scale, void* stream) {
  AttnArgs a{};
  bool empty = false;
  const hca_status st = attn_prepare(q, H, kv, block_table, bt_stride, win, win_block_table, wbt_stride, seq_lens, B,
                                     max_seq_len, m, window, sel_idx, sel_n, k, softmax_scale, rope_theta, out, lse,
                                     out_fp8, out_scale, a, empty);
  if (st != HCA_OK || empty) return st;
  if (a.plan.total > kNoAllocScratchBytes) return HCA_ERR_WORKSPACE;
  void* p = nullptr;
  const hca_status sp = scratch_of_current_device(&p);
  if (sp != HCA_OK) return sp;
  a.ws = static_cast<unsigned char*>(p);
  return from_hip(launch_attention(a, (hipStream_t)stream));
}

hca_status kv_gather(hca_paged_cache src, const int32_t* block_table, int32_t bt_stride, const int32_t* n_rows,
                     int32_t B, int32_t max_rows, void* dst_codes, void* dst_scales, void* stream) {
  if (B < 0 || max_rows < 0 || bt_stride < 1) return HCA_ERR_INVALID;
  if (!cache_ok(src)) return HCA_ERR_INVALID;
  if ((int64_t)bt_stride * src.epp < max_rows) return HCA_ERR_INVALID;
  if (B == 0 || max_rows == 0) return HCA_OK;
  if (!block_table || !n_rows || !dst_codes) return HCA_ERR_INVALID;
  if (src.dtype != HCA_BF16 && !dst_scales) return HCA_ERR_INVALID;
  if (!aligned(dst_codes, 4)) return HCA_ERR_INVALID;
  GatherArgs a{src, block_table, bt_stride, n_rows, B, max_rows, dst_codes, dst_scales};
  return from_hip(launch_gather(a, (hipStream_t)stream));
}

// ------------------------------------------------------------------ checking hooks
hca_status hca_host_e4m3_encode(const float* in, uint8_t* out, int64_t n) {
  if (!in || !out || n < 0) return HCA_ERR_INVALID;
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode(in[i]);
  return HCA_OK;
}
hca_status hca_host_e2m1_encode(const float* in, uint8_t* out, int64_t n) {
  if (!in || !out || n < 0) return HCA_ERR_INVALID;
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)e2m1_encode(in[i]);
  return HCA_OK;
}
hca_status hca_host_bf16_encode(const float* in, uint16_t* out, int64_t n) {
  if (!in || !out || n < 0) return HCA_ERR_INVALID;
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_encode(in[i]);
  return HCA_OK;
}

}  // extern "C"

// probes: same conversions / MFMA as the kernels, on known data
namespace hca {

__global__ void probe_decode_kernel(const uint8_t* codes, float* out, int n, int kind) {
  const int i = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i >= n) return;
  if (kind == 0) {
    const uint32_t w0 = *reinterpret_cast<const uint32_t*>(codes + i);
    const uint32_t w1 = *reinterpret_cast<const uint32_t*>(codes + i + 4);
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false), b = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
    const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false), d = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
    out[i + 0] = a[0]; out[i + 1] = a[1]; out[i + 2] = b[0]; out[i + 3] = b[1];
    out[i + 4] = c[0]; out[i + 5] = c[1]; out[i + 6] = d[0]; out[i + 7] = d[1];
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + i / 2);
    uint32_t r[4];
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
    for (int sel = 0; sel < 4; ++sel) {
      out[i + 2 * sel] = u2f(r[sel] << 16);
      out[i + 2 * sel + 1] = u2f(r[sel] & 0xFFFF0000u);
    }
  }
}

__global__ void probe_mfma_kernel(const uint16_t* A, const uint16_t* B, float* D, int kind) {
  const int l = threadIdx.x;
  u32x4 ra, rb;
  uint16_t av[8], bv[8];
  for (int j = 0; j < 8; ++j) {
    av[j] = A[(l % 16) * 32 + 8 * (l / 16) + j];
    bv[j] = B[(8 * (l / 16) + j) * 16 + (l % 16)];
  }
  for (int j = 0; j < 4; ++j) {
    ra[j] = (uint32_t)av[2 * j] | ((uint32_t)av[2 * j + 1] << 16);
    rb[j] = (uint32_t)bv[2 * j] | ((uint32_t)bv[2 * j + 1] << 16);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (kind == 0)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, ra), __builtin_bit_cast(f16x8, rb), acc, 0, 0, 0);
  else
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ra), __builtin_bit_cast(bf16x8, rb), acc, 0, 0, 0);
  for (int i = 0; i < 4; ++i) D[(4 * (l / 16) + i) * 16 + (l % 16)] = acc[i];
}

// Every binary32 pattern lo .. lo + n - 1 except NaNs through both E4M3
// encoders; res[0] counts the patterns where they differ, res[1] keeps the
// largest such pattern (0 if none).
__global__ void probe_e4m3_sweep_kernel(uint32_t lo, uint32_t n, uint32_t* res) {
  uint32_t bad = 0, last = 0;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint32_t bits = lo + i;
    const float x = u2f(bits);
    if (x != x) continue;
    const uint32_t hw = e4m3_encode2_hw<false>(x, 0.0f, 0u) & 0xFFu;
    if (hw != e4m3_encode(x)) {
      ++bad;
      last = bits > last ? bits : last;
    }
  }
  if (bad) {
    atomicAdd(&res[0], bad);
    atomicMax(&res[1], last);
  }
}

}  // namespace hca

extern "C" {

hca_status hca_probe_e4m3_sweep(uint32_t lo, uint32_t n, uint32_t* res, void* stream) {
  if (!res) return HCA_ERR_INVALID;
  if (n == 0) return HCA_OK;
  hipLaunchKernelGGL(probe_e4m3_sweep_kernel, dim3(4096), dim3(256), 0, (hipStream_t)stream, lo, n, res);
  return from_hip(hipGetLastError());
}

hca_status hca_probe_decode(const uint8_t* codes, float* out, int32_t n, int32_t kind, void* stream) {
  if (!codes || !out || n < 0 || (n % 8) != 0 || (kind != 0 && kind != 1)) return HCA_ERR_INVALID;
  if (n == 0) return HCA_OK;
  const int threads = n / 8;
  hipLaunchKernelGGL(probe_decode_kernel, dim3((threads + 255) / 256), dim3(256), 0, (hipStream_t)stream, codes, out, n,
                     kind);
  return from_hip(hipGetLastError());
}

hca_status hca_probe_mfma(const uint16_t* A, const uint16_t* B, float* D, int32_t kind, void* stream) {
  if (!A || !B || !D || (kind != 0 && kind != 1)) return HCA_ERR_INVALID;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, A, B, D, kind);
  return from_hip(hipGetLastError());
}

}  // extern "C"
