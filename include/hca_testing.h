/*
 * hca_testing.h -- checking and measurement hooks of libhca (not part of the
 * decode path).
 *
 * The host hooks run the very encoder functions the kernels use, compiled for
 * the host, so their rounding can be checked exhaustively on a machine without
 * a GPU.  The GPU probes run one hardware conversion or one MFMA on known data
 * so that the lane layouts the kernels rely on can be checked in isolation.
 * All return HCA_OK or HCA_ERR_INVALID (NULL pointer / bad size / bad kind).
 */
#ifndef HCA_TESTING_H
#define HCA_TESTING_H

#include "hca.h"

#ifdef __cplusplus
extern "C" {
#endif

/* host: in[n] fp32 -> E4M3 codes (RNE, saturating, sign kept) */
hca_status hca_host_e4m3_encode(const float* in, uint8_t* out, int64_t n);
/* host: in[n] fp32 -> E2M1 codes (low 4 bits of each byte) */
hca_status hca_host_e2m1_encode(const float* in, uint8_t* out, int64_t n);
/* host: in[n] fp32 -> bfloat16 bit patterns (RNE) */
hca_status hca_host_bf16_encode(const float* in, uint16_t* out, int64_t n);

/* GPU: decode n codes with the conversions the kernels use.
 *   kind 0: E4M3 bytes codes[n] -> out[n] (hardware fp8 -> fp32)
 *   kind 1: E2M1 packed bytes codes[n/2] -> out[n] (hardware fp4 -> bf16)
 * codes, out: device; n a multiple of 8. */
hca_status hca_probe_decode(const uint8_t* codes, float* out, int32_t n, int32_t kind, void* stream);

/* GPU: every binary32 bit pattern lo .. lo + n - 1 (n < 2^32; NaNs skipped)
 * through the kernels' two E4M3 encoders, the exact-step one (as
 * hca_host_e4m3_encode) and the hardware conversion after a saturating clamp;
 * res (device, two words, zeroed by the caller) accumulates the number of
 * patterns where they differ and the largest such pattern. */
hca_status hca_probe_e4m3_sweep(uint32_t lo, uint32_t n, uint32_t* res, void* stream);

/* GPU: one wave computes D[16][16] = A[16][32] . B[32][16] with one
 * v_mfma_f32_16x16x32 (kind 0: f16 operands, kind 1: bf16 operands), loading
 * lane l's operands as A[l%16][8(l/16) .. +8] and B[8(l/16) .. +8][l%16] and
 * storing its accumulator as D[4(l/16)+i][l%16].  A, B: 16-bit patterns,
 * row-major; D: fp32 row-major; all device. */
hca_status hca_probe_mfma(const uint16_t* A, const uint16_t* B, float* D, int32_t kind, void* stream);

/* Measurement: the scoring kernel of indexer_topk alone, same arguments and
 * launch configuration, no selection.  It accumulates into the workspace's
 * score histogram, so use a workspace reserved for it (never one that
 * indexer_topk will use afterwards).  The fp32 scores land at the start of the
 * workspace: sequence b's row of 2048 * ceil(ceil(max_seq_len / m) / 2048)
 * floats, entry j at j (entries at or past ceil(seq_lens[b] / m) unwritten). */
hca_status hca_indexer_score(const uint16_t* q_idx, const float* head_w, int32_t HI, hca_paged_cache idx_keys,
                             const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens, int32_t B,
                             int32_t max_seq_len, int32_t m, int32_t k, void* ws, size_t ws_bytes, void* stream);

/* Measurement: the split kernel of paged_hybrid_decode alone, with the same
 * arguments (outputs omitted), launch configuration and workspace; it writes
 * only the per-split partials in the workspace, so a workspace reserved for it
 * is needed when paged_hybrid_decode's results must stay untouched. */
hca_status hca_attention_split(const uint16_t* q, int32_t H, hca_paged_cache kv, const int32_t* block_table,
                               int32_t bt_stride, hca_paged_cache win, const int32_t* win_block_table,
                               int32_t wbt_stride, const int32_t* seq_lens, int32_t B, int32_t max_seq_len, int32_t m,
                               int32_t window, const int32_t* sel_idx, const int32_t* sel_n, int32_t k,
                               float softmax_scale, float rope_theta, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HCA_TESTING_H */
