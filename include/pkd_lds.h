/*
 * pkd_lds.h -- the two direct-output kernels of the MI355X (gfx950) paged-KV
 * decode library side by side, for measurement.
 *
 * The AstrAI commit log's kernel double-buffers its K/V tiles in shared memory
 * with asynchronous copies (two stages).  The library has both arrangements:
 * the grid kernel keeps the next tile's loads in flight in registers and
 * copies each tile into LDS only to form the matrix-core operands; the
 * LDS-staged kernel cycles two LDS stages of one 16-token tile per wave, the
 * next tile's direct-to-LDS loads (global_load_lds_dwordx4) in flight while
 * the current one is computed from LDS.  Both compute paged_decode with
 * num_splits = 1 (one workgroup of four waves per (sequence, KV head), out and
 * lse written directly) with the same matrix-core steps, softmax and combine,
 * so they give the same bits.  paged_decode picks one by shape
 * (paged_decode_path); these entries run each on any shape it takes, so that
 * the two pipelines can be timed on the same inputs.
 *
 * pkd_decode_lds -- the LDS-staged kernel.  Supported: a bfloat16 cache,
 * head_dim 128, G = num_q_heads / num_kv_heads at most 16, page_size a
 * multiple of 16, max_pages_per_seq at most 512, one query token per sequence
 * (no window or sinks through this entry).  Other shapes return
 * PKD_ERR_BAD_DIMS, PKD_ERR_HEAD_DIM, PKD_ERR_DTYPE or PKD_ERR_GQA and enqueue
 * nothing.
 *
 *   dims, q, k_cache, v_cache, block_table, seq_lens, scale, out, lse, stream:
 *   as for paged_decode (lse may be NULL).  Same contract for device contents,
 *   alignment and asynchrony.
 * Returns PKD_OK or a negative status of paged_kv_decode.h.
 */
#ifndef PKD_LDS_H
#define PKD_LDS_H
#include "paged_kv_decode.h"
#ifdef __cplusplus
extern "C" {
#endif
int32_t pkd_decode_lds(const pkd_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, const int32_t* seq_lens, float scale, void* out, float* lse,
                       void* stream);

/*
 * pkd_decode_registers -- the other side of the comparison: paged_decode with
 * num_splits = 1 on the register-staged grid kernel, whatever the shape (where
 * paged_decode itself would take the LDS-staged kernel).  A BF16 cache (FP8
 * returns PKD_ERR_SCALES); otherwise the arguments, checks and results of
 * paged_decode(dims, q, k_cache, v_cache, block_table, seq_lens, NULL, NULL,
 * scale, out, lse, 1, NULL, 0, stream).
 */
int32_t pkd_decode_registers(const pkd_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens, float scale, void* out, float* lse,
                             void* stream);
#ifdef __cplusplus
}
#endif
#endif /* PKD_LDS_H */
