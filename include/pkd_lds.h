/*
 * pkd_lds.h -- a direct-output paged decode whose K/V tiles are loaded
 * straight into LDS, for measurement beside the register-staged kernels of the
 * MI355X (gfx950) paged-KV decode library.  No decode entry point calls it.
 *
 * The AstrAI commit log's kernel double-buffers its K/V tiles in shared memory
 * with asynchronous copies (two stages).  The library's kernels instead keep
 * the next tile's loads in flight in registers and copy each tile into LDS
 * only to form the matrix-core operands.  This entry computes the same
 * attention as paged_decode with num_splits = 1 (one workgroup of four waves
 * per (sequence, KV head), out and lse written directly) with the pages'
 * arrangement: each wave cycles two LDS stages of one 16-token tile, the
 * next tile's direct-to-LDS loads (global_load_lds_dwordx4) in flight while
 * the current one is computed from LDS, so that the two pipelines can be timed
 * on the same shapes.  The matrix-core steps, the softmax and the final
 * combine are the library's own.
 *
 * Supported: a bfloat16 cache, head_dim 128, G = num_q_heads / num_kv_heads
 * at most 16, page_size a multiple of 16, max_pages_per_seq at most 512, one
 * query token per sequence, no window or sinks.  Other shapes return
 * PKD_ERR_BAD_DIMS, PKD_ERR_HEAD_DIM, PKD_ERR_DTYPE or PKD_ERR_GQA and enqueue
 * nothing.
 *
 *   dims, q, k_cache, v_cache, block_table, seq_lens, scale, out, lse, stream:
 *   as for paged_decode (lse may be NULL).  Same contract for device contents,
 *   alignment and asynchrony.  Results equal paged_decode's with num_splits = 1
 *   bit for bit (the same products, sums and roundings in the same order).
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
#ifdef __cplusplus
}
#endif
#endif /* PKD_LDS_H */
