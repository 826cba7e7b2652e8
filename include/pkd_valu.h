/*
 * pkd_valu.h -- a direct-output paged decode whose inner loop runs on the
 * vector ALU, for measurement beside the matrix-core kernels of the MI355X
 * (gfx950) paged-KV decode library.  No decode entry point calls it.
 *
 * The library's kernels compute QK^T and PV with 16x16x32 matrix-core products,
 * packing the query heads of a KV head into the 16 columns (the head packing
 * of the AstrAI log's MMA variant); with 4 query heads per KV head 12 columns
 * are padding.  This entry computes the same attention as paged_decode with
 * num_splits = 1 (one workgroup per (sequence, KV head), out and lse written
 * directly) with bf16 dot products on the vector ALU and cross-lane sums by
 * DPP instead (the warp-level reduction of the log's scalar variant), so that
 * the two inner loops can be timed on the same shapes.
 *
 * Supported: a bfloat16 cache, head_dim 64 or 128, G = num_q_heads /
 * num_kv_heads in {1, 2, 4}, page_size a multiple of 16, one query token per
 * sequence, no window or sinks.  Other shapes return PKD_ERR_BAD_DIMS,
 * PKD_ERR_HEAD_DIM, PKD_ERR_DTYPE or PKD_ERR_GQA and enqueue nothing.
 *
 *   dims, q, k_cache, v_cache, block_table, seq_lens, scale, out, lse, stream:
 *   as for paged_decode (lse may be NULL).  Same contract for device contents,
 *   alignment and asynchrony.  Results agree with paged_decode within the
 *   rounding of the bf16 output, not bit for bit (sums are taken in another
 *   order).
 * Returns PKD_OK or a negative status of paged_kv_decode.h.
 */
#ifndef PKD_VALU_H
#define PKD_VALU_H

#include "paged_kv_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

int32_t pkd_decode_valu(const pkd_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_table, const int32_t* seq_lens, float scale, void* out, float* lse,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKD_VALU_H */
