/*
 * pkd_stream.h -- a read-only stream kernel of the MI355X (gfx950) paged-KV
 * decode library, for measurement only.
 *
 * The decode step is bound by HBM bandwidth: its K/V rows are streamed once.
 * The bandwidth a plain load stream reaches with the same access pattern is
 * the practical ceiling the decode kernels are compared with (the chip's
 * 8 TB/s is the theoretical one).  This entry point is that stream: it reads
 * a buffer and computes nothing but an XOR of what it read.  It is not part of
 * the decode and no decode entry point calls it.
 *
 * The buffer is seen as bytes / row_bytes rows of row_bytes bytes, each row cut
 * into columns of chunk_bytes.  Each column is one stream: chunk_bytes of
 * every row (chunk_bytes = 256 with row_bytes = 2048 is one KV head's slice of
 * each token row of a bf16 cache with 8 KV heads of 128 dims; chunk_bytes =
 * row_bytes reads the buffer front to back).  With pattern 0 a wave's 16-byte
 * lane loads read 1 KB of a column in order; with pattern 1 (the operand layout
 * of a 16x16x32 matrix-core instruction, whose 16 rows sit in lanes l % 16)
 * they read 64 bytes of each of 16 consecutive rows, the next load the next
 * 64 bytes of those rows; pattern 2 is pattern 0 issued as direct-to-LDS loads
 * (global_load_lds_dwordx4), the load path of a pipeline staged in shared
 * memory rather than registers, each wave cycling its two batches through an
 * LDS ring of 2 * batch_kb KB.  The 1 KB blocks of the
 * column-major stream order are divided evenly among `workgroups` workgroups of
 * `waves` waves; a wave keeps two batches of batch_kb blocks (16 bytes per lane
 * per block) in flight, with nontemporal = 1 using non-temporal loads.
 *
 *   buf          device, 16-byte aligned, `bytes` bytes.
 *   bytes        > 0, a multiple of row_bytes and of 1024.
 *   row_bytes    a multiple of chunk_bytes.
 *   chunk_bytes  a power of two >= 16; (bytes / row_bytes) * chunk_bytes a multiple of 1024.
 *   pattern      0, 1 or 2 (1: chunk_bytes >= 64 and bytes / row_bytes a multiple of 16;
 *                2: waves * 2 * batch_kb <= 128, the KB of LDS rings per workgroup).
 *   workgroups   1 .. 2^20;  waves 1 .. 8;  batch_kb in {4, 8, 16, 32};  nontemporal 0 or 1.
 *   sink         device uint32 array of pkd_stream_read_sink_bytes(workgroups, waves) bytes,
 *                overwritten (one word per thread: patterns 0 and 1 the XOR of every word the
 *                thread loaded, pattern 2 the first word of the thread's 16 bytes in the
 *                ring's first block after the last batch, 0 for a wave with no block).
 * Returns PKD_OK or a negative status of paged_kv_decode.h; argument errors enqueue nothing.
 * Enqueued on `stream` (a hipStream_t) without synchronising.
 */
#ifndef PKD_STREAM_H
#define PKD_STREAM_H

#include "paged_kv_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

int32_t pkd_stream_read(const void* buf, int64_t bytes, int32_t row_bytes, int32_t chunk_bytes,
                        int32_t pattern, int32_t workgroups, int32_t waves, int32_t batch_kb,
                        int32_t nontemporal, uint32_t* sink, void* stream);

/* Bytes of the sink array for a launch shape (0 for an invalid one). */
size_t pkd_stream_read_sink_bytes(int32_t workgroups, int32_t waves);

#ifdef __cplusplus
}
#endif

#endif /* PKD_STREAM_H */
