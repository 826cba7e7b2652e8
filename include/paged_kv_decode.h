/*
 * paged_kv_decode.h -- C ABI of the MI355X (gfx950) paged-KV decode attention library.
 *
 * The operation: for each sequence b of a decode batch there is one query
 * token with Hq heads; its keys and values live in a paged KV cache and are
 * found through the sequence's block table.  Query head h attends to KV head
 * floor(h / G), G = Hq / Hkv (grouped-query attention: consecutive query heads
 * share a KV head):
 *
 *   s_t = scale * <q[b,h,:], K[t]>,  out[b,h,:] = sum_t softmax(s)_t * V[t],
 *   lse[b,h] = ln sum_t exp(s_t)                        (natural log)
 *
 * over the tokens t < seq_lens[b], where token t is slot t % page_size of
 * physical page block_table[b][t / page_size].  This is the paged decode that
 * the AstrAI commit log for csrc/kernels/attn_paged_decode_split_kv_mma.cuh
 * builds its split-KV kernels for (per-token page lookup that works for any
 * page size; one unified paged_decode entry; split partials written without
 * a memset), and that the b12x 0.30.0 inventory lists in its "Paged attention"
 * row (BF16 and FP8-E4M3 KV caches, GQA, "split-KV or direct output", a
 * persistent merge kernel).
 *
 * Several query tokens per sequence (ext.q_len > 1, paged_decode_ext): the speculative-verify /
 * extend form that the same b12x row lists beside decode ("decode/verify",
 * "extend"), with the causal mask the AstrAI log expresses as the position of
 * the first query token.  Sequence b then has q_len query tokens, the last
 * q_len positions of the sequence: query token i sits at position
 * seq_lens[b] - q_len + i.  Without the mask (ext.causal = 0) every query
 * token attends over all seq_lens[b] tokens; with it (ext.causal = 1) query
 * token i attends over positions <= seq_lens[b] - q_len + i only, and a token
 * that sees no position gets out = 0 and lse = -inf.  q, out and lse gain a
 * q_len dimension after the batch: row (b, i, h) of each is at
 * (b * q_len + i) * Hq + h.  All the q_len * G rows that share a KV head are
 * computed from one read of its K/V rows.
 *
 * Sliding window and attention sinks: two variants the same b12x row lists
 * for its paged attention.  With ext.window = W > 0, query token i (position
 * p = seq_lens[b] - q_len + i) sees only positions t > p - W, besides the
 * limit above (t < seq_lens[b], and t <= p with the causal mask); for plain
 * decode that is the last W tokens.  K/V rows below the lowest window start of
 * a sequence (rounded down to a multiple of 16) are not read.  With a sinks
 * array, query head h has a logit sinks[h] that joins the softmax denominator
 * and contributes no value:
 *
 *   out = sum_t exp(s_t) V[t] / (exp(sinks[h]) + sum_t exp(s_t)),
 *   lse = ln(exp(sinks[h]) + sum_t exp(s_t)),
 *
 * so a token that sees no position gets out = 0 and lse = sinks[h].  Split
 * partials never include the sink; it is folded in where out is written.
 *
 * Split-KV: each sequence's tokens are cut into num_splits ranges; each range
 * produces a normalised partial output and its log-sum-exp, and a merge
 * combines them (out = sum_j exp(lse_j - lse) * o_j, lse = ln sum_j exp(lse_j)),
 * the same recombination as the merge_attn_states kernels in the vLLM section
 * of the sglang fuse/overlap catalogue.  num_splits == 1 writes out and lse
 * directly with no partials and no second kernel.
 *
 * Conventions for every entry point below:
 *  - Pointers are device pointers unless marked "host".  The caller owns all
 *    memory; the library allocates and frees nothing and keeps no state other
 *    than cached device attributes.  Calls are thread-safe.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns without synchronising and without any device-to-host
 *    copy.
 *  - All arguments are checked on the host before anything is enqueued; on a
 *    negative status nothing was enqueued and no output was written.
 *  - Device-side contents are the caller's contract: every block-table entry
 *    for a page a sequence uses (i < ceil(seq_lens[b] / page_size)) must lie
 *    in [0, num_pages), and 0 <= seq_lens[b] <= max_pages_per_seq * page_size.
 *    Entries past a sequence's last page are never used: their values do not
 *    matter (they may hold -1), although the kernels may load them, since
 *    every row of block_table is read only within its max_pages_per_seq
 *    entries.  Cache slots past seq_lens[b] in its last page never contribute
 *    (they may hold anything, NaN included).  Violations are undefined
 *    behaviour; paged_decode_check_tables reports them.
 *  - Outputs must not alias inputs.  Results are bitwise deterministic for
 *    fixed inputs and num_splits.
 *  - Alignment: q, k_cache, v_cache, out, workspace and o_part must be 16-byte
 *    aligned; every other pointer must be aligned to its element size (4 bytes
 *    for int32 and fp32 arrays, 2 for the merge entry's bf16 out).  Memory from
 *    hipMalloc or a torch allocation always is.  Misaligned pointers are
 *    rejected with PKD_ERR_ALIGNMENT.
 */
#ifndef PAGED_KV_DECODE_H
#define PAGED_KV_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define PKD_OK 0
#define PKD_ERR_NULL_POINTER (-1)    /* a required pointer is NULL */
#define PKD_ERR_BAD_DIMS (-2)        /* a dimension is out of range */
#define PKD_ERR_GQA (-3)             /* num_q_heads is not a multiple of num_kv_heads */
#define PKD_ERR_HEAD_DIM (-4)        /* head_dim not in {32, 64, 128, 256} */
#define PKD_ERR_DTYPE (-5)           /* kv_dtype not a pkd_dtype value */
#define PKD_ERR_SCALES (-6)          /* FP8 cache without scales, or scales given for BF16 */
#define PKD_ERR_NUM_SPLITS (-7)      /* num_splits above PKD_MAX_SPLITS */
#define PKD_ERR_WORKSPACE (-8)       /* workspace NULL or smaller than required */
#define PKD_ERR_LAUNCH (-9)          /* the HIP runtime refused a launch */
#define PKD_ERR_DEVICE (-10)         /* the current device is not a usable gfx950 */
#define PKD_ERR_ALIGNMENT (-11)      /* a pointer is not aligned as required (see below) */
#define PKD_ERR_SCRATCH_LIMIT (-12)  /* paged_decode_ext_noalloc: the mode needs more than its fixed scratch */

/* Largest num_splits accepted. */
#define PKD_MAX_SPLITS 512

/* Largest q_len accepted.  The q_len * G query rows of a KV head are computed
 * 16 at a time, each group of 16 reading the KV head's K/V rows once, so the
 * cost grows with q_len * G / 16: a verify / short-extend form, not prefill. */
#define PKD_MAX_Q_LEN 64

/* Special num_splits values.  PKD_SPLITS_AUTO lets the library choose
 * (paged_decode_num_splits).  PKD_SPLITS_BALANCED selects the balanced
 * partition: a persistent grid sized to the device in which every workgroup
 * gets an equal share of all (sequence, KV head, 16-token group) work and
 * writes one partial per (workgroup, segment) piece, merged afterwards.  It needs
 * page_size % 16 == 0 and batch <= PKD_BALANCED_MAX_BATCH. */
#define PKD_SPLITS_AUTO 0
#define PKD_SPLITS_BALANCED (-1000)
#define PKD_BALANCED_MAX_BATCH 1024

/* PKD_SPLITS_PAIRED selects whole items paired by length: the balanced
 * partition's grid, in which each workgroup takes one or two whole
 * (sequence, KV head, head group) items, so that nothing is split or merged.
 * The device ranks the items by length (from seq_lens, with the window);
 * with N items on W workgroups and N > W, the 2(N - W) shortest are taken in
 * pairs, the shortest with the longest of them, and the rest one each.  When
 * that would give some workgroup more than 1.6 times the mean work per
 * workgroup, or N > 2W, the kernel uses the balanced partition's equal ranges
 * instead, merging in place.  It needs what the balanced mode needs, and
 * batch <= PKD_PAIRED_MAX_BATCH and max_pages_per_seq * page_size < 2^27; one
 * kernel, paged_decode_ext only (the two-phase entries reject it).  This is the
 * split-or-not choice of the AstrAI commit log's shared split-count helper
 * (compute_num_splits), taken per item from the lengths on the device. */
#define PKD_SPLITS_PAIRED (-1001)
#define PKD_PAIRED_MAX_BATCH 256

/* Split boundaries: with S splits, sequence b's split j covers tokens
 * [min(lo_b + j*c, L_b), min(lo_b + (j+1)*c, L_b)) where
 * c = PKD_SPLIT_ALIGN * ceil(ceil(N / S) / PKD_SPLIT_ALIGN),
 * N = max_pages_per_seq * page_size, the same for every sequence of the batch,
 * so that every split carries about the same work; trailing splits of shorter
 * sequences are empty.  lo_b = 0 without a window; with window W,
 * lo_b = max(L_b - q_len - W + 1, 0) rounded down to a multiple of 16 (the
 * sequence's first visible 16-token group) and N = min(N, W + q_len + 14). */
#define PKD_SPLIT_ALIGN 64

/* KV-cache element types.  q and out are always bfloat16. */
typedef enum {
  PKD_DTYPE_BF16 = 0,     /* bfloat16 K and V */
  PKD_DTYPE_FP8_E4M3 = 1  /* OCP FP8 E4M3FN codes with a per-KV-head fp32 scale each for K and V */
} pkd_dtype;

/* Problem dimensions (passed as a host pointer). */
typedef struct {
  int32_t batch;              /* B >= 0 (B == 0 enqueues nothing) */
  int32_t num_q_heads;        /* Hq >= 1 */
  int32_t num_kv_heads;       /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;           /* D in {32, 64, 128, 256} */
  int32_t page_size;          /* tokens per page, >= 1 (any value) */
  int32_t num_pages;          /* pages in the pool, >= 1 */
  int32_t max_pages_per_seq;  /* row length of block_table, >= 1 */
  int32_t kv_dtype;           /* a pkd_dtype */
} pkd_dims;

/* The extended forms (passed as a host pointer; NULL means q_len = 1, no mask,
 * no window: plain decode). */
typedef struct {
  int32_t q_len;              /* query tokens per sequence, 1..PKD_MAX_Q_LEN (1 = decode) */
  int32_t causal;             /* 0: every query token sees all tokens; 1: causal mask (above) */
  int32_t window;             /* 0: no window; W > 0: sliding window of W positions (above) */
  int32_t reserved;           /* must be 0 */
} pkd_ext;

/*
 * paged_decode -- the whole decode-attention step (split-KV partition + merge):
 * the single paged_decode entry of the AstrAI log (the bullets on
 * attn_pack_paged_params and on unifying the paged decode path), one query
 * token per sequence.
 *
 *   dims         host; see pkd_dims.
 *   q            [B][Hq][D] bfloat16, contiguous.
 *   k_cache      [num_pages][page_size][Hkv][D] of kv_dtype, contiguous.
 *   v_cache      same layout as k_cache.
 *   block_table  [B][max_pages_per_seq] int32 physical page ids.
 *   seq_lens     [B] int32 tokens per sequence (0 allowed: out = 0, lse = -inf).
 *   k_scale      [Hkv] fp32 dequantisation scales for an FP8 cache (K = code * k_scale[kv]);
 *                must be NULL for BF16.
 *   v_scale      [Hkv] fp32, as k_scale for V.
 *   scale        softmax scale applied to q.k (typically 1/sqrt(D)); included in lse.
 *   out          [B][Hq][D] bfloat16 result (fp32 accumulate, round-to-nearest-even).
 *   lse          [B][Hq] fp32 natural-log log-sum-exp of the scaled scores, or NULL.
 *   num_splits   <= 0: the heuristic's choice, paged_decode_num_splits(dims, 0) (the log's
 *                compute_num_splits helper names such a choice but not its rule);
 *                1: direct output (one kernel);
 *                2..PKD_MAX_SPLITS: split-KV + merge (two kernels).  Above: PKD_ERR_NUM_SPLITS.
 *   workspace    device scratch for partials (the log's alloc_split_partials bullet: taken per
 *                call and never cleared), at least paged_decode_workspace_bytes(dims, num_splits)
 *                bytes; may be NULL when that is 0.  Its contents on entry do not matter.
 *   workspace_bytes  size of workspace.
 *   stream       hipStream_t.
 * Returns PKD_OK or a negative status.
 */
int32_t paged_decode(const pkd_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, const int32_t* seq_lens, const float* k_scale,
                     const float* v_scale, float scale, void* out, float* lse, int32_t num_splits,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_decode_ext -- paged_decode with the extended forms and the special
 * split modes.
 *   ext          host; see pkd_ext (NULL: plain decode).  With q_len > 1, q is
 *                [B][q_len][Hq][D], out [B][q_len][Hq][D] and lse [B][q_len][Hq].
 *   sinks        [Hq] fp32 sink logits (above; -inf means no sink for that head), or NULL.
 *   num_splits   PKD_SPLITS_AUTO: chosen by paged_decode_num_splits_ext(dims, ext, 0);
 *                1: direct output; 2..PKD_MAX_SPLITS: split-KV + merge;
 *                PKD_SPLITS_BALANCED: balanced partition, which merges the pieces of each
 *                (sequence, KV head) itself when few are expected (one kernel; see
 *                paged_decode_launches), else partition + merge (two kernels);
 *                PKD_SPLITS_PAIRED: whole items paired by length (one kernel; above).
 *                Any other value is PKD_ERR_NUM_SPLITS.
 *   workspace    at least paged_decode_workspace_bytes_ext(dims, ext, num_splits) bytes.
 * Other arguments as for paged_decode.  With ext NULL, sinks NULL and num_splits
 * in 1..PKD_MAX_SPLITS it is paged_decode, bit for bit.
 */
int32_t paged_decode_ext(const pkd_dims* dims, const pkd_ext* ext, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                         const float* k_scale, const float* v_scale, const float* sinks, float scale, void* out,
                         float* lse, int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the fixed device array paged_decode_ext_noalloc uses as its workspace. */
#define PKD_NOALLOC_SCRATCH_BYTES 16777216  /* 16 MiB */

/*
 * paged_decode_ext_noalloc -- paged_decode_ext for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid it): the workspace is a fixed array of PKD_NOALLOC_SCRATCH_BYTES
 * inside the library, one per device, which each device holds until the
 * process ends.  The call itself allocates and frees nothing.
 *   Arguments as for paged_decode_ext, without workspace and workspace_bytes.
 *   A mode whose paged_decode_workspace_bytes_ext exceeds
 *   PKD_NOALLOC_SCRATCH_BYTES returns PKD_ERR_SCRATCH_LIMIT and enqueues nothing
 *   (the balanced mode needs a few MB for batches up to 1024; many grid splits of
 *   large batches need more).
 *   All calls on one device share its array: calls that overlap in time there
 *   (on different streams, or from different threads) race and their results
 *   are undefined; calls in one stream's order are safe.  The array is never
 *   cleared and never needs to be.
 * Returns PKD_OK or a negative status.
 */
int32_t paged_decode_ext_noalloc(const pkd_dims* dims, const pkd_ext* ext, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                                 const float* k_scale, const float* v_scale, const float* sinks, float scale,
                                 void* out, float* lse, int32_t num_splits, void* stream);

/*
 * paged_decode_partition / paged_decode_finish -- the two phases of
 * paged_decode_ext for a split mode (num_splits = 2..PKD_MAX_SPLITS or
 * PKD_SPLITS_BALANCED, or PKD_SPLITS_AUTO when it resolves to one of them; a
 * resolution to direct output is PKD_ERR_NUM_SPLITS here): the partition kernel
 * writes its partials into the workspace, then the merge kernel reads them and
 * writes out and lse.  Issued back to back on one stream with the same dims,
 * ext, num_splits and workspace they are exactly paged_decode_ext; split apart
 * they let a caller schedule or time the phases.  Arguments as for
 * paged_decode_ext; the sinks are folded in by paged_decode_finish.
 */
int32_t paged_decode_partition(const pkd_dims* dims, const pkd_ext* ext, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_table,
                               const int32_t* seq_lens, const float* k_scale, const float* v_scale,
                               float scale, int32_t num_splits, void* workspace,
                               size_t workspace_bytes, void* stream);
int32_t paged_decode_finish(const pkd_dims* dims, const pkd_ext* ext, int32_t num_splits, const void* workspace,
                            size_t workspace_bytes, const float* sinks, void* out, float* lse,
                            void* stream);

/*
 * paged_decode_num_splits -- what paged_decode does for num_splits <= 0 (and
 * paged_decode_num_splits_ext what paged_decode_ext does for PKD_SPLITS_AUTO).
 * Work items are (sequence, KV head, head group), a head group being up to 16
 * of a KV head's q_len * G query rows.
 *  - 1 (direct output) for a BF16 cache with head_dim >= 64 when the items
 *    number between three quarters of the current device's compute units and
 *    all of them (one whole item per unit, nothing to merge);
 *  - else 1 when no sequence can show more than 256 tokens
 *    (max_pages_per_seq * page_size, or with a window window + q_len + 14,
 *    whichever is smaller);
 *  - else, for more items than compute units and at most twice as many: 1 for
 *    a paged cache (BF16 or FP8) with head_dim 128, q_len 1, no window, G <= 16,
 *    page_size % 16 == 0, max_pages_per_seq <= 512, batch <= PKD_PAIRED_MAX_BATCH
 *    and max_pages_per_seq * page_size < 2^23 (direct output, whole items paired
 *    by length on the device: see paged_decode_path), else PKD_SPLITS_PAIRED
 *    wherever it applies.  Whole items in pairs measured faster than the equal
 *    cuts for ragged lengths; when every length is equal, pairs cost up to
 *    twice an item's time on some units and PKD_SPLITS_BALANCED is faster;
 *  - else, with at most one item per 64 compute units (a few long sequences),
 *    S = units / items split by the grid kernel (one workgroup per unit),
 *    capped by the longest sequence expected (at least 256 tokens per split)
 *    and by PKD_MAX_SPLITS, when that gives S >= 2;
 *  - else PKD_SPLITS_BALANCED wherever it applies;
 *  - else 1 when the items alone fill the device's compute units, else a split
 *    count in [2, PKD_MAX_SPLITS] bounded by the longest sequence expected,
 *    max_seq_len_hint (<= 0: max_pages_per_seq * page_size).
 * Host only; returns that value, or a status in [-11, -1] for invalid dims.
 * Since the value may be PKD_SPLITS_BALANCED, pass it to paged_decode_ext (to
 * paged_decode it would mean the heuristic again, which is the same choice).
 */
int32_t paged_decode_num_splits(const pkd_dims* dims, int32_t max_seq_len_hint);
int32_t paged_decode_num_splits_ext(const pkd_dims* dims, const pkd_ext* ext, int32_t max_seq_len_hint);

/*
 * paged_decode_launches -- kernels paged_decode_ext enqueues for num_splits
 * (PKD_SPLITS_AUTO: the heuristic's choice): 1 for direct output and for the
 * balanced mode when its partition kernel merges in place (when the
 * (sequence, KV head, head group) segments are at least as many as the
 * current device's compute units; a head group is 16 of the q_len * G query
 * rows of a KV head), else 2.  ext may be NULL.
 * Host only; returns a status in [-11, -1] for invalid dims or num_splits.
 */
int32_t paged_decode_launches(const pkd_dims* dims, const pkd_ext* ext, int32_t num_splits);

/*
 * paged_decode_path -- which partition kernel paged_decode_ext runs for
 * num_splits (PKD_SPLITS_AUTO: the heuristic's choice), for profilers and
 * tests that need the kernel by name.  Returns
 *   PKD_PATH_DIRECT          direct output, the next K/V tile's loads held in registers;
 *   PKD_PATH_DIRECT_LDS      direct output, K/V tiles loaded straight into two LDS stages per
 *                            wave (the same arithmetic; the same bits for BF16, while FP8
 *                            runs eight waves per workgroup whose grouping of the tiles
 *                            rounds differently), taken for a paged cache with
 *                            head_dim 128, q_len 1, no window, G <= 16,
 *                            page_size a multiple of 16, max_pages_per_seq <= 512, and
 *                            batch * num_kv_heads at most the current device's compute units
 *                            (one workgroup per item), or at most twice that with
 *                            batch <= PKD_PAIRED_MAX_BATCH and max_pages_per_seq * page_size
 *                            < 2^23 (one workgroup per compute unit, each taking one or two
 *                            whole items paired by length rank on the device, as in
 *                            PKD_SPLITS_PAIRED but never falling back);
 *   PKD_PATH_SPLITS          split-KV partials, then the merge kernel;
 *   PKD_PATH_BALANCED        the balanced partition, merging in place;
 *   PKD_PATH_BALANCED_MERGE  the balanced partition, then the merge kernel;
 *   PKD_PATH_PAIRED          the balanced kernel in paired mode (whole items, or equal
 *                            ranges merged in place when pairing balances too poorly).
 * Sinks do not change the path.  Host only; returns a status in [-11, -1] for
 * invalid dims or num_splits.
 */
#define PKD_PATH_DIRECT 1
#define PKD_PATH_DIRECT_LDS 2
#define PKD_PATH_SPLITS 3
#define PKD_PATH_BALANCED 4
#define PKD_PATH_BALANCED_MERGE 5
#define PKD_PATH_PAIRED 6
int32_t paged_decode_path(const pkd_dims* dims, const pkd_ext* ext, int32_t num_splits);

/*
 * paged_decode_workspace_bytes -- workspace paged_decode needs for num_splits
 * (<= 0: the heuristic's choice); paged_decode_workspace_bytes_ext the same
 * for paged_decode_ext (PKD_SPLITS_AUTO: the heuristic's choice).  0 for one
 * split; for S splits the fp32 partials [B][q_len][Hq][S][D] and
 * [B][q_len][Hq][S]; for PKD_SPLITS_BALANCED, with R = q_len * G query rows per
 * KV head, the fp32 partials of D floats per row in (W + B*Hkv*ceil(R/16))
 * slots of min(R,16) rows, W the workgroups of the device-sized grid (one per
 * compute unit), B+1 int64 prefix sums, and B*Hkv*ceil(R/16) uint64 merge
 * counters; each part rounded up to 256 bytes.  When KV heads are read in
 * pairs (head rows under 128 bytes, no window, 2R <= 16: two heads sharing each
 * cache line are read together), Hkv counts pairs and R doubles.  Returns 0 for
 * invalid dims or an unsupported num_splits.  The counters carry a per-call
 * tag, so the workspace never needs initialising.
 */
size_t paged_decode_workspace_bytes(const pkd_dims* dims, int32_t num_splits);
size_t paged_decode_workspace_bytes_ext(const pkd_dims* dims, const pkd_ext* ext, int32_t num_splits);

/*
 * paged_decode_partials -- the split-KV partition step alone: every split of
 * every (sequence, query row) writes its normalised partial output and
 * natural-log LSE.  An empty split writes o = 0 and lse = -inf, so every slot
 * is written and no clearing is needed.
 *   o_part    [B][q_len][Hq][num_splits][D] fp32.
 *   lse_part  [B][q_len][Hq][num_splits] fp32.
 *   num_splits 1..PKD_MAX_SPLITS (no heuristic here).
 * Other arguments as for paged_decode_ext (no sinks: partials never hold them).
 */
int32_t paged_decode_partials(const pkd_dims* dims, const pkd_ext* ext, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens, const float* k_scale, const float* v_scale,
                              float scale, int32_t num_splits, float* o_part, float* lse_part,
                              void* stream);

/*
 * paged_decode_merge -- the log-sum-exp merge of split partials alone:
 * for each of `rows` rows, M = max_j lse_j, lse = M + ln sum_j exp(lse_j - M),
 * out = sum_j exp(lse_j - lse) * o_j rounded to bfloat16.  Rows whose partials
 * are all -inf give out = 0, lse = -inf.
 *   rows       number of rows (B * Hq for paged_decode), >= 0.
 *   num_splits partials per row, 1..PKD_MAX_SPLITS.
 *   head_dim   D in {32, 64, 128, 256}.
 *   o_part     [rows][num_splits][D] fp32;  lse_part [rows][num_splits] fp32.
 *   out        [rows][D] bfloat16;  lse [rows] fp32 or NULL.
 */
int32_t paged_decode_merge(int64_t rows, int32_t num_splits, int32_t head_dim, const float* o_part,
                           const float* lse_part, void* out, float* lse, void* stream);

/*
 * paged_decode_check_tables -- optional validation of the device-side
 * contract (not part of the decode step): counts sequences whose length is
 * outside [0, max_pages_per_seq * page_size] plus used block-table entries
 * outside [0, num_pages), and writes the count to *d_error_count (device int32;
 * written, not accumulated).  Only the used entries are inspected.
 */
int32_t paged_decode_check_tables(const pkd_dims* dims, const int32_t* block_table,
                                  const int32_t* seq_lens, int32_t* d_error_count, void* stream);

/*
 * paged_kv_append -- write new K/V rows into the paged cache: the step before
 * decode that the sglang fuse/overlap catalogue lists as fused FP8 quantisation
 * + paged K/V cache write (section 1, the TRTLLM FP8 KV row) and as RoPE fused
 * with the KV cache store (sections 1 and 14).
 *
 *   dims          host; num_kv_heads, head_dim, page_size, num_pages and
 *                 kv_dtype are used (the other fields are ignored).
 *   num_tokens    N >= 0 (0 enqueues nothing).
 *   k_new, v_new  [N][Hkv][D] bfloat16, contiguous.
 *   slot_mapping  [N] int64: token n goes to page slot_mapping[n] / page_size,
 *                 position slot_mapping[n] % page_size.  A negative slot
 *                 (padding) or one >= num_pages * page_size writes nothing.
 *                 Slots of one call must be distinct.
 *   positions     [N] int64 and cos_sin [max_position][D] fp32, or both NULL:
 *                 with them K is rotated first, NeoX rotate-half form: for
 *                 d < D/2, c = cos_sin[pos][d], s = cos_sin[pos][D/2 + d],
 *                 k'[d] = k[d] c - k[d + D/2] s, k'[d + D/2] = k[d + D/2] c + k[d] s,
 *                 each an fp32 product followed by one fused multiply-add.  A
 *                 position outside [0, max_position) writes nothing.
 *   k_cache, v_cache  [num_pages][page_size][Hkv][D] of kv_dtype, updated in
 *                 place: bf16 values rounded to nearest even; FP8 codes of
 *                 clamp(x / scale[h], -448, 448) (fp32 division, nearest code,
 *                 ties to even) with
 *   k_scale, v_scale  [Hkv] fp32 per-KV-head scales (FP8 only; NULL for BF16),
 *                 the same scales paged_decode dequantises with.
 * Alignment: k_new, v_new, caches and cos_sin 16 bytes; slot_mapping and
 * positions 8; scales 4.  Returns PKD_OK or a negative status; argument errors
 * enqueue nothing.
 */
int32_t paged_kv_append(const pkd_dims* dims, int64_t num_tokens, const void* k_new, const void* v_new,
                        const int64_t* slot_mapping, const int64_t* positions, const float* cos_sin,
                        int32_t max_position, void* k_cache, void* v_cache, const float* k_scale,
                        const float* v_scale, void* stream);

/* Dimensions of paged_decode_metadata (passed as a host pointer). */
typedef struct {
  int32_t batch;              /* B, 0..65535 (0: only cu_seqlens_k[0] = 0 and the error count are
                                 written, and the other arrays may be NULL) */
  int32_t req_rows;           /* rows of req_to_token, >= 1 */
  int32_t req_stride;         /* columns of req_to_token (token slots per request row), >= 1 */
  int32_t page_size;          /* tokens per page, >= 1 */
  int32_t max_pages_per_seq;  /* row length of page_table / swa_page_table, >= 1 */
  int32_t q_len;              /* query tokens per sequence, 1..PKD_MAX_Q_LEN (for the window) */
  int32_t window;             /* 0: no window tables; W > 0: sliding window (as pkd_ext.window) */
  int32_t extend;             /* tokens this step adds to every seq_lens[b], >= 0 */
} pkd_meta_dims;

/*
 * paged_decode_metadata -- build the block table and lengths that paged_decode
 * reads from a serving runtime's token map, in one launch (the decode metadata
 * step that the sglang fuse/overlap catalogue, section 1, lists as fused for
 * the flashattention backend).  It extends each length by the step's new
 * tokens, forms their running sums, looks up each page through the token map
 * and, with a window, also builds the tables without the pages below it;
 * the outputs below define each of these.
 *
 *   md                host; see pkd_meta_dims.
 *   req_to_token      [req_rows][req_stride] int32: the KV slot (page * page_size +
 *                     position) of every token of every request row.
 *   req_pool_indices  [B] int64: the request row r_b of batch entry b.
 *   seq_lens          [B] int64: tokens of entry b before this step.
 * Outputs (device, written for every entry):
 *   cache_seqlens     [B] int32: L_b = seq_lens[b] + extend (paged_decode's seq_lens).
 *   cu_seqlens_k      [B + 1] int32: 0, L_0, L_0 + L_1, ...
 *   page_table        [B][max_pages_per_seq] int32: entry j < ceil(L_b / page_size) is
 *                     req_to_token[r_b][j * page_size] / page_size (the page of the page's
 *                     first token; -1 for a negative slot); the rest -1.  This is
 *                     paged_decode's block_table.
 *   swa_seqlens, swa_page_table  (window > 0; may be NULL otherwise): the same
 *                     sequence without its first f_b = max(L_b - q_len - W + 1, 0) /
 *                     page_size pages, which hold no visible position:
 *                     swa_page_table[b][j] = page_table[b][f_b + j] (then -1),
 *                     swa_seqlens[b] = L_b - f_b * page_size.  paged_decode with the
 *                     same window gives the same result on these as on the full ones.
 *   d_error_count     int32 or NULL: the number of invalid entries, written (not
 *                     accumulated).  An entry is invalid when r_b is outside
 *                     [0, req_rows) or L_b outside [0, min(max_pages_per_seq *
 *                     page_size, req_stride)]; its lengths are written as 0 and its
 *                     table rows as -1, so decode reads nothing for it.
 * Requires batch * max_pages_per_seq * page_size <= INT32_MAX (the prefix sums are
 * int32).  Alignment: int64 arrays 8 bytes, int32 arrays 4.  Returns PKD_OK or a
 * negative status; argument errors enqueue nothing.
 */
int32_t paged_decode_metadata(const pkd_meta_dims* md, const int32_t* req_to_token,
                              const int64_t* req_pool_indices, const int64_t* seq_lens, int32_t* cache_seqlens,
                              int32_t* cu_seqlens_k, int32_t* page_table, int32_t* swa_seqlens,
                              int32_t* swa_page_table, int32_t* d_error_count, void* stream);

/* Dimensions and strides of contiguous_decode (passed as a host pointer). */
typedef struct {
  int32_t batch;              /* B >= 0 */
  int32_t num_q_heads;        /* Hq >= 1 */
  int32_t num_kv_heads;       /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;           /* D in {32, 64, 128, 256} */
  int32_t max_seq_len;        /* token capacity of the K/V tensors, >= 1; every seq_lens[b] <= it */
  int32_t kv_dtype;           /* a pkd_dtype */
  int32_t q_len;              /* query tokens per sequence, 1..PKD_MAX_Q_LEN */
  int32_t causal;             /* as in pkd_ext */
  int32_t window;             /* as in pkd_ext */
  int32_t reserved;           /* must be 0 */
  int64_t q_strides[3];       /* element strides of q: sequence, query token, head (>= 0, multiples of 8) */
  int64_t kv_strides[3];      /* element strides of k and v: sequence, token, KV head (>= 0; each a multiple
                                 of 16 bytes; 16 * token stride in bytes < 2^31) */
  int64_t out_strides[3];     /* element strides of out: sequence, query token, head (>= 0, multiples of 8) */
} pkd_contig_dims;

/*
 * contiguous_decode -- the same attention as paged_decode (GQA, several query
 * tokens, causal mask, window, sinks, BF16 or FP8 K/V, every num_splits mode)
 * over K/V held in one contiguous tensor each rather than in pages: the
 * contiguous decode kernels of the AstrAI commit log, with its stride-based
 * addressing for Q, K/V and O, which reads any layout in place (for instance
 * [B][L][Hkv][D], or [B][Hkv][L][D] with strides (Hkv L D, D, L D)).
 *
 *   k, v      key element (b, t, h, d) at k[b*kv_strides[0] + t*kv_strides[1] +
 *             h*kv_strides[2] + d] (of kv_dtype; v alike with the same strides).
 *             Tokens t >= seq_lens[b] are never read.
 *   q         query row (b, i, h) at q + b*q_strides[0] + i*q_strides[1] + h*q_strides[2].
 *   out       row (b, i, h) at out + b*out_strides[0] + i*out_strides[1] +
 *             h*out_strides[2] (bfloat16; rows must not overlap).
 *   lse       [B][q_len][Hq] fp32, dense, or NULL.
 *   seq_lens, k_scale, v_scale, sinks, scale, num_splits, workspace, stream:
 *             as for paged_decode.
 * The head dimension of every tensor is contiguous.  Internally each sequence
 * is one page of max_seq_len rounded up to 16 tokens, so num_splits and the
 * workspace size follow paged_decode's rules for that paged problem
 * (contiguous_decode_workspace_bytes).  Pointer alignment as for paged_decode.
 * Returns PKD_OK or a negative status.
 */
int32_t contiguous_decode(const pkd_contig_dims* dims, const void* q, const void* k, const void* v,
                          const int32_t* seq_lens, const float* k_scale, const float* v_scale, const float* sinks,
                          float scale, void* out, float* lse, int32_t num_splits, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Workspace bytes contiguous_decode needs for num_splits (0 for invalid dims). */
size_t contiguous_decode_workspace_bytes(const pkd_contig_dims* dims, int32_t num_splits);

/* Human-readable text for a status code (static storage). */
const char* paged_decode_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_DECODE_H */
