// Internal declarations shared by the HIP kernels and the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkd {

// Rows.  Each sequence has q_len query tokens (1 for plain decode); the memory
// row of (sequence b, query token i, head h) in q, out and lse is
// (b * q_len + i) * Hq + h.  The q_len * G rows of one KV head are "packed
// rows" r = i * G + (h - kvh * G), grouped 16 to a head group.

// Element strides of a (sequence, query token, head) row of q or out; the
// head dimension is contiguous.  Dense [B][q_len][Hq][D]: (q_len Hq D, Hq D, D).
struct RowStrides {
  int64_t b, i, h;
  __host__ __device__ int64_t at(int64_t bb, int64_t ii, int64_t hh) const { return bb * b + ii * i + hh * h; }
};

// Where K/V rows sit, in bytes: row (page, slot, KV head) at page * page_stride
// + slot * tok_stride + head * head_stride.  A paged cache [P][ps][Hkv][D] has
// (ps Hkv D e, Hkv D e, D e).  A contiguous cache is read as one page per
// sequence (page = b, no block table) whose page_size covers every length, with
// the tensor's own sequence, token and head strides.
struct KvLayout {
  int64_t page_stride;
  int64_t head_stride;
  int32_t tok_stride;          // 16 * tok_stride < 2^31 (offsets inside a 16-token group are 32-bit)
};

// Arguments of the split-KV partition kernel (one launch).
struct SplitParams {
  const uint16_t* q;           // rows at qs.at(b, i, h), bf16
  const uint8_t* k;            // kv elements (bf16 or fp8 codes) placed by kv
  const uint8_t* v;
  const int32_t* block_table;  // [B][max_pages], or null: page b holds sequence b (contiguous K/V)
  const int32_t* seq_lens;     // [B]
  const float* k_scale;        // [Hkv] (fp8) or null
  const float* v_scale;
  uint16_t* out;               // direct mode: rows at os.at(b, i, h), bf16
  float* lse;                  // direct mode: [B][q_len][Hq] or null
  float* o_part;               // split mode: [B][q_len][Hq][S][D]
  float* lse_part;             // split mode: [B][q_len][Hq][S]
  float qk_scale_log2;         // scale * log2(e): scores are kept in base-2 units
  int32_t hq, hkv, group;      // group = G = Hq / Hkv
  int32_t q_len, causal;       // query tokens per sequence; causal mask on (1) or off (0)
  int32_t window;              // sliding window in tokens (0: none)
  const float* sinks;          // [Hq] sink logits or null (direct mode only)
  int32_t rows_kv;             // packed rows per KV head: q_len * G
  int32_t head_groups;         // ceil(rows_kv / 16): packed rows are taken 16 per workgroup
  int32_t page_size, max_pages;
  int32_t num_splits;
  int32_t chunk;               // tokens per split (a multiple of kSplitAlign, or >= every visible span);
                               // splits start at the sequence's first visible 16-token group
  RowStrides qs, os;
  KvLayout kv;
  int32_t strided;             // 1: qs, os, kv and a null block table are honoured (host picks the kernel)
};

// Arguments of the balanced persistent partition kernel.
struct BalancedParams {
  const uint16_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const float* k_scale;
  const float* v_scale;
  float* o_part;               // [slots][hpg][D], slots = num_workers + batch * hkv * head_groups
  float* lse_part;             // [slots][hpg]
  int64_t* prefix;             // [batch + 1] group prefix sums, written for the merge kernel
  float qk_scale_log2;
  int32_t batch, hq, hkv, group, head_groups;
  int32_t q_len, causal, rows_kv;  // as in SplitParams
  int32_t window;              // as in SplitParams; a sequence's groups start at its first visible one
  const float* sinks;          // [Hq] or null (fused: applied to out/lse)
  int32_t hpg;                 // rows per slot: min(rows_kv, 16)
  int32_t page_size, max_pages;
  int32_t num_workers;         // workgroups in the grid
  // In-kernel merge (fused != 0): segments held by one piece write out/lse
  // directly; for the others the last piece to finish (found with seg_count)
  // merges the segment's partials.  seg_count[s] holds (epoch << 24) | pieces
  // done; a word with another epoch counts as zero, and the merging piece
  // resets it to (epoch << 24), so no initialisation is ever needed.
  int32_t fused;
  uint16_t* out;               // [B][q_len][Hq][D] bf16 (fused)
  float* lse;                  // [B][q_len][Hq] or null (fused)
  uint64_t* seg_count;         // [B * Hkv * head_groups] (fused)
  uint64_t epoch;              // distinct per call, 1 .. 2^40 - 1 (fused)
  RowStrides qs, os;           // as in SplitParams
  KvLayout kv;
  int32_t strided;
  int32_t xcd_ranges;          // give each XCD a contiguous part of the work space (heads sharing cache lines)
  int32_t pair_heads;          // 1, or 2: hkv / group / head dims count wide heads of two real KV heads
                               // (q / out rows, partials and scales stay per real head)
  int32_t paired;              // 1 (with fused): one or two whole segments per workgroup, paired by
                               // length rank on the device, when that balances well enough (else the
                               // equal ranges); batch <= kPairedMaxBatch
};

// ---- Arithmetic shared by the kernels and the host, in one place so that a
// host-only test can check it (the in-place merge's counter words, the
// balanced partition's pieces, the paired deal of whole items). ----

// An in-place merge counter word is (tag << 24) | pieces counted.  A word
// carrying another tag counts as zero, so a workspace left by any earlier call
// (or never initialised) needs no clearing; the piece that completes the count
// writes count_word_reset, which any later tag, the same one included, again
// reads as zero.  Tags are 40 bits and never 0.
__host__ __device__ inline uint64_t count_word_add(uint64_t old, uint64_t tag) {
  return ((old >> 24) == tag ? old : (tag << 24)) + 1;
}
__host__ __device__ inline int count_word_pieces(uint64_t word) { return (int)(word & 0xFFFFFF); }
__host__ __device__ inline uint64_t count_word_reset(uint64_t tag) { return tag << 24; }
// The tag of the call numbered n (a process-wide counter): its low 40 bits, 0
// read as 1.
__host__ __device__ inline uint64_t call_tag(uint64_t n) {
  const uint64_t e = n & ((1ull << 40) - 1);
  return e != 0 ? e : 1;
}

// The balanced partition: T groups on nwe workgroups, workgroup w taking
// groups [w T / nwe, (w + 1) T / nwe).  A segment holding groups
// [seg_pos, seg_pos + nb) (nb >= 1) is split among the workgroups w_first ..
// w_first + npieces - 1, one piece each.
__host__ __device__ inline void segment_pieces(int64_t seg_pos, int64_t nb, int64_t nwe, int64_t T,
                                               int64_t* w_first, int* npieces) {
  const int64_t f = ((seg_pos + 1) * nwe - 1) / T;
  *w_first = f;
  *npieces = (int)(((seg_pos + nb) * nwe - 1) / T - f + 1);
}

// The paired deal of N whole items, ranked by length ascending, on W
// workgroups: with E = N - W > 0, workgroup g < E takes items 2E - 1 - g
// (first) and g, every other workgroup g < W item g + E; with E <= 0
// workgroup g < N takes item g.  -1: none.  Each item goes to exactly one
// workgroup when N <= 2W.
__host__ __device__ inline void paired_items(int g, int N, int W, int* first, int* second) {
  const int E = N - W;
  if (E > 0) {
    *first = g < E ? 2 * E - 1 - g : (g + E < N ? g + E : -1);
    *second = g < E ? g : -1;
  } else {
    *first = g < N ? g : -1;
    *second = -1;
  }
}

// True when the balanced mode merges inside the partition kernel: when there
// are at least as many segments as workgroups, so a segment spans one or two
// pieces and a multi-piece merge is short.  (Measured: the same or faster
// there; slower with ~8 pieces per segment, where the last piece's merge
// lengthens the tail.)  The merge kernel then uses one wave per row, so both
// paths run the same per-row merge and give the same bits.
__host__ __device__ inline bool balanced_merge_in_kernel(int64_t workers, int64_t segments) {
  return segments > 0 && workers <= segments;
}

// Arguments of the log-sum-exp merge kernel.  Grid-kernel partials sit at
// [row][j] (j < num_splits); balanced-kernel partials of a row's segment sit at
// consecutive slots found from the prefix sums.
struct MergeParams {
  const float* o_part;
  const float* lse_part;
  uint16_t* out;               // [rows][D] bf16
  float* lse;                  // [rows] or null
  int64_t rows;
  int32_t num_splits;          // grid layout
  int32_t balanced;            // 0: grid layout; 1: balanced layout
  const int64_t* prefix;       // balanced layout fields
  int32_t batch, hq, hkv, group, head_groups, hpg, num_workers;
  int32_t q_len;               // balanced layout: rows are (b * q_len + i) * Hq + h
  const float* sinks;          // [Hq] sink logits or null; row r has head r % hq (hq set whenever sinks is)
  int32_t strided_out;         // 0: out row r at r * D; 1: at os.at(b, i, h) of row r = (b q_len + i) Hq + h
  RowStrides os;               //    (q_len and hq set)
};

// Arguments of the paged KV append kernel.
struct AppendParams {
  const uint16_t* k_new;       // [N][Hkv][D] bf16
  const uint16_t* v_new;
  const int64_t* slot_mapping; // [N] page * page_size + position; < 0 or >= capacity: not written
  const int64_t* positions;    // [N] or null (no RoPE)
  const float* cos_sin;        // [max_position][D]: cos of the D/2 angles, then their sin
  void* k_cache;               // [num_pages][page_size][Hkv][D] bf16 or fp8 codes
  void* v_cache;
  const float* k_scale;        // [Hkv] (fp8)
  const float* v_scale;
  int64_t num_tokens;
  int64_t capacity;            // num_pages * page_size
  int64_t max_position;
  int32_t hkv;
};

// Arguments of the decode metadata kernel.
struct MetaParams {
  const int32_t* req_to_token;      // [req_rows][req_stride] KV slot of every token of every request row
  const int64_t* req_pool_indices;  // [batch]
  const int64_t* seq_lens;          // [batch] tokens before this step
  int32_t* cache_seqlens;           // [batch] out
  int32_t* cu_seqlens_k;            // [batch + 1] out
  int32_t* page_table;              // [batch][max_pages] out
  int32_t* swa_seqlens;             // [batch] out (window > 0)
  int32_t* swa_page_table;          // [batch][max_pages] out (window > 0)
  int32_t* error_count;             // out or null: invalid batch entries
  int64_t req_rows, req_stride;
  int64_t max_len;                  // min(max_pages * page_size, req_stride)
  int32_t batch, page_size, max_pages, q_len, window, extend;
};

constexpr int kWaves = 4;            // waves per split-kernel workgroup
constexpr int kSplitAlign = 64;      // tokens; split boundaries are multiples of this
constexpr int kHeadsPerGroup = 16;   // query heads packed into one MFMA N dimension
constexpr int kBalancedMaxBatch = 1024;  // largest batch the balanced kernel's prefix scan takes
constexpr int kPairedMaxBatch = 256;     // largest batch of the balanced kernel's paired mode
constexpr int kXcds = 8;                 // accelerator complex dies of an MI355X (gfx950), each with its own L2

// Launchers (defined in the .hip files).  head_dim in {32, 64, 128, 256}.
// strided: take the q/out strides and the K/V layout from the parameters (and
// allow a null block table); otherwise the dense q/out and paged cache layouts.
hipError_t launch_split_kv(const SplitParams& p, int batch, int head_dim, bool fp8, bool direct,
                           bool paged16, bool strided, hipStream_t stream);
hipError_t launch_balanced(const BalancedParams& p, int head_dim, bool fp8, bool strided, hipStream_t stream);
hipError_t launch_lse_merge(const MergeParams& p, int head_dim, hipStream_t stream);
hipError_t launch_kv_append(const AppendParams& p, int head_dim, bool fp8, hipStream_t stream);
hipError_t launch_decode_metadata(const MetaParams& p, hipStream_t stream);
hipError_t launch_check_tables(const int32_t* block_table, const int32_t* seq_lens, int batch,
                               int max_pages, int page_size, int num_pages, int32_t* d_count,
                               hipStream_t stream);

// Direct output with K/V tiles loaded straight into LDS stages (lds_decode.hip):
// the grid kernel's arithmetic, bit for bit, for the shapes lds_direct_applies
// accepts (paged bf16 cache, D = 128, no window, one query token, G <= 16,
// page_size % 16 == 0, max_pages <= 512; sinks or not).  One workgroup per
// (KV head, sequence); reads the direct-mode fields of p.
bool lds_direct_applies(int head_dim, bool fp8, int q_len, int window, int group, int page_size, int max_pages,
                        bool strided);
// workers = 0: one workgroup per (KV head, sequence); workers = W > 0: the
// pairs form, W workgroups for B * Hkv items, W < B * Hkv <= 2W, B <= kPairedMaxBatch,
// lengths below 2^23.
hipError_t launch_lds_direct(const SplitParams& p, bool fp8, int batch, int workers, hipStream_t stream);

}  // namespace pkd
