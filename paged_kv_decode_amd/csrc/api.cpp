// C-ABI entry points: host-side validation, the num-splits heuristic,
// workspace sizing and kernel launches.  Nothing here synchronises with the
// device or copies device memory to the host.
#include <atomic>
#include <cstring>
#include <chrono>
#include <climits>
#include <cmath>
#include <unistd.h>

#include "../../include/paged_kv_decode.h"
#include "../../include/pkd_lds.h"
#include "pkd_internal.hpp"

namespace {

// The whole problem shape: pkd_dims plus the extensions of pkd_ext (one query
// token, no mask and no window for the plain paged_decode).
struct Dims {
  int32_t batch, num_q_heads, num_kv_heads, head_dim;
  int32_t page_size, num_pages, max_pages_per_seq;
  int32_t kv_dtype;
  int32_t q_len, causal, window;
};

// Dims of a call: the plain shape and its extensions (ext may be NULL).  An
// extension record with a non-zero reserved field gives q_len 0, which
// check_dims rejects.
Dims make_dims(const pkd_dims& d, const pkd_ext* e) {
  Dims f{d.batch, d.num_q_heads, d.num_kv_heads, d.head_dim, d.page_size, d.num_pages, d.max_pages_per_seq,
         d.kv_dtype, 1, 0, 0};
  if (e) {
    f.q_len = e->reserved == 0 ? e->q_len : 0;
    f.causal = e->causal;
    f.window = e->window;
  }
  return f;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not yet queried

// Compute units of the current device (cached per device id), or -1.
// Compute units of the current device, or -1 when there is none or it is not
// a gfx950 (the only target the kernels are built for).  Cached per device.
int current_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached != 0) return cached;
  }
  int cus = 0;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return -1;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0 || (prop.gcnArchName[6] != '\0' && prop.gcnArchName[6] != ':'))
    cus = -1;
  else if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return -1;
  if (dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

bool valid_head_dim(int d) { return d == 32 || d == 64 || d == 128 || d == 256; }

// Query rows per KV head: the q_len query tokens of each of its G heads.
int rows_per_kv(const Dims& d) { return d.q_len * (d.num_q_heads / d.num_kv_heads); }

// Head groups: the rows of a KV head taken 16 at a time.
int head_groups(const Dims& d) {
  return (rows_per_kv(d) + pkd::kHeadsPerGroup - 1) / pkd::kHeadsPerGroup;
}

// Shape checks shared by every entry that takes dims.
int32_t check_dims(const Dims* d) {
  if (!d) return PKD_ERR_NULL_POINTER;
  if (d->batch < 0 || d->batch > 65535 || d->num_q_heads < 1 || d->num_kv_heads < 1 ||
      d->page_size < 1 || d->num_pages < 1 || d->max_pages_per_seq < 1 || d->q_len < 1 ||
      d->q_len > PKD_MAX_Q_LEN || (d->causal != 0 && d->causal != 1) || d->window < 0)
    return PKD_ERR_BAD_DIMS;
  if (d->num_q_heads % d->num_kv_heads != 0) return PKD_ERR_GQA;
  if (!valid_head_dim(d->head_dim)) return PKD_ERR_HEAD_DIM;
  if (d->kv_dtype != PKD_DTYPE_BF16 && d->kv_dtype != PKD_DTYPE_FP8_E4M3) return PKD_ERR_DTYPE;
  if ((int64_t)d->max_pages_per_seq * d->page_size > INT32_MAX) return PKD_ERR_BAD_DIMS;
  // Query rows per sequence (and so per KV head) stay far inside int32.
  if ((int64_t)d->q_len * d->num_q_heads > (1 << 24)) return PKD_ERR_BAD_DIMS;
  if ((int64_t)d->num_kv_heads * head_groups(*d) > 65535) return PKD_ERR_BAD_DIMS;
  // Offsets inside one 16-token group of a page are computed in 32 bits.
  if ((int64_t)d->num_kv_heads * d->head_dim * 2 * 16 > INT32_MAX) return PKD_ERR_BAD_DIMS;
  return PKD_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workgroups of the balanced grid: one per compute unit.  Its four waves then
// sit on the unit's four SIMDs; with a second workgroup on the unit the
// hardware favours the older one's waves, the two finish far apart, and the
// whole measured 2-8% slower on every workload shape.
int balanced_workers(const Dims&) {
  const int cus = current_cu_count();
  return cus > 0 ? cus : 256;
}

int heads_per_slot(const Dims& d) {
  const int R = rows_per_kv(d);
  return R < pkd::kHeadsPerGroup ? R : pkd::kHeadsPerGroup;
}

// Whether the balanced partition applies: aligned 16-token groups lie in one
// page, the prefix scan takes the batch, and the work-space arithmetic stays
// far inside int64 (T * workers < 2^62).
bool balanced_ok(const Dims& d) {
  if (d.page_size % 16 != 0 || d.batch > PKD_BALANCED_MAX_BATCH) return false;
  const int64_t groups = ((int64_t)d.max_pages_per_seq * d.page_size + 15) / 16;
  const int64_t T = groups * d.batch * d.num_kv_heads * head_groups(d);
  return T < ((int64_t)1 << 46);
}

// Whether the paired mode applies: the balanced partition applies (it is the
// paired mode's fallback), the batch fits the kernel's ranking of sequences by
// length, and a segment's group count fits the 23 bits of its ranking key.
static_assert(pkd::kPairedMaxBatch == PKD_PAIRED_MAX_BATCH, "paired-mode batch limit");
bool paired_ok(const Dims& d) {
  return balanced_ok(d) && d.batch <= pkd::kPairedMaxBatch &&
         (int64_t)d.max_pages_per_seq * d.page_size < ((int64_t)1 << 27);
}

// KV heads the balanced kernel reads as one: 2 when adjacent heads of the paged
// layout share 128-byte lines (head rows of fewer than 128 bytes), the pair's
// query rows still fit one 16-row group and the pair's width has a kernel
// instance (64 or 128); else 1.  A pair is then one wide head (see the
// kernel), so that each line is fetched once.  Not with a window or strided
// (contiguous) K/V.  A function of the shape alone, so workspace sizes agree.
int pair_heads(const Dims& d, bool strided) {
  if (strided || d.window != 0) return 1;
  const int e = d.kv_dtype == PKD_DTYPE_FP8_E4M3 ? 1 : 2;
  if (d.head_dim * e >= 128 || d.num_kv_heads % 2 != 0) return 1;
  if (2 * rows_per_kv(d) > pkd::kHeadsPerGroup) return 1;
  if (2 * d.head_dim != 64 && 2 * d.head_dim != 128) return 1;
  return 2;
}

// The problem as the balanced kernel's work space sees it: pair KV heads of
// head_dim D become one KV head of pair * D dims.
Dims balanced_view(const Dims& d, int pair) {
  Dims v = d;
  v.num_kv_heads /= pair;
  v.head_dim *= pair;
  return v;
}

// Balanced workspace: partials [slots][hpg][D] fp32 (D of a real head), LSEs
// [slots][hpg] fp32, prefix sums [B + 1] int64, then one in-kernel-merge
// counter per segment [B * Hkv * head_groups] uint64 (its contents never need
// initialising); slots, hpg and the segments as in balanced_view.
size_t balanced_bytes(const Dims& d, int pair, size_t* lse_offset, size_t* prefix_offset,
                      size_t* count_offset) {
  const Dims v = balanced_view(d, pair);
  const size_t segments = (size_t)v.batch * v.num_kv_heads * head_groups(v);
  const size_t slots = (size_t)balanced_workers(v) + segments;
  const size_t hpg = (size_t)heads_per_slot(v);
  const size_t o = align256(slots * hpg * d.head_dim * sizeof(float));
  const size_t l = align256(slots * hpg * sizeof(float));
  const size_t pre = align256(((size_t)d.batch + 1) * sizeof(int64_t));
  if (lse_offset) *lse_offset = o;
  if (prefix_offset) *prefix_offset = o + l;
  if (count_offset) *count_offset = o + l + pre;
  return o + l + pre + align256(segments * sizeof(uint64_t));
}

// Whether the balanced mode merges inside the partition kernel (paged_decode only).
bool balanced_fused(const Dims& d, int pair) {
  const Dims v = balanced_view(d, pair);
  return pkd::balanced_merge_in_kernel(balanced_workers(v), (int64_t)v.batch * v.num_kv_heads * head_groups(v));
}

// Call tags for the in-kernel merge counters: distinct for every call in this
// process (40 bits, never 0), starting from a value that differs between
// processes, so that a counter word left by an earlier call never matches.
std::atomic<uint64_t> g_epoch{0};
uint64_t next_epoch() {
  uint64_t cur = g_epoch.load(std::memory_order_relaxed);
  if (cur == 0) {
    const uint64_t seed = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() ^
                          ((uint64_t)getpid() << 20);
    uint64_t expect = 0;
    g_epoch.compare_exchange_strong(expect, (seed & ((1ull << 40) - 1)) | 1);
  }
  return pkd::call_tag(g_epoch.fetch_add(1, std::memory_order_relaxed));
}

size_t partial_bytes(const Dims& d, int S, size_t* lse_offset) {
  const size_t rows = (size_t)d.batch * d.q_len * d.num_q_heads;
  const size_t o = align256(rows * (size_t)S * d.head_dim * sizeof(float));
  if (lse_offset) *lse_offset = o;
  return o + align256(rows * (size_t)S * sizeof(float));
}

// Most tokens one sequence's splits cover: what the block table can hold, or
// with a sliding window the visible span of the q_len query tokens (window +
// q_len - 1) plus up to 15 tokens before it (splits start on a 16-token group).
int64_t visible_span(const Dims& d) {
  const int64_t cap = (int64_t)d.max_pages_per_seq * d.page_size;
  if (d.window <= 0) return cap;
  const int64_t span = (int64_t)d.window + d.q_len - 1 + 15;
  return span < cap ? span : cap;
}

// Tokens per split: the longest span a sequence can need, cut into S equal
// pieces rounded up to PKD_SPLIT_ALIGN.  Every split of every sequence then
// covers the same number of tokens (or is the sequence's shorter last piece,
// or empty), so workgroups carry equal work whatever the length mix.
int32_t split_chunk(const Dims& d, int S) {
  const int64_t cap = visible_span(d);
  const int64_t per = (cap + S - 1) / S;
  const int64_t c = (per + PKD_SPLIT_ALIGN - 1) / PKD_SPLIT_ALIGN * PKD_SPLIT_ALIGN;
  return (int32_t)(c < INT32_MAX ? c : INT32_MAX);
}

bool lds_direct_ok(const Dims& d, bool strided);

// The split mode for PKD_SPLITS_AUTO.
//  - Direct output (one split) when a bf16 cache whose head rows are at least
//    128 bytes has between three quarters of one and one (sequence, KV head,
//    head group) item per compute unit: each unit streams one whole item and
//    nothing is merged.  There the balanced partition's even cuts give most
//    workgroups two pieces, and the second piece's combine, acknowledged
//    partial store, count and merge cost more than the length imbalance that
//    whole items leave (measured, lengths 1024-4096, 8 KV heads: direct output
//    faster by 2.5% at 192 items and by 5-7% at 224-256; with 264 items or
//    more, where a second round of workgroups would follow, and for an FP8
//    cache, the balanced partition was faster).
//  - Direct output when no sequence can show more than 256 tokens (the block
//    table's capacity, or the window's span): a whole item is then at most 16
//    groups, which one workgroup streams in about the time the balanced
//    partition takes to spread it and launch its merge (the two-sequence,
//    112-token case: 8.5 against 16.4 us).
//  - Between one and two items per compute unit: direct output in the
//    LDS-staged kernel's pairs form where it applies (bf16 or FP8, head_dim
//    128, one query token, no window, paged), else the paired mode where it
//    applies; both keep whole items, the longest alone and the shortest in
//    pairs, which measured faster than the balanced partition's equal cuts for
//    lengths 1024-4096 (bf16, 8 KV heads, B = 33-64: 5.5-6.4 against 4.9-5.5
//    TB/s) and 512-8192 (FP8, B = 40-64: 4.4-5.5 against 4.0-4.7 TB/s); the
//    LDS-staged form led the paired mode by 2-7%.
//  - At most one item per 64 compute units (a few long sequences): grid
//    splits, about one workgroup per unit (S = units / items, at least 256
//    tokens per split).  The grid kernel's start-up (length, q and block table
//    loaded together) is shorter than the balanced partition's (lengths, prefix
//    sums, page window, q in turn), which weighs at these sizes: B = 1 with
//    131072 tokens and 2 KV heads ran 15.5 / 18.7 / 51.9 us against 18.6 /
//    22.3 / 55.4 balanced at D = 32 / 64 / 256.
//  - Otherwise the balanced partition wherever it applies (it balances any
//    length mix and pays each workgroup's start-up once).
//  - Otherwise direct output when the items alone fill the device, else
//    enough splits to fill it, bounded by the longest sequence.
int32_t heuristic_splits(const Dims& d, int32_t max_len, bool strided) {
  const int cus = current_cu_count();
  const int64_t items = (int64_t)d.batch * d.num_kv_heads * head_groups(d);
  if (d.kv_dtype == PKD_DTYPE_BF16 && d.head_dim >= 64 && cus > 0 && items <= cus && 4 * items >= 3LL * cus)
    return 1;
  if (visible_span(d) <= 256) return 1;
  if (cus > 0 && items > cus && items <= 2LL * cus) {
    if (lds_direct_ok(d, strided)) return 1;
    if (paired_ok(d)) return PKD_SPLITS_PAIRED;
  }
  if (cus > 0 && items > 0 && items * 64 <= cus) {
    // A few long items: grid splits, about one workgroup per unit.
    const int64_t span = max_len < visible_span(d) ? max_len : visible_span(d);
    int64_t s = cus / items;
    const int64_t by_len = (span + 255) / 256;  // at least ~256 tokens per split
    if (s > by_len) s = by_len;
    if (s > PKD_MAX_SPLITS) s = PKD_MAX_SPLITS;
    if (s >= 2) return (int32_t)s;
  }
  if (balanced_ok(d)) return PKD_SPLITS_BALANCED;
  const int64_t target = 4LL * (cus > 0 ? cus : 256);  // workgroups to keep every CU busy
  if (items <= 0 || items >= target) return 1;
  int64_t s = (target + items - 1) / items;
  const int64_t span = max_len < visible_span(d) ? max_len : visible_span(d);
  const int64_t by_len = (span + 255) / 256;  // keep at least ~256 tokens per split
  if (s > by_len) s = by_len;
  if (s < 1) s = 1;
  if (s > PKD_MAX_SPLITS) s = PKD_MAX_SPLITS;
  return (int32_t)s;
}

// Where q, out and the K/V rows are.  Paged caches use the dense layouts of the
// header; contiguous K/V and strided q / out come from contiguous_decode.
struct Layout {
  pkd::RowStrides qs, os;
  pkd::KvLayout kv;
  bool dense_out;  // os is the dense [B][q_len][Hq][D] layout
  bool strided;    // not the paged_decode layouts: run the kernels that read the strides
};

int64_t kv_elem_bytes(const Dims& d) { return d.kv_dtype == PKD_DTYPE_FP8_E4M3 ? 1 : 2; }

Layout paged_layout(const Dims& d) {
  Layout L;
  const int64_t D = d.head_dim;
  L.qs = {(int64_t)d.q_len * d.num_q_heads * D, (int64_t)d.num_q_heads * D, D};
  L.os = L.qs;
  L.kv.head_stride = D * kv_elem_bytes(d);
  L.kv.tok_stride = (int32_t)(d.num_kv_heads * L.kv.head_stride);
  L.kv.page_stride = (int64_t)d.page_size * L.kv.tok_stride;
  L.dense_out = true;
  L.strided = false;
  return L;
}

pkd::SplitParams make_split_params(const Dims& d, const Layout& lay, const void* q, const void* k,
                                   const void* v, const int32_t* bt, const int32_t* lens, const float* ks,
                                   const float* vs, float scale, int S) {
  pkd::SplitParams p{};
  p.qs = lay.qs;
  p.os = lay.os;
  p.kv = lay.kv;
  p.strided = lay.strided ? 1 : 0;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint8_t*>(k);
  p.v = static_cast<const uint8_t*>(v);
  p.block_table = bt;
  p.seq_lens = lens;
  p.k_scale = ks;
  p.v_scale = vs;
  p.qk_scale_log2 = scale * 1.44269504088896340736f;
  p.hq = d.num_q_heads;
  p.hkv = d.num_kv_heads;
  p.group = d.num_q_heads / d.num_kv_heads;
  p.q_len = d.q_len;
  p.causal = d.causal;
  p.window = d.window;
  p.rows_kv = rows_per_kv(d);
  p.head_groups = head_groups(d);
  p.page_size = d.page_size;
  p.max_pages = d.max_pages_per_seq;
  p.num_splits = S;
  p.chunk = split_chunk(d, S);
  return p;
}

// Whether p is a multiple of `bytes` (NULL passes: NULL is checked separately).
bool aligned(const void* p, uintptr_t bytes) { return ((uintptr_t)p & (bytes - 1)) == 0; }

int32_t check_inputs(const Dims* dims, const void* q, const void* k, const void* v,
                     const int32_t* bt, const int32_t* lens, const float* ks, const float* vs,
                     float scale, const float* sinks = nullptr) {
  const int32_t st = check_dims(dims);
  if (st != PKD_OK) return st;
  if (!q || !k || !v || !bt || !lens) return PKD_ERR_NULL_POINTER;
  const bool fp8 = dims->kv_dtype == PKD_DTYPE_FP8_E4M3;
  if (fp8 && (!ks || !vs)) return PKD_ERR_SCALES;
  if (!fp8 && (ks || vs)) return PKD_ERR_SCALES;
  if (!std::isfinite(scale)) return PKD_ERR_BAD_DIMS;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(bt, 4) || !aligned(lens, 4) ||
      !aligned(ks, 4) || !aligned(vs, 4) || !aligned(sinks, 4))
    return PKD_ERR_ALIGNMENT;
  return PKD_OK;
}

// Alignment of the output and workspace pointers of paged_decode and its phases.
int32_t check_out_ws(const void* out, const float* lse, const void* ws) {
  return aligned(out, 16) && aligned(lse, 4) && aligned(ws, 16) ? PKD_OK : PKD_ERR_ALIGNMENT;
}

// Direct output with K/V tiles loaded straight into LDS stages, where that
// kernel applies and the (sequence, KV head) items fit in one round of
// workgroups, or in the pairs form (lds_pairs_workers) in two.  For bf16 it
// gives the grid kernel's bits (FP8: the same arithmetic over eight waves,
// rounding differently); measured back to back it was about 0.7% faster at
// B = 32 (256 items on 256 units; ahead in five of six comparisons) and
// 1-1.5% slower at B = 128 (1024 items, four rounds).
bool lds_direct_ok(const Dims& d, bool strided) {
  const int cus = current_cu_count();
  if (!pkd::lds_direct_applies(d.head_dim, d.kv_dtype == PKD_DTYPE_FP8_E4M3, d.q_len, d.window,
                               d.num_q_heads / d.num_kv_heads, d.page_size, d.max_pages_per_seq, strided) ||
      cus <= 0)
    return false;
  const int64_t items = (int64_t)d.batch * d.num_kv_heads;
  if (items <= cus) return true;
  return items <= 2LL * cus && d.batch <= pkd::kPairedMaxBatch &&
         (int64_t)d.max_pages_per_seq * d.page_size < ((int64_t)1 << 23);
}

bool use_lds_direct(const Dims& d, const Layout& lay) { return lds_direct_ok(d, lay.strided); }

// Workgroups of the LDS-staged direct kernel's pairs form (one or two whole
// items each, paired by length on the device) when the items exceed the
// compute units, else 0 (one workgroup per item).  Only where use_lds_direct.
int lds_pairs_workers(const Dims& d) {
  const int cus = current_cu_count();
  return (int64_t)d.batch * d.num_kv_heads > cus ? cus : 0;
}

int32_t launch_partition(const Dims& d, const pkd::SplitParams& p, bool direct, hipStream_t s) {
  if (current_cu_count() < 0) return PKD_ERR_DEVICE;
  const bool paged16 = d.page_size % 16 == 0;
  const hipError_t e = pkd::launch_split_kv(p, d.batch, d.head_dim, d.kv_dtype == PKD_DTYPE_FP8_E4M3, direct,
                                            paged16, p.strided != 0, s);
  return e == hipSuccess ? PKD_OK : PKD_ERR_LAUNCH;
}

// The heuristic's choice for a checked shape, and the workspace of a mode
// (PKD_SPLITS_AUTO: of the heuristic's choice); 0 for an unsupported mode.
int32_t num_splits_of(const Dims& d, int32_t max_seq_len_hint) {
  const int32_t max_len = max_seq_len_hint > 0 ? max_seq_len_hint : d.max_pages_per_seq * d.page_size;
  return heuristic_splits(d, max_len, false);
}

size_t workspace_of(const Dims& d, int32_t num_splits) {
  int S = num_splits;
  if (S == PKD_SPLITS_AUTO) S = heuristic_splits(d, d.max_pages_per_seq * d.page_size, false);
  if (S == PKD_SPLITS_BALANCED)
    return balanced_ok(d) ? balanced_bytes(d, pair_heads(d, false), nullptr, nullptr, nullptr) : 0;
  if (S == PKD_SPLITS_PAIRED)
    return paired_ok(d) ? balanced_bytes(d, pair_heads(d, false), nullptr, nullptr, nullptr) : 0;
  if (S < 1 || S > PKD_MAX_SPLITS) return 0;
  if (S == 1) return 0;
  return partial_bytes(d, S, nullptr);
}

}  // namespace

extern "C" {

int32_t paged_decode_num_splits(const pkd_dims* dims, int32_t max_seq_len_hint) {
  return paged_decode_num_splits_ext(dims, nullptr, max_seq_len_hint);
}

int32_t paged_decode_num_splits_ext(const pkd_dims* dims, const pkd_ext* ext, int32_t max_seq_len_hint) {
  if (!dims) return PKD_ERR_NULL_POINTER;
  const Dims d = make_dims(*dims, ext);
  const int32_t st = check_dims(&d);
  if (st != PKD_OK) return st;
  return num_splits_of(d, max_seq_len_hint);
}

size_t paged_decode_workspace_bytes(const pkd_dims* dims, int32_t num_splits) {
  // Every num_splits <= 0 asks for the heuristic here.
  return paged_decode_workspace_bytes_ext(dims, nullptr, num_splits <= 0 ? PKD_SPLITS_AUTO : num_splits);
}

size_t paged_decode_workspace_bytes_ext(const pkd_dims* dims, const pkd_ext* ext, int32_t num_splits) {
  if (!dims) return 0;
  const Dims d = make_dims(*dims, ext);
  if (check_dims(&d) != PKD_OK) return 0;
  return workspace_of(d, num_splits);
}

int32_t paged_decode_partials(const pkd_dims* dims, const pkd_ext* ext, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens, const float* k_scale, const float* v_scale,
                              float scale, int32_t num_splits, float* o_part, float* lse_part,
                              void* stream) {
  if (!dims) return PKD_ERR_NULL_POINTER;
  const Dims d = make_dims(*dims, ext);
  int32_t st = check_inputs(&d, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, scale);
  if (st != PKD_OK) return st;
  if (!o_part || !lse_part) return PKD_ERR_NULL_POINTER;
  if (!aligned(o_part, 16) || !aligned(lse_part, 4)) return PKD_ERR_ALIGNMENT;
  if (num_splits < 1 || num_splits > PKD_MAX_SPLITS) return PKD_ERR_NUM_SPLITS;
  if (d.batch == 0) return PKD_OK;
  pkd::SplitParams p = make_split_params(d, paged_layout(d), q, k_cache, v_cache, block_table, seq_lens,
                                         k_scale, v_scale, scale, num_splits);
  p.o_part = o_part;
  p.lse_part = lse_part;
  return launch_partition(d, p, false, static_cast<hipStream_t>(stream));
}

int32_t paged_decode_merge(int64_t rows, int32_t num_splits, int32_t head_dim, const float* o_part,
                           const float* lse_part, void* out, float* lse, void* stream) {
  if (rows < 0 || rows > (int64_t)UINT_MAX * 4) return PKD_ERR_BAD_DIMS;
  if (!valid_head_dim(head_dim)) return PKD_ERR_HEAD_DIM;
  if (num_splits < 1 || num_splits > PKD_MAX_SPLITS) return PKD_ERR_NUM_SPLITS;
  if (!o_part || !lse_part || !out) return PKD_ERR_NULL_POINTER;
  if (!aligned(o_part, 4) || !aligned(lse_part, 4) || !aligned(out, 2) || !aligned(lse, 4))
    return PKD_ERR_ALIGNMENT;
  if (rows == 0) return PKD_OK;
  if (current_cu_count() < 0) return PKD_ERR_DEVICE;
  pkd::MergeParams m{};
  m.o_part = o_part;
  m.lse_part = lse_part;
  m.out = static_cast<uint16_t*>(out);
  m.lse = lse;
  m.rows = rows;
  m.num_splits = num_splits;
  return pkd::launch_lse_merge(m, head_dim, static_cast<hipStream_t>(stream)) == hipSuccess
             ? PKD_OK : PKD_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// Resolved split mode of one call.
struct Plan {
  int S;           // 1 = direct output, 2.. = grid splits, PKD_SPLITS_BALANCED or _PAIRED
  bool balanced;   // the balanced kernel runs (balanced or paired mode)
  bool paired;     // paired mode: whole segments paired by length, merging in place if it falls back
  int pair;        // balanced: KV heads read as one (pair_heads), else 1
  size_t need;     // workspace bytes
  size_t lse_off, prefix_off, count_off;
};

int32_t make_plan(const Dims& d, int32_t num_splits, bool strided, Plan* pl) {
  int S = num_splits;
  if (S == PKD_SPLITS_AUTO) S = heuristic_splits(d, d.max_pages_per_seq * d.page_size, strided);
  pl->S = S;
  pl->paired = S == PKD_SPLITS_PAIRED;
  pl->balanced = S == PKD_SPLITS_BALANCED || pl->paired;
  if (pl->paired ? !paired_ok(d)
                 : pl->balanced ? !balanced_ok(d) : (S < 1 || S > PKD_MAX_SPLITS))
    return PKD_ERR_NUM_SPLITS;
  pl->pair = pl->balanced ? pair_heads(d, strided) : 1;
  pl->lse_off = pl->prefix_off = pl->count_off = 0;
  pl->need = pl->balanced ? balanced_bytes(d, pl->pair, &pl->lse_off, &pl->prefix_off, &pl->count_off)
                          : (S > 1 ? partial_bytes(d, S, &pl->lse_off) : 0);
  return PKD_OK;
}

pkd::BalancedParams make_balanced_params(const Dims& d, const Layout& lay, const void* q, const void* k,
                                         const void* v, const int32_t* bt, const int32_t* lens, const float* ks,
                                         const float* vs, float scale, void* ws, const Plan& pl) {
  pkd::BalancedParams b{};
  b.qs = lay.qs;
  b.os = lay.os;
  b.kv = lay.kv;
  b.strided = lay.strided ? 1 : 0;
  b.pair_heads = pl.pair;
  // Head rows shorter than a 128-byte line put several KV heads in each line;
  // those heads' workgroups are kept on one XCD so each line is fetched once.
  b.xcd_ranges = !lay.strided && pl.pair == 1 && lay.kv.head_stride < 128 && d.num_kv_heads > 1 ? 1 : 0;
  b.q = static_cast<const uint16_t*>(q);
  b.k = static_cast<const uint8_t*>(k);
  b.v = static_cast<const uint8_t*>(v);
  b.block_table = bt;
  b.seq_lens = lens;
  b.k_scale = ks;
  b.v_scale = vs;
  b.o_part = static_cast<float*>(ws);
  b.lse_part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + pl.lse_off);
  b.prefix = reinterpret_cast<int64_t*>(static_cast<uint8_t*>(ws) + pl.prefix_off);
  b.qk_scale_log2 = scale * 1.44269504088896340736f;
  b.batch = d.batch;
  const Dims bv = balanced_view(d, pl.pair);  // segments count wide heads when paired
  b.hq = bv.num_q_heads;
  b.hkv = bv.num_kv_heads;
  b.group = bv.num_q_heads / bv.num_kv_heads;
  b.q_len = bv.q_len;
  b.causal = bv.causal;
  b.window = bv.window;
  b.rows_kv = rows_per_kv(bv);
  b.head_groups = head_groups(bv);
  b.hpg = heads_per_slot(bv);
  b.page_size = d.page_size;
  b.max_pages = d.max_pages_per_seq;
  b.num_workers = balanced_workers(d);
  return b;
}

// Partition phase of a split plan (S > 1 or balanced) into the workspace.
int32_t run_partition(const Dims& d, const Layout& lay, const void* q, const void* k, const void* v,
                      const int32_t* bt, const int32_t* lens, const float* ks, const float* vs, float scale,
                      void* ws, const Plan& pl, hipStream_t s) {
  if (pl.balanced) {
    const pkd::BalancedParams b = make_balanced_params(d, lay, q, k, v, bt, lens, ks, vs, scale, ws, pl);
    return pkd::launch_balanced(b, d.head_dim * pl.pair, d.kv_dtype == PKD_DTYPE_FP8_E4M3, b.strided != 0, s) ==
                   hipSuccess
               ? PKD_OK : PKD_ERR_LAUNCH;
  }
  pkd::SplitParams p = make_split_params(d, lay, q, k, v, bt, lens, ks, vs, scale, pl.S);
  p.o_part = static_cast<float*>(ws);
  p.lse_part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + pl.lse_off);
  return launch_partition(d, p, false, s);
}

// Merge phase of a split plan from the workspace (sinks: [Hq] or null).
int32_t run_finish(const Dims& d, const Layout& lay, const void* ws, const float* sinks, void* out,
                   float* lse, const Plan& pl, hipStream_t s) {
  pkd::MergeParams m{};
  m.sinks = sinks;
  m.hq = d.num_q_heads;
  m.q_len = d.q_len;
  m.strided_out = lay.dense_out ? 0 : 1;
  m.os = lay.os;
  m.o_part = static_cast<const float*>(ws);
  m.lse_part = reinterpret_cast<const float*>(static_cast<const uint8_t*>(ws) + pl.lse_off);
  m.out = static_cast<uint16_t*>(out);
  m.lse = lse;
  m.rows = (int64_t)d.batch * d.q_len * d.num_q_heads;
  if (pl.balanced) {
    m.balanced = 1;
    m.prefix = reinterpret_cast<const int64_t*>(static_cast<const uint8_t*>(ws) + pl.prefix_off);
    const Dims v = balanced_view(d, pl.pair);  // the partition's segments
    m.batch = v.batch;
    m.hkv = v.num_kv_heads;
    m.group = v.num_q_heads / v.num_kv_heads;
    m.head_groups = head_groups(v);
    m.hpg = heads_per_slot(v);
    m.num_workers = balanced_workers(v);
    m.q_len = v.q_len;
  } else {
    m.num_splits = pl.S;
  }
  return pkd::launch_lse_merge(m, d.head_dim, s) == hipSuccess ? PKD_OK : PKD_ERR_LAUNCH;
}

// The whole decode once every argument has been checked: plan, then one
// partition kernel (direct output or in-kernel merge) or partition + merge.
int32_t decode_checked(const Dims& d, const Layout& lay, const void* q, const void* k, const void* v,
                       const int32_t* bt, const int32_t* lens, const float* ks, const float* vs, const float* sinks,
                       float scale, void* out, float* lse, int32_t num_splits, void* workspace,
                       size_t workspace_bytes, hipStream_t s) {
  Plan pl;
  int32_t st = make_plan(d, num_splits, lay.strided, &pl);
  if (st != PKD_OK) return st;
  if (pl.need > 0 && (!workspace || workspace_bytes < pl.need)) return PKD_ERR_WORKSPACE;
  if (d.batch == 0) return PKD_OK;
  if (current_cu_count() < 0) return PKD_ERR_DEVICE;
  if (pl.S == 1) {
    pkd::SplitParams p = make_split_params(d, lay, q, k, v, bt, lens, ks, vs, scale, 1);
    p.out = static_cast<uint16_t*>(out);
    p.lse = lse;
    p.sinks = sinks;
    if (use_lds_direct(d, lay))
      return pkd::launch_lds_direct(p, d.kv_dtype == PKD_DTYPE_FP8_E4M3, d.batch, lds_pairs_workers(d), s) ==
                     hipSuccess
                 ? PKD_OK : PKD_ERR_LAUNCH;
    return launch_partition(d, p, true, s);
  }
  if (pl.balanced && (pl.paired || balanced_fused(d, pl.pair))) {
    // One kernel: the partition merges each segment's pieces itself (or, in
    // paired mode, takes whole segments).
    pkd::BalancedParams b = make_balanced_params(d, lay, q, k, v, bt, lens, ks, vs, scale, workspace, pl);
    b.fused = 1;
    b.paired = pl.paired ? 1 : 0;
    b.out = static_cast<uint16_t*>(out);
    b.lse = lse;
    b.sinks = sinks;
    b.seg_count = reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(workspace) + pl.count_off);
    b.epoch = next_epoch();
    return pkd::launch_balanced(b, d.head_dim * pl.pair, d.kv_dtype == PKD_DTYPE_FP8_E4M3, b.strided != 0, s) ==
                   hipSuccess
               ? PKD_OK : PKD_ERR_LAUNCH;
  }
  st = run_partition(d, lay, q, k, v, bt, lens, ks, vs, scale, workspace, pl, s);
  if (st != PKD_OK) return st;
  return run_finish(d, lay, workspace, sinks, out, lse, pl, s);
}

// Argument checks and the decode of paged_decode / paged_decode_ext.
int32_t decode_entry(const pkd_dims* dims, const pkd_ext* ext, const void* q, const void* k_cache,
                     const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                     const float* k_scale, const float* v_scale, const float* sinks, float scale, void* out,
                     float* lse, int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (!dims) return PKD_ERR_NULL_POINTER;
  const Dims d = make_dims(*dims, ext);
  int32_t st = check_inputs(&d, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, scale, sinks);
  if (st != PKD_OK) return st;
  if (!out) return PKD_ERR_NULL_POINTER;
  st = check_out_ws(out, lse, workspace);
  if (st != PKD_OK) return st;
  return decode_checked(d, paged_layout(d), q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, sinks,
                        scale, out, lse, num_splits, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

int32_t paged_decode_launches(const pkd_dims* dims, const pkd_ext* ext, int32_t num_splits) {
  if (!dims) return PKD_ERR_NULL_POINTER;
  const Dims d = make_dims(*dims, ext);
  const int32_t st = check_dims(&d);
  if (st != PKD_OK) return st;
  Plan pl;
  const int32_t pst = make_plan(d, num_splits, false, &pl);
  if (pst != PKD_OK) return pst;
  if (pl.S == 1 || (pl.balanced && (pl.paired || balanced_fused(d, pl.pair)))) return 1;
  return 2;
}

int32_t pkd_decode_registers(const pkd_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens, float scale, void* out, float* lse,
                             void* stream) {
  if (!dims) return PKD_ERR_NULL_POINTER;
  const Dims d = make_dims(*dims, nullptr);
  int32_t st = check_inputs(&d, q, k_cache, v_cache, block_table, seq_lens, nullptr, nullptr, scale);
  if (st != PKD_OK) return st;
  if (!out) return PKD_ERR_NULL_POINTER;
  st = check_out_ws(out, lse, nullptr);
  if (st != PKD_OK) return st;
  if (d.batch == 0) return PKD_OK;
  if (current_cu_count() < 0) return PKD_ERR_DEVICE;
  pkd::SplitParams p =
      make_split_params(d, paged_layout(d), q, k_cache, v_cache, block_table, seq_lens, nullptr, nullptr, scale, 1);
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  return launch_partition(d, p, true, static_cast<hipStream_t>(stream));
}

int32_t paged_decode_path(const pkd_dims* dims, const pkd_ext* ext, int32_t num_splits) {
  if (!dims) return PKD_ERR_NULL_POINTER;
  const Dims d = make_dims(*dims, ext);
  const int32_t st = check_dims(&d);
  if (st != PKD_OK) return st;
  Plan pl;
  const int32_t pst = make_plan(d, num_splits, false, &pl);
  if (pst != PKD_OK) return pst;
  if (pl.S == 1) return use_lds_direct(d, paged_layout(d)) ? PKD_PATH_DIRECT_LDS : PKD_PATH_DIRECT;
  if (pl.paired) return PKD_PATH_PAIRED;
  if (pl.balanced) return balanced_fused(d, pl.pair) ? PKD_PATH_BALANCED : PKD_PATH_BALANCED_MERGE;
  return PKD_PATH_SPLITS;
}

int32_t paged_decode(const pkd_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, const int32_t* seq_lens, const float* k_scale,
                     const float* v_scale, float scale, void* out, float* lse, int32_t num_splits,
                     void* workspace, size_t workspace_bytes, void* stream) {
  // Every num_splits <= 0 asks for the heuristic here.
  return decode_entry(dims, nullptr, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, nullptr, scale,
                      out, lse, num_splits <= 0 ? PKD_SPLITS_AUTO : num_splits, workspace, workspace_bytes, stream);
}

int32_t paged_decode_ext(const pkd_dims* dims, const pkd_ext* ext, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                         const float* k_scale, const float* v_scale, const float* sinks, float scale, void* out,
                         float* lse, int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_entry(dims, ext, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, sinks, scale, out,
                      lse, num_splits, workspace, workspace_bytes, stream);
}

int32_t paged_decode_partition(const pkd_dims* dims, const pkd_ext* ext, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_table,
                               const int32_t* seq_lens, const float* k_scale, const float* v_scale,
                               float scale, int32_t num_splits, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!dims) return PKD_ERR_NULL_POINTER;
  const Dims d = make_dims(*dims, ext);
  int32_t st = check_inputs(&d, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, scale);
  if (st != PKD_OK) return st;
  Plan pl;
  st = make_plan(d, num_splits, false, &pl);
  if (st != PKD_OK) return st;
  if (pl.S == 1 || pl.paired) return PKD_ERR_NUM_SPLITS;
  if (!workspace || workspace_bytes < pl.need) return PKD_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return PKD_ERR_ALIGNMENT;
  if (d.batch == 0) return PKD_OK;
  if (current_cu_count() < 0) return PKD_ERR_DEVICE;
  return run_partition(d, paged_layout(d), q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, scale,
                       workspace, pl, static_cast<hipStream_t>(stream));
}

int32_t paged_decode_finish(const pkd_dims* dims, const pkd_ext* ext, int32_t num_splits, const void* workspace,
                            size_t workspace_bytes, const float* sinks, void* out, float* lse, void* stream) {
  if (!dims) return PKD_ERR_NULL_POINTER;
  const Dims d = make_dims(*dims, ext);
  int32_t st = check_dims(&d);
  if (st != PKD_OK) return st;
  if (!out) return PKD_ERR_NULL_POINTER;
  st = check_out_ws(out, lse, workspace);
  if (st != PKD_OK) return st;
  if (!aligned(sinks, 4)) return PKD_ERR_ALIGNMENT;
  Plan pl;
  st = make_plan(d, num_splits, false, &pl);
  if (st != PKD_OK) return st;
  if (pl.S == 1 || pl.paired) return PKD_ERR_NUM_SPLITS;
  if (!workspace || workspace_bytes < pl.need) return PKD_ERR_WORKSPACE;
  if (d.batch == 0) return PKD_OK;
  if (current_cu_count() < 0) return PKD_ERR_DEVICE;
  return run_finish(d, paged_layout(d), workspace, sinks, out, lse, pl, static_cast<hipStream_t>(stream));
}

int32_t paged_decode_check_tables(const pkd_dims* dims, const int32_t* block_table,
                                  const int32_t* seq_lens, int32_t* d_error_count, void* stream) {
  if (!dims) return PKD_ERR_NULL_POINTER;
  const Dims d = make_dims(*dims, nullptr);
  const int32_t st = check_dims(&d);
  if (st != PKD_OK) return st;
  if (!block_table || !seq_lens || !d_error_count) return PKD_ERR_NULL_POINTER;
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(d_error_count, 4)) return PKD_ERR_ALIGNMENT;
  if (current_cu_count() < 0) return PKD_ERR_DEVICE;
  const hipError_t e = pkd::launch_check_tables(block_table, seq_lens, dims->batch,
                                                dims->max_pages_per_seq, dims->page_size,
                                                dims->num_pages, d_error_count,
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKD_OK : PKD_ERR_LAUNCH;
}

int32_t paged_kv_append(const pkd_dims* dims, int64_t num_tokens, const void* k_new, const void* v_new,
                        const int64_t* slot_mapping, const int64_t* positions, const float* cos_sin,
                        int32_t max_position, void* k_cache, void* v_cache, const float* k_scale,
                        const float* v_scale, void* stream) {
  if (!dims) return PKD_ERR_NULL_POINTER;
  if (dims->num_kv_heads < 1 || dims->page_size < 1 || dims->num_pages < 1 || num_tokens < 0 ||
      num_tokens > ((int64_t)1 << 40))
    return PKD_ERR_BAD_DIMS;
  if (!valid_head_dim(dims->head_dim)) return PKD_ERR_HEAD_DIM;
  if (dims->kv_dtype != PKD_DTYPE_BF16 && dims->kv_dtype != PKD_DTYPE_FP8_E4M3) return PKD_ERR_DTYPE;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PKD_ERR_NULL_POINTER;
  if ((positions == nullptr) != (cos_sin == nullptr)) return PKD_ERR_NULL_POINTER;
  if (positions && max_position < 1) return PKD_ERR_BAD_DIMS;
  const bool fp8 = dims->kv_dtype == PKD_DTYPE_FP8_E4M3;
  if (fp8 && (!k_scale || !v_scale)) return PKD_ERR_SCALES;
  if (!fp8 && (k_scale || v_scale)) return PKD_ERR_SCALES;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 8) || !aligned(positions, 8) || !aligned(cos_sin, 16) || !aligned(k_scale, 4) ||
      !aligned(v_scale, 4))
    return PKD_ERR_ALIGNMENT;
  if (num_tokens == 0) return PKD_OK;
  if (current_cu_count() < 0) return PKD_ERR_DEVICE;
  pkd::AppendParams a{};
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.slot_mapping = slot_mapping;
  a.positions = positions;
  a.cos_sin = cos_sin;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.num_tokens = num_tokens;
  a.capacity = (int64_t)dims->num_pages * dims->page_size;
  a.max_position = max_position;
  a.hkv = dims->num_kv_heads;
  return pkd::launch_kv_append(a, dims->head_dim, fp8, static_cast<hipStream_t>(stream)) == hipSuccess
             ? PKD_OK : PKD_ERR_LAUNCH;
}

int32_t paged_decode_metadata(const pkd_meta_dims* md, const int32_t* req_to_token,
                              const int64_t* req_pool_indices, const int64_t* seq_lens, int32_t* cache_seqlens,
                              int32_t* cu_seqlens_k, int32_t* page_table, int32_t* swa_seqlens,
                              int32_t* swa_page_table, int32_t* d_error_count, void* stream) {
  if (!md) return PKD_ERR_NULL_POINTER;
  if (md->batch < 0 || md->batch > 65535 || md->req_rows < 1 || md->req_stride < 1 || md->page_size < 1 ||
      md->max_pages_per_seq < 1 || md->q_len < 1 || md->q_len > PKD_MAX_Q_LEN || md->window < 0 ||
      md->extend < 0)
    return PKD_ERR_BAD_DIMS;
  // Every length and prefix sum fits int32.
  const int64_t cap = (int64_t)md->max_pages_per_seq * md->page_size;
  if (cap > INT32_MAX || (int64_t)md->batch * cap > INT32_MAX) return PKD_ERR_BAD_DIMS;
  // With an empty batch only cu_seqlens_k[0] (and the error count) is written.
  if (!cu_seqlens_k) return PKD_ERR_NULL_POINTER;
  if (md->batch > 0) {
    if (!req_to_token || !req_pool_indices || !seq_lens || !cache_seqlens || !page_table)
      return PKD_ERR_NULL_POINTER;
    if (md->window > 0 && (!swa_seqlens || !swa_page_table)) return PKD_ERR_NULL_POINTER;
  }
  if (!aligned(req_to_token, 4) || !aligned(req_pool_indices, 8) || !aligned(seq_lens, 8) ||
      !aligned(cache_seqlens, 4) || !aligned(cu_seqlens_k, 4) || !aligned(page_table, 4) ||
      !aligned(swa_seqlens, 4) || !aligned(swa_page_table, 4) || !aligned(d_error_count, 4))
    return PKD_ERR_ALIGNMENT;
  if (current_cu_count() < 0) return PKD_ERR_DEVICE;
  pkd::MetaParams m{};
  m.req_to_token = req_to_token;
  m.req_pool_indices = req_pool_indices;
  m.seq_lens = seq_lens;
  m.cache_seqlens = cache_seqlens;
  m.cu_seqlens_k = cu_seqlens_k;
  m.page_table = page_table;
  m.swa_seqlens = md->window > 0 ? swa_seqlens : nullptr;
  m.swa_page_table = md->window > 0 ? swa_page_table : nullptr;
  m.error_count = d_error_count;
  m.req_rows = md->req_rows;
  m.req_stride = md->req_stride;
  m.max_len = cap < md->req_stride ? cap : md->req_stride;
  m.batch = md->batch;
  m.page_size = md->page_size;
  m.max_pages = md->max_pages_per_seq;
  m.q_len = md->q_len;
  m.window = md->window;
  m.extend = md->extend;
  return pkd::launch_decode_metadata(m, static_cast<hipStream_t>(stream)) == hipSuccess ? PKD_OK
                                                                                         : PKD_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// The paged problem a contiguous one is run as (one page per sequence, page b
// = sequence b, page_size the capacity rounded up to 16) and its layout.
int32_t contiguous_plan(const pkd_contig_dims* c, Dims* d, Layout* lay) {
  if (!c) return PKD_ERR_NULL_POINTER;
  if (c->max_seq_len < 1 || c->reserved != 0) return PKD_ERR_BAD_DIMS;
  const int64_t ps = ((int64_t)c->max_seq_len + 15) / 16 * 16;
  if (ps > INT32_MAX) return PKD_ERR_BAD_DIMS;
  *d = Dims{c->batch, c->num_q_heads, c->num_kv_heads, c->head_dim, (int32_t)ps, c->batch > 0 ? c->batch : 1,
                1, c->kv_dtype, c->q_len, c->causal, c->window};
  const int32_t st = check_dims(d);
  if (st != PKD_OK) return st;
  for (int i = 0; i < 3; ++i)
    if (c->q_strides[i] < 0 || c->kv_strides[i] < 0 || c->out_strides[i] < 0) return PKD_ERR_BAD_DIMS;
  const int64_t e = kv_elem_bytes(*d);
  if (c->kv_strides[1] * e > INT32_MAX / 16) return PKD_ERR_BAD_DIMS;
  for (int i = 0; i < 3; ++i)
    if (c->q_strides[i] % 8 != 0 || c->out_strides[i] % 8 != 0 || (c->kv_strides[i] * e) % 16 != 0)
      return PKD_ERR_ALIGNMENT;
  lay->qs = {c->q_strides[0], c->q_strides[1], c->q_strides[2]};
  lay->os = {c->out_strides[0], c->out_strides[1], c->out_strides[2]};
  lay->kv.page_stride = c->kv_strides[0] * e;
  lay->kv.tok_stride = (int32_t)(c->kv_strides[1] * e);
  lay->kv.head_stride = c->kv_strides[2] * e;
  const Layout dense = paged_layout(*d);
  lay->dense_out = lay->os.b == dense.os.b && lay->os.i == dense.os.i && lay->os.h == dense.os.h;
  lay->strided = true;
  return PKD_OK;
}

}  // namespace

extern "C" {

size_t contiguous_decode_workspace_bytes(const pkd_contig_dims* dims, int32_t num_splits) {
  Dims d;
  Layout lay;
  if (contiguous_plan(dims, &d, &lay) != PKD_OK) return 0;
  Plan pl;
  if (make_plan(d, num_splits, true, &pl) != PKD_OK) return 0;
  return pl.need;
}

int32_t contiguous_decode(const pkd_contig_dims* dims, const void* q, const void* k, const void* v,
                          const int32_t* seq_lens, const float* k_scale, const float* v_scale, const float* sinks,
                          float scale, void* out, float* lse, int32_t num_splits, void* workspace,
                          size_t workspace_bytes, void* stream) {
  Dims d;
  Layout lay;
  int32_t st = contiguous_plan(dims, &d, &lay);
  if (st != PKD_OK) return st;
  if (!q || !k || !v || !seq_lens || !out) return PKD_ERR_NULL_POINTER;
  const bool fp8 = d.kv_dtype == PKD_DTYPE_FP8_E4M3;
  if (fp8 && (!k_scale || !v_scale)) return PKD_ERR_SCALES;
  if (!fp8 && (k_scale || v_scale)) return PKD_ERR_SCALES;
  if (!std::isfinite(scale)) return PKD_ERR_BAD_DIMS;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(seq_lens, 4) || !aligned(k_scale, 4) ||
      !aligned(v_scale, 4) || !aligned(sinks, 4))
    return PKD_ERR_ALIGNMENT;
  st = check_out_ws(out, lse, workspace);
  if (st != PKD_OK) return st;
  return decode_checked(d, lay, q, k, v, nullptr, seq_lens, k_scale, v_scale, sinks, scale, out, lse, num_splits,
                        workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

const char* paged_decode_status_string(int32_t status) {
  switch (status) {
    case PKD_OK: return "ok";
    case PKD_ERR_NULL_POINTER: return "a required pointer is NULL";
    case PKD_ERR_BAD_DIMS: return "a dimension is out of range";
    case PKD_ERR_GQA: return "num_q_heads is not a multiple of num_kv_heads";
    case PKD_ERR_HEAD_DIM: return "head_dim must be 32, 64, 128 or 256";
    case PKD_ERR_DTYPE: return "unknown kv_dtype";
    case PKD_ERR_SCALES: return "FP8 caches need k_scale and v_scale; BF16 caches take none";
    case PKD_ERR_NUM_SPLITS: return "num_splits out of range";
    case PKD_ERR_WORKSPACE: return "workspace missing or too small";
    case PKD_ERR_LAUNCH: return "kernel launch failed";
    case PKD_ERR_DEVICE: return "the current device is not a usable gfx950";
    case PKD_ERR_SCRATCH_LIMIT: return "the mode needs more workspace than the fixed scratch array holds";
    case PKD_ERR_ALIGNMENT: return "a pointer is not aligned as required";
    default: return "unknown status";
  }
}

}  // extern "C"
