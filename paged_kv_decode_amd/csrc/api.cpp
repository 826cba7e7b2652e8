// C-ABI entry points: host-side validation, the num-splits heuristic,
// workspace sizing and kernel launches.  Nothing here synchronises with the
// device or copies device memory to the host.
#include <atomic>
#include <climits>
#include <cmath>

#include "../../include/paged_kv_decode.h"
#include "pkd_internal.hpp"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not yet queried

// Compute units of the current device (cached per device id), or -1.
int current_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return -1;
  if (dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

bool valid_head_dim(int d) { return d == 32 || d == 64 || d == 128 || d == 256; }

int head_groups(const pkd_dims& d) {
  const int G = d.num_q_heads / d.num_kv_heads;
  return (G + pkd::kHeadsPerGroup - 1) / pkd::kHeadsPerGroup;
}

// Shape checks shared by every entry that takes dims.
int32_t check_dims(const pkd_dims* d) {
  if (!d) return PKD_ERR_NULL_POINTER;
  if (d->batch < 0 || d->batch > 65535 || d->num_q_heads < 1 || d->num_kv_heads < 1 ||
      d->page_size < 1 || d->num_pages < 1 || d->max_pages_per_seq < 1)
    return PKD_ERR_BAD_DIMS;
  if (d->num_q_heads % d->num_kv_heads != 0) return PKD_ERR_GQA;
  if (!valid_head_dim(d->head_dim)) return PKD_ERR_HEAD_DIM;
  if (d->kv_dtype != PKD_DTYPE_BF16 && d->kv_dtype != PKD_DTYPE_FP8_E4M3) return PKD_ERR_DTYPE;
  if ((int64_t)d->max_pages_per_seq * d->page_size > INT32_MAX) return PKD_ERR_BAD_DIMS;
  if ((int64_t)d->num_kv_heads * head_groups(*d) > 65535) return PKD_ERR_BAD_DIMS;
  // Offsets inside one 16-token group of a page are computed in 32 bits.
  if ((int64_t)d->num_kv_heads * d->head_dim * 2 * 16 > INT32_MAX) return PKD_ERR_BAD_DIMS;
  return PKD_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t partial_bytes(const pkd_dims& d, int S, size_t* lse_offset) {
  const size_t rows = (size_t)d.batch * d.num_q_heads;
  const size_t o = align256(rows * (size_t)S * d.head_dim * sizeof(float));
  if (lse_offset) *lse_offset = o;
  return o + align256(rows * (size_t)S * sizeof(float));
}

int32_t heuristic_splits(const pkd_dims& d, int32_t max_len) {
  const int cus = current_cu_count();
  const int64_t target = 4LL * (cus > 0 ? cus : 256);  // workgroups to keep every CU busy
  const int64_t work = (int64_t)d.batch * d.num_kv_heads * head_groups(d);
  if (work <= 0 || work >= target) return 1;
  int64_t s = (target + work - 1) / work;
  const int64_t by_len = (max_len + 255) / 256;  // keep at least ~256 tokens per split
  if (s > by_len) s = by_len;
  if (s < 1) s = 1;
  if (s > PKD_MAX_SPLITS) s = PKD_MAX_SPLITS;
  return (int32_t)s;
}

pkd::SplitParams make_split_params(const pkd_dims& d, const void* q, const void* k, const void* v,
                                   const int32_t* bt, const int32_t* lens, const float* ks,
                                   const float* vs, float scale, int S) {
  pkd::SplitParams p{};
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
  p.head_groups = head_groups(d);
  p.page_size = d.page_size;
  p.max_pages = d.max_pages_per_seq;
  p.num_splits = S;
  return p;
}

int32_t check_inputs(const pkd_dims* dims, const void* q, const void* k, const void* v,
                     const int32_t* bt, const int32_t* lens, const float* ks, const float* vs,
                     float scale) {
  const int32_t st = check_dims(dims);
  if (st != PKD_OK) return st;
  if (!q || !k || !v || !bt || !lens) return PKD_ERR_NULL_POINTER;
  const bool fp8 = dims->kv_dtype == PKD_DTYPE_FP8_E4M3;
  if (fp8 && (!ks || !vs)) return PKD_ERR_SCALES;
  if (!fp8 && (ks || vs)) return PKD_ERR_SCALES;
  if (!std::isfinite(scale)) return PKD_ERR_BAD_DIMS;
  return PKD_OK;
}

int32_t launch_partition(const pkd_dims& d, const pkd::SplitParams& p, bool direct, hipStream_t s) {
  if (current_cu_count() < 0) return PKD_ERR_DEVICE;
  const bool paged16 = d.page_size % 16 == 0;
  const hipError_t e = pkd::launch_split_kv(p, d.batch, d.head_dim,
                                            d.kv_dtype == PKD_DTYPE_FP8_E4M3, direct, paged16, s);
  return e == hipSuccess ? PKD_OK : PKD_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int32_t paged_decode_num_splits(const pkd_dims* dims, int32_t max_seq_len_hint) {
  const int32_t st = check_dims(dims);
  if (st != PKD_OK) return st;
  const int32_t max_len = max_seq_len_hint > 0 ? max_seq_len_hint
                                               : dims->max_pages_per_seq * dims->page_size;
  return heuristic_splits(*dims, max_len);
}

size_t paged_decode_workspace_bytes(const pkd_dims* dims, int32_t num_splits) {
  if (check_dims(dims) != PKD_OK) return 0;
  int S = num_splits;
  if (S <= 0) S = heuristic_splits(*dims, dims->max_pages_per_seq * dims->page_size);
  if (S > PKD_MAX_SPLITS) return 0;
  if (S == 1) return 0;
  return partial_bytes(*dims, S, nullptr);
}

int32_t paged_decode_partials(const pkd_dims* dims, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens, const float* k_scale, const float* v_scale,
                              float scale, int32_t num_splits, float* o_part, float* lse_part,
                              void* stream) {
  int32_t st = check_inputs(dims, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, scale);
  if (st != PKD_OK) return st;
  if (!o_part || !lse_part) return PKD_ERR_NULL_POINTER;
  if (num_splits < 1 || num_splits > PKD_MAX_SPLITS) return PKD_ERR_NUM_SPLITS;
  if (dims->batch == 0) return PKD_OK;
  pkd::SplitParams p = make_split_params(*dims, q, k_cache, v_cache, block_table, seq_lens, k_scale,
                                         v_scale, scale, num_splits);
  p.o_part = o_part;
  p.lse_part = lse_part;
  return launch_partition(*dims, p, false, static_cast<hipStream_t>(stream));
}

int32_t paged_decode_merge(int64_t rows, int32_t num_splits, int32_t head_dim, const float* o_part,
                           const float* lse_part, void* out, float* lse, void* stream) {
  if (rows < 0 || rows > (int64_t)UINT_MAX * 4) return PKD_ERR_BAD_DIMS;
  if (!valid_head_dim(head_dim)) return PKD_ERR_HEAD_DIM;
  if (num_splits < 1 || num_splits > PKD_MAX_SPLITS) return PKD_ERR_NUM_SPLITS;
  if (!o_part || !lse_part || !out) return PKD_ERR_NULL_POINTER;
  if (rows == 0) return PKD_OK;
  if (current_cu_count() < 0) return PKD_ERR_DEVICE;
  pkd::MergeParams m{o_part, lse_part, static_cast<uint16_t*>(out), lse, rows, num_splits};
  return pkd::launch_lse_merge(m, head_dim, static_cast<hipStream_t>(stream)) == hipSuccess
             ? PKD_OK : PKD_ERR_LAUNCH;
}

int32_t paged_decode(const pkd_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, const int32_t* seq_lens, const float* k_scale,
                     const float* v_scale, float scale, void* out, float* lse, int32_t num_splits,
                     void* workspace, size_t workspace_bytes, void* stream) {
  int32_t st = check_inputs(dims, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, scale);
  if (st != PKD_OK) return st;
  if (!out) return PKD_ERR_NULL_POINTER;
  if (num_splits > PKD_MAX_SPLITS) return PKD_ERR_NUM_SPLITS;
  const int S = num_splits > 0
                    ? num_splits
                    : heuristic_splits(*dims, dims->max_pages_per_seq * dims->page_size);
  size_t lse_off = 0;
  if (S > 1) {
    const size_t need = partial_bytes(*dims, S, &lse_off);
    if (!workspace || workspace_bytes < need) return PKD_ERR_WORKSPACE;
  }
  if (dims->batch == 0) return PKD_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  pkd::SplitParams p = make_split_params(*dims, q, k_cache, v_cache, block_table, seq_lens, k_scale,
                                         v_scale, scale, S);
  if (S == 1) {
    p.out = static_cast<uint16_t*>(out);
    p.lse = lse;
    return launch_partition(*dims, p, true, s);
  }
  p.o_part = static_cast<float*>(workspace);
  p.lse_part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + lse_off);
  st = launch_partition(*dims, p, false, s);
  if (st != PKD_OK) return st;
  pkd::MergeParams m{p.o_part, p.lse_part, static_cast<uint16_t*>(out), lse,
                     (int64_t)dims->batch * dims->num_q_heads, S};
  return pkd::launch_lse_merge(m, dims->head_dim, s) == hipSuccess ? PKD_OK : PKD_ERR_LAUNCH;
}

int32_t paged_decode_check_tables(const pkd_dims* dims, const int32_t* block_table,
                                  const int32_t* seq_lens, int32_t* d_error_count, void* stream) {
  const int32_t st = check_dims(dims);
  if (st != PKD_OK) return st;
  if (!block_table || !seq_lens || !d_error_count) return PKD_ERR_NULL_POINTER;
  if (current_cu_count() < 0) return PKD_ERR_DEVICE;
  const hipError_t e = pkd::launch_check_tables(block_table, seq_lens, dims->batch,
                                                dims->max_pages_per_seq, dims->page_size,
                                                dims->num_pages, d_error_count,
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKD_OK : PKD_ERR_LAUNCH;
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
    case PKD_ERR_DEVICE: return "no usable device is current";
    default: return "unknown status";
  }
}

}  // extern "C"
