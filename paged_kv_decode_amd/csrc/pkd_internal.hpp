// Internal declarations shared by the HIP kernels and the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkd {

// Arguments of the split-KV partition kernel (one launch).
struct SplitParams {
  const uint16_t* q;           // [B][Hq][D] bf16
  const uint8_t* k;            // [num_pages][ps][Hkv][D] kv elements (bf16 or fp8 codes)
  const uint8_t* v;
  const int32_t* block_table;  // [B][max_pages]
  const int32_t* seq_lens;     // [B]
  const float* k_scale;        // [Hkv] (fp8) or null
  const float* v_scale;
  uint16_t* out;               // direct mode: [B][Hq][D] bf16
  float* lse;                  // direct mode: [B][Hq] or null
  float* o_part;               // split mode: [B][Hq][S][D]
  float* lse_part;             // split mode: [B][Hq][S]
  float qk_scale_log2;         // scale * log2(e): scores are kept in base-2 units
  int32_t hq, hkv, group;      // group = G = Hq / Hkv
  int32_t head_groups;         // ceil(G / 16): query heads are packed 16 per workgroup
  int32_t page_size, max_pages;
  int32_t num_splits;
};

// Arguments of the log-sum-exp merge kernel.
struct MergeParams {
  const float* o_part;         // [rows][S][D]
  const float* lse_part;       // [rows][S] natural log
  uint16_t* out;               // [rows][D] bf16
  float* lse;                  // [rows] or null
  int64_t rows;
  int32_t num_splits;
};

constexpr int kWaves = 4;            // waves per split-kernel workgroup
constexpr int kSplitAlign = 64;      // tokens; split boundaries are multiples of this
constexpr int kHeadsPerGroup = 16;   // query heads packed into one MFMA N dimension

// Launchers (defined in the .hip files).  head_dim in {32, 64, 128, 256}.
hipError_t launch_split_kv(const SplitParams& p, int batch, int head_dim, bool fp8, bool direct,
                           bool paged16, hipStream_t stream);
hipError_t launch_lse_merge(const MergeParams& p, int head_dim, hipStream_t stream);
hipError_t launch_check_tables(const int32_t* block_table, const int32_t* seq_lens, int batch,
                               int max_pages, int page_size, int num_pages, int32_t* d_count,
                               hipStream_t stream);

}  // namespace pkd
