// Decode metadata preparation for gfx950: the block table and lengths that
// decode reads, built on the device from the serving runtime's token map.
//
// The sglang fuse/overlap catalogue (section 1) lists this step as one fused
// kernel for its flashattention backend's decode.  Here it is one launch that
// derives, for batch entry b with request row r = req_pool_indices[b] and
// L = seq_lens[b] + extend (the lengths after this step's new tokens):
//   cache_seqlens[b] = L (int32), cu_seqlens_k = exclusive prefix sums,
//   page_table[b][j] = req_to_token[r][j * ps] / ps for j < ceil(L / ps), else -1,
//   with a window W: f = max(L - q_len - W + 1, 0) / ps pages are dropped:
//   swa_page_table[b][j] = page_table[b][f + j], swa_seqlens[b] = L - f * ps.
// An entry with r outside [0, req_rows) or L outside
// [0, min(max_pages * ps, req_stride)] is invalid: lengths 0, rows -1, counted.
//
// Grid: one workgroup per batch entry writes its table rows (the gather reads
// one int32 per page, the first token's slot); one more workgroup computes
// the lengths, their validity and the prefix sums for the whole batch (a
// wave-shuffle scan per 256-entry chunk with a running carry) and writes the
// invalid count.  The entries need each other only through the prefix sums,
// which the last workgroup computes from the lengths alone, so nothing waits.
#include "pkd_internal.hpp"

namespace pkd {
namespace {

constexpr int kMetaThreads = 256;  // threads per workgroup

__device__ __forceinline__ bool meta_len(const MetaParams& p, int b, int64_t* len, int64_t* row) {
  const int64_t r = p.req_pool_indices[b];
  const int64_t L = p.seq_lens[b] + p.extend;
  const bool ok = r >= 0 && r < p.req_rows && L >= 0 && L <= p.max_len;
  *len = ok ? L : 0;
  *row = ok ? r : 0;
  return ok;
}

__device__ __forceinline__ int32_t slot_page(int32_t slot, int ps) { return slot >= 0 ? slot / ps : -1; }

__global__ void __launch_bounds__(kMetaThreads) decode_metadata_kernel(const MetaParams p) {
  const int tid = threadIdx.x;
  if ((int)blockIdx.x < p.batch) {
    const int b = blockIdx.x;
    int64_t L, r;
    meta_len(p, b, &L, &r);
    const int ps = p.page_size;
    const int64_t n = (L + ps - 1) / ps;
    const int32_t* src = p.req_to_token + r * p.req_stride;
    int32_t* pt = p.page_table + (int64_t)b * p.max_pages;
    for (int j = tid; j < p.max_pages; j += kMetaThreads) pt[j] = j < n ? slot_page(src[(int64_t)j * ps], ps) : -1;
    if (p.window > 0) {
      const int64_t lo = max(L - p.q_len - p.window + 1, (int64_t)0);
      const int64_t f = lo / ps;
      int32_t* st = p.swa_page_table + (int64_t)b * p.max_pages;
      for (int j = tid; j < p.max_pages; j += kMetaThreads)
        st[j] = j < n - f ? slot_page(src[(f + j) * ps], ps) : -1;
      if (tid == 0) p.swa_seqlens[b] = (int32_t)(L - f * ps);
    }
    return;
  }
  // The prefix-sum workgroup.
  __shared__ int32_t wsum[kMetaThreads / 64];
  __shared__ int32_t s_bad[kMetaThreads / 64];
  const int lane = tid & 63, wave = tid >> 6;
  int32_t carry = 0, bad = 0;
  if (tid == 0) p.cu_seqlens_k[0] = 0;
  for (int base = 0; base < p.batch; base += kMetaThreads) {
    const int b = base + tid;
    int64_t L = 0, r;
    if (b < p.batch) {
      bad += !meta_len(p, b, &L, &r);
      p.cache_seqlens[b] = (int32_t)L;
    }
    int32_t x = (int32_t)L;  // inclusive scan within the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t up = __shfl_up(x, off);
      if (lane >= off) x += up;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int32_t before = carry;
    for (int v = 0; v < wave; ++v) before += wsum[v];
    if (b < p.batch) p.cu_seqlens_k[b + 1] = before + x;
    int32_t total = 0;
    for (int v = 0; v < kMetaThreads / 64; ++v) total += wsum[v];
    carry += total;
    __syncthreads();  // wsum is rewritten by the next chunk
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) bad += __shfl_xor(bad, off);
  if (lane == 0) s_bad[wave] = bad;
  __syncthreads();
  if (tid == 0) {
    int32_t total = 0;
    for (int v = 0; v < kMetaThreads / 64; ++v) total += s_bad[v];
    if (p.error_count) *p.error_count = total;
  }
}

}  // namespace

hipError_t launch_decode_metadata(const MetaParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(decode_metadata_kernel, dim3(p.batch + 1), dim3(kMetaThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkd
