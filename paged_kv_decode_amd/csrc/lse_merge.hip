// Log-sum-exp merge of split-KV partials for gfx950.
//
// One wave per output row (sequence, query head).  With M = max_j lse_j,
// w_j = exp(lse_j - M) and W = sum_j w_j, the merged row is
// out = sum_j w_j o_j / W (bf16, round-to-nearest-even) and lse = M + ln W.
// This is the recombination behind split-KV decoding (the AstrAI commit log's
// split partials, b12x's PagedPersistentMergeKernel, vLLM's merge_attn_states
// in the sglang fuse/overlap catalogue).  Partials of empty splits carry
// lse = -inf and weigh 0; a row with no non-empty split gets out = 0 and
// lse = -inf.  Splits are summed in index order, so the result is
// deterministic.
//
// Also: the optional block-table / length validation kernel.
#include "pkd_internal.hpp"

namespace pkd {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

template <int D>
__global__ void __launch_bounds__(256) lse_merge_kernel(const MergeParams p) {
  constexpr int EPL = D >= 64 ? D / 64 : 1;  // elements per lane
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const int S = p.num_splits;
  const float* lp = p.lse_part + row * S;
  const float* op = p.o_part + row * S * D;

  float M = -INFINITY;
  for (int j = lane; j < S; j += 64) M = fmaxf(M, lp[j]);
  M = wave_max(M);

  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  float W = 0.f;
  if (M != -INFINITY) {
    for (int j = 0; j < S; ++j) {
      const float w = __builtin_amdgcn_exp2f((lp[j] - M) * kLog2e);
      W += w;
      const float* oj = op + (int64_t)j * D;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int d = lane * EPL + e;
        if (d < D) o[e] += w * oj[d];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int d = lane * EPL + e;
    if (d < D) {
      const float v = M != -INFINITY ? o[e] / W : 0.f;
      const __bf16 h = (__bf16)v;
      uint16_t bits;
      __builtin_memcpy(&bits, &h, 2);
      p.out[row * D + d] = bits;
    }
  }
  if (lane == 0 && p.lse) p.lse[row] = M != -INFINITY ? M + log2f(W) * kLn2 : -INFINITY;
}

// Counts sequences with a length outside [0, max_pages * page_size] and used
// block-table entries outside [0, num_pages).  One workgroup; the count is
// written, not accumulated.
__global__ void __launch_bounds__(256)
check_tables_kernel(const int32_t* bt, const int32_t* lens, int batch, int max_pages, int page_size,
                    int num_pages, int32_t* d_count) {
  __shared__ int32_t partial[256];
  int32_t bad = 0;
  for (int b = 0; b < batch; ++b) {
    const int L = lens[b];
    const bool len_ok = L >= 0 && (int64_t)L <= (int64_t)max_pages * page_size;
    if (!len_ok) {
      if (threadIdx.x == 0) ++bad;
      continue;
    }
    const int used = (L + page_size - 1) / page_size;
    for (int i = threadIdx.x; i < used; i += 256) {
      const int32_t pg = bt[(int64_t)b * max_pages + i];
      if (pg < 0 || pg >= num_pages) ++bad;
    }
  }
  partial[threadIdx.x] = bad;
  __syncthreads();
  for (int s = 128; s >= 1; s >>= 1) {
    if ((int)threadIdx.x < s) partial[threadIdx.x] += partial[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) *d_count = partial[0];
}

template <int D>
hipError_t launch_merge_t(const MergeParams& p, hipStream_t stream) {
  const int64_t blocks = (p.rows + 3) / 4;
  hipLaunchKernelGGL((lse_merge_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(const MergeParams& p, int head_dim, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  switch (head_dim) {
    case 32: return launch_merge_t<32>(p, stream);
    case 64: return launch_merge_t<64>(p, stream);
    case 128: return launch_merge_t<128>(p, stream);
    case 256: return launch_merge_t<256>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_check_tables(const int32_t* block_table, const int32_t* seq_lens, int batch,
                               int max_pages, int page_size, int num_pages, int32_t* d_count,
                               hipStream_t stream) {
  hipLaunchKernelGGL(check_tables_kernel, dim3(1), dim3(256), 0, stream, block_table, seq_lens, batch,
                     max_pages, page_size, num_pages, d_count);
  return hipGetLastError();
}

}  // namespace pkd
