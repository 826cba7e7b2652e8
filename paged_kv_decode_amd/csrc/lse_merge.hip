// Log-sum-exp merge of split-KV partials for gfx950.
//
// One wave per output row (sequence, query token, query head).  With M = max_j lse_j,
// w_j = exp(lse_j - M) and W = sum_j w_j, the merged row is
// out = sum_j w_j o_j / W (bf16, round-to-nearest-even) and lse = M + ln W.
// This is the recombination behind split-KV decoding (the AstrAI commit log's
// split partials, b12x's PagedPersistentMergeKernel, vLLM's merge_attn_states
// in the sglang fuse/overlap catalogue).  Partials of empty splits carry
// lse = -inf and weigh 0; a row with no non-empty split gets out = 0 and
// lse = -inf.  Splits are summed in index order, so the result is
// deterministic.  With sink logits the head's sink joins the denominator at
// the end (out scaled by e^(lse - lse'), lse' = ln(e^lse + e^sink)).
//
// Also: the optional block-table / length validation kernel.
#include "merge_row.hpp"
#include "pkd_internal.hpp"

namespace pkd {
namespace {

// WPR waves per output row (WPR = 1: four rows per workgroup).  Wave `part`
// of a row takes the row's partials j = part, part + WPR, ...: their LSEs are
// read one per lane and reduced across the wave to M_w and W_w = sum exp(lse_j
// - M_w), and their rows are read with lanes along the head dimension, several
// partials per batch of independent loads, accumulated with weights
// exp(lse_j - M_w).  With WPR > 1 the waves' (M_w, W_w, o_w) are then combined
// in LDS by the same rule.
// The merge kernel's waves take up to 16 partials in one round trip of loads
// (a wave of the partition kernel's in-place merge, at the edge of its
// registers, takes 8).
template <int D>
using KernelRowMerge = RowMerge<D, false, 16>;

template <int D, int WPR>
__global__ void __launch_bounds__(64 * (WPR == 1 ? 4 : WPR)) lse_merge_kernel(const MergeParams p) {
  constexpr int EPL = KernelRowMerge<D>::EPL;
  constexpr int WAVES = WPR == 1 ? 4 : WPR;
  __shared__ float sm_m[WAVES], sm_w[WAVES];
  __shared__ float sm_o[WPR == 1 ? 1 : WAVES * D];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row = WPR == 1 ? (int64_t)blockIdx.x * 4 + wave : (int64_t)blockIdx.x;
  const int part = WPR == 1 ? 0 : wave;
  if (row >= p.rows) return;  // with WPR > 1 the whole workgroup shares the row

  // Where this row's partials are: lp[j * ls] and op[j * os + d], j < S.
  int S;
  const float* lp;
  const float* op;
  int64_t ls, os;
  if (!p.balanced) {
    S = p.num_splits;
    lp = p.lse_part + row * S;
    op = p.o_part + row * S * D;
    ls = 1;
    os = D;
  } else {
    // Row (b * q_len + i) * Hq + h is packed row r = i * G + h % G of KV head
    // h / G.  Segment s = (b * Hkv + kvh) * HG + hg starts at group P_s of the
    // work space; its pieces were written by workgroups w_first .. w_last at
    // slots w + s.
    const int64_t per_seq = (int64_t)p.q_len * p.hq;
    const int b = (int)(row / per_seq);
    const int rem = (int)(row - (int64_t)b * per_seq);
    const int qi = rem / p.hq;
    const int h = rem - qi * p.hq;
    const int kvh = h / p.group;
    const int hin = qi * p.group + (h - kvh * p.group);
    const int hg = hin / kHeadsPerGroup;
    const int nh = hin - hg * kHeadsPerGroup;
    const int spb = p.hkv * p.head_groups;
    const int seg = kvh * p.head_groups + hg;
    const int64_t T = p.prefix[p.batch];
    const int64_t nb = (p.prefix[b + 1] - p.prefix[b]) / spb;
    S = 0;
    int64_t slot0 = 0;
    if (nb > 0) {
      const int64_t ps_ = p.prefix[b] + seg * nb;
      const int64_t nwe = min((int64_t)p.num_workers, T);
      int64_t w_first;
      segment_pieces(ps_, nb, nwe, T, &w_first, &S);
      slot0 = w_first + (int64_t)b * spb + seg;
    }
    lp = p.lse_part + slot0 * p.hpg + nh;
    op = p.o_part + (slot0 * p.hpg + nh) * D;
    ls = p.hpg;
    os = (int64_t)p.hpg * D;
  }
  // This wave's partials: j = part + WPR * k, k < mine.
  const int mine = S > part ? (S - part + WPR - 1) / WPR : 0;
  lp += (int64_t)part * ls;
  op += (int64_t)part * os;
  ls *= WPR;
  os *= WPR;

  KernelRowMerge<D> r;
  r.run(lp, ls, op, os, mine, lane);

  if constexpr (WPR > 1) {
    // Combine the waves: M = max M_w, W = sum e_w W_w, o = sum e_w o_w, e_w = exp(M_w - M).
    const bool live = lane * EPL < D;
    if (lane == 0) {
      sm_m[wave] = r.M;
      sm_w[wave] = r.W;
    }
    if (live)
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_o[wave * D + lane * EPL + e] = r.o[e];
    __syncthreads();
    if (wave != 0) return;
    float Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) Mx = fmaxf(Mx, sm_m[w]);
    r.W = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) r.o[e] = 0.f;
    if (Mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float ew = __builtin_amdgcn_exp2f((sm_m[w] - Mx) * kMergeLog2e);  // 0 for an empty wave
        r.W += ew * sm_w[w];
        if (live)
#pragma unroll
          for (int e = 0; e < EPL; ++e) r.o[e] += ew * sm_o[w * D + lane * EPL + e];
      }
    }
    r.M = Mx;
  }
  int64_t ooff = row * D;
  if (p.strided_out) {
    const int64_t per_seq = (int64_t)p.q_len * p.hq;
    const int64_t b = row / per_seq;
    const int rem = (int)(row - b * per_seq);
    const int qi = rem / p.hq;
    ooff = p.os.at(b, qi, rem - qi * p.hq);
  }
  r.store(p.out + ooff, p.lse ? p.lse + row : nullptr, lane, p.sinks ? p.sinks[(int)(row % p.hq)] : -INFINITY);
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

template <int D, int WPR>
hipError_t launch_merge_t(const MergeParams& p, hipStream_t stream) {
  const int64_t blocks = WPR == 1 ? (p.rows + 3) / 4 : p.rows;
  hipLaunchKernelGGL((lse_merge_kernel<D, WPR>), dim3((unsigned)blocks), dim3(64 * (WPR == 1 ? 4 : WPR)), 0,
                     stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_merge_d(const MergeParams& p, hipStream_t stream) {
  // Waves per row from the partials a row is expected to hold.  In the
  // balanced layout one wave per row exactly when the partition kernel would
  // merge in-kernel, so that both paths give the same bits.
  const int64_t segments = (int64_t)p.batch * p.hkv * p.head_groups;
  if (p.balanced && balanced_merge_in_kernel(p.num_workers, segments)) return launch_merge_t<D, 1>(p, stream);
  const int64_t per_row = p.balanced ? p.num_workers / segments + 2 : p.num_splits;
  if (per_row >= 64) return launch_merge_t<D, 16>(p, stream);
  if (per_row >= 12) return launch_merge_t<D, 4>(p, stream);
  return launch_merge_t<D, 1>(p, stream);
}

}  // namespace

hipError_t launch_lse_merge(const MergeParams& p, int head_dim, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  switch (head_dim) {
    case 32: return launch_merge_d<32>(p, stream);
    case 64: return launch_merge_d<64>(p, stream);
    case 128: return launch_merge_d<128>(p, stream);
    case 256: return launch_merge_d<256>(p, stream);
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
