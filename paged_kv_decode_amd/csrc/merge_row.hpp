// Log-sum-exp merge of one output row's partials by one wave, shared by the
// merge kernel and the balanced kernel's in-kernel merge so that both give the
// same bits.
//
// With M = max_j lse_j, w_j = exp(lse_j - M) and W = sum_j w_j, the merged row
// is out = sum_j w_j o_j / W and lse = M + ln W: the recombination behind
// split-KV decoding (the AstrAI commit log's split partials, b12x's
// PagedPersistentMergeKernel, vLLM's merge_attn_states in the sglang
// fuse/overlap catalogue).  Partials with lse = -inf weigh 0; when all are
// -inf the row is 0 with lse = -inf.  Partials are summed in index order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkd {

constexpr float kMergeLog2e = 1.44269504088896340736f;
constexpr float kMergeLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float merge_wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

// Folds a query head's sink logit into a finished row (natural-log lse):
// lse' = ln(e^lse + e^sink); returns the factor e^(lse - lse') that scales the
// output (0 for a row that saw no token, whose lse becomes the sink).
__device__ __forceinline__ float fold_sink(float& lse, float sink) {
  if (sink == -INFINITY) return 1.f;
  if (lse == -INFINITY) {
    lse = sink;
    return 0.f;
  }
  const float mx = fmaxf(lse, sink);
  const float l2 = mx + log1pf(expf(-fabsf(lse - sink)));
  const float f = expf(lse - l2);
  lse = l2;
  return f;
}

// One wave's share of a row: partials k < mine, LSE at lp[k * ls], row at
// op[k * os + d].  Lanes run along the head dimension (EPL elements each).
// After run(), M is the maximum LSE seen, W the (wave-reduced) sum of
// exp(lse_k - M) and o the unnormalised row.
// With few partials (mine <= UNROLL) the same result can be had in two steps,
// issue() then finish(), so that a wave merging several rows has all of their
// loads in flight before it combines any; both run the same code as run().
// COHERENT: read the partials with agent-scope atomic loads, which see the
// coherent copy even when another XCD's workgroup wrote them during this
// kernel (ordinary loads may hit a stale line of this XCD's L2).
// UNROLL: partials loaded per batch (and the most the one-round-trip path
// takes).  For up to 64 partials both paths add the same products in the same
// order, so the choice changes no bit of the result (but for the sign of a
// row that sums to zero exactly).
template <int D, bool COHERENT = false, int UNROLL_ = 8>
struct RowMerge {
  static constexpr int EPL = D >= 64 ? D / 64 : 1;  // elements per lane
  static constexpr int UNROLL = UNROLL_;
  float M, W;
  float o[EPL];

  // Loads of the few-partials path, held between issue() and finish().
  struct Staged {
    float l_own;            // this lane's partial LSE
    float v[UNROLL][EPL];   // the partial rows
  };

  static __device__ __forceinline__ float ld(const float* a) {
    if constexpr (COHERENT)
      return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      return *a;
  }

  __device__ __forceinline__ void begin() {
    M = -INFINITY;
    W = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  }

  // Few partials: their LSEs and rows are loaded together, in one round trip ...
  static __device__ __forceinline__ void load_few(const float* lp, int64_t ls, const float* op, int64_t os,
                                                  int mine, int lane, float& l_own, float (&v)[UNROLL][EPL]) {
    const bool live = lane * EPL < D;
    l_own = lane < mine ? ld(lp + lane * ls) : -INFINITY;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        v[u][e] = (live && u < mine) ? ld(op + (int64_t)u * os + lane * EPL + e) : 0.f;
  }

  // ... and combined once the maximum is known.
  __device__ __forceinline__ void combine_few(float l_own, const float (&v)[UNROLL][EPL], int mine, int lane) {
    M = merge_wave_max(l_own);
    if (M != -INFINITY) {
      const float wl = lane < mine ? __builtin_amdgcn_exp2f((l_own - M) * kMergeLog2e) : 0.f;
      W = wl;
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const float wgt = __shfl(wl, u);
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] += wgt * v[u][e];
      }
    }
  }

  __device__ __forceinline__ void reduce_w() {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) W += __shfl_xor(W, m);
  }

  __device__ __forceinline__ void run(const float* lp, int64_t ls, const float* op, int64_t os, int mine,
                                      int lane) {
    begin();
    const bool live = lane * EPL < D;
    if (mine <= UNROLL) {
      float l_own;
      float v[UNROLL][EPL];
      load_few(lp, ls, op, os, mine, lane, l_own, v);
      combine_few(l_own, v, mine, lane);
    } else {
      for (int k = lane; k < mine; k += 64) M = fmaxf(M, ld(lp + k * ls));
      M = merge_wave_max(M);
      if (M != -INFINITY) {
        for (int k0 = 0; k0 < mine; k0 += 64) {
          // weights of partials k0 .. k0+63, one per lane
          const int kl = k0 + lane;
          const float wl = kl < mine ? __builtin_amdgcn_exp2f((ld(lp + kl * ls) - M) * kMergeLog2e) : 0.f;
          W += wl;
          const int kn = min(64, mine - k0);
          int k = 0;
          for (; k + UNROLL <= kn; k += UNROLL) {
            float v[UNROLL][EPL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
#pragma unroll
              for (int e = 0; e < EPL; ++e)
                v[u][e] = live ? ld(op + (int64_t)(k0 + k + u) * os + lane * EPL + e) : 0.f;
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
              const float wgt = __shfl(wl, k + u);
#pragma unroll
              for (int e = 0; e < EPL; ++e) o[e] += wgt * v[u][e];
            }
          }
          for (; k < kn; ++k) {
            const float wgt = __shfl(wl, k);
#pragma unroll
            for (int e = 0; e < EPL; ++e)
              o[e] += wgt * (live ? ld(op + (int64_t)(k0 + k) * os + lane * EPL + e) : 0.f);
          }
        }
      }
    }
    reduce_w();
  }

  // The two-step form of run() for mine <= UNROLL.
  static __device__ __forceinline__ void issue(const float* lp, int64_t ls, const float* op, int64_t os, int mine,
                                               int lane, Staged& st) {
    load_few(lp, ls, op, os, mine, lane, st.l_own, st.v);
  }
  __device__ __forceinline__ void finish(const Staged& st, int mine, int lane) {
    begin();
    combine_few(st.l_own, st.v, mine, lane);
    reduce_w();
  }

  // Writes the normalised row (bf16, round-to-nearest-even) and, from lane 0,
  // its natural-log LSE (when lse is not null).  A finite sink logit joins the
  // denominator: the row is scaled by 1 / (1 + e^(sink - lse)) and the LSE
  // becomes ln(e^lse + e^sink); a row with no partial then gets 0 and the sink.
  __device__ __forceinline__ void store(uint16_t* out_row, float* lse, int lane, float sink = -INFINITY) const {
    float l = M != -INFINITY ? M + log2f(W) * kMergeLn2 : -INFINITY;
    const float f = fold_sink(l, sink);
    if (lane * EPL < D) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float v = M != -INFINITY ? (o[e] / W) * f : 0.f;
        const __bf16 h = (__bf16)v;
        uint16_t bits;
        __builtin_memcpy(&bits, &h, 2);
        out_row[lane * EPL + e] = bits;
      }
    }
    if (lane == 0 && lse) *lse = l;
  }
};

}  // namespace pkd
