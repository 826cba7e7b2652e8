// Direct-output paged decode with a vector-ALU inner loop, for measurement
// beside the matrix-core kernels (not called by any decode entry point).
//
// The decode kernels run QK^T and PV as 16x16x32 matrix-core products with the
// query rows of a KV head packed along N: with G = 4 query heads per KV head,
// 12 of the 16 columns are padding.  This kernel does the same work on the
// vector ALU instead, for G <= 4, bf16 K/V, page sizes that are multiples of
// 16 and head dims 64 or 128, so that the two inner loops can be timed on the
// same shapes.  It keeps no tile in LDS:
//
//  * K and V rows are loaded in row order, 16 bytes per lane: a row of D
//    bf16 values is CPR = D / 8 lanes, one load instruction covers RPI =
//    64 / CPR rows, and a wave's 16-token tile is NL = 16 / RPI instructions
//    for K and as many for V.  Lane (row group r, column c) holds dims
//    8c .. 8c + 7 of tokens RPI * i + r, i < NL, of every tile.
//  * QK: v_dot2 of bf16 pairs of q and K over the lane's 8 dims, then a sum
//    across the CPR lanes of the row with DPP adds (quad swaps, half-row and
//    row mirrors).  Every lane of the row then holds the token's score.
//  * Each row group keeps its own online softmax (running max, sum and output
//    rows) over the tokens it sees, so no reduction across row groups is needed
//    per tile; the weights are rounded to bf16 for PV, as the matrix-core path
//    rounds its P operand.
//  * PV: v_dot2 over token pairs: the V values of tokens i and i + 1 for one
//    dim are paired with v_perm, and the two weights packed to bf16.
//  * At the end the row groups of the four waves are combined in LDS.
//
// One workgroup of four waves per (KV head, sequence); wave w takes tiles
// w, w + 4, ..., with the next tile's loads in flight while one is processed.
#include "../../include/pkd_valu.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>
#include <cmath>

#include "pkd_internal.hpp"

namespace pkd {
namespace {

typedef __bf16 vbf16x2 __attribute__((ext_vector_type(2)));
typedef float vf32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t vu32x4 __attribute__((ext_vector_type(4)));

struct ValuParams {
  const uint16_t* q;           // [B][Hq][D] bf16
  const uint8_t* k;            // [P][ps][Hkv][D] bf16
  const uint8_t* v;
  const int32_t* block_table;  // [B][max_pages]
  const int32_t* seq_lens;     // [B]
  uint16_t* out;               // [B][Hq][D] bf16
  float* lse;                  // [B][Hq] or null
  float qk_scale_log2;
  int32_t hq, hkv, page_size, max_pages;
  int32_t tok_stride;          // bytes between slots of a page: Hkv * D * 2
  int64_t page_stride;         // bytes between pages
};

constexpr int kValuWaves = 4;
constexpr int kValuBtEntries = 512;  // block-table entries staged in LDS

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(vbf16x2, a), __builtin_bit_cast(vbf16x2, b), c, false);
}

// x + x of the lane whose index differs in the bits the DPP control selects.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF,
                                                                   false));
}

// Sum over the CPR lanes of a row (aligned groups of 8 or 16 lanes).
template <int CPR>
__device__ __forceinline__ float row_sum(float x) {
  x = dpp_add<0xB1>(x);   // quad_perm [1,0,3,2]
  x = dpp_add<0x4E>(x);   // quad_perm [2,3,0,1]
  x = dpp_add<0x141>(x);  // row_half_mirror: the two quads of each half row
  if constexpr (CPR == 16) x = dpp_add<0x140>(x);  // row_mirror: the two half rows
  return x;
}

template <int D, int G>
struct ValuCfg {
  static constexpr int CPR = D * 2 / 16;  // lanes per row
  static constexpr int RPI = 64 / CPR;    // rows per load instruction
  static constexpr int NL = 16 / RPI;     // load instructions per 16-token tile (each of K and V)
  static constexpr int NP = kValuWaves * RPI;  // independent softmax streams of a workgroup
  static_assert(NL % 2 == 0, "PV pairs tokens");
};

template <int D, int G>
struct ValuTile {
  vu32x4 k[ValuCfg<D, G>::NL];
  vu32x4 v[ValuCfg<D, G>::NL];
};

template <int D, int G>
__global__ void __launch_bounds__(kValuWaves * 64) valu_direct_kernel(const ValuParams p) {
  typedef ValuCfg<D, G> C;
  constexpr int NL = C::NL, RPI = C::RPI, CPR = C::CPR, NP = C::NP;
  __shared__ int32_t sbt[kValuBtEntries];
  __shared__ float s_acc[NP][G][D];
  __shared__ float s_m[NP][G], s_l[NP][G];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane / CPR, c = lane % CPR;
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int L = p.seq_lens[b];
  const int ps = p.page_size;
  const int ntiles = (L + 15) / 16;
  const int n_pages = (L + ps - 1) / ps;
  const int32_t* bt = p.block_table + (int64_t)b * p.max_pages;
  const bool staged = n_pages <= kValuBtEntries;
  if (staged)
    for (int i = tid; i < n_pages; i += kValuWaves * 64) sbt[i] = bt[i];

  // This lane's 8 dims of each of the G query rows, as bf16 pairs.
  vu32x4 qv[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qv[h] = *reinterpret_cast<const vu32x4*>(p.q + ((int64_t)b * p.hq + kvh * G + h) * D + c * 8);
  __syncthreads();

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  const int64_t head_off = (int64_t)kvh * D * 2 + c * 16;
  auto issue = [&](int t, ValuTile<D, G>& T) {
    const int t0 = t * 16;
    const int page = __builtin_amdgcn_readfirstlane(staged ? sbt[t0 / ps] : bt[t0 / ps]);
    const int64_t base = (int64_t)page * p.page_stride + head_off;
    const int slot0 = t0 % ps;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int tok = min(t0 + i * RPI + r, L - 1);  // rows past the sequence reload its last row
      const int64_t off = base + (int64_t)(slot0 + tok - t0) * p.tok_stride;
      T.k[i] = __builtin_nontemporal_load(reinterpret_cast<const vu32x4*>(p.k + off));
      T.v[i] = __builtin_nontemporal_load(reinterpret_cast<const vu32x4*>(p.v + off));
    }
  };
  auto process = [&](int t, const ValuTile<D, G>& T) {
    const int t0 = t * 16;
    float s[G][NL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        float x = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) x = dot2(qv[h][j], T.k[i][j], x);
        x = row_sum<CPR>(x) * p.qk_scale_log2;
        s[h][i] = t0 + i * RPI + r < L ? x : -INFINITY;
      }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = s[h][0];
#pragma unroll
      for (int i = 1; i < NL; ++i) mx = fmaxf(mx, s[h][i]);
      const float m_new = fmaxf(m[h], mx);
      if (m_new == -INFINITY) continue;  // nothing seen yet by this row group
      const float alpha = __builtin_amdgcn_exp2f(m[h] - m_new);
      m[h] = m_new;
      float pr[NL];
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        pr[i] = __builtin_amdgcn_exp2f(s[h][i] - m_new);
        sum += pr[i];
      }
      l[h] = l[h] * alpha + sum;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int i = 0; i < NL; i += 2) {
        const uint32_t pp = __builtin_bit_cast(uint32_t, __builtin_convertvector((vf32x2){pr[i], pr[i + 1]}, vbf16x2));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // (V[i][2j], V[i+1][2j]) and (V[i][2j+1], V[i+1][2j+1])
          const uint32_t lo = __builtin_amdgcn_perm(T.v[i + 1][j], T.v[i][j], 0x05040100u);
          const uint32_t hi = __builtin_amdgcn_perm(T.v[i + 1][j], T.v[i][j], 0x07060302u);
          acc[h][2 * j] = dot2(pp, lo, acc[h][2 * j]);
          acc[h][2 * j + 1] = dot2(pp, hi, acc[h][2 * j + 1]);
        }
      }
    }
  };

  // Tiles wave, wave + 4, ...: the next tile's loads are in flight while one is processed.
  if (wave < ntiles) {
    ValuTile<D, G> ta, tb;
    int t = wave;
    issue(t, ta);
    while (true) {
      const int t1 = t + kValuWaves;
      if (t1 < ntiles) issue(t1, tb);
      process(t, ta);
      if (t1 >= ntiles) break;
      const int t2 = t1 + kValuWaves;
      if (t2 < ntiles) issue(t2, ta);
      process(t1, tb);
      if (t2 >= ntiles) break;
      t = t2;
    }
  }

  // Combine the NP streams (row groups of the waves).
  const int part = wave * RPI + r;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (c == 0) {
      s_m[part][h] = m[h];
      s_l[part][h] = l[h];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s_acc[part][h][c * 8 + e] = acc[h][e];
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kValuWaves * 64) {
    const int h = idx / D, d = idx - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < NP; ++q) M = fmaxf(M, s_m[q][h]);
    float den = 0.f, o = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        const float w = __builtin_amdgcn_exp2f(s_m[q][h] - M);  // 0 for a stream that saw nothing
        den += w * s_l[q][h];
        o += w * s_acc[q][h][d];
      }
    }
    const int64_t row = (int64_t)b * p.hq + kvh * G + h;
    const __bf16 hv = (__bf16)(den > 0.f ? o / den : 0.f);
    p.out[row * D + d] = __builtin_bit_cast(uint16_t, hv);
    if (d == 0 && p.lse) p.lse[row] = den > 0.f ? (M + __builtin_log2f(den)) * 0.69314718055994530942f : -INFINITY;
  }
}

template <int D, int G>
void launch_valu(const ValuParams& p, int batch, hipStream_t s) {
  hipLaunchKernelGGL((valu_direct_kernel<D, G>), dim3(p.hkv, batch), dim3(kValuWaves * 64), 0, s, p);
}

}  // namespace
}  // namespace pkd

extern "C" {

int32_t pkd_decode_valu(const pkd_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_table, const int32_t* seq_lens, float scale, void* out, float* lse,
                        void* stream) {
  if (!dims) return PKD_ERR_NULL_POINTER;
  const pkd_dims& d = *dims;
  if (d.batch < 0 || d.num_q_heads < 1 || d.num_kv_heads < 1 || d.page_size < 1 || d.num_pages < 1 ||
      d.max_pages_per_seq < 1 || d.batch > 65535 || d.num_kv_heads > 65535)
    return PKD_ERR_BAD_DIMS;
  if (d.num_q_heads % d.num_kv_heads != 0) return PKD_ERR_GQA;
  const int G = d.num_q_heads / d.num_kv_heads;
  if (d.head_dim != 64 && d.head_dim != 128) return PKD_ERR_HEAD_DIM;
  if (d.kv_dtype != PKD_DTYPE_BF16) return PKD_ERR_DTYPE;
  if ((G != 1 && G != 2 && G != 4) || d.page_size % 16 != 0) return PKD_ERR_BAD_DIMS;
  if ((int64_t)d.max_pages_per_seq * d.page_size > INT32_MAX) return PKD_ERR_BAD_DIMS;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out) return PKD_ERR_NULL_POINTER;
  if (!std::isfinite(scale)) return PKD_ERR_BAD_DIMS;
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out) & 15) return PKD_ERR_ALIGNMENT;
  if (((uintptr_t)block_table | (uintptr_t)seq_lens | (uintptr_t)lse) & 3) return PKD_ERR_ALIGNMENT;
  if (d.batch == 0) return PKD_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PKD_ERR_DEVICE;
  pkd::ValuParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint8_t*>(k_cache);
  p.v = static_cast<const uint8_t*>(v_cache);
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.qk_scale_log2 = scale * 1.44269504088896340736f;
  p.hq = d.num_q_heads;
  p.hkv = d.num_kv_heads;
  p.page_size = d.page_size;
  p.max_pages = d.max_pages_per_seq;
  p.tok_stride = d.num_kv_heads * d.head_dim * 2;
  p.page_stride = (int64_t)d.page_size * p.tok_stride;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d.head_dim == 128) {
    if (G == 4) pkd::launch_valu<128, 4>(p, d.batch, s);
    else if (G == 2) pkd::launch_valu<128, 2>(p, d.batch, s);
    else pkd::launch_valu<128, 1>(p, d.batch, s);
  } else {
    if (G == 4) pkd::launch_valu<64, 4>(p, d.batch, s);
    else if (G == 2) pkd::launch_valu<64, 2>(p, d.batch, s);
    else pkd::launch_valu<64, 1>(p, d.batch, s);
  }
  return hipGetLastError() == hipSuccess ? PKD_OK : PKD_ERR_LAUNCH;
}

}  // extern "C"
