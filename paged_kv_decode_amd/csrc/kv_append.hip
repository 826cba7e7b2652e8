// Paged KV append for gfx950 (CDNA4): new K/V rows written into the paged
// cache, with optional rotate-half RoPE on K and FP8 E4M3FN quantisation.
//
// This is the write that precedes decode, which the sglang fuse/overlap
// catalogue lists as fused FP8 quantisation + paged K/V cache write and as RoPE
// fused with the KV cache store.  Token n's rows go to slot slot_mapping[n]
// (page * page_size + position in the page); padding tokens (slot < 0), slots
// past the pool and, with RoPE, positions outside the cos/sin table write
// nothing.  With RoPE, for d < D/2, c = cos_sin[pos][d], s = cos_sin[pos][D/2 + d]:
//     k'[d] = k[d] c - k[d + D/2] s,   k'[d + D/2] = k[d + D/2] c + k[d] s,
// each as an fp32 product followed by one fused multiply-add.  The stored value
// is k' rounded to bf16 (nearest even), or for an FP8 cache the code of
// clamp(k' / scale[h], -448, 448) (fp32 division, nearest code, ties to even).
//
// One thread per (token, KV head, 8-dim chunk of the first half): it handles
// dims 8j .. 8j + 7 and their rotate-half partners 8j + D/2 .., so the rotation
// needs no cross-lane exchange, and moves 16-byte words (8-byte FP8 codes).
// The work is HBM-bound: per token and KV head it reads 2 D bf16 values of K
// and V, writes 2 D cache elements, and with RoPE reads one D-float table row
// per token.
#include "pkd_internal.hpp"

namespace pkd {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void bf16x8_to_f32(u32x4 w, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// fp32 -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ u32x4 f32_to_bf16x8(const float (&y)[8]) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = bf16_bits(y[2 * i]) | (bf16_bits(y[2 * i + 1]) << 16);
  return w;
}

// Eight E4M3FN codes of clamp(y / scale, -448, 448).
__device__ __forceinline__ u32x2 f32_to_fp8x8(const float (&y)[8], float scale) {
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = fminf(fmaxf(__fdiv_rn(y[i], scale), -448.0f), 448.0f);
  u32x2 w;
  uint32_t a = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0u, false);
  w[0] = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], a, true);
  uint32_t b = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0u, false);
  w[1] = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], b, true);
  return w;
}

template <int D, bool FP8, bool ROPE>
__global__ void __launch_bounds__(256) kv_append_kernel(const AppendParams p) {
  constexpr int CH = D / 16;  // threads per (token, head) row
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = t / CH;  // (token, head)
  if (row >= p.num_tokens * p.hkv) return;
  const int j = (int)(t - row * CH);
  const int64_t n = row / p.hkv;
  const int h = (int)(row - n * p.hkv);
  const int64_t slot = p.slot_mapping[n];
  if (slot < 0 || slot >= p.capacity) return;
  int64_t pos = 0;
  if constexpr (ROPE) {
    pos = p.positions[n];
    if (pos < 0 || pos >= p.max_position) return;
  }
  const int64_t src = row * D + 8 * j;                 // element of dims 8j of token n, head h
  const int64_t dst = (slot * p.hkv + h) * D + 8 * j;  // page * ps + position, then head

  float x0[8], x1[8];
  bf16x8_to_f32(*reinterpret_cast<const u32x4*>(p.k_new + src), x0);
  bf16x8_to_f32(*reinterpret_cast<const u32x4*>(p.k_new + src + D / 2), x1);
  float y0[8], y1[8];
  if constexpr (ROPE) {
    const float* cs = p.cos_sin + pos * D + 8 * j;
    const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs), c1 = *reinterpret_cast<const f32x4*>(cs + 4);
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(cs + D / 2), s1 = *reinterpret_cast<const f32x4*>(cs + D / 2 + 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float c = i < 4 ? c0[i] : c1[i - 4], s = i < 4 ? s0[i] : s1[i - 4];
      y0[i] = fmaf(x0[i], c, -__fmul_rn(x1[i], s));
      y1[i] = fmaf(x1[i], c, __fmul_rn(x0[i], s));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      y0[i] = x0[i];
      y1[i] = x1[i];
    }
  }
  float v0[8], v1[8];
  bf16x8_to_f32(*reinterpret_cast<const u32x4*>(p.v_new + src), v0);
  bf16x8_to_f32(*reinterpret_cast<const u32x4*>(p.v_new + src + D / 2), v1);
  if constexpr (FP8) {
    uint8_t* kc = static_cast<uint8_t*>(p.k_cache);
    uint8_t* vc = static_cast<uint8_t*>(p.v_cache);
    const float ks = p.k_scale[h], vsc = p.v_scale[h];
    *reinterpret_cast<u32x2*>(kc + dst) = f32_to_fp8x8(y0, ks);
    *reinterpret_cast<u32x2*>(kc + dst + D / 2) = f32_to_fp8x8(y1, ks);
    *reinterpret_cast<u32x2*>(vc + dst) = f32_to_fp8x8(v0, vsc);
    *reinterpret_cast<u32x2*>(vc + dst + D / 2) = f32_to_fp8x8(v1, vsc);
  } else {
    uint16_t* kc = static_cast<uint16_t*>(p.k_cache);
    uint16_t* vc = static_cast<uint16_t*>(p.v_cache);
    *reinterpret_cast<u32x4*>(kc + dst) = f32_to_bf16x8(y0);
    *reinterpret_cast<u32x4*>(kc + dst + D / 2) = f32_to_bf16x8(y1);
    *reinterpret_cast<u32x4*>(vc + dst) = *reinterpret_cast<const u32x4*>(p.v_new + src);
    *reinterpret_cast<u32x4*>(vc + dst + D / 2) = *reinterpret_cast<const u32x4*>(p.v_new + src + D / 2);
  }
}

template <int D, bool FP8>
hipError_t launch_a(const AppendParams& p, hipStream_t s) {
  const int64_t threads = p.num_tokens * p.hkv * (D / 16);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (p.positions)
    hipLaunchKernelGGL((kv_append_kernel<D, FP8, true>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((kv_append_kernel<D, FP8, false>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_ad(const AppendParams& p, bool fp8, hipStream_t s) {
  return fp8 ? launch_a<D, true>(p, s) : launch_a<D, false>(p, s);
}

}  // namespace

hipError_t launch_kv_append(const AppendParams& p, int head_dim, bool fp8, hipStream_t stream) {
  if (p.num_tokens == 0) return hipSuccess;
  switch (head_dim) {
    case 32: return launch_ad<32>(p, fp8, stream);
    case 64: return launch_ad<64>(p, fp8, stream);
    case 128: return launch_ad<128>(p, fp8, stream);
    case 256: return launch_ad<256>(p, fp8, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkd
