// Direct-output paged decode with K/V tiles loaded straight into LDS, for
// measurement beside the register-staged kernels (not called by any decode
// entry point).
//
// The grid kernel keeps its next tile's loads in flight in registers and
// writes each tile into LDS when it is processed.  Here each wave owns two LDS
// stages of one 16-token tile (4 KiB of K, then 4 KiB of V) and fills them
// with direct-to-LDS loads (global_load_lds_dwordx4: each lane's 16 bytes land
// in LDS at the instruction's base + 16 * lane, never in registers), so that
// the tile after the current one is in flight while the current one is
// computed from LDS: the two-stage shared-memory pipeline of the AstrAI commit
// log, on gfx950.
//
//  * Layout.  A load instruction covers 4 rows of 256 bytes (D = 128 bf16) and
//    writes 1 KiB of LDS in lane order, so a tile is row-major with no padding.
//    To keep the matrix-core operand reads free of bank conflicts, lane l of
//    the instruction covering row r fetches the row's 16-byte chunk
//    (l % 16) ^ swz(r): chunk c of row r sits in slot c ^ swz(r) (swz below
//    keeps the 16-row K operand reads and the 4- and 8-row transposing V reads
//    in distinct bank groups).  Each lane's read offsets inside a stage, and
//    its part of every load instruction, are computed once; a load then takes
//    the page's row address as a scalar base plus the lane's 32-bit offset.
//  * Waits.  The compiler's own bookkeeping would wait for every outstanding
//    direct-to-LDS load before any LDS read, which leaves one tile in flight.
//    The loads are therefore issued from inline assembly (the LDS address
//    passed in M0; they write no register), and the wave waits by count: with two
//    tiles issued (8 instructions each), vmcnt(8) means the older one has
//    landed.  No other vector-memory load is issued inside the tile loop (the
//    block table is staged in LDS first), so the count is exact.  Before a
//    stage is refilled the wave's LDS reads of it have completed (lgkmcnt(0)).
//  * The matrix-core steps, the reference-maximum softmax and the workgroup
//    combine are those of the grid kernel, so the results equal paged_decode's
//    with num_splits = 1 bit for bit.
#include "../../include/pkd_lds.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <type_traits>

#include "wave_attn.hpp"

namespace pkd {
namespace {


constexpr int kLD = 128;                   // head dim
constexpr int kLT = 16;                    // tokens per tile
constexpr int kLW = 4;                     // waves per workgroup
constexpr int kLS = 2;                     // LDS stages per wave (tiles in flight)
constexpr int kRowB = kLD * 2;             // bytes of one token's K (or V) row
constexpr int kTileB = kLT * kRowB;        // 4 KiB of K, as many of V
constexpr int kStageB = 2 * kTileB;        // one stage: K tile, then V tile
constexpr int kWaveB = kLS * kStageB;      // this wave's stages
constexpr int kBtOff = kLW * kWaveB;       // staged block-table entries after the stages
constexpr int kBtEntries = 512;
constexpr int kLdsBytes = kBtOff + kBtEntries * 4;
constexpr int kLoadsPerHalf = kTileB / 1024;  // load instructions per K (or V) tile
// The workgroup combine's staging (per-wave rows and weights) reuses the stages.
static_assert(kLW * 16 * (2 + Cfg<kLD, false>::OW_STRIDE) * 4 + 16 * (kLW + 4) * 4 <= kBtOff, "combine staging");

// Slot permutation of tile row r (see the header comment): for s = r % 8,
// 2s on s < 4 and 2s + 1 on s >= 4, then XOR 8 on rows 8 .. 15.  The 16 rows
// take 16 distinct values and any 8 consecutive rows distinct values modulo 8,
// so a K operand read (16 rows, one chunk) finds every row's chunk in another
// bank group whether the LDS serves 8 or 16 lanes of 16 bytes per pass; and
// slot >> 1 is distinct on any 8 consecutive rows, so the 32-byte pieces of a
// transposing V read land in distinct bank groups for 4 and for 8 rows.
__device__ __forceinline__ int swz(int r) {
  const int s = r & 7;
  return ((s << 1) + (s >> 2)) ^ (r & 8);
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// LDS byte address of a pointer into this workgroup's shared memory.
__device__ __forceinline__ uint32_t lds_address(uint8_t* p) { return (uint32_t)(uintptr_t)(lds_u8*)p; }

// One direct-to-LDS load: 16 bytes from base + off (base wave-uniform, off per
// lane) to LDS lds + 16 * lane.  The LDS address goes to M0 through the operand
// constraint (the compiler writes M0 itself); one wait state separates that
// write from the load.
__device__ __forceinline__ void load_to_lds(const uint8_t* base, uint32_t off, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(off), "s"(base), "{m0}"(lds) : "memory");
}

// Wait until at most N direct-to-LDS loads of this wave are outstanding (they
// complete in issue order).
template <int N>
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory"); }
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

// Two waves per SIMD as the register budget (as the grid kernel): the
// accumulators then stay in ordinary VGPRs, where the rescale reaches them.
__global__ void __launch_bounds__(kLW * 64) __attribute__((amdgpu_waves_per_eu(2)))
lds_direct_kernel(const SplitParams p) {
  typedef WaveAttn<kLD, false> WA;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kvh = blockIdx.x;
  const int b = blockIdx.y;
  const int G = p.group;
  WA A;
  A.init_lane(lane);

  // Issued while the length is in flight: the block-table row (every entry of
  // the sequence's row) and the query rows.
  int32_t* sbt = reinterpret_cast<int32_t*>(smem + kBtOff);
  for (int i = tid; i < p.max_pages; i += kLW * 64) sbt[i] = p.block_table[(int64_t)b * p.max_pages + i];
  const bool hv = A.n < G;
  const int64_t row_n = (int64_t)b * p.hq + kvh * G + (hv ? A.n : 0);
  A.load_q(p.q + row_n * kLD, hv);
  A.qk_scale = p.qk_scale_log2;
  A.reset();
  const int L = __builtin_amdgcn_readfirstlane(p.seq_lens[b]);  // uniform: tile bookkeeping stays scalar
  __shared__ int64_t s_rows[kHeadsPerGroup];
  if (tid < kHeadsPerGroup) s_rows[tid] = (int64_t)b * p.hq + kvh * G + tid;
  __syncthreads();

  const int ntiles = (L + kLT - 1) / kLT;
  const int lim = L - 1;
  const int ps = p.page_size;
  const int ts = p.kv.tok_stride;
  // This lane's part of every load instruction: instruction i covers tile rows
  // 4i .. 4i + 3; the lane fetches row 4i + lane / 16, chunk (lane % 16) ^
  // swz(row), at byte loff[i] of the tile's first row (32-bit: a 16-token group
  // lies in one page).
  int drow[kLoadsPerHalf];
  uint32_t dchunk[kLoadsPerHalf], loff[kLoadsPerHalf];
#pragma unroll
  for (int i = 0; i < kLoadsPerHalf; ++i) {
    drow[i] = 4 * i + (lane >> 4);
    dchunk[i] = (uint32_t)(kvh * kRowB + (((lane & 15) ^ swz(drow[i])) << 4));
    loff[i] = (uint32_t)(drow[i] * ts) + dchunk[i];
  }
  // This lane's LDS read offsets inside a stage: K row n, chunk 4 kk + g; V row
  // 4g + n / 4, chunk 2 nb + (n / 2) % 2, bytes 8 (n % 2) ..
  const int wofs = wave * kWaveB;
  int kofs[WA::C::KK], vofs[WA::C::NB];
#pragma unroll
  for (int kk = 0; kk < WA::C::KK; ++kk) kofs[kk] = wofs + A.n * kRowB + (((4 * kk + A.g) ^ swz(A.n)) << 4);
  {
    const int vr = 4 * A.g + (A.n >> 2);
#pragma unroll
    for (int nb = 0; nb < WA::C::NB; ++nb)
      vofs[nb] = wofs + kTileB + vr * kRowB + (((2 * nb + ((A.n >> 1) & 1)) ^ swz(vr)) << 4) + ((A.n & 1) << 3);
  }
  const uint32_t wlds = __builtin_amdgcn_readfirstlane(lds_address(smem)) + wofs;

  auto issue = [&](int t, auto stage_c) {
    constexpr int ST = decltype(stage_c)::value;
    const int tb = t * kLT;
    const int page = __builtin_amdgcn_readfirstlane(sbt[tb / ps]);
    const int64_t row0 = (int64_t)page * p.kv.page_stride + (int64_t)(tb % ps) * ts;
    const uint8_t* kb = p.k + row0;
    const uint8_t* vb = p.v + row0;
    const uint32_t lk = wlds + ST * kStageB;
    const int rl = lim - tb;  // last row of the tile inside the sequence; later rows re-read it
    if (rl >= kLT - 1) {
#pragma unroll
      for (int i = 0; i < kLoadsPerHalf; ++i) load_to_lds(kb, loff[i], lk + i * 1024);
#pragma unroll
      for (int i = 0; i < kLoadsPerHalf; ++i) load_to_lds(vb, loff[i], lk + kTileB + i * 1024);
    } else {
      uint32_t o[kLoadsPerHalf];
#pragma unroll
      for (int i = 0; i < kLoadsPerHalf; ++i) o[i] = (uint32_t)(min(drow[i], rl) * ts) + dchunk[i];
#pragma unroll
      for (int i = 0; i < kLoadsPerHalf; ++i) load_to_lds(kb, o[i], lk + i * 1024);
#pragma unroll
      for (int i = 0; i < kLoadsPerHalf; ++i) load_to_lds(vb, o[i], lk + kTileB + i * 1024);
    }
  };
  // Loads issued after a tile's K half: its V half and the next tile.
  constexpr int kAfterK = 3 * kLoadsPerHalf;
  constexpr int kAfterV = 2 * kLoadsPerHalf;

  // One tile from LDS stage ST: QK^T, the softmax against the reference
  // maximum, PV.  The arithmetic is the grid kernel's (WaveAttn::process) step
  // for step; only the LDS addresses differ.
  auto compute = [&](int t, auto stage_c) {
    constexpr int ST = decltype(stage_c)::value;
    const int tb = t * kLT;
    wait_loads<kAfterK>();  // the tile's K has landed (its V may still be in flight)
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < WA::C::KK; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(smem + kofs[kk] + ST * kStageB);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, A.qf[kk], s, 0, 0, 0);
    }
    float mt = -INFINITY;
    if (tb + kLT <= L) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] *= A.qk_scale;
        mt = fmaxf(mt, s[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = tb + 4 * A.g + i;
        const float x = s[i] * A.qk_scale;
        s[i] = tok < L ? x : -INFINITY;
        mt = fmaxf(mt, s[i]);
      }
    }
    if (__builtin_amdgcn_ballot_w64(mt > A.m_run + kRescaleSlack) != 0) {
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = mt > A.m_run + kRescaleSlack ? mt : A.m_run;
      const float alpha = __builtin_amdgcn_exp2f(A.m_run - (m_new == -INFINITY ? 0.f : m_new));
      A.m_run = m_new;
      A.l_run *= alpha;
#pragma unroll
      for (int nb = 0; nb < WA::C::NB; ++nb) A.acc[nb] *= alpha;
    }
    const float m_use = A.m_run == -INFINITY ? 0.f : A.m_run;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = __builtin_amdgcn_exp2f(s[i] - m_use);
      s[i] = e;
      psum += e;
    }
    A.l_run += psum;
    bf16x4 pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) pb[i] = (__bf16)s[i];
    const s16x4 pbs = bit_cast_dev<s16x4>(pb);
    wait_loads<kAfterV>();  // and its V
#pragma unroll
    for (int nb = 0; nb < WA::C::NB; ++nb) {
      const s16x4 a = lds_read_tr16(reinterpret_cast<const uint16_t*>(smem + vofs[nb] + ST * kStageB));
      A.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pbs, A.acc[nb], 0, 0, 0);
    }
    wait_lds_reads();  // this stage's reads are done before it is refilled
  };

  // Tiles wave, wave + kLW, ...: two in flight, the older one computed while
  // the newer one loads.  After the last tile the refill repeats the newer tile
  // (rows already loaded) so that every wait sees the same count; it is never
  // read.
  if (wave < ntiles) {
    typedef std::integral_constant<int, 0> S0;
    typedef std::integral_constant<int, 1> S1;
    auto nxt = [&](int t) { return t + kLW < ntiles ? t + kLW : t; };
    int t = wave;
    issue(t, S0());
    int t1 = nxt(t);
    issue(t1, S1());
    while (true) {
      compute(t, S0());
      if (t1 == t) break;
      int t2 = nxt(t1);
      issue(t2, S0());
      t = t1;
      t1 = t2;
      compute(t, S1());
      if (t1 == t) break;
      t2 = nxt(t1);
      issue(t2, S1());
      t = t1;
      t1 = t2;
    }
  }
  wait_loads<0>();  // the combine below reuses the stages

  auto store = [&](int hh, int d0, f32x4 o, float lse_nat) {
    const int64_t row = s_rows[hh];
    *reinterpret_cast<bf16x4*>(p.out + row * kLD + d0) = to_bf16x4(o);
    if (d0 == 0 && p.lse) p.lse[row] = lse_nat;
  };
  wg_combine<kLD, false, kLW>(A, smem, wave, tid, G, 1.0f, store, NoSink());
}

}  // namespace

bool lds_direct_applies(int head_dim, bool fp8, int q_len, int window, bool sinks, int group, int page_size,
                        int max_pages, bool strided) {
  return head_dim == kLD && !fp8 && q_len == 1 && window == 0 && !sinks && group >= 1 && group <= kHeadsPerGroup &&
         page_size % 16 == 0 && max_pages >= 1 && max_pages <= kBtEntries && !strided;
}

hipError_t launch_lds_direct(const SplitParams& p, int batch, hipStream_t stream) {
  hipLaunchKernelGGL(lds_direct_kernel, dim3(p.hkv, batch), dim3(kLW * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkd

extern "C" {

int32_t pkd_decode_lds(const pkd_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, const int32_t* seq_lens, float scale, void* out, float* lse,
                       void* stream) {
  if (!dims) return PKD_ERR_NULL_POINTER;
  const pkd_dims& d = *dims;
  if (d.batch < 0 || d.num_q_heads < 1 || d.num_kv_heads < 1 || d.page_size < 1 || d.num_pages < 1 ||
      d.max_pages_per_seq < 1 || d.batch > 65535 || d.num_kv_heads > 65535)
    return PKD_ERR_BAD_DIMS;
  if (d.num_q_heads % d.num_kv_heads != 0) return PKD_ERR_GQA;
  const int G = d.num_q_heads / d.num_kv_heads;
  if (d.head_dim != 128) return PKD_ERR_HEAD_DIM;
  if (d.kv_dtype != PKD_DTYPE_BF16) return PKD_ERR_DTYPE;
  if (!pkd::lds_direct_applies(d.head_dim, false, 1, 0, false, G, d.page_size, d.max_pages_per_seq, false))
    return PKD_ERR_BAD_DIMS;
  if ((int64_t)d.num_kv_heads * 256 * d.page_size > INT32_MAX) return PKD_ERR_BAD_DIMS;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out) return PKD_ERR_NULL_POINTER;
  if (!std::isfinite(scale)) return PKD_ERR_BAD_DIMS;
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out) & 15) return PKD_ERR_ALIGNMENT;
  if (((uintptr_t)block_table | (uintptr_t)seq_lens | (uintptr_t)lse) & 3) return PKD_ERR_ALIGNMENT;
  if (d.batch == 0) return PKD_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PKD_ERR_DEVICE;
  pkd::SplitParams p{};
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
  p.group = G;
  p.q_len = 1;
  p.page_size = d.page_size;
  p.max_pages = d.max_pages_per_seq;
  p.kv.head_stride = 256;
  p.kv.tok_stride = d.num_kv_heads * 256;
  p.kv.page_stride = (int64_t)d.page_size * p.kv.tok_stride;
  return pkd::launch_lds_direct(p, d.batch, static_cast<hipStream_t>(stream)) == hipSuccess ? PKD_OK
                                                                                            : PKD_ERR_LAUNCH;
}

}  // extern "C"
