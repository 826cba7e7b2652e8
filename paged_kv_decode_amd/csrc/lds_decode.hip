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
//    (l % 16) ^ swz(r): chunk c of row r sits in slot c ^ swz(r).  swz gives
//    16 distinct values on 16 consecutive rows (the K operand reads 16 rows) and
//    distinct slot pairs on each 4 consecutive rows (a transposing V read
//    takes 32 bytes of 4 rows per 16 lanes).
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

// Slot permutation of a tile row (see the header comment).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8); }

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// LDS byte address of a pointer into this workgroup's shared memory.
__device__ __forceinline__ uint32_t lds_address(uint8_t* p) { return (uint32_t)(uintptr_t)(lds_u8*)p; }

// One direct-to-LDS load: 16 bytes from src (per lane) to LDS lds + 16 * lane.
// The LDS address goes to M0 through the operand constraint (the compiler
// writes M0 itself); one wait state separates that write from the load.
__device__ __forceinline__ void load_to_lds(const uint8_t* src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(src), "{m0}"(lds) : "memory");
}

// Wait until at most N direct-to-LDS loads of this wave are outstanding (they
// complete in issue order).
template <int N>
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory"); }
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

__global__ void __launch_bounds__(kLW * 64) lds_direct_kernel(const SplitParams p) {
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
  const int L = p.seq_lens[b];
  __shared__ int64_t s_rows[kHeadsPerGroup];
  if (tid < kHeadsPerGroup) s_rows[tid] = (int64_t)b * p.hq + kvh * G + tid;
  __syncthreads();

  const int ntiles = (L + kLT - 1) / kLT;
  const int lim = L - 1;
  // This lane's part of every load instruction: instruction i covers tile rows
  // 4i .. 4i + 3; the lane fetches row 4i + lane / 16, chunk (lane % 16) ^ swz(row).
  int drow[4], dchunk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    drow[i] = 4 * i + (lane >> 4);
    dchunk[i] = ((lane & 15) ^ swz(drow[i])) * 16;
  }
  uint8_t* wbase = smem + wave * kWaveB;
  const uint32_t wlds = __builtin_amdgcn_readfirstlane(lds_address(wbase));
  const int64_t head_off = (int64_t)kvh * kRowB;
  const int ps = p.page_size;

  auto issue = [&](int t, int stage) {
    const int tb = t * kLT;
    const int page = __builtin_amdgcn_readfirstlane(sbt[tb / ps]);
    const int64_t base = (int64_t)page * p.kv.page_stride + (int64_t)(tb % ps) * p.kv.tok_stride + head_off;
    const int rl = lim - tb;  // last row of the tile inside the sequence; later rows re-read it
    int64_t off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) off[i] = base + (int64_t)min(drow[i], rl) * p.kv.tok_stride + dchunk[i];
    const uint32_t lk = wlds + stage * kStageB;
#pragma unroll
    for (int i = 0; i < kLoadsPerHalf; ++i) load_to_lds(p.k + off[i], lk + i * 1024);
#pragma unroll
    for (int i = 0; i < kLoadsPerHalf; ++i) load_to_lds(p.v + off[i], lk + kTileB + i * 1024);
  };
  // Loads issued after a tile's K half: its V half and the later tiles.
  constexpr int kAfterK = kLoadsPerHalf + (kLS - 1) * 2 * kLoadsPerHalf;
  constexpr int kAfterV = (kLS - 1) * 2 * kLoadsPerHalf;

  // One tile from LDS stage `stage`: QK^T, the softmax against the reference
  // maximum, PV.  The arithmetic is the grid kernel's (WaveAttn::process) step
  // for step; only the LDS addresses differ.
  auto compute = [&](int t, int stage) {
    const uint8_t* kt = wbase + stage * kStageB;
    const uint8_t* vt = kt + kTileB;
    const int tb = t * kLT;
    wait_loads<kAfterK>();  // the tile's K has landed (its V may still be in flight)
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < WA::C::KK; ++kk) {
      // row n, dims kk * 32 + g * 8 .. + 8: chunk 4 kk + g
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + A.n * kRowB + (((4 * kk + A.g) ^ swz(A.n)) << 4));
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
    // lane (n, g) addresses row 4g + n/4, dims 16 nb + 4 (n % 4) .. + 3: chunk
    // 2 nb + (n / 2) % 2, bytes 8 (n % 2) .. of it.
    const int vr = 4 * A.g + (A.n >> 2);
    const uint8_t* vrow = vt + vr * kRowB + ((A.n & 1) << 3);
    const int vsw = swz(vr);
    const int vhalf = (A.n >> 1) & 1;
    wait_loads<kAfterV>();  // and its V
#pragma unroll
    for (int nb = 0; nb < WA::C::NB; ++nb) {
      const s16x4 a = lds_read_tr16(reinterpret_cast<const uint16_t*>(vrow + (((2 * nb + vhalf) ^ vsw) << 4)));
      A.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pbs, A.acc[nb], 0, 0, 0);
    }
    wait_lds_reads();  // this stage's reads are done before it is refilled
  };

  // Tiles wave, wave + kLW, ...: kLS in flight, the oldest computed while the
  // others load.  After the last tile the refills repeat the newest tile
  // (rows already loaded) so that every wait sees the same count; they are
  // never read.
  if (wave < ntiles) {
    auto nxt = [&](int t) { return t + kLW < ntiles ? t + kLW : t; };
    int tl[kLS];  // the tiles in the stages, oldest first
    tl[0] = wave;
    issue(tl[0], 0);
#pragma unroll
    for (int i = 1; i < kLS; ++i) {
      tl[i] = nxt(tl[i - 1]);
      issue(tl[i], i);
    }
    int stage = 0;
    while (true) {
      compute(tl[0], stage);
      if (tl[1] == tl[0]) break;
      const int tn = nxt(tl[kLS - 1]);
      issue(tn, stage);
#pragma unroll
      for (int i = 0; i + 1 < kLS; ++i) tl[i] = tl[i + 1];
      tl[kLS - 1] = tn;
      stage = stage + 1 == kLS ? 0 : stage + 1;
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
