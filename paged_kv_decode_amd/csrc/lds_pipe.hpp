// The LDS-staged tile pipeline for bf16 K/V with head_dim 128: each wave owns
// two LDS stages of one 16-token tile (4 KiB of K, then 4 KiB of V) and fills
// them with direct-to-LDS loads (global_load_lds_dwordx4: each lane's 16 bytes
// land in LDS at the instruction's base + 16 * lane, never in registers), so
// that the tile after the current one is in flight while the current one is
// computed from LDS: the two-stage shared-memory pipeline of the AstrAI commit
// log, on gfx950.  Used by the LDS-staged direct kernel (lds_decode.hip).
//
//  * Layout.  A load instruction covers 4 rows of 256 bytes and writes 1 KiB of
//    LDS in lane order, so a tile is row-major with no padding.  Lane l of the
//    instruction covering row r fetches the row's 16-byte chunk (l % 16) ^
//    swz(r): chunk c of row r sits in slot c ^ swz(r), which keeps the 16-row K
//    operand reads and the 4- and 8-row transposing V reads in distinct bank
//    groups.  Each lane's read offsets inside a stage, and its part of every
//    load instruction, are computed once; a load then takes the tile's first
//    row address (page, slot, KV head) as a scalar base plus the lane's 32-bit
//    offset.
//  * Waits.  The compiler's own bookkeeping would wait for every outstanding
//    direct-to-LDS load before any LDS read, which leaves one tile in flight.
//    The loads are therefore issued from inline assembly (the LDS address
//    passed in M0; they write no register), and the wave waits by count: with
//    two tiles issued (4 + 4 instructions each), vmcnt(12) means the older
//    tile's K has landed and vmcnt(8) its V.  Loads issued before a pipeline
//    starts complete first (loads complete in issue order), and no other
//    vector-memory load is issued while it runs, so the counts are exact.
//    Before a stage is refilled the wave's LDS reads of it have completed
//    (lgkmcnt(0)); after the last tile every load is waited for (vmcnt(0)), so
//    the caller may reuse the stages.
//  * The matrix-core steps and the reference-maximum softmax are those of
//    WaveAttn::process, step for step, so the results equal the register-staged
//    kernels' bit for bit.  There is no window: a lane masks the tokens at or
//    past its row's end (the range's end, or under the causal mask its query
//    token's position + 1), nothing below.
#pragma once

#include <type_traits>

#include "wave_attn.hpp"

namespace pkd {
namespace {

constexpr int kLpD = 128;                  // head dim
constexpr int kLpTT = 16;                  // tokens per tile
constexpr int kLpRowB = kLpD * 2;          // bytes of one token's K (or V) row of one head
constexpr int kLpTileB = kLpTT * kLpRowB;  // 4 KiB of K, as many of V
constexpr int kLpStageB = 2 * kLpTileB;    // one stage: K tile, then V tile
constexpr int kLpWaveB = 2 * kLpStageB;    // two stages per wave
constexpr int kLpLoads = kLpTileB / 1024;  // load instructions per K (or V) tile

// Slot permutation of tile row r: for s = r % 8, 2s on s < 4 and 2s + 1 on
// s >= 4, then XOR 8 on rows 8 .. 15.  The 16 rows take 16 distinct values and
// any 8 consecutive rows distinct values modulo 8, so a K operand read (16
// rows, one chunk) finds every row's chunk in another bank group whether the
// LDS serves 8 or 16 lanes of 16 bytes per pass; and slot >> 1 is distinct on
// any 8 consecutive rows, so the 32-byte pieces of a transposing V read land
// in distinct bank groups for 4 and for 8 rows.
__device__ __forceinline__ int lp_swz(int r) {
  const int s = r & 7;
  return ((s << 1) + (s >> 2)) ^ (r & 8);
}

typedef __attribute__((address_space(3))) uint8_t lp_lds_u8;

// LDS byte address of a pointer into this workgroup's shared memory.
__device__ __forceinline__ uint32_t lp_lds_address(uint8_t* p) { return (uint32_t)(uintptr_t)(lp_lds_u8*)p; }

// One direct-to-LDS load: 16 bytes from base + off (base wave-uniform, off per
// lane) to LDS lds + 16 * lane.  The LDS address goes to M0 through the operand
// constraint (the compiler writes M0 itself); one wait state separates that
// write from the load.
__device__ __forceinline__ void lp_load(const uint8_t* base, uint32_t off, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(off), "s"(base), "{m0}"(lds) : "memory");
}

// Wait until at most N direct-to-LDS loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void lp_wait_loads() { asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory"); }
__device__ __forceinline__ void lp_wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

struct LdsPipe {
  typedef WaveAttn<kLpD, false> WA;
  uint8_t* smem;                 // the workgroup's shared memory (its stages start at wofs)
  int drow[kLpLoads];            // tile row of this lane in load instruction i
  uint32_t dchunk[kLpLoads];     // byte of its chunk within the row
  uint32_t loff[kLpLoads];       // its offset from the tile's first row
  int kofs[WA::C::KK];           // its K operand read offsets (stage 0)
  int vofs[WA::C::NB];           // its V operand read offsets (stage 0)
  uint32_t wlds;                 // LDS address of this wave's stage 0
  int ts;                        // bytes between consecutive slots of a page

  // wofs: byte offset of this wave's two stages (kLpWaveB bytes) in smem.
  __device__ __forceinline__ void init(uint8_t* smem_, int wofs, const WA& A, int lane, int tok_stride) {
    smem = smem_;
    ts = tok_stride;
#pragma unroll
    for (int i = 0; i < kLpLoads; ++i) {
      drow[i] = 4 * i + (lane >> 4);
      dchunk[i] = (uint32_t)(((lane & 15) ^ lp_swz(drow[i])) << 4);
      loff[i] = (uint32_t)(drow[i] * ts) + dchunk[i];
    }
    // K row n, chunk 4 kk + g; V row 4g + n / 4, chunk 2 nb + (n / 2) % 2, bytes 8 (n % 2) ..
#pragma unroll
    for (int kk = 0; kk < WA::C::KK; ++kk) kofs[kk] = wofs + A.n * kLpRowB + (((4 * kk + A.g) ^ lp_swz(A.n)) << 4);
    const int vr = 4 * A.g + (A.n >> 2);
#pragma unroll
    for (int nb = 0; nb < WA::C::NB; ++nb)
      vofs[nb] = wofs + kLpTileB + vr * kLpRowB + (((2 * nb + ((A.n >> 1) & 1)) ^ lp_swz(vr)) << 4) + ((A.n & 1) << 3);
    wlds = __builtin_amdgcn_readfirstlane(lp_lds_address(smem)) + wofs;
  }

  // Loads of the tile whose first row is at kb / vb (uniform), rows past rl
  // re-reading row rl, into stage ST.
  template <int ST>
  __device__ __forceinline__ void issue(const uint8_t* kb, const uint8_t* vb, int rl) const {
    const uint32_t lk = wlds + ST * kLpStageB;
    if (rl >= kLpTT - 1) {
#pragma unroll
      for (int i = 0; i < kLpLoads; ++i) lp_load(kb, loff[i], lk + i * 1024);
#pragma unroll
      for (int i = 0; i < kLpLoads; ++i) lp_load(vb, loff[i], lk + kLpTileB + i * 1024);
    } else {
      uint32_t o[kLpLoads];
#pragma unroll
      for (int i = 0; i < kLpLoads; ++i) o[i] = (uint32_t)(min(drow[i], rl) * ts) + dchunk[i];
#pragma unroll
      for (int i = 0; i < kLpLoads; ++i) lp_load(kb, o[i], lk + i * 1024);
#pragma unroll
      for (int i = 0; i < kLpLoads; ++i) lp_load(vb, o[i], lk + kLpTileB + i * 1024);
    }
  }

  // The tile of tokens tb .. tb + 15 from stage ST: QK^T, the softmax against
  // the reference maximum, PV.  Tokens at or past end (this lane's row's end)
  // are masked; end_min (uniform) bounds every lane's end from below.
  template <int ST>
  __device__ __forceinline__ void compute(WA& A, int tb, int end, int end_min) const {
    lp_wait_loads<3 * kLpLoads>();  // the tile's K has landed (its V may still be in flight)
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < WA::C::KK; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(smem + kofs[kk] + ST * kLpStageB);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, A.qf[kk], s, 0, 0, 0);
    }
    float mt = -INFINITY;
    if (tb + kLpTT <= end_min) {
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
        s[i] = tok < end ? x : -INFINITY;
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
    lp_wait_loads<2 * kLpLoads>();  // and its V
#pragma unroll
    for (int nb = 0; nb < WA::C::NB; ++nb) {
      const s16x4 a = lds_read_tr16(reinterpret_cast<const uint16_t*>(smem + vofs[nb] + ST * kLpStageB));
      A.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pbs, A.acc[nb], 0, 0, 0);
    }
    lp_wait_lds_reads();  // this stage's reads are done before it is refilled
  }

  // Tiles first, first + step, ... (< ntiles) of the token range [s0, s1)
  // (s0 a multiple of 16; the tiles' 16-token groups each lie in one page):
  // two in flight, the older computed while the newer loads.  row_of(tb)
  // gives the byte offset of token tb's row (page, slot and KV head) in the
  // caches, uniform.  end / end_min: as for compute.  After the last tile the
  // refill repeats the newer tile (rows already loaded) so that every wait sees
  // the same count; it is never read.  Returns with every load complete.
  template <typename RowOf>
  __device__ __forceinline__ void run(WA& A, int first, int step, int ntiles, int s0, int s1, int end, int end_min,
                                      const uint8_t* k, const uint8_t* v, RowOf row_of) const {
    if (first < ntiles) {
      const int lim = s1 - 1;
      auto nxt = [&](int t) { return t + step < ntiles ? t + step : t; };
      auto put = [&](int t, auto stage_c) {
        constexpr int ST = decltype(stage_c)::value;
        const int tb = s0 + t * kLpTT;
        const int64_t row0 = row_of(tb);
        issue<ST>(k + row0, v + row0, lim - tb);
      };
      typedef std::integral_constant<int, 0> S0;
      typedef std::integral_constant<int, 1> S1;
      int t = first;
      put(t, S0());
      int t1 = nxt(t);
      put(t1, S1());
      while (true) {
        compute<0>(A, s0 + t * kLpTT, end, end_min);
        if (t1 == t) break;
        int t2 = nxt(t1);
        put(t2, S0());
        t = t1;
        t1 = t2;
        compute<1>(A, s0 + t * kLpTT, end, end_min);
        if (t1 == t) break;
        t2 = nxt(t1);
        put(t2, S1());
        t = t1;
        t1 = t2;
      }
    }
    lp_wait_loads<0>();
  }
};

}  // namespace
}  // namespace pkd
