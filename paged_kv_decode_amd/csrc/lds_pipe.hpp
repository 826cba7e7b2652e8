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
//    the next tile issued after the current one (4 + 4 instructions each),
//    vmcnt(12) means the current tile's K has landed and vmcnt(8) its V; with
//    none (the wave's last tile), vmcnt(4) and vmcnt(0).  Loads issued before
//    a pipeline starts complete first (loads complete in issue order), and no
//    other vector-memory load is issued while it runs, so the counts are
//    exact.
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

// lp_wait_loads<STEP * a + BASE>() for a runtime a in [0, MAXA] (uniform).
template <int STEP, int BASE, int MAXA>
__device__ __forceinline__ void lp_wait_loads_rt(int a) {
  if constexpr (MAXA == 0) {
    lp_wait_loads<BASE>();
  } else {
    if (a >= MAXA)
      lp_wait_loads<STEP * MAXA + BASE>();
    else
      lp_wait_loads_rt<STEP, BASE, MAXA - 1>(a);
  }
}

// Scores to weights, as WaveAttn::process does them, step for step: s[blk][i]
// (the raw dot products of token tok_of(blk, i)) is scaled and, unless
// `unmasked`, set to -inf at or past `end`; the reference maximum is raised
// (and l and O rescaled) when a row's tile maximum exceeds it by more than the
// slack; then s becomes 2^(s - m) and l takes the sum of the weights, added
// in the order blk, i.
template <int NBLK, typename WA, typename TokOf>
__device__ __forceinline__ void lp_softmax(WA& A, f32x4 (&s)[NBLK], bool unmasked, int end, TokOf tok_of) {
  float mt = -INFINITY;
  if (unmasked) {
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[blk][i] *= A.qk_scale;
        mt = fmaxf(mt, s[blk][i]);
      }
  } else {
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = s[blk][i] * A.qk_scale;
        s[blk][i] = tok_of(blk, i) < end ? x : -INFINITY;
        mt = fmaxf(mt, s[blk][i]);
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
  for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = __builtin_amdgcn_exp2f(s[blk][i] - m_use);
      s[blk][i] = e;
      psum += e;
    }
  A.l_run += psum;
}

struct LdsPipe {
  typedef WaveAttn<kLpD, false> WA;
  static constexpr int TT = kLpTT;
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
  // `ahead` (uniform, 0 or 1) tiles were issued after this one: its K has
  // landed at (2 ahead + 1) kLpLoads outstanding loads, its V at 2 ahead
  // kLpLoads.
  template <int ST>
  __device__ __forceinline__ void compute(WA& A, int tb, int end, int end_min, int ahead) const {
    lp_wait_loads_rt<2 * kLpLoads, kLpLoads, 1>(ahead);  // the tile's K has landed (its V may still be in flight)
    f32x4 s[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kk = 0; kk < WA::C::KK; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(smem + kofs[kk] + ST * kLpStageB);
      s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, A.qf[kk], s[0], 0, 0, 0);
    }
    lp_softmax(A, s, tb + kLpTT <= end_min, end, [&](int, int i) { return tb + 4 * A.g + i; });
    bf16x4 pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) pb[i] = (__bf16)s[0][i];
    const s16x4 pbs = bit_cast_dev<s16x4>(pb);
    lp_wait_loads_rt<2 * kLpLoads, 0, 1>(ahead);  // and its V
#pragma unroll
    for (int nb = 0; nb < WA::C::NB; ++nb) {
      const s16x4 a = lds_read_tr16(reinterpret_cast<const uint16_t*>(smem + vofs[nb] + ST * kLpStageB));
      A.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pbs, A.acc[nb], 0, 0, 0);
    }
    lp_wait_lds_reads();  // this stage's reads are done before it is refilled
  }

  // The tile of tokens tb .. tb + 15 into stage ST: row_of(tb) (uniform) is
  // the byte offset of its first row in the caches; rows past lim re-read
  // row lim.
  template <int ST, typename RowOf>
  __device__ __forceinline__ void put(const uint8_t* k, const uint8_t* v, int tb, int lim, RowOf row_of) const {
    const int64_t row0 = row_of(tb);
    issue<ST>(k + row0, v + row0, lim - tb);
  }

  template <typename RowOf>
  __device__ __forceinline__ void run(WA& A, int first, int step, int ntiles, int s0, int s1, int end, int end_min,
                                      const uint8_t* k, const uint8_t* v, RowOf row_of) const;
};

// ---- FP8 (E4M3) codes, head_dim 128 --------------------------------------
//
// The same pipeline over code tiles of 32 tokens (4 KiB of K codes, then 4 KiB
// of V codes, per stage).  A load instruction covers 8 rows of 128 bytes.  The
// codes are widened to bf16 after they are read from LDS, exactly as the
// register path widens them after loading: the K operand of row block blk is
// two 16-byte reads of its row (the dims q_dim0 gives the query), the V^T
// operand one transposing 8-byte read (ds_read_b64_tr_b8) of 8 rows per
// 16-dim block, and the matrix-core steps, softmax and PV order are those of
// WaveAttn::process for 32-token tiles, so the results equal the register
// path's bit for bit.  A tile's two 16-token groups may lie in different
// pages; each has its own base.
constexpr int kLfTT = 32;
constexpr int kLfRowB = kLpD;              // bytes of one token's K (or V) codes of one head
constexpr int kLfTileB = kLfTT * kLfRowB;  // 4 KiB
constexpr int kLfStageB = 2 * kLfTileB;
constexpr int kLfStages = 2;               // stages per wave
constexpr int kLfWaveB = kLfStages * kLfStageB;
constexpr int kLfLoads = kLfTileB / 1024;  // load instructions per K (or V) tile, 8 rows each

// Slot permutation of tile row r (0..31) on its 8 chunks of 16 bytes: chunk c
// sits in slot c ^ lf_swz(r), with lf_swz's three bits r1, r3 ^ r0 and
// r2 ^ r0 ^ r4.  A K operand read of row block blk (one chunk of rows
// 4 blk + {0..3, 8..11, 16..19, 24..27}, by lanes 0..15 of a lane group) and a
// transposing V read (one chunk of rows 8 g .. 8 g + 7, two lanes a row) then
// find their chunks in distinct 16-byte bank groups, whether the LDS serves
// 128 bytes per pass (8 lanes of 16 bytes, 16 of 8: the slot alone must
// differ) or 256 (16 lanes of 16 bytes, 32 of 8: slot and row parity).
__device__ __forceinline__ int lf_swz(int r) {
  return ((r >> 1) & 1) | ((((r >> 3) ^ r) & 1) << 1) | ((((r >> 2) ^ r ^ (r >> 4)) & 1) << 2);
}

typedef int lf_v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) lf_v2i lf_lds_v2i;

// Transposing byte read (ds_read_b64_tr_b8).  Within each group of 16 lanes,
// lane k addresses 8 bytes: if they are bytes 8 (k % 2) .. + 7 of row k / 2 of
// a row-major byte tile (two lanes a row), lane i receives byte column i of
// rows 0 .. 7, row r in byte r.
__device__ __forceinline__ u32x2 lds_read_tr8(const uint8_t* p) {
  const lf_v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lf_lds_v2i*)(p));
  return u32x2{(uint32_t)r[0], (uint32_t)r[1]};
}

struct LdsPipeF8 {
  typedef WaveAttn<kLpD, true> WA;
  static constexpr int TT = kLfTT;
  static_assert(WA::C::TT == kLfTT && WA::C::KP == 32 && WA::C::NBLK == 2 && WA::C::R == 2,
                "the register path's FP8 tile shape");
  uint8_t* smem;
  int rig[kLfLoads];          // row within its 16-row half of this lane in load instruction i (half i / 2)
  uint32_t dchunk[kLfLoads];  // byte of its chunk within the row
  uint32_t loff[kLfLoads];    // its offset from its half's first row
  int kofs[2][2];             // K operand reads (stage 0): row block, then dims 64 j + 16 g ..
  int vofs[WA::C::NB];        // V^T operand reads (stage 0)
  uint32_t wlds;
  int ts;

  __device__ __forceinline__ void init(uint8_t* smem_, int wofs, const WA& A, int lane, int tok_stride) {
    smem = smem_;
    ts = tok_stride;
#pragma unroll
    for (int i = 0; i < kLfLoads; ++i) {
      const int r = 8 * i + (lane >> 3);
      rig[i] = r & 15;
      dchunk[i] = (uint32_t)(((lane & 7) ^ lf_swz(r)) << 4);
      loff[i] = (uint32_t)(rig[i] * ts) + dchunk[i];
    }
    // K: row k_row_token(blk, n), chunk 4 j + g holds the dims of MFMAs 2 j and 2 j + 1.
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int r = k_row_token<32>(blk, A.n);
#pragma unroll
      for (int j = 0; j < 2; ++j) kofs[blk][j] = wofs + r * kLfRowB + (((4 * j + A.g) ^ lf_swz(r)) << 4);
    }
    // V: row 8 g + n / 2, chunk nb, bytes 8 (n % 2) ..
    const int vr = 8 * A.g + (A.n >> 1);
#pragma unroll
    for (int nb = 0; nb < WA::C::NB; ++nb)
      vofs[nb] = wofs + kLfTileB + vr * kLfRowB + ((nb ^ lf_swz(vr)) << 4) + ((A.n & 1) << 3);
    wlds = __builtin_amdgcn_readfirstlane(lp_lds_address(smem)) + wofs;
  }

  // The tile of tokens tb .. tb + 31 into stage ST: row_of(t) (uniform) is the
  // byte offset of token t's row; rows past lim are replaced by row lim's
  // group's rows up to lim (as the register path clamps them).
  template <int ST, typename RowOf>
  __device__ __forceinline__ void put(const uint8_t* k, const uint8_t* v, int tb, int lim, RowOf row_of) const {
    const uint32_t lk = wlds + ST * kLfStageB;
    if (tb + kLfTT - 1 <= lim) {
      const int64_t r0 = row_of(tb), r1 = row_of(tb + 16);
#pragma unroll
      for (int i = 0; i < kLfLoads; ++i) lp_load(k + (i < 2 ? r0 : r1), loff[i], lk + i * 1024);
#pragma unroll
      for (int i = 0; i < kLfLoads; ++i) lp_load(v + (i < 2 ? r0 : r1), loff[i], lk + kLfTileB + i * 1024);
    } else {
      const int g1 = min(tb + 16, lim) & ~15;  // the second half's group (the first's when it is past lim)
      const int64_t r0 = row_of(tb), r1 = row_of(g1);
      const int l0 = lim - tb, l1 = lim - g1;
      uint32_t o[kLfLoads];
#pragma unroll
      for (int i = 0; i < kLfLoads; ++i) o[i] = (uint32_t)(min(rig[i], i < 2 ? l0 : l1) * ts) + dchunk[i];
#pragma unroll
      for (int i = 0; i < kLfLoads; ++i) lp_load(k + (i < 2 ? r0 : r1), o[i], lk + i * 1024);
#pragma unroll
      for (int i = 0; i < kLfLoads; ++i) lp_load(v + (i < 2 ? r0 : r1), o[i], lk + kLfTileB + i * 1024);
    }
  }

  // The tile of tokens tb .. tb + 31 from stage ST (as LdsPipe::compute).
  // `ahead` tiles (uniform, 0 .. kLfStages - 1) were issued after it, 2
  // kLfLoads loads each: its K codes have landed at (2 ahead + 1) kLfLoads
  // outstanding loads, its V codes at 2 ahead kLfLoads.
  template <int ST>
  __device__ __forceinline__ void compute(WA& A, int tb, int end, int end_min, int ahead) const {
    lp_wait_loads_rt<2 * kLfLoads, kLfLoads, kLfStages - 1>(ahead);  // the tile's K codes have landed
    f32x4 s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      s[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(smem + kofs[blk][j] + ST * kLfStageB);
        s[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(u32x2{raw[0], raw[1]}), A.qf[2 * j], s[blk],
                                                          0, 0, 0);
        s[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(u32x2{raw[2], raw[3]}), A.qf[2 * j + 1],
                                                          s[blk], 0, 0, 0);
      }
    }
    lp_softmax(A, s, tb + kLfTT <= end_min, end,
               [&](int blk, int i) { return tb + s_out_token<32>(blk, A.g, i); });
    bf16x8 pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pb[i] = (__bf16)s[0][i];
      pb[4 + i] = (__bf16)s[1][i];
    }
    lp_wait_loads_rt<2 * kLfLoads, 0, kLfStages - 1>(ahead);  // and its V codes
#pragma unroll
    for (int nb = 0; nb < WA::C::NB; ++nb) {
      const bf16x8 a = fp8x8_to_bf16(lds_read_tr8(smem + vofs[nb] + ST * kLfStageB));
      A.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, A.acc[nb], 0, 0, 0);
    }
    lp_wait_lds_reads();
  }
};

// Stage S of an NS-stage round: f(stage) computes the tile in that stage and
// refills it; false ends the rounds.
template <int S, int NS, typename F>
__device__ __forceinline__ bool lp_stage_round(F& f) {
  if constexpr (S == NS) {
    return true;
  } else {
    if (!f(std::integral_constant<int, S>())) return false;
    return lp_stage_round<S + 1, NS>(f);
  }
}

// The loop of both pipelines: tiles first, first + step, ... (< ntiles) of the
// token range [s0, s1) (s0 a multiple of 16; every 16-token group lies in one
// page), with NS stages per wave, so that up to NS tiles are in flight and the
// oldest is computed while the newer ones load.  The stages are filled with
// the wave's first tiles (at most NS); then, stage by stage, a tile is
// computed and its stage refilled with the next tile not yet loaded, if there
// is one.  compute is told how many tiles were issued after the one it
// computes, which sets its wait counts.  row_of(t) gives the byte offset of
// token t's row (page, slot and KV head) in the caches, uniform, for t a
// multiple of 16.  end / end_min: as for compute.  Returns with every load
// complete.
template <int NS, typename Pipe, typename WA, typename RowOf>
__device__ __forceinline__ void lds_pipe_run_ns(const Pipe& P, WA& A, int first, int step, int ntiles, int s0,
                                                int s1, int end, int end_min, const uint8_t* k, const uint8_t* v,
                                                RowOf row_of) {
  constexpr int TT = Pipe::TT;
  if (first < ntiles) {
    const int lim = s1 - 1;
    auto nxt = [&](int t) { return t + step < ntiles ? t + step : t; };
    int newest = first;
    int ahead = 0;  // tiles issued after cur
    auto fill = [&](auto stage_c) {
      constexpr int ST = decltype(stage_c)::value;
      if constexpr (ST > 0) {
        const int n = nxt(newest);
        if (n == newest) return false;  // fewer tiles than stages
        newest = n;
        ++ahead;
      }
      P.template put<ST>(k, v, s0 + newest * TT, lim, row_of);
      return true;
    };
    lp_stage_round<0, NS>(fill);
    int cur = first;
    auto turn = [&](auto stage_c) {
      constexpr int ST = decltype(stage_c)::value;
      P.template compute<ST>(A, s0 + cur * TT, end, end_min, ahead);
      const int n2 = nxt(cur);
      if (n2 == cur) return false;  // that was the wave's last tile
      const int n = nxt(newest);
      if (n != newest) {
        newest = n;
        P.template put<ST>(k, v, s0 + newest * TT, lim, row_of);
      } else {
        --ahead;
      }
      cur = n2;
      return true;
    };
    while (lp_stage_round<0, NS>(turn)) {
    }
  }
  lp_wait_loads<0>();
}

template <typename RowOf>
__device__ __forceinline__ void LdsPipe::run(WA& A, int first, int step, int ntiles, int s0, int s1, int end,
                                             int end_min, const uint8_t* k, const uint8_t* v, RowOf row_of) const {
  lds_pipe_run_ns<2>(*this, A, first, step, ntiles, s0, s1, end, end_min, k, v, row_of);
}

}  // namespace
}  // namespace pkd
