// Per-wave attention machinery for gfx950 (CDNA4), shared by the split-KV
// partition kernels: compile-time tile shapes, K/V loads, the WaveAttn tile
// step (QK^T and PV on MFMA with an online softmax), the tile pipeline, the
// workgroup combine and the query-row mapping.
//
// A wave owns a token range of one (sequence b, KV head) pair and up to 16
// query rows of that KV head (GQA head packing: every K/V row read from HBM
// serves all query heads that share the KV head), and keeps its own
// online-softmax state for them.
//
// Per tile of TT tokens a wave:
//   1. resolves the page of every row through the block table (per-token
//      lookup as in the AstrAI commit log's unified paged path; with page_size
//      a multiple of 16 one lookup per 16-token group suffices),
//   2. has issued the tile's 16-byte K/V loads one tile earlier (register
//      double buffering: the next tile's loads are in flight while this one
//      computes),
//   3. writes V (and K, for rows of a 128-byte line or more) row-major into
//      wave-private LDS tiles: those loads read whole lines of consecutive rows,
//   4. QK^T on MFMA (v_mfma_f32_16x16x32_bf16): A = 16 K rows x 32 dims read
//      from the LDS tile (or, for shorter rows, loaded straight in that layout),
//      B = the packed query heads (zero-padded to 16),
//   5. online softmax in base 2 against a per-row reference maximum, common
//      to the four lane groups that hold the row's scores (formed with
//      cross-lane xor shuffles only in the tiles that raise it),
//   6. PV on MFMA: A = V^T gathered by transposing LDS reads
//      (ds_read_b64_tr_b16), B = P^T taken from the QK accumulator registers
//      without any shuffle (token order inside each 32-token chunk is permuted
//      so that the QK output layout is already the PV operand layout).
//
// Rows past the end of a range are clamped to the last valid row for
// addressing (so no page past the sequence and no tail slot is ever read) and
// masked to -inf by selection.  An empty range writes o = 0 and lse = -inf.
//
// Several query tokens per sequence (speculative verify / extend, q_len > 1):
// the q_len * G query rows of one KV head are packed 16 to an MFMA N dimension
// exactly like G query heads, packed row r being query token r / G of head
// kvh * G + r % G, so every K/V row read still serves all of them.  Under the
// causal mask query token i of a length-L sequence sees positions
// <= L - q_len + i (the position of that token), so each lane, which holds one
// packed row, masks scores at its own end; a row that sees no token of a tile
// or of a whole range keeps m = -inf and contributes nothing.
//
// A sliding window adds a per-lane lower bound (the row's window start) to the
// same select; per-head sink logits are folded into the finished rows (see
// fold_sink).  K/V rows are addressed through byte strides of a page (or, for
// contiguous K/V, a sequence), a token and a head (Geometry), and with paired
// heads a wave's D dims span two real heads, each query row zero-padded
// outside its own (load_q).
#pragma once

#include "merge_row.hpp"
#include "pkd_internal.hpp"

namespace pkd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int BYTES> struct VecT;
template <> struct VecT<16> { typedef u32x4 T; };
template <> struct VecT<8> { typedef u32x2 T; };

// Compile-time shape of one (head_dim, kv dtype) instance.
template <int D, bool FP8>
struct Cfg {
  static constexpr int ELEM = FP8 ? 1 : 2;                 // bytes per cached element
  static constexpr int ROWB = D * ELEM;                    // bytes of one token's row for one KV head
  // Tokens per wave tile: 2048 / D for bf16 (4 KiB of K and 4 KiB of V, at
  // least 16 tokens) and 4096 / D for fp8 (4 KiB of codes each).  Two tiles of
  // loads are in flight per wave; with 8 KiB tiles instead, the B = 32 and
  // B = 128 steps measured 1-2 us slower (a read stream likewise ran faster
  // with 8-16 KiB in flight per wave than with 16-32 KiB).
  static constexpr int TT = FP8 ? 4096 / D : (2048 / D > 16 ? 2048 / D : 16);
  static constexpr int NBLK = TT / 16;                     // QK MFMA row blocks per tile
  static constexpr int KP = TT >= 32 ? 32 : 16;            // tokens per PV MFMA (its K depth)
  static constexpr int NCH = TT / KP;                      // PV chunks per tile
  static constexpr int PIECE = (FP8 && D >= 64) ? 16 : 8;  // dims per lane per K load
  static constexpr int KLB = PIECE * ELEM;                 // K load bytes (16, or 8 for fp8 D=32)
  static constexpr int NPIECE = D / (4 * PIECE);           // K loads per lane per row block
  static constexpr int R = PIECE / 8;                      // QK MFMAs fed by one K load
  static constexpr int KK = D / 32;                        // QK MFMAs per row block
  static constexpr int VLB = ROWB >= 64 ? 16 : 8;          // V load bytes
  static constexpr int VEPL = VLB / ELEM;                  // elements per V load
  static constexpr int CPR = ROWB / VLB;                   // V loads per row
  static constexpr int RPI = 64 / CPR;                     // rows per V load instruction (<= 16)
  static constexpr int NV = TT * ROWB / (64 * VLB);        // V loads per lane per tile
  static constexpr int VS = D + 16;                        // V tile LDS row stride (bf16 elements)
  // K rows of at least one 128-byte line are loaded like V (each instruction
  // reads whole lines of consecutive rows) and staged in LDS, from where the
  // matrix-core operand (16 rows x 32 dims, a row per lane) is read.  Loaded
  // straight in the operand layout, every instruction would read half lines of
  // 16 rows, a pattern a plain read stream measured about 20% slower than whole
  // lines.  Shorter rows (64 bytes) are whole lines in the operand layout too
  // and are loaded straight into it.  FP8 K stays in registers: its tile loop is
  // bound by instruction issue (the code conversions), and staging measured
  // slower there (B = 64: 128.4 -> 134.6 us).
  static constexpr bool KLDS = !FP8 && ROWB >= 128;
  static constexpr int KS = D + 8;                         // K tile LDS row stride (bf16 elements)
  static constexpr int NKL = KLDS ? NV : NBLK * NPIECE;    // K loads per lane per tile
  static constexpr int KLOAD = KLDS ? VLB : KLB;           // bytes per K load
  static constexpr int WT = TT * VS + (KLDS ? TT * KS : 0);  // LDS elements of one wave's tiles (V, then K)
  static constexpr int NB = D / 16;                        // PV output blocks of 16 dims
  static constexpr int NGRP = TT / 16;                     // 16-token groups per tile
  static constexpr int VT_BYTES = kWaves * WT * 2;
  static constexpr int BT_OFFSET = VT_BYTES;                // staged block-table entries
  static constexpr int BT_ENTRIES = 512;
  static constexpr int OW_STRIDE = D + 4;                  // merge staging row stride (floats)
  static constexpr int MERGE_BYTES = kWaves * 16 * (2 + OW_STRIDE) * 4 + 16 * (kWaves + 4) * 4;
  static constexpr int LOOP_BYTES = VT_BYTES + BT_ENTRIES * 4;
  static constexpr int LDS_BYTES = LOOP_BYTES > MERGE_BYTES ? LOOP_BYTES : MERGE_BYTES;
  static_assert(KK == NPIECE * R, "K pieces must feed whole MFMAs");
  static_assert(RPI <= 16 && 16 % RPI == 0, "a V load instruction must stay in one 16-row group");
  static_assert(NV * 64 * VLB == TT * ROWB, "V loads must tile the rows exactly");
  static_assert(LDS_BYTES <= 81920 + BT_ENTRIES * 4, "LDS budget");
};

typedef typename VecT<16>::T Ld16;

template <typename To, typename From>
__device__ __forceinline__ To bit_cast_dev(const From& f) {
  static_assert(sizeof(To) == sizeof(From), "size mismatch");
  To t;
  __builtin_memcpy(&t, &f, sizeof(To));
  return t;
}

// V rows are streamed exactly once, each load instruction covering whole
// rows: non-temporal loads keep them from displacing reusable lines in L2 and
// the Infinity Cache.
template <int BYTES>
__device__ __forceinline__ typename VecT<BYTES>::T gload(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const typename VecT<BYTES>::T*>(p));
}

// K loads are laid out for the MFMA A operand: one instruction reads 16 rows,
// 4 lanes x 16 bytes of each, so every 128-byte line of a row is requested by
// two consecutive instructions.  They are ordinary cached loads so that the
// second request hits in the vector L1; streamed non-temporally, both went to
// L2 and the step ran 3-6% slower (K streams at some row offsets 20-30% slower).
template <int BYTES>
__device__ __forceinline__ typename VecT<BYTES>::T kload(const uint8_t* p) {
  return *reinterpret_cast<const typename VecT<BYTES>::T*>(p);
}

// Wave-local LDS ordering: all of this wave's LDS writes have landed before any
// later LDS read of another lane's data, and the compiler does not move LDS
// accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// result lane i, element r is element i % 4 of the 8 bytes that lane 4r + i/4
// addressed.  So if lane k of a group addresses row r0 + k/4, columns
// c0 + 4(k%4) .. +3 of a row-major bf16 tile, lane i receives column c0 + i of
// rows r0 .. r0 + 3.
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// 8 fp8 E4M3FN codes (two dwords) -> 8 bf16 (exact: every E4M3 value is a bf16 value).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(u32x2 c) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, true);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, false);
  bf16x2 e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = d[0]; r[5] = d[1]; r[6] = e[0]; r[7] = e[1];
  return r;
}

// Row tokens.  Inside each 32-token chunk c, QK row block 2c+h, MFMA row r holds
// token 32c + 8*(r/4) + 4h + r%4.  Then QK output lane group g, register i holds
// token 32c + 8g + 4h + i, which is exactly element 4h+i of the 8-token P^T
// operand lane group g needs for PV over tokens 32c + 8g .. 32c + 8g + 7.
template <int KP>
__device__ __forceinline__ int k_row_token(int blk, int r) {
  if constexpr (KP == 32) {
    return 32 * (blk >> 1) + 8 * (r >> 2) + 4 * (blk & 1) + (r & 3);
  } else {
    return 16 * blk + r;
  }
}
template <int KP>
__device__ __forceinline__ int s_out_token(int blk, int g, int i) {
  if constexpr (KP == 32) {
    return 32 * (blk >> 1) + 8 * g + 4 * (blk & 1) + i;
  } else {
    return 16 * blk + 4 * g + i;
  }
}

template <int D, bool FP8>
struct TileRegs {
  typedef Cfg<D, FP8> C;
  // K: load i covers the rows of V load i (KLDS), or piece pc of row block
  // blk at i = blk * NPIECE + pc (operand layout).
  typename VecT<C::KLOAD>::T k[C::NKL];
  typename VecT<C::VLB>::T v[C::NV];
};

// Block-table entries of one tile, fetched one tile before they are used so
// that address computation never waits on a block-table read.
template <int D, bool FP8, bool PAGED16>
struct TilePages {
  typedef Cfg<D, FP8> C;
  // PAGED16: per 16-token group; else per row a lane loads (K rows in the
  // operand layout, then V rows; or V rows alone, which K shares, with KLDS).
  int pg[PAGED16 ? C::NGRP : (C::KLDS ? C::NV : C::NBLK + C::NV)];
};


// How far (base-2 units) a tile's score maximum may exceed a row's reference
// maximum before the reference is raised: softmax weights then stay at most
// 2^8, far inside the range of the bf16 P operand and the fp32 sums.
constexpr float kRescaleSlack = 8.f;

// First of the 8 dims lane group g contributes to QK MFMA kk.  K staged in LDS
// is read as dims kk * 32 + g * 8 .. + 8; K loaded straight into the operand
// layout takes dims (kk / R) * 4 * PIECE + g * PIECE + (kk % R) * 8 .., those
// its 16-byte (or 8-byte) piece of a row holds.  q uses the same assignment,
// so each MFMA sums the products of matching dims.
template <int D, bool FP8>
__device__ __forceinline__ int q_dim0(int kk, int g) {
  typedef Cfg<D, FP8> C;
  if constexpr (C::KLDS) return kk * 32 + g * 8;
  else return (kk / C::R) * 4 * C::PIECE + g * C::PIECE + (kk % C::R) * 8;
}

// Per-wave attention state and tile operations, shared by both launch shapes.
// Lane (n, g) = (lane % 16, lane / 16) in the MFMA operand layouts.
template <int D, bool FP8>
struct WaveAttn {
  typedef Cfg<D, FP8> C;
  typedef TileRegs<D, FP8> Regs;

  int lane, n, g;
  int k_rig[C::NBLK];  // position of this lane's K row (of each row block) inside its 16-token group
  int v_rig;           // + (i * RPI) % 16: position of this lane's row of V load i
  int k_doff, v_doff;  // byte offsets of this lane's K dims / V chunk inside a row
  bf16x8 qf[C::KK];    // query heads as the B operand of QK^T
  float qk_scale;      // scale * log2(e) (* k_scale for fp8)
  float m_run;         // reference max (base-2 units) of head n, equal in all lane groups
  float l_run;         // this lane's partial sum of exp2(s - m_run) for head n
  f32x4 acc[C::NB];    // O^T: acc[nb][i] = out[head n][16 nb + 4 g + i] (unnormalised)

  __device__ __forceinline__ void init_lane(int lane_) {
    lane = lane_;
    n = lane & 15;
    g = lane >> 4;
#pragma unroll
    for (int blk = 0; blk < C::NBLK; ++blk) k_rig[blk] = k_row_token<C::KP>(blk, n) & 15;
    v_rig = lane / C::CPR;
    k_doff = g * C::PIECE * C::ELEM;
    v_doff = (lane % C::CPR) * C::VLB;
  }

  // Lane (n, g) holds packed row n's dims q_dim0(kk, g) + [0, 8) for MFMA kk;
  // the K operand uses the same dim assignment.  qrow_n is the memory
  // row of packed row n (any valid row when hv is false); rows past the group are zero.
  // This lane's query row.  With paired KV heads (VK > 1) the wave's D dims are
  // VK real heads of DR = D / VK dims each; the row (of real head slice s)
  // fills dims [s DR, (s + 1) DR) and is zero elsewhere, so that its scores
  // take only its own head's keys.
  template <int VK = 1>
  __device__ __forceinline__ void load_q(const uint16_t* qrow, bool hv, int s = 0) {
    constexpr int DR = D / VK;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      const int d0 = q_dim0<D, FP8>(kk, g);
      const bool mine = VK == 1 || d0 / DR == s;
      Ld16 raw = Ld16{0, 0, 0, 0};
      if (hv && mine) raw = *reinterpret_cast<const Ld16*>(qrow + (d0 - s * DR));
      qf[kk] = bit_cast_dev<bf16x8>(raw);
    }
  }

  __device__ __forceinline__ void reset() {
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Issue every K and V load of the tile starting at token tb (a multiple of
  // 16).  pages[q] is the physical page of the tile's 16-token group q (every
  // aligned group lies in one page when page_size % 16 == 0); a row past lim is
  // replaced by a valid row of its group (position min(pos, lim - group start))
  // and masked later.
  // idle: read the same rows of physical page 0 instead (shared by every
  // workgroup, so they come from cache); the data is not used.
  __device__ __forceinline__ void issue_paged16(const uint8_t* kc, const uint8_t* vc, int tb, int lim,
                                                const int* pages, int ps, int tok_stride, int64_t page_stride,
                                                int64_t head_off, Regs& R, bool idle) const {
    int64_t gbase[C::NGRP];
    int glim[C::NGRP];
#pragma unroll
    for (int q = 0; q < C::NGRP; ++q) {
      const int gt = min(tb + 16 * q, lim) & ~15;
      const int page = idle ? 0 : __builtin_amdgcn_readfirstlane(pages[q]);
      gbase[q] = (int64_t)page * page_stride + (int64_t)(gt - (gt / ps) * ps) * tok_stride + head_off;
      glim[q] = lim - gt;
    }
    if constexpr (C::KLDS) {
      // K rows are loaded exactly like V rows (whole lines per instruction).
#pragma unroll
      for (int i = 0; i < C::NV; ++i) {
        const int q = (i * C::RPI) >> 4;
        const int rig = ((i * C::RPI) & 15) + v_rig;
        R.k[i] = gload<C::VLB>(kc + gbase[q] + min(rig, glim[q]) * tok_stride + v_doff);
      }
    }
#pragma unroll
    for (int blk = 0; blk < (C::KLDS ? 0 : C::NBLK); ++blk) {
      int64_t base;
      int gl;
      if constexpr (C::KP == 32) {
        // The two halves of a 32-token row block come from groups 2c and 2c+1.
        const int q0 = 2 * (blk >> 1);
        const bool hi = (k_row_token<C::KP>(blk, n) >> 4) != q0;
        base = hi ? gbase[q0 + 1] : gbase[q0];
        gl = hi ? glim[q0 + 1] : glim[q0];
      } else {
        base = gbase[blk];
        gl = glim[blk];
      }
      const uint8_t* src = kc + base + min(k_rig[blk], gl) * tok_stride + k_doff;
#pragma unroll
      for (int pc = 0; pc < C::NPIECE; ++pc)
        R.k[blk * C::NPIECE + pc] = kload<C::KLB>(src + pc * 4 * C::PIECE * C::ELEM);
    }
#pragma unroll
    for (int i = 0; i < C::NV; ++i) {
      const int q = (i * C::RPI) >> 4;
      const int rig = ((i * C::RPI) & 15) + v_rig;
      R.v[i] = gload<C::VLB>(vc + gbase[q] + min(rig, glim[q]) * tok_stride + v_doff);
    }
  }

  // Any page size: pages[blk] is the page of this lane's K row of row block
  // blk, pages[NBLK + i] that of its row of V load i (rows clamped to lim);
  // with KLDS, pages[i] is the page of its row of V load i, which K shares.
  __device__ __forceinline__ void issue_generic(const uint8_t* kc, const uint8_t* vc, int tb, int lim,
                                                const int* pages, int ps, int tok_stride, int64_t page_stride,
                                                int64_t head_off, Regs& R, bool idle) const {
    constexpr int VP = C::KLDS ? 0 : C::NBLK;  // index of the first V row's page
    if constexpr (C::KLDS) {
#pragma unroll
      for (int i = 0; i < C::NV; ++i) {
        const int tok = min(tb + i * C::RPI + v_rig, lim);
        const int64_t off = (int64_t)(idle ? 0 : pages[i]) * page_stride +
                            (int64_t)(tok - (tok / ps) * ps) * tok_stride + head_off;
        R.k[i] = gload<C::VLB>(kc + off + v_doff);
      }
    }
#pragma unroll
    for (int blk = 0; blk < (C::KLDS ? 0 : C::NBLK); ++blk) {
      const int tok = min(tb + k_row_token<C::KP>(blk, n), lim);
      const int64_t off = (int64_t)(idle ? 0 : pages[blk]) * page_stride + (int64_t)(tok - (tok / ps) * ps) * tok_stride +
                          head_off;
      const uint8_t* src = kc + off + k_doff;
#pragma unroll
      for (int pc = 0; pc < C::NPIECE; ++pc)
        R.k[blk * C::NPIECE + pc] = kload<C::KLB>(src + pc * 4 * C::PIECE * C::ELEM);
    }
#pragma unroll
    for (int i = 0; i < C::NV; ++i) {
      const int tok = min(tb + i * C::RPI + v_rig, lim);
      const int64_t off = (int64_t)(idle ? 0 : pages[VP + i]) * page_stride +
                          (int64_t)(tok - (tok / ps) * ps) * tok_stride + head_off;
      R.v[i] = gload<C::VLB>(vc + off + v_doff);
    }
  }

  // Tokens (relative to tb) whose pages the generic path needs, per lane.
  __device__ __forceinline__ int generic_row(int idx) const {
    if constexpr (C::KLDS) return idx * C::RPI + v_rig;
    return idx < C::NBLK ? k_row_token<C::KP>(idx, n) : (idx - C::NBLK) * C::RPI + v_rig;
  }

  // One row-pattern load (V, or K with KLDS) into a row-major bf16 LDS tile of
  // row stride STRIDE: lane `lane` of load i holds row (i * 64 + lane) / CPR,
  // elements VEPL * ((i * 64 + lane) % CPR) ..; FP8 codes are widened to bf16
  // (exactly).
  template <int STRIDE>
  __device__ __forceinline__ void stage_rows(const typename VecT<C::VLB>::T& raw, int i, uint16_t* tile) const {
    const int lin = i * 64 + lane;
    uint16_t* dst = tile + (lin / C::CPR) * STRIDE + (lin % C::CPR) * C::VEPL;
    if constexpr (FP8) {
#pragma unroll
      for (int h = 0; h < C::VEPL / 8; ++h) {
        u32x2 c8;
        c8[0] = raw[2 * h];
        c8[1] = raw[2 * h + 1];
        *reinterpret_cast<bf16x8*>(dst + 8 * h) = fp8x8_to_bf16(c8);
      }
    } else if constexpr (C::VLB == 16) {
      *reinterpret_cast<u32x4*>(dst) = raw;
    } else {
      *reinterpret_cast<u32x2*>(dst) = raw;
    }
  }

  // One tile: V (and K) to LDS, QK^T, online softmax, PV.  Tokens before s_lo or at or
  // past s1 (this lane's packed row's window start and end) are masked.
  // lo_all and hi_all (uniform) bound every lane's s_lo from above and s1 from
  // below: tiles starting at lo_all or later skip the lower-bound test, and
  // tiles inside [lo_all, hi_all) skip masking altogether.
  __device__ __forceinline__ void process(const Regs& R, int tb, int s_lo, int s1, int lo_all, int hi_all,
                                          uint16_t* vs) {
    // V -> LDS, row-major bf16 (16-byte writes); K too when it is staged there.
#pragma unroll
    for (int i = 0; i < C::NV; ++i) stage_rows<C::VS>(R.v[i], i, vs);
    uint16_t* ks = vs + C::TT * C::VS;  // this wave's K[TT][KS] (KLDS)
    if constexpr (C::KLDS) {
#pragma unroll
      for (int i = 0; i < C::NV; ++i) stage_rows<C::KS>(R.k[i], i, ks);
      wave_lds_sync();  // the K and V tiles are complete in LDS
    }

    // S^T = K Q^T for each 16-row block.
    f32x4 sacc[C::NBLK];
#pragma unroll
    for (int blk = 0; blk < C::NBLK; ++blk) {
      sacc[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) {
        bf16x8 a;
        if constexpr (C::KLDS) {
          // Row n of the block, dims kk * 32 + g * 8 .. + 8 (ds_read_b128).
          a = *reinterpret_cast<const bf16x8*>(ks + k_row_token<C::KP>(blk, n) * C::KS + kk * 32 + g * 8);
        } else if constexpr (FP8) {
          const auto& raw = R.k[blk * C::NPIECE + kk / C::R];
          u32x2 c8;
          c8[0] = raw[2 * (kk % C::R)];
          c8[1] = raw[2 * (kk % C::R) + 1];
          a = fp8x8_to_bf16(c8);
        } else {
          a = bit_cast_dev<bf16x8>(R.k[blk * C::NPIECE + kk]);
        }
        sacc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[kk], sacc[blk], 0, 0, 0);
      }
    }

    // Online softmax (base 2).  Lane (n, g) holds scores of head n for tokens
    // s_out_token(blk, g, i).
    float mt = -INFINITY;
    if (tb >= lo_all && tb + C::TT <= hi_all) {
#pragma unroll
      for (int blk = 0; blk < C::NBLK; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sacc[blk][i] *= qk_scale;
          mt = fmaxf(mt, sacc[blk][i]);
        }
    } else if (tb >= lo_all) {
#pragma unroll
      for (int blk = 0; blk < C::NBLK; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = tb + s_out_token<C::KP>(blk, g, i);
          const float x = sacc[blk][i] * qk_scale;
          sacc[blk][i] = tok < s1 ? x : -INFINITY;
          mt = fmaxf(mt, sacc[blk][i]);
        }
    } else {
#pragma unroll
      for (int blk = 0; blk < C::NBLK; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = tb + s_out_token<C::KP>(blk, g, i);
          const float x = sacc[blk][i] * qk_scale;
          sacc[blk][i] = (tok < s1 && tok >= s_lo) ? x : -INFINITY;
          mt = fmaxf(mt, sacc[blk][i]);
        }
    }
    // m_run is a reference maximum rather than the exact running maximum: it
    // is raised (and l and O rescaled by 2^(old - new)) only when a tile's
    // maximum exceeds it by more than kRescaleSlack, so every weight
    // 2^(s - m_run) stays at most 2^kRescaleSlack and, after the first tiles,
    // the rescale of the accumulators is skipped.  Raised, it becomes the
    // tile's maximum.  A row that has seen no unmasked token keeps m = -inf;
    // subtracting 0 then gives e = 0 instead of NaN.
    // A row's tile maximum exceeds the threshold exactly when one of its four
    // lane groups' maxima does, so the wave-wide test needs no cross-lane
    // exchange; the row maximum (two shuffles through LDS) is formed only when
    // some row is raised.
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleSlack) != 0) {
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = mt > m_run + kRescaleSlack ? mt : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) acc[nb] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float psum = 0.f;
#pragma unroll
    for (int blk = 0; blk < C::NBLK; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(sacc[blk][i] - m_use);
        sacc[blk][i] = e;
        psum += e;
      }
    l_run += psum;

    if constexpr (!C::KLDS) wave_lds_sync();  // the V tile is complete in LDS

    // O^T += V^T P^T; the V^T operand comes from transposing LDS reads.
    if constexpr (C::KP == 32) {
#pragma unroll
      for (int c = 0; c < C::NCH; ++c) {
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[i] = (__bf16)sacc[2 * c][i];
          pb[4 + i] = (__bf16)sacc[2 * c + 1][i];
        }
        // lane (n, g) needs V[32c + 8g + j][16 nb + n], j = 0..7
        const uint16_t* rowp = vs + (32 * c + 8 * g + (n >> 2)) * C::VS + 4 * (n & 3);
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          const s16x4 lo = lds_read_tr16(rowp + 16 * nb);
          const s16x4 hi = lds_read_tr16(rowp + 4 * C::VS + 16 * nb);
          s16x4 both[2] = {lo, hi};
          const bf16x8 a = bit_cast_dev<bf16x8>(both);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, acc[nb], 0, 0, 0);
        }
      }
    } else {
      bf16x4 pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[i] = (__bf16)sacc[0][i];
      const s16x4 pbs = bit_cast_dev<s16x4>(pb);
      // lane (n, g) needs V[4g + j][16 nb + n], j = 0..3
      const uint16_t* rowp = vs + (4 * g + (n >> 2)) * C::VS + 4 * (n & 3);
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        const s16x4 a = lds_read_tr16(rowp + 16 * nb);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pbs, acc[nb], 0, 0, 0);
      }
    }
    wave_lds_sync();  // PV reads done before the next tile overwrites the V tile
  }

  // Sum of l over the four lane groups (every lane of head n gets it).
  __device__ __forceinline__ float l_total() const {
    const float l = l_run + __shfl_xor(l_run, 16);
    return l + __shfl_xor(l, 32);
  }
};

// Memory row ((b * q_len + i) * Hq + h) of packed row r of KV head kvh of
// sequence b: query token i = r / G, head h = kvh * G + r % G.
__device__ __forceinline__ int64_t packed_row(int b, int kvh, int r, int q_len, int hq, int group) {
  const int i = r / group;
  return ((int64_t)b * q_len + i) * hq + kvh * group + (r - i * group);
}

// Per lane (packed row n = lane % 16 of head group hg): the row index of its
// query (a valid row even past the group), the element offsets of that row in
// q and out, whether the row exists, and the range of tokens it sees within
// [.., s1): to s1, or under the causal mask min(s1, L - q_len + i + 1) for
// query token i; from its window start.
struct LaneRow {
  int64_t row;
  int64_t qoff, ooff;
  int head;       // query head of the row
  bool valid;
  int start;      // first position the row sees (its sliding window's lower end; 0 without a window)
  int end;
  int start_max;  // uniform: no row of the sequence starts later (L - window, or 0)
  int end_min;    // uniform: no row of the group ends earlier
};
template <int D, bool STRIDED, typename P>
__device__ __forceinline__ LaneRow lane_row(const P& p, int b, int kvh, int hg, int n, int L, int s1, int window) {
  const int r = hg * kHeadsPerGroup + n;
  LaneRow lr;
  lr.valid = r < p.rows_kv;
  const int rr = lr.valid ? r : hg * kHeadsPerGroup;
  const int i = rr / p.group, h = kvh * p.group + (rr - i * p.group);
  lr.row = ((int64_t)b * p.q_len + i) * p.hq + h;
  lr.head = h;
  if constexpr (STRIDED) {
    lr.qoff = p.qs.at(b, i, h);
    lr.ooff = p.os.at(b, i, h);
  } else {
    lr.qoff = lr.ooff = lr.row * D;
  }
  const int pos = L - p.q_len + i;  // the query token's position
  lr.end = p.causal ? min(s1, pos + 1) : s1;
  // The group's first row holds its earliest query token.
  lr.end_min = p.causal ? min(s1, L - p.q_len + (hg * kHeadsPerGroup) / p.group + 1) : s1;
  lr.start = window > 0 ? max(pos - window + 1, 0) : 0;
  lr.start_max = window > 0 ? max(L - window, 0) : 0;
  return lr;
}

// Where q/out rows and K/V rows are.  STRIDED: the strides the host passed
// (contiguous K/V, strided q / out).  Otherwise the dense q/out layout and the
// paged [P][ps][Hkv][D] cache, derived from the shape, so that the paged
// kernels keep no stride parameters in scalar registers.
template <int D, bool FP8, bool STRIDED>
struct Geometry {
  typedef Cfg<D, FP8> C;
  template <typename P>
  static __device__ __forceinline__ RowStrides qs(const P& p) {
    if constexpr (STRIDED) return p.qs;
    else return RowStrides{(int64_t)p.q_len * p.hq * D, (int64_t)p.hq * D, D};
  }
  template <typename P>
  static __device__ __forceinline__ RowStrides os(const P& p) {
    if constexpr (STRIDED) return p.os;
    else return RowStrides{(int64_t)p.q_len * p.hq * D, (int64_t)p.hq * D, D};
  }
  template <typename P>
  static __device__ __forceinline__ int tok_stride(const P& p) {
    if constexpr (STRIDED) return p.kv.tok_stride;
    else return p.hkv * C::ROWB;
  }
  template <typename P>
  static __device__ __forceinline__ int64_t page_stride(const P& p) {
    if constexpr (STRIDED) return p.kv.page_stride;
    else return (int64_t)p.page_size * (p.hkv * C::ROWB);
  }
  template <typename P>
  static __device__ __forceinline__ int64_t head_stride(const P& p) {
    if constexpr (STRIDED) return p.kv.head_stride;
    else return C::ROWB;
  }
  // No block table: sequence b is page b (contiguous K/V).
  template <typename P>
  static __device__ __forceinline__ bool contiguous(const P& p) {
    if constexpr (STRIDED) return p.block_table == nullptr;
    else return false;
  }
};

// First token of sequence b that any of its query tokens sees, rounded down to
// a multiple of 16 (tiles start on 16-token groups): the lowest window start
// when there is a window, else 0.  Tokens below it are never read.
template <typename P>
__device__ __forceinline__ int seq_first_token(const P& p, int L, int window) {
  if (window <= 0) return 0;
  return max(L - p.q_len - window + 1, 0) & ~15;
}

// Tiles first, first + step, ... (< ntiles): while tile t is processed the
// next tile's K/V loads are in flight and the page entries of the tile after
// that are being read.  After the last tile the "next" loads stay in the
// instruction stream (so the wait counts are the same on every iteration) but
// are pointed at rows every workgroup shares by passing idle = true; they are
// never consumed.
template <int D, bool FP8, typename Pages, typename Fetch, typename Issue>
__device__ __forceinline__ void run_tiles(WaveAttn<D, FP8>& A, int first, int step, int ntiles, int s0,
                                          const LaneRow& lr, uint16_t* vs, Fetch fetch, Issue issue) {
  typedef Cfg<D, FP8> C;
  if (first >= ntiles) return;
  auto nxt = [&](int t) { return t + step < ntiles ? t + step : t; };
  TileRegs<D, FP8> ra, rb;
  Pages pa, pb;
  int t = first;
  fetch(t, pa);
  issue(t, pa, ra, false);
  int t1 = nxt(t);
  fetch(t1, pb);
  while (true) {
    issue(t1, pb, rb, t1 == t);
    int t2 = nxt(t1);
    fetch(t2, pa);
    __builtin_amdgcn_sched_barrier(0);
    A.process(ra, s0 + t * C::TT, lr.start, lr.end, lr.start_max, lr.end_min, vs);
    if (t1 == t) break;
    t = t1;
    t1 = t2;
    issue(t1, pa, ra, t1 == t);
    t2 = nxt(t1);
    fetch(t2, pb);
    __builtin_amdgcn_sched_barrier(0);
    A.process(rb, s0 + t * C::TT, lr.start, lr.end, lr.start_max, lr.end_min, vs);
    if (t1 == t) break;
    t = t1;
    t1 = t2;
  }
}

// Combine the waves' (m, l, O) of one workgroup in LDS (smem must hold
// NWV * 16 * (2 + OW_STRIDE) * 4 + 16 * (NWV + 4) * 4 bytes) and hand every
// row of the group to store, four dims at a time: store(hh, d0, o4, lse_nat),
// o4 = dims d0 .. d0 + 3 of o = sum_w e_w O_w * vsc / sum_w e_w l_w with
// e_w = 2^(m_w - max m), and the natural-log LSE.  A row that saw no token in
// any wave gets o = 0 and lse = -inf.  sink_of(hh) is row hh's sink logit
// (-inf for none), folded in as fold_sink describes; partials take none.  The
// per-row weights e_w * vsc / den (vsc_of(hh) for row hh) are computed once per row, then each element
// is a short weighted sum of the staged wave rows.  Ends with the LDS still in
// use: synchronise before reusing it.
template <int D, bool FP8, int NWV = kWaves, typename Store, typename SinkOf, typename VscOf>
__device__ __forceinline__ void wg_combine_rows(const WaveAttn<D, FP8>& A, uint8_t* smem, int wave, int tid,
                                                int heads_here, VscOf vsc_of, Store store, SinkOf sink_of) {
  typedef Cfg<D, FP8> C;
  constexpr int RWS = NWV + 4;                 // per-row table stride (floats): NWV weights, then the LSE
  const float l_tot = A.l_total();
  __syncthreads();
  float* mw = reinterpret_cast<float*>(smem);  // [NWV][16]
  float* lw = mw + NWV * 16;                   // [NWV][16]
  float* ow = lw + NWV * 16;                   // [NWV][16][OW_STRIDE]
  float* rw = ow + NWV * 16 * C::OW_STRIDE;    // [16][RWS]
  if (A.g == 0) {
    mw[wave * 16 + A.n] = A.m_run;
    lw[wave * 16 + A.n] = l_tot;
  }
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
    *reinterpret_cast<f32x4*>(ow + (wave * 16 + A.n) * C::OW_STRIDE + 16 * nb + 4 * A.g) = A.acc[nb];
  __syncthreads();
  if (tid < heads_here) {
    const int hh = tid;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) M = fmaxf(M, mw[w * 16 + hh]);
    const float M_use = M == -INFINITY ? 0.f : M;
    float e[NWV];
    float den = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      e[w] = __builtin_amdgcn_exp2f(mw[w * 16 + hh] - M_use);
      den += e[w] * lw[w * 16 + hh];
    }
    float lse_nat = (M_use + log2f(den)) * 0.69314718055994530942f;
    const float f = fold_sink(lse_nat, sink_of(hh));
    const float sc = den > 0.f ? vsc_of(hh) * f / den : 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) rw[hh * RWS + w] = e[w] * sc;
    rw[hh * RWS + NWV] = lse_nat;
  }
  __syncthreads();
  constexpr int Q4 = D / 4;
  for (int idx = tid; idx < heads_here * Q4; idx += NWV * 64) {
    const int hh = idx / Q4, d0 = (idx - hh * Q4) * 4;
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NWV; ++w)
      o += rw[hh * RWS + w] * *reinterpret_cast<const f32x4*>(ow + (w * 16 + hh) * C::OW_STRIDE + d0);
    store(hh, d0, o, rw[hh * RWS + NWV]);
  }
}

// wg_combine_rows with one V scale for every row.
template <int D, bool FP8, int NWV = kWaves, typename Store, typename SinkOf>
__device__ __forceinline__ void wg_combine(const WaveAttn<D, FP8>& A, uint8_t* smem, int wave, int tid,
                                           int heads_here, float vsc, Store store, SinkOf sink_of) {
  wg_combine_rows<D, FP8, NWV>(A, smem, wave, tid, heads_here, [vsc](int) { return vsc; }, store, sink_of);
}

// No sink (partials, and rows of a call without sinks).
struct NoSink {
  __device__ __forceinline__ float operator()(int) const { return -INFINITY; }
};

// Four fp32 values rounded to bf16 (round-to-nearest-even), as one 8-byte word.
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 o) {
  bf16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (__bf16)o[i];
  return r;
}

}  // namespace
}  // namespace pkd
