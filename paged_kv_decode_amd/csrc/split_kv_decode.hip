// Split-KV paged decode attention for gfx950 (CDNA4): the partition kernel.
//
// One workgroup = one (split j, KV head, sequence b) and up to 16 query heads of
// that KV head (GQA head packing: all query heads that share a KV head are
// served by each K/V row read from HBM).  Four waves per workgroup; each wave
// streams its own tiles of the split's token range and keeps its own online
// softmax state, and the workgroup combines the four wave states at the end.
//
// Per tile of TT tokens a wave:
//   1. resolves the page of every row through the block table (per-token
//      lookup as in the AstrAI commit log's unified paged path; with page_size
//      a multiple of 16 one scalar lookup per 16-token group suffices),
//   2. has already issued 16-byte HBM loads for this tile one tile earlier
//      (register double buffering; the next tile's loads are in flight while
//      this one computes),
//   3. writes V transposed into a wave-private LDS tile,
//   4. QK^T on MFMA (v_mfma_f32_16x16x32_bf16): A = 16 K rows x 32 dims straight
//      from the load registers, B = the packed query heads (zero-padded to 16),
//   5. online softmax in base 2 with the running max shared across the four
//      lane groups by cross-lane xor shuffles,
//   6. PV on MFMA: A = V^T from LDS, B = P^T taken from the QK accumulator
//      registers without any shuffle (token order inside each 32-token chunk is
//      permuted so that the QK output layout is already the PV operand layout).
//
// Rows past the end of the split are clamped to the last valid row for
// addressing (so no page past the sequence and no tail slot is ever read) and
// masked to -inf by selection.  An empty split writes o = 0 and lse = -inf.
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
  // Tokens per wave tile: 8 KiB of K (and of V) per tile for bf16; fp8 keeps
  // the same bytes except at D = 32 where the tile would be 256 rows.
  static constexpr int TT = FP8 ? (D == 32 ? 128 : 8192 / D) : 4096 / D;
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
  static constexpr int RS = TT + 8;                        // V^T LDS row stride (bf16 elements)
  static constexpr int NB = D / 16;                        // PV output blocks of 16 dims
  static constexpr int NGRP = TT / 16;                     // 16-token groups per tile
  static constexpr int VT_BYTES = kWaves * D * RS * 2;
  static constexpr int OW_STRIDE = D + 4;                  // merge staging row stride (floats)
  static constexpr int MERGE_BYTES = kWaves * 16 * (2 + OW_STRIDE) * 4;
  static constexpr int LDS_BYTES = VT_BYTES > MERGE_BYTES ? VT_BYTES : MERGE_BYTES;
  static_assert(KK == NPIECE * R, "K pieces must feed whole MFMAs");
  static_assert(RPI <= 16 && 16 % RPI == 0, "a V load instruction must stay in one 16-row group");
  static_assert(NV * 64 * VLB == TT * ROWB, "V loads must tile the rows exactly");
  static_assert(LDS_BYTES <= 81920, "two workgroups per CU must fit in LDS");
};

typedef typename VecT<16>::T Ld16;

template <typename To, typename From>
__device__ __forceinline__ To bit_cast_dev(const From& f) {
  static_assert(sizeof(To) == sizeof(From), "size mismatch");
  To t;
  __builtin_memcpy(&t, &f, sizeof(To));
  return t;
}

template <int BYTES>
__device__ __forceinline__ typename VecT<BYTES>::T gload(const uint8_t* p) {
  return *reinterpret_cast<const typename VecT<BYTES>::T*>(p);
}

// Wave-local LDS ordering: all of this wave's LDS writes have landed before any
// later LDS read of another lane's data, and the compiler does not move LDS
// accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
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
  typename VecT<C::KLB>::T k[C::NBLK][C::NPIECE];
  typename VecT<C::VLB>::T v[C::NV];
};

template <int D, bool FP8, bool PAGED16, bool DIRECT>
__global__ void __launch_bounds__(kWaves * 64)
split_kv_kernel(const SplitParams p) {
  typedef Cfg<D, FP8> C;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;   // MFMA row/column index of this lane
  const int g = lane >> 4;   // MFMA k-group of this lane

  const int split = blockIdx.x;
  const int kvh = blockIdx.y / p.head_groups;
  const int hg = blockIdx.y - kvh * p.head_groups;
  const int b = blockIdx.z;
  const int S = p.num_splits;

  const int L = p.seq_lens[b];
  const int per = (L + S - 1) / S;
  const int chunk = ((per + kSplitAlign - 1) / kSplitAlign) * kSplitAlign;
  const int s0 = split * chunk;
  const int s1 = min(s0 + chunk, L);
  const int heads_here = min(kHeadsPerGroup, p.group - hg * kHeadsPerGroup);
  const int h0 = kvh * p.group + hg * kHeadsPerGroup;
  const int64_t row0 = (int64_t)b * p.hq + h0;  // first output row of this workgroup

  if (s0 >= s1) {
    // Empty split (or an empty sequence): o = 0, lse = -inf.
    for (int idx = tid; idx < heads_here * D; idx += kWaves * 64) {
      const int hh = idx / D, d = idx - (idx / D) * D;
      if constexpr (DIRECT) {
        p.out[(row0 + hh) * D + d] = 0;
        if (d == 0 && p.lse) p.lse[row0 + hh] = -INFINITY;
      } else {
        p.o_part[((row0 + hh) * S + split) * D + d] = 0.f;
        if (d == 0) p.lse_part[(row0 + hh) * S + split] = -INFINITY;
      }
    }
    return;
  }

  const int ntiles = (s1 - s0 + C::TT - 1) / C::TT;
  const int lim = s1 - 1;
  const int tok_stride = p.hkv * C::ROWB;  // bytes between consecutive slots of a page
  const int64_t head_off = (int64_t)kvh * C::ROWB;
  // The block table is read-only for the whole launch: reading it through the
  // constant address space makes the uniform lookups scalar loads, which do not
  // wait behind the vector loads of K/V in flight.
  const __attribute__((address_space(4))) int32_t* bt =
      (const __attribute__((address_space(4))) int32_t*)(p.block_table + (int64_t)b * p.max_pages);
  const int ps = p.page_size;

  // Query heads as the B operand of QK^T: lane (n, g) holds head n's dims for
  // MFMA kk: (kk / R) * 4 * PIECE + g * PIECE + (kk % R) * 8 + [0, 8).  The K
  // loads below use the same dim assignment.  Heads past the group are zero.
  bf16x8 qf[C::KK];
  {
    const bool hv = n < heads_here;
    const uint16_t* qrow = p.q + (row0 + (hv ? n : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      const int d0 = (kk / C::R) * 4 * C::PIECE + g * C::PIECE + (kk % C::R) * 8;
      Ld16 raw = *reinterpret_cast<const Ld16*>(qrow + d0);
      if (!hv) raw = Ld16{0, 0, 0, 0};
      qf[kk] = bit_cast_dev<bf16x8>(raw);
    }
  }

  float qk_scale = p.qk_scale_log2;
  if constexpr (FP8) qk_scale *= p.k_scale[kvh];

  // Lane-constant parts of the row addressing.  Row tau of a tile (K row block
  // blk uses tau = k_row_token(blk, n); V load i uses tau = i*RPI + lane/CPR)
  // sits in 16-token group tau/16 at position tau%16.
  int k_rig[C::NBLK];   // position inside its 16-group, per K row block
#pragma unroll
  for (int blk = 0; blk < C::NBLK; ++blk) k_rig[blk] = k_row_token<C::KP>(blk, n) & 15;
  const int v_rig = lane / C::CPR;                     // + (i*RPI) % 16 for load i
  const int k_doff = g * C::PIECE * C::ELEM;           // byte offset of this lane's K dims
  const int v_doff = (lane % C::CPR) * C::VLB;         // byte offset of this lane's V chunk

  auto issue_loads = [&](int tile, TileRegs<D, FP8>& R) {
    const int tb = s0 + tile * C::TT;
    if constexpr (PAGED16) {
      // Every aligned 16-token group lies in one page: one scalar lookup per
      // group.  A row past the end is replaced by a valid row of its group
      // (position min(pos, lim - group start)); it is masked out later.
      int64_t gbase[C::NGRP];
      int glim[C::NGRP];
#pragma unroll
      for (int q = 0; q < C::NGRP; ++q) {
        const int gt = min(tb + 16 * q, lim) & ~15;
        const int pidx = gt / ps;
        const int page = bt[pidx];
        gbase[q] = ((int64_t)page * ps + (gt - pidx * ps)) * tok_stride + head_off;
        glim[q] = lim - gt;
      }
#pragma unroll
      for (int blk = 0; blk < C::NBLK; ++blk) {
        const int q = k_row_token<C::KP>(blk, n) >> 4;
        // For KP == 32 the two halves of a row block come from groups 2c, 2c+1.
        int64_t base;
        int gl;
        if constexpr (C::KP == 32) {
          const int q0 = 2 * (blk >> 1);
          base = q == q0 ? gbase[q0] : gbase[q0 + 1];
          gl = q == q0 ? glim[q0] : glim[q0 + 1];
        } else {
          base = gbase[blk];
          gl = glim[blk];
        }
        const uint8_t* src = p.k + base + min(k_rig[blk], gl) * tok_stride + k_doff;
#pragma unroll
        for (int pc = 0; pc < C::NPIECE; ++pc)
          R.k[blk][pc] = gload<C::KLB>(src + pc * 4 * C::PIECE * C::ELEM);
      }
#pragma unroll
      for (int i = 0; i < C::NV; ++i) {
        const int q = (i * C::RPI) >> 4;
        const int rig = ((i * C::RPI) & 15) + v_rig;
        R.v[i] = gload<C::VLB>(p.v + gbase[q] + min(rig, glim[q]) * tok_stride + v_doff);
      }
    } else {
      // Any page size: one lookup per row.
#pragma unroll
      for (int blk = 0; blk < C::NBLK; ++blk) {
        const int tok = min(tb + k_row_token<C::KP>(blk, n), lim);
        const int pidx = tok / ps;
        const int64_t off = ((int64_t)p.block_table[(int64_t)b * p.max_pages + pidx] * ps + (tok - pidx * ps)) *
                                tok_stride + head_off;
        const uint8_t* src = p.k + off + k_doff;
#pragma unroll
        for (int pc = 0; pc < C::NPIECE; ++pc)
          R.k[blk][pc] = gload<C::KLB>(src + pc * 4 * C::PIECE * C::ELEM);
      }
#pragma unroll
      for (int i = 0; i < C::NV; ++i) {
        const int tok = min(tb + i * C::RPI + v_rig, lim);
        const int pidx = tok / ps;
        const int64_t off = ((int64_t)p.block_table[(int64_t)b * p.max_pages + pidx] * ps + (tok - pidx * ps)) *
                                tok_stride + head_off;
        R.v[i] = gload<C::VLB>(p.v + off + v_doff);
      }
    }
  };

  float m_run = -INFINITY;  // running max (base-2 units) of head n, same in all lane groups
  float l_run = 0.f;        // this lane's partial sum of exp2(s - m_run) for head n
  f32x4 acc[C::NB];         // O^T: acc[nb][i] = out[head n][16 nb + 4 g + i] (unnormalised)
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint16_t* vt = reinterpret_cast<uint16_t*>(smem) + wave * D * C::RS;  // this wave's V^T[D][RS]

  auto process = [&](int tile, const TileRegs<D, FP8>& R) {
    const int tb = s0 + tile * C::TT;
    // V -> LDS, transposed to [dim][token] as bf16.
#pragma unroll
    for (int i = 0; i < C::NV; ++i) {
      const int lin = i * 64 + lane;
      const int vrow = lin / C::CPR;
      const int d0 = (lin % C::CPR) * C::VEPL;
      if constexpr (FP8) {
#pragma unroll
        for (int h = 0; h < C::VEPL / 8; ++h) {
          u32x2 c8;
          c8[0] = R.v[i][2 * h];
          c8[1] = R.v[i][2 * h + 1];
          const bf16x8 x = fp8x8_to_bf16(c8);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            vt[(d0 + 8 * h + e) * C::RS + vrow] = bit_cast_dev<uint16_t>(x[e]);
        }
      } else {
#pragma unroll
        for (int w = 0; w < C::VEPL / 2; ++w) {
          const uint32_t two = R.v[i][w];
          vt[(d0 + 2 * w) * C::RS + vrow] = (uint16_t)(two & 0xffffu);
          vt[(d0 + 2 * w + 1) * C::RS + vrow] = (uint16_t)(two >> 16);
        }
      }
    }

    // S^T = K Q^T for each 16-row block.
    f32x4 sacc[C::NBLK];
#pragma unroll
    for (int blk = 0; blk < C::NBLK; ++blk) {
      sacc[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) {
        bf16x8 a;
        if constexpr (FP8) {
          const auto& raw = R.k[blk][kk / C::R];
          u32x2 c8;
          c8[0] = raw[2 * (kk % C::R)];
          c8[1] = raw[2 * (kk % C::R) + 1];
          a = fp8x8_to_bf16(c8);
        } else {
          a = bit_cast_dev<bf16x8>(R.k[blk][kk]);
        }
        sacc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[kk], sacc[blk], 0, 0, 0);
      }
    }

    // Online softmax (base 2).  Lane (n, g) holds scores of head n for tokens
    // s_out_token(blk, g, i).
    float mt = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < C::NBLK; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = tb + s_out_token<C::KP>(blk, g, i);
        const float x = sacc[blk][i] * qk_scale;
        sacc[blk][i] = tok < s1 ? x : -INFINITY;
        mt = fmaxf(mt, sacc[blk][i]);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int blk = 0; blk < C::NBLK; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(sacc[blk][i] - m_new);
        sacc[blk][i] = e;
        psum += e;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) acc[nb] *= alpha;

    wave_lds_sync();  // V^T of this tile is complete

    // O^T += V^T P^T.
    if constexpr (C::KP == 32) {
#pragma unroll
      for (int c = 0; c < C::NCH; ++c) {
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[i] = (__bf16)sacc[2 * c][i];
          pb[4 + i] = (__bf16)sacc[2 * c + 1][i];
        }
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + (16 * nb + n) * C::RS + 32 * c + 8 * g);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, acc[nb], 0, 0, 0);
        }
      }
    } else {
      bf16x4 pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[i] = (__bf16)sacc[0][i];
      const s16x4 pbs = bit_cast_dev<s16x4>(pb);
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        const s16x4 a = *reinterpret_cast<const s16x4*>(vt + (16 * nb + n) * C::RS + 4 * g);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pbs, acc[nb], 0, 0, 0);
      }
    }
    wave_lds_sync();  // PV reads done before the next tile's V^T overwrites the tile
  };

  // Tiles wave, wave + 4, wave + 8, ... with the next tile's loads in flight.
  // At the end the "next" tile repeats the last one so the loads stay
  // unconditional (they hit in cache and are not consumed).
  if (wave < ntiles) {
    TileRegs<D, FP8> ra, rb;
    int t = wave;
    issue_loads(t, ra);
    while (true) {
      const int t1 = t + kWaves < ntiles ? t + kWaves : t;
      issue_loads(t1, rb);
      process(t, ra);
      if (t1 == t) break;
      t = t1;
      const int t2 = t + kWaves < ntiles ? t + kWaves : t;
      issue_loads(t2, ra);
      process(t, rb);
      if (t2 == t) break;
      t = t2;
    }
  }

  // Combine the four waves' (m, l, O) in LDS.
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  __syncthreads();
  float* mw = reinterpret_cast<float*>(smem);  // [kWaves][16]
  float* lw = mw + kWaves * 16;                // [kWaves][16]
  float* ow = lw + kWaves * 16;                // [kWaves][16][OW_STRIDE]
  if (g == 0) {
    mw[wave * 16 + n] = m_run;
    lw[wave * 16 + n] = l_tot;
  }
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
    *reinterpret_cast<f32x4*>(ow + (wave * 16 + n) * C::OW_STRIDE + 16 * nb + 4 * g) = acc[nb];
  __syncthreads();

  const float vsc = FP8 ? p.v_scale[kvh] : 1.0f;
  for (int idx = tid; idx < heads_here * D; idx += kWaves * 64) {
    const int hh = idx / D, d = idx - (idx / D) * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mw[w * 16 + hh]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = __builtin_amdgcn_exp2f(mw[w * 16 + hh] - M);
      num += e * ow[(w * 16 + hh) * C::OW_STRIDE + d];
      den += e * lw[w * 16 + hh];
    }
    const float o = (num / den) * vsc;
    const float lse_nat = (M + log2f(den)) * 0.69314718055994530942f;
    if constexpr (DIRECT) {
      p.out[(row0 + hh) * D + d] = bit_cast_dev<uint16_t>((__bf16)o);
      if (d == 0 && p.lse) p.lse[row0 + hh] = lse_nat;
    } else {
      p.o_part[((row0 + hh) * S + split) * D + d] = o;
      if (d == 0) p.lse_part[(row0 + hh) * S + split] = lse_nat;
    }
  }
}

template <int D, bool FP8, bool PAGED16, bool DIRECT>
hipError_t launch_t(const SplitParams& p, int batch, hipStream_t stream) {
  const dim3 grid(DIRECT ? 1 : p.num_splits, p.hkv * p.head_groups, batch);
  hipLaunchKernelGGL((split_kv_kernel<D, FP8, PAGED16, DIRECT>), grid, dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool FP8>
hipError_t launch_d(const SplitParams& p, int batch, bool direct, bool paged16, hipStream_t s) {
  if (paged16) return direct ? launch_t<D, FP8, true, true>(p, batch, s) : launch_t<D, FP8, true, false>(p, batch, s);
  return direct ? launch_t<D, FP8, false, true>(p, batch, s) : launch_t<D, FP8, false, false>(p, batch, s);
}

}  // namespace

hipError_t launch_split_kv(const SplitParams& p, int batch, int head_dim, bool fp8, bool direct,
                           bool paged16, hipStream_t stream) {
  switch (head_dim) {
    case 32: return fp8 ? launch_d<32, true>(p, batch, direct, paged16, stream) : launch_d<32, false>(p, batch, direct, paged16, stream);
    case 64: return fp8 ? launch_d<64, true>(p, batch, direct, paged16, stream) : launch_d<64, false>(p, batch, direct, paged16, stream);
    case 128: return fp8 ? launch_d<128, true>(p, batch, direct, paged16, stream) : launch_d<128, false>(p, batch, direct, paged16, stream);
    case 256: return fp8 ? launch_d<256, true>(p, batch, direct, paged16, stream) : launch_d<256, false>(p, batch, direct, paged16, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkd
