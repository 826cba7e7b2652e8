// Split-KV paged decode attention for gfx950 (CDNA4): the partition kernels.
// Included by one translation unit per head dimension (decode_d*.hip), which
// instantiates the launchers below for its D, so the many kernel instances
// compile in parallel.
//
// Work is done by waves.  A wave owns a token range of one (sequence b, KV head)
// pair and up to 16 query heads of that KV head (GQA head packing: every K/V
// row read from HBM serves all query heads that share the KV head), and keeps
// its own online-softmax state for them.  Two launch shapes share that wave
// machinery (WaveAttn below):
//
//  * grid kernel: one workgroup of four waves per (split j, KV head, sequence);
//    the waves interleave the tiles of the split and combine their states in
//    LDS at the end.  One split writes out/lse directly; several write
//    partials for the merge kernel.
//  * balanced kernel: a persistent grid of one workgroup per compute unit;
//    every workgroup gets an equal share of the flattened (sequence, KV head,
//    head group, 16-token group) space, walks it segment by segment (its waves
//    interleaving each piece's tiles) and writes one partial per (workgroup,
//    segment) piece, or merges a segment's pieces itself when it completes
//    the segment.  Work per workgroup is equal whatever the length mix, and the
//    start-up latency chain (lengths -> block table -> first K/V) is paid once
//    per workgroup rather than once per split.
//
// The per-tile machinery (loads, MFMA tile step, pipeline, combine) is in
// wave_attn.hpp.
#pragma once

#include "lds_pipe.hpp"

namespace pkd {
namespace {

// Waves per SIMD the register allocation targets.  Two resident waves per
// SIMD hide the load latency of one another's tiles; the compiler keeps the
// MFMA accumulators in ordinary VGPRs to fit 256 registers.  The instances
// that would spill at two (bf16 K/V with per-row page lookups at D = 32 or
// 256) are left at one.  The balanced kernel runs one workgroup per compute
// unit, so it is not constrained.
template <int D, bool FP8, bool PAGED16>
constexpr int waves_per_simd() {
  if (!FP8 && !PAGED16 && (D == 32 || D == 256)) return 1;
  return 2;
}

// ---- grid kernel ----------------------------------------------------------

template <int D, bool FP8, bool PAGED16, bool DIRECT, bool STRIDED>
__global__ void __launch_bounds__(kWaves * 64)
    __attribute__((amdgpu_waves_per_eu(waves_per_simd<D, FP8, PAGED16>())))
split_kv_kernel(const SplitParams p) {
  typedef Cfg<D, FP8> C;
  typedef Geometry<D, FP8, STRIDED> Geo;
  typedef TilePages<D, FP8, PAGED16> Pages;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  WaveAttn<D, FP8> A;
  A.init_lane(tid & 63);

  const int split = blockIdx.x;
  const int kvh = blockIdx.y / p.head_groups;
  const int hg = blockIdx.y - kvh * p.head_groups;
  const int b = blockIdx.z;
  const int S = p.num_splits;

  const int L = p.seq_lens[b];
  const int chunk = p.chunk;  // tokens per split, the same for every sequence

  // Loads that do not depend on the length, issued while it is in flight: the
  // query rows, and (without a window, so that the split starts at token
  // split * chunk) the block-table entries the split can use, staged in LDS.
  // Entries past the sequence's last page may be among them; they are not used.
  int32_t* sbt = reinterpret_cast<int32_t*>(smem + C::BT_OFFSET);
  const bool contiguous = Geo::contiguous(p);
  const int ps = p.page_size;
  const int64_t spec_tok = (int64_t)split * chunk;
  const int spec_first = (int)min(spec_tok / ps, (int64_t)p.max_pages);
  const int spec_n = (int)min((int64_t)p.max_pages - spec_first, (int64_t)chunk / ps + 2);
  const bool spec = !contiguous && p.window == 0 && spec_n <= C::BT_ENTRIES;
  if (spec)
    for (int i = tid; i < spec_n; i += kWaves * 64) sbt[i] = p.block_table[(int64_t)b * p.max_pages + spec_first + i];
  {
    const LaneRow lq = lane_row<D, STRIDED>(p, b, kvh, hg, A.n, 0, 0, 0);
    A.load_q(p.q + lq.qoff, lq.valid);
  }

  // Splits cover [lo, L): tokens below the first visible 16-token group (with
  // a sliding window) are never read.
  const int lo = seq_first_token(p, L, p.window);
  const int s0 = (int)min((int64_t)lo + (int64_t)split * chunk, (int64_t)L);
  const int s1 = (int)min((int64_t)s0 + chunk, (int64_t)L);
  const int heads_here = min(kHeadsPerGroup, p.rows_kv - hg * kHeadsPerGroup);
  // Row indices and out offsets of the workgroup's packed rows (query token, head).
  __shared__ int64_t s_rows[kHeadsPerGroup];
  __shared__ int64_t s_orow[kHeadsPerGroup];

  if (s0 >= s1) {
    // Empty split (or an empty sequence): o = 0, lse = -inf (the sink logit
    // for a direct row with a sink).
    for (int idx = tid; idx < heads_here * D; idx += kWaves * 64) {
      const int hh = idx / D, d = idx - (idx / D) * D;
      const int r = hg * kHeadsPerGroup + hh;
      const int qi = r / p.group, h = kvh * p.group + (r - qi * p.group);
      const int64_t row = ((int64_t)b * p.q_len + qi) * p.hq + h;
      if constexpr (DIRECT) {
        p.out[Geo::os(p).at(b, qi, h) + d] = 0;
        if (d == 0 && p.lse) p.lse[row] = p.sinks ? p.sinks[(int)(row % p.hq)] : -INFINITY;
      } else {
        p.o_part[(row * S + split) * D + d] = 0.f;
        if (d == 0) p.lse_part[row * S + split] = -INFINITY;
      }
    }
    return;
  }

  const int ntiles = (s1 - s0 + C::TT - 1) / C::TT;
  const int lim = s1 - 1;
  const int tok_stride = Geo::tok_stride(p);  // bytes between consecutive slots of a page
  const int64_t page_stride = Geo::page_stride(p);
  const int64_t head_off = (int64_t)kvh * Geo::head_stride(p);
  // The block table is read-only for the whole launch (constant address space).
  const __attribute__((address_space(4))) int32_t* bt =
      (const __attribute__((address_space(4))) int32_t*)(p.block_table + (int64_t)b * p.max_pages);

  const LaneRow lr = lane_row<D, STRIDED>(p, b, kvh, hg, A.n, L, s1, p.window);
  if (tid < kHeadsPerGroup) {  // read after the barriers below
    s_rows[tid] = lr.row;
    s_orow[tid] = lr.ooff;
  }
  A.qk_scale = p.qk_scale_log2;
  if constexpr (FP8) A.qk_scale *= p.k_scale[kvh];
  A.reset();

  // The split's block-table entries are staged in LDS once (when they fit), so
  // that per-tile page lookups are short LDS reads rather than dependent HBM
  // reads on the path of every tile's loads (already done above without a
  // window: there the split's first page is spec_first).  Without a block
  // table (contiguous K/V) sequence b is page b.
  const int first_page = s0 / ps;
  const int n_pages = lim / ps - first_page + 1;
  const bool staged = spec || (!contiguous && n_pages <= C::BT_ENTRIES);
  if (staged && !spec)
    for (int i = tid; i < n_pages; i += kWaves * 64) sbt[i] = bt[first_page + i];
  __syncthreads();
  auto page_of = [&](int pidx) -> int { return contiguous ? b : staged ? sbt[pidx - first_page] : bt[pidx]; };

  auto fetch = [&](int tile, Pages& P) {
    const int tb = s0 + tile * C::TT;
    if constexpr (PAGED16) {
#pragma unroll
      for (int q = 0; q < C::NGRP; ++q) P.pg[q] = page_of((min(tb + 16 * q, lim) & ~15) / ps);
    } else {
#pragma unroll
      for (int i = 0; i < (C::KLDS ? C::NV : C::NBLK + C::NV); ++i)
        P.pg[i] = page_of(min(tb + A.generic_row(i), lim) / ps);
    }
  };
  auto issue = [&](int tile, const Pages& P, TileRegs<D, FP8>& R, bool idle) {
    const int tb = s0 + tile * C::TT;
    if constexpr (PAGED16)
      A.issue_paged16(p.k, p.v, tb, lim, P.pg, ps, tok_stride, page_stride, head_off, R, idle);
    else
      A.issue_generic(p.k, p.v, tb, lim, P.pg, ps, tok_stride, page_stride, head_off, R, idle);
  };

  uint16_t* vs = reinterpret_cast<uint16_t*>(smem) + wave * C::WT;  // this wave's V[TT][VS] (and K[TT][KS])
  // Tiles wave, wave + 4, wave + 8, ...
  run_tiles<D, FP8, Pages>(A, wave, kWaves, ntiles, s0, lr, vs, fetch, issue);

  const float vsc = FP8 ? p.v_scale[kvh] : 1.0f;
  auto store = [&](int hh, int d0, f32x4 o, float lse_nat) {
    const int64_t row = s_rows[hh];
    if constexpr (DIRECT) {
      *reinterpret_cast<bf16x4*>(p.out + s_orow[hh] + d0) = to_bf16x4(o);
      if (d0 == 0 && p.lse) p.lse[row] = lse_nat;
    } else {
      *reinterpret_cast<f32x4*>(p.o_part + (row * S + split) * D + d0) = o;
      if (d0 == 0) p.lse_part[row * S + split] = lse_nat;
    }
  };
  if (DIRECT && p.sinks)
    wg_combine<D, FP8>(A, smem, wave, tid, heads_here, vsc, store,
                       [&](int hh) { return p.sinks[(int)(s_rows[hh] % p.hq)]; });
  else
    wg_combine<D, FP8>(A, smem, wave, tid, heads_here, vsc, store, NoSink());
}

// ---- balanced persistent kernel ---------------------------------------------
//
// The work space is the sequence of segments s = (b * Hkv + kvh) * HG + hg
// (HG head groups of up to 16 query rows per KV head), segment s holding the
// n_b = ceil((L_b - lo_b) / 16) 16-token groups of sequence b, from its first
// visible group lo_b (0 without a sliding window); T groups in all.  With
// NWE = min(workgroups, T) active workgroups, workgroup w takes groups
// [floor(w T / NWE), floor((w + 1) T / NWE)); its waves interleave the
// tiles of each piece (the part of one segment inside the range) and combine
// in LDS.  Each (workgroup, segment) piece writes its normalised partial and
// LSE to slot w + s, which is unique and increasing along the work space; the
// merge kernel finds segment s's pieces from the same formula.  page_size
// must be a multiple of 16.

// Paired whole items (the balanced kernel's paired mode).  Items are the
// segments of the non-empty sequences, ranked by length (groups per segment,
// ties by sequence).  With N items on W workgroups and E = N - W: for E <= 0
// each workgroup takes one item, for 0 < E <= W the E workgroups of the 2E
// shortest items take two (folded: the shortest with the longest of them), the
// others one.  The plan is taken when no workgroup then holds more than 1.6x
// the mean work per workgroup (T / W groups): whole items need no partial, no
// count and no merge, which measured worth that much imbalance.  Otherwise
// (or with more than 2W items) the kernel uses its equal ranges.
// Every thread computes the same plan; rank_b[r] is the sequence of rank r.
struct PairPlan {
  bool ok;
  int items;
};

template <int NWV>
__device__ PairPlan pair_plan(const int64_t* spre, int B, int SPB, int64_t T, int W, int tid, int64_t* red,
                              int16_t* rank_b, uint32_t* keys) {
  constexpr int NT = NWV * 64;
  static_assert(NT >= kPairedMaxBatch, "one thread per sequence");
  PairPlan r{false, 0};
  if (B > kPairedMaxBatch) return r;
  const int B4 = (B + 3) & ~3;
  // Key of sequence i: groups per segment above its index (0xFFFFFFFF: empty).
  if (tid < B4) {
    uint32_t k = 0xFFFFFFFFu;
    if (tid < B) {
      const int64_t g = (spre[tid + 1] - spre[tid]) / SPB;
      if (g > 0) k = ((uint32_t)g << 8) | (uint32_t)tid;
    }
    keys[tid] = k;
  }
  __syncthreads();
  int nonempty = 0;
  if (tid < B) {
    const uint32_t mk = keys[tid];
    if (mk != 0xFFFFFFFFu) {
      int rank = 0;
      for (int j = 0; j < B4; j += 4) {
        const uint4 k4 = *reinterpret_cast<const uint4*>(keys + j);
        rank += (int)(k4.x < mk) + (int)(k4.y < mk) + (int)(k4.z < mk) + (int)(k4.w < mk);
      }
      rank_b[rank] = (int16_t)tid;
      nonempty = 1;
    }
  }
  const int N = __syncthreads_count(nonempty) * SPB;
  const int E = N - W;
  r.items = N;
  if (E > W) return r;
  auto nb_of = [&](int item) -> int64_t {
    const int bb = rank_b[item / SPB];
    return (spre[bb + 1] - spre[bb]) / SPB;
  };
  int64_t m = (tid == 0 && N > 0) ? nb_of(N - 1) : 0;
  for (int g = tid; g < E; g += NT) m = max(m, nb_of(g) + nb_of(2 * E - 1 - g));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (int64_t)__shfl_xor(m, off));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  int64_t M = 0;
#pragma unroll
  for (int v = 0; v < NWV; ++v) M = max(M, red[v]);
  r.ok = 5 * M * W <= 8 * T;
  __syncthreads();  // red and keys are reused
  return r;
}

// VK > 1 pairs KV heads whose rows share 128-byte lines: the kernel runs on
// "wide" heads of D = VK * DR dims (VK adjacent real heads, the parameters'
// hkv and group counting wide heads), each query row zero-padded outside its
// own head's dims, and writes only its own head's DR dims (see load_q).  Each
// line is then read once, by one workgroup.
// LDSP: the tiles are loaded straight into LDS stages by the FP8 pipeline of
// lds_pipe.hpp (LdsPipeF8) instead of being held in registers (run_tiles):
// FP8 D = 128 in the paged layout, without a window or paired heads.  Its two
// waves per SIMD as the register budget keep the accumulators in VGPRs.
template <int D, bool FP8, int NWV, bool STRIDED, bool WINDOW, bool SINKS, int VK, bool LDSP = false>
__global__ void __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(LDSP ? 2 : NWV / 4)))
balanced_kernel(const BalancedParams p) {
  static_assert(!LDSP || (D == kLpD && FP8 && !STRIDED && !WINDOW && VK == 1), "LDS-staged instance");
  typedef Cfg<D, FP8> C;
  constexpr int DR = D / VK;  // dims of a real head
  typedef Geometry<D, FP8, STRIDED> Geo;    // K/V rows (of wide heads when paired)
  typedef Geometry<DR, FP8, STRIDED> GeoQ;  // q / out rows, which are real heads' rows
  // Without a window (the instance for window = 0) nothing of it stays live.
  const int win = WINDOW ? p.window : 0;
  typedef TilePages<D, FP8, true> Pages;
  constexpr int VT_BYTES = LDSP ? NWV * kLfWaveB : NWV * C::WT * 2;  // wave-private tiles or LDS stages
  constexpr int MERGE_BYTES = NWV * 16 * (2 + C::OW_STRIDE) * 4 + 16 * (NWV + 4) * 4;  // combine staging
  constexpr int SMEM = VT_BYTES > MERGE_BYTES ? VT_BYTES : MERGE_BYTES;
  static_assert(SMEM >= kPairedMaxBatch * 4, "paired-mode keys");
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  __shared__ int64_t spre[kBalancedMaxBatch + 1];  // spre[b] = groups of all segments of sequences < b
  __shared__ int64_t stot[NWV];
  __shared__ int s_last;                           // in-kernel merge: this piece completes its segment
  __shared__ int64_t s_rows[kHeadsPerGroup];       // row indices of the current piece's packed rows
  __shared__ int64_t s_orow[kHeadsPerGroup];       // their out offsets
  __shared__ int s_slice[kHeadsPerGroup];          // paired heads: the row's head within its wide head
  __shared__ int16_t s_rank_b[kPairedMaxBatch];    // paired mode: the non-empty sequences by length rank

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int B = p.batch;
  const int SPB = p.hkv * p.head_groups;  // segments per sequence

  // Prefix sums of the group counts (every workgroup computes them; workgroup 0
  // also stores them for the merge kernel): thread t sums sequences 4t..4t+3,
  // a shuffle scan runs inside each wave, and the wave totals are added across
  // waves through LDS.
  {
    constexpr int PER = kBalancedMaxBatch / (NWV * 64);
    const int lane = tid & 63;
    int64_t run[PER];
    int64_t sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int bb = tid * PER + i;
      const int L = bb < B ? p.seq_lens[bb] : 0;
      sum += (int64_t)((L - seq_first_token(p, L, win) + 15) >> 4) * SPB;
      run[i] = sum;
    }
    int64_t incl = sum;  // inclusive scan of the thread sums within the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t up = __shfl_up(incl, off);
      if (lane >= off) incl += up;
    }
    if (lane == 63) stot[wave] = incl;
    __syncthreads();
    int64_t base = incl - sum;
    for (int v = 0; v < wave; ++v) base += stot[v];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int bb = tid * PER + i;
      if (bb < B) spre[bb + 1] = base + run[i];
    }
    if (tid == 0) spre[0] = 0;
    __syncthreads();
  }
  const int64_t T = spre[B];
  if (blockIdx.x == 0)
    for (int i = tid; i <= B; i += NWV * 64) p.prefix[i] = spre[i];
  const int64_t nwe = min((int64_t)p.num_workers, T);
  // Workgroups are dealt to the XCDs round-robin (workgroup i runs on XCD
  // i % kXcds).  With xcd_ranges, and every worker busy, worker ranges are
  // assigned so that each XCD takes one contiguous 1/kXcds of the work space:
  // the KV heads of a sequence then stream the same tokens on the same XCD, so
  // that heads whose rows share 128-byte lines fetch each line from HBM once
  // and find it in that XCD's L2 for the other head.
  const int N = p.num_workers;
  const int64_t w = (p.xcd_ranges && T >= N && N % kXcds == 0)
                        ? (int64_t)(blockIdx.x % kXcds) * (N / kXcds) + blockIdx.x / kXcds
                        : (int64_t)blockIdx.x;
  if (p.fused) {
    // Sequences of length 0 have no piece: out = 0, lse = -inf (or the head's
    // sink logit) for all their q_len * Hq rows (workgroup bb % W).
    const int rows_seq = p.q_len * p.hq;
    for (int bb = (int)w; bb < B; bb += p.num_workers) {
      if (spre[bb + 1] != spre[bb]) continue;
      for (int i = tid; i < rows_seq * DR; i += NWV * 64) {
        const int rr = i / DR, qi = rr / p.hq;
        p.out[GeoQ::os(p).at(bb, qi, rr - qi * p.hq) + (i - rr * DR)] = 0;
      }
      if (p.lse)
        for (int i = tid; i < rows_seq; i += NWV * 64)
          p.lse[(int64_t)bb * rows_seq + i] = SINKS ? p.sinks[i % p.hq] : -INFINITY;
    }
  }
  // Paired whole items (p.paired): each workgroup takes one or two whole
  // segments, chosen from the lengths, or the ranges below when that choice
  // would leave a workgroup too much work.
  int pi_n = 0;              // segments this workgroup takes in paired mode (0: ranges)
  int pi_b[2] = {0, 0}, pi_s[2] = {0, 0};
  bool paired = false;
  if (p.paired) {
    const PairPlan pl = pair_plan<NWV>(spre, B, SPB, T, p.num_workers, tid, stot, s_rank_b,
                                       reinterpret_cast<uint32_t*>(smem));
    paired = pl.ok;
    if (paired) {
      const int wi = blockIdx.x;
      // Items by rank, ascending in length: with E = N - W > 0 extra items,
      // workgroup g < E takes items g and 2E - 1 - g (the 2E shortest, folded
      // so that each pair's lengths add up to about the same), every other
      // workgroup one item of the N - 2E longest.
      int it0, it1;
      paired_items(wi, pl.items, p.num_workers, &it0, &it1);
      if (it0 >= 0) {
        pi_n = it1 >= 0 ? 2 : 1;
        pi_b[0] = s_rank_b[it0 / SPB];
        pi_s[0] = it0 % SPB;
        if (it1 >= 0) {
          pi_b[1] = s_rank_b[it1 / SPB];
          pi_s[1] = it1 % SPB;
        }
      }
    }
  }
  if (paired ? pi_n == 0 : w >= nwe) return;  // the whole workgroup leaves together

  int64_t pos = paired ? 0 : w * T / nwe;
  const int64_t hi = paired ? 0 : (w + 1) * T / nwe;
  int pi = 0;  // paired mode: index of the current item

  // The sequence holding group pos: spre[b] <= pos < spre[b + 1].
  int b = 0;
  if (paired) {
    b = pi_b[0];
  } else {
    int lo_b = 0, hi_b = B;
    while (hi_b - lo_b > 1) {
      const int mid = (lo_b + hi_b) >> 1;
      if (spre[mid] <= pos) lo_b = mid; else hi_b = mid;
    }
    b = lo_b;
  }
  int64_t nb = (spre[b + 1] - spre[b]) / SPB;  // groups per segment of sequence b
  int seg = paired ? pi_s[0] : (int)((pos - spre[b]) / nb);
  int grp = paired ? 0 : (int)((pos - spre[b]) - (int64_t)seg * nb);

  WaveAttn<D, FP8> A;
  A.init_lane(tid & 63);
  uint16_t* vs = reinterpret_cast<uint16_t*>(smem) + wave * C::WT;
  const int ps = p.page_size;
  const int tok_stride = Geo::tok_stride(p);
  const int64_t page_stride = Geo::page_stride(p);
  LdsPipeF8 pipe;
  if constexpr (LDSP) pipe.init(smem, wave * kLfWaveB, A, tid & 63, tok_stride);

  // Page window of a piece: lane j holds block-table entry first_page + j of
  // sequence bb (entries past the row are not read; entries past the pieces's
  // last page are never used).  The next piece's window is loaded while the
  // current piece runs.  Without a block table (contiguous K/V) sequence bb is
  // page bb, its only page.
  auto load_window = [&](int bb, int first_page) -> int {
    if (Geo::contiguous(p)) return bb;
    const int idx = first_page + A.lane;
    return idx < p.max_pages ? p.block_table[(int64_t)bb * p.max_pages + idx] : 0;
  };
  // First visible token (16-aligned) of a sequence: where its groups start.
  auto first_of = [&](int bb) -> int { return WINDOW ? seq_first_token(p, p.seq_lens[bb], win) : 0; };
  int lo = first_of(b);
  int window = load_window(b, (lo + grp * 16) / ps);

  for (;;) {
    const int gend = paired ? (int)nb : (int)min(nb, (int64_t)grp + (hi - pos));
    const int L = p.seq_lens[b];
    const int s0 = lo + grp * 16;
    const int s1 = min(lo + gend * 16, L);
    const int lim = s1 - 1;
    const int kvh = seg / p.head_groups;
    const int hg = seg - kvh * p.head_groups;
    const int heads_here = min(kHeadsPerGroup, p.rows_kv - hg * kHeadsPerGroup);
    const LaneRow lr = lane_row<DR, STRIDED>(p, b, kvh, hg, A.n, L, s1, win);
    // Paired heads: the lane's row belongs to real head kvh * VK + slice.
    const int slice = VK > 1 ? (lr.head / (p.group / VK)) % VK : 0;
    if (tid < kHeadsPerGroup) {  // read after the combine's barriers
      s_rows[tid] = lr.row;
      s_orow[tid] = lr.ooff;
      s_slice[tid] = slice;
    }
    const int64_t head_off = (int64_t)kvh * Geo::head_stride(p);

    // The next piece: the following segment (of this or a later sequence), or
    // in paired mode this workgroup's second item.
    const int64_t npos = pos + (gend - grp);
    int nseg = seg + 1, nbq = b;
    bool more;
    if (paired) {
      more = pi + 1 < pi_n;
      nbq = more ? pi_b[1] : B;
      nseg = more ? pi_s[1] : 0;
    } else {
      if (nseg == SPB) {
        nseg = 0;
        do { ++nbq; } while (nbq < B && spre[nbq + 1] == spre[nbq]);
      }
      more = npos < hi;
    }
    const int nlo = more ? (nbq == b ? lo : first_of(nbq)) : 0;
    const int next_window = more ? load_window(nbq, nlo / ps) : 0;

    A.template load_q<VK>(p.q + lr.qoff, lr.valid, slice);
    A.qk_scale = p.qk_scale_log2;
    if constexpr (FP8) A.qk_scale *= p.k_scale[kvh * VK + slice];
    A.reset();

    const int first_page = s0 / ps;
    const __attribute__((address_space(4))) int32_t* btc =
        (const __attribute__((address_space(4))) int32_t*)(p.block_table + (int64_t)b * p.max_pages);
    auto page_of = [&](int pidx) -> int {
      const int rel = pidx - first_page;
      return rel < 64 ? __builtin_amdgcn_readlane(window, rel) : btc[pidx];
    };
    auto fetch = [&](int tile, Pages& P) {
      const int tb = s0 + tile * C::TT;
#pragma unroll
      for (int q = 0; q < C::NGRP; ++q) P.pg[q] = page_of((min(tb + 16 * q, lim) & ~15) / ps);
    };
    auto issue = [&](int tile, const Pages& P, TileRegs<D, FP8>& R, bool idle) {
      A.issue_paged16(p.k, p.v, s0 + tile * C::TT, lim, P.pg, ps, tok_stride, page_stride, head_off, R, idle);
    };
    const int ntiles = (s1 - s0 + C::TT - 1) / C::TT;
    if constexpr (LDSP)
      lds_pipe_run_ns<kLfStages>(pipe, A, wave, NWV, ntiles, s0, s1, lr.end, lr.end_min, p.k, p.v, [&](int t) -> int64_t {
        return (int64_t)page_of(t / ps) * page_stride + (int64_t)(t % ps) * tok_stride + head_off;
      });
    else
      run_tiles<D, FP8, Pages>(A, wave, NWV, ntiles, s0, lr, vs, fetch, issue);

    // This segment's pieces are those of workgroups w_first .. w_last, at
    // slots w + s (s = b * SPB + seg).
    const int64_t sidx = (int64_t)b * SPB + seg;
    const int64_t seg_pos = spre[b] + (int64_t)seg * nb;
    int64_t w_first;
    int npieces;
    segment_pieces(seg_pos, nb, nwe, T, &w_first, &npieces);
    if (paired) npieces = 1;
    // Row hh's V scale, and whether dims d0.. of the wide row are its own head's
    // (always, without pairing); own_dim gives their place in the real row.
    const float vsc = FP8 ? p.v_scale[kvh * VK] : 1.0f;
    auto vsc_of = [&](int hh) -> float { return FP8 && VK > 1 ? p.v_scale[kvh * VK + s_slice[hh]] : vsc; };
    auto mine = [&](int hh, int d0) -> bool { return VK == 1 || d0 / DR == s_slice[hh]; };
    auto own_dim = [&](int hh, int d0) -> int { return VK == 1 ? d0 : d0 - s_slice[hh] * DR; };
    if (p.fused && npieces == 1) {
      // The whole segment is this piece: write the result directly.
      auto store = [&](int hh, int d0, f32x4 o, float lse_nat) {
        if (!mine(hh, d0)) return;
        const int64_t row = s_rows[hh];
        const int dd = own_dim(hh, d0);
        *reinterpret_cast<bf16x4*>(p.out + s_orow[hh] + dd) = to_bf16x4(o);
        if (dd == 0 && p.lse) p.lse[row] = lse_nat;
      };
      if constexpr (SINKS)
        wg_combine_rows<D, FP8, NWV>(A, smem, wave, tid, heads_here, vsc_of, store,
                                     [&](int hh) { return p.sinks[(int)(s_rows[hh] % p.hq)]; });
      else
        wg_combine_rows<D, FP8, NWV>(A, smem, wave, tid, heads_here, vsc_of, store, NoSink());
      __syncthreads();  // the LDS is reused by the next piece
    } else {
      // This piece's partial, for the group's heads (DR dims per row).
      const int64_t slot = w + sidx;
      float* orow = p.o_part + slot * p.hpg * DR;
      float* lrow = p.lse_part + slot * p.hpg;
      if (!p.fused) {
        wg_combine_rows<D, FP8, NWV>(A, smem, wave, tid, heads_here, vsc_of,
                                     [&](int hh, int d0, f32x4 o, float lse_nat) {
          if (!mine(hh, d0)) return;
          const int dd = own_dim(hh, d0);
          *reinterpret_cast<f32x4*>(orow + hh * DR + dd) = o;
          if (dd == 0) lrow[hh] = lse_nat;
        }, NoSink());
      } else {
        // Release, done by hand: agent-scope atomic stores write through this
        // XCD's L2 to the agent's coherent memory, and vmcnt(0) waits until the
        // memory has acknowledged every one of them, so the partial is visible to
        // any agent-scope reader before the count below is taken.  That is what
        // an agent-scope release fence does for such stores; the fence would
        // also write back the XCD's whole L2 (for ordinary stores, of which
        // there are none here), which is far too costly per piece.
        wg_combine_rows<D, FP8, NWV>(A, smem, wave, tid, heads_here, vsc_of,
                                     [&](int hh, int d0, f32x4 o, float lse_nat) {
          if (!mine(hh, d0)) return;
          const int dd = own_dim(hh, d0);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            __hip_atomic_store(orow + hh * DR + dd + i, o[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (dd == 0) __hip_atomic_store(lrow + hh, lse_nat, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }, NoSink());
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's stores are acknowledged
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        // Count this piece in; the last of the segment's pieces merges them.
        __syncthreads();
        if (tid == 0) {
          const uint64_t E = p.epoch;
          uint64_t* cw = p.seg_count + sidx;
          uint64_t old = __hip_atomic_load(cw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          uint64_t nv;
          do {
            nv = count_word_add(old, E);
          } while (!__hip_atomic_compare_exchange_weak(cw, &old, nv, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT));
          const bool last = count_word_pieces(nv) == npieces;
          if (last) {
            // Acquire at agent scope: the other pieces' partials, which their
            // counts made visible before this count saw them, are read after it.
            // Only a merging piece pays for it (one per multi-piece segment).
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            __hip_atomic_store(cw, count_word_reset(E), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          s_last = last;
        }
        __syncthreads();
        const bool last = s_last != 0;
        if (last) {
          // The pieces' partials, read from the coherent copy.  Wave w merges
          // rows w, w + NWV, ...  With few pieces the loads of RC rows at a
          // time are issued before any of them is combined (RC rows of staged
          // partials take at most 64 registers under a one-wave-per-SIMD
          // register budget, 32 under two); otherwise, or when only one row
          // fits, one row at a time.
          const int64_t slot0 = w_first + sidx;
          typedef RowMerge<DR, true> RM;
          constexpr int MAXR = kHeadsPerGroup / NWV;
          constexpr int RC_REG = (NWV > 4 || LDSP ? 32 : 64) / (RM::UNROLL * RM::EPL);
          constexpr int RC = RC_REG < MAXR ? RC_REG : MAXR;
          const float* lp0 = p.lse_part + slot0 * p.hpg;
          const float* op0 = p.o_part + slot0 * p.hpg * DR;
          const int64_t ls = p.hpg, os = (int64_t)p.hpg * DR;
          const int lane = tid & 63;
          if (RC < 2 || npieces > RM::UNROLL) {
            for (int hh = wave; hh < heads_here; hh += NWV) {
              RM r;
              r.run(lp0 + hh, ls, op0 + hh * DR, os, npieces, lane);
              const int64_t row = s_rows[hh];
              r.store(p.out + s_orow[hh], p.lse ? p.lse + row : nullptr, lane,
                      SINKS ? p.sinks[(int)(row % p.hq)] : -INFINITY);
            }
          } else {
            constexpr int RCS = RC < 2 ? 2 : RC;  // (the branch above takes RC < 2)
#pragma unroll
            for (int k0 = 0; k0 < MAXR; k0 += RCS) {
              typename RM::Staged st[RCS];
#pragma unroll
              for (int k = 0; k < RCS; ++k) {
                const int hh = wave + (k0 + k) * NWV;
                if (hh < heads_here) RM::issue(lp0 + hh, ls, op0 + hh * DR, os, npieces, lane, st[k]);
              }
#pragma unroll
              for (int k = 0; k < RCS; ++k) {
                const int hh = wave + (k0 + k) * NWV;
                if (hh < heads_here) {
                  RM r;
                  r.finish(st[k], npieces, lane);
                  const int64_t row = s_rows[hh];
                  r.store(p.out + s_orow[hh], p.lse ? p.lse + row : nullptr, lane,
                          SINKS ? p.sinks[(int)(row % p.hq)] : -INFINITY);
                }
              }
            }
          }
        }
      }
      __syncthreads();  // the LDS is reused by the next piece
    }
    if (!more) break;
    pos = npos;
    ++pi;
    grp = 0;
    seg = nseg;
    if (nbq != b) {
      b = nbq;
      lo = nlo;
      nb = (spre[b + 1] - spre[b]) / SPB;
    }
    window = next_window;
  }
}

template <int D, bool FP8, bool PAGED16, bool DIRECT>
hipError_t launch_t(const SplitParams& p, int batch, bool strided, hipStream_t stream) {
  const dim3 grid(DIRECT ? 1 : p.num_splits, p.hkv * p.head_groups, batch);
  if (strided)
    hipLaunchKernelGGL((split_kv_kernel<D, FP8, PAGED16, DIRECT, true>), grid, dim3(kWaves * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((split_kv_kernel<D, FP8, PAGED16, DIRECT, false>), grid, dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool FP8>
hipError_t launch_d(const SplitParams& p, int batch, bool direct, bool paged16, bool strided, hipStream_t s) {
  if (paged16)
    return direct ? launch_t<D, FP8, true, true>(p, batch, strided, s) : launch_t<D, FP8, true, false>(p, batch, strided, s);
  return direct ? launch_t<D, FP8, false, true>(p, batch, strided, s) : launch_t<D, FP8, false, false>(p, batch, strided, s);
}


// Waves per balanced workgroup: four (one per SIMD) for bf16 K/V; eight for
// FP8, whose tiles carry half the bytes, so that as many bytes are in flight
// per compute unit (measured: 3% faster for FP8, 4-20% slower for bf16).
constexpr int balanced_waves(bool fp8) { return fp8 ? 8 : 4; }
// Waves per workgroup of the LDS-staged FP8 instance (16 KiB of stages each).
constexpr int kBalancedLdsWaves = 8;

// Instances without a window or without sinks keep none of their state live
// (the kernel is at the edge of its scalar registers).
// FP8 D = 128 in the paged layout without a window or pairing runs the
// LDS-staged tile pipeline.
template <int D, bool FP8, bool STRIDED, bool WINDOW, int VK = 1>
void launch_bw(const BalancedParams& p, hipStream_t stream) {
  constexpr bool LDSP = D == kLpD && FP8 && !STRIDED && !WINDOW && VK == 1;
  constexpr int NWV = LDSP ? kBalancedLdsWaves : balanced_waves(FP8);
  if (p.sinks)
    hipLaunchKernelGGL((balanced_kernel<D, FP8, NWV, STRIDED, WINDOW, true, VK, LDSP>), dim3(p.num_workers),
                       dim3(NWV * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((balanced_kernel<D, FP8, NWV, STRIDED, WINDOW, false, VK, LDSP>), dim3(p.num_workers),
                       dim3(NWV * 64), 0, stream, p);
}

template <int D, bool FP8, bool STRIDED>
void launch_bs(const BalancedParams& p, hipStream_t stream) {
  if (p.window > 0)
    launch_bw<D, FP8, STRIDED, true>(p, stream);
  else
    launch_bw<D, FP8, STRIDED, false>(p, stream);
}

template <int D, bool FP8>
hipError_t launch_b(const BalancedParams& p, bool strided, hipStream_t stream) {
  if (p.pair_heads > 1) {
    // Paired KV heads (D is the wide head's dims): the paged layout without a window.
    if constexpr (D == 64 || D == 128) {
      if (strided || p.window > 0 || p.pair_heads != 2) return hipErrorInvalidValue;
      launch_bw<D, FP8, false, false, 2>(p, stream);
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (strided)
    launch_bs<D, FP8, true>(p, stream);
  else
    launch_bs<D, FP8, false>(p, stream);
  return hipGetLastError();
}

}  // namespace

// The launchers for one head dimension (explicitly instantiated per D).
template <int D>
hipError_t launch_split_kv_dim(const SplitParams& p, int batch, bool fp8, bool direct, bool paged16, bool strided,
                               hipStream_t stream) {
  return fp8 ? launch_d<D, true>(p, batch, direct, paged16, strided, stream)
             : launch_d<D, false>(p, batch, direct, paged16, strided, stream);
}

template <int D>
hipError_t launch_balanced_dim(const BalancedParams& p, bool fp8, bool strided, hipStream_t stream) {
  return fp8 ? launch_b<D, true>(p, strided, stream) : launch_b<D, false>(p, strided, stream);
}

}  // namespace pkd
