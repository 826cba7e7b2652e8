// Direct output (out and lse written directly, nothing merged) with the K/V
// tiles loaded straight into LDS stages by the pipelines of lds_pipe.hpp,
// instead of being held in registers for one tile as the grid kernel does:
// four waves per workgroup for a bf16 cache, eight for FP8 codes.  paged_decode
// runs it for D = 128 decode of one query token per sequence without a window
// (sinks or not) whose (sequence, KV head) items fit one round of workgroups
// (one workgroup per item) or two (the pairs form: one workgroup per compute
// unit, each taking one or two whole items paired by length on the device);
// pkd_decode_lds exposes the bf16 one-per-item form for measurement beside the
// grid kernel.  It also computes several query tokens under the causal mask
// (q_len * G <= 16 rows, bit for bit the grid kernel's), but four tokens at
// B = 32 ran 1% slower than the grid kernel, so paged_decode does not send
// them.  The arithmetic is the grid kernel's: bf16 results equal the grid
// kernel's bit for bit; FP8 runs eight waves, whose grouping of the tiles in
// the workgroup combine rounds differently from the grid kernel's four.
#include "../../include/pkd_lds.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "lds_pipe.hpp"

namespace pkd {
namespace {

constexpr int kBtEntries = 512;                // staged block-table entries (after the stages)

// The two instances: bf16 K/V (16-token tiles, two stages of 8 KiB per wave,
// four waves) and FP8 codes (32-token tiles, two stages of 8 KiB per wave,
// eight waves, so that a compute unit keeps about as many bytes in flight).
template <bool FP8>
struct LdsDirect {
  typedef LdsPipe Pipe;
  static constexpr int NW = 4;          // waves per workgroup
  static constexpr int WAVE_B = kLpWaveB;
};
template <>
struct LdsDirect<true> {
  typedef LdsPipeF8 Pipe;
  static constexpr int NW = 8;
  static constexpr int WAVE_B = kLfWaveB;
};
template <bool FP8>
constexpr int lds_bt_offset() { return LdsDirect<FP8>::NW * LdsDirect<FP8>::WAVE_B; }
template <bool FP8>
constexpr int lds_bytes() { return lds_bt_offset<FP8>() + kBtEntries * 4; }
// The workgroup combine's staging (per-wave rows and weights) reuses the stages.
static_assert(4 * 16 * (2 + Cfg<kLpD, false>::OW_STRIDE) * 4 + 16 * (4 + 4) * 4 <= lds_bt_offset<false>(),
              "combine staging");
static_assert(8 * 16 * (2 + Cfg<kLpD, true>::OW_STRIDE) * 4 + 16 * (8 + 4) * 4 <= lds_bt_offset<true>(),
              "combine staging");

// Items (sequence, KV head) of one launch, in the pairs form: with N = B * Hkv
// items on W workgroups (W < N <= 2W), the sequences are ranked by length
// (ties by index), items by their sequence's rank; workgroup g < E = N - W
// takes items 2E - 1 - g and g (the 2E shortest, folded so that the pairs'
// lengths come out about even), every other workgroup the one item g + E.
// The longest items thus run alone, and the pairs finish inside the time of
// the longest item unless the shortest are nearly as long as it.  Every
// workgroup computes the same ranking; keys are staged in LDS (kb, B + 3
// words) and rank_b[r] receives the sequence of rank r.
__device__ void lds_pair_items(const SplitParams& p, int batch, int tid, uint32_t* kb, int16_t* rank_b,
                               int (&items)[2]) {
  const int B4 = (batch + 3) & ~3;
  if (tid < B4) {
    // Lengths are clamped to [0, 2^23) (the host admits no larger capacity), so
    // keys are distinct and below 2^31 and the ranks a permutation.
    const int L = tid < batch ? min(max(p.seq_lens[tid], 0), (1 << 23) - 1) : 0;
    kb[tid] = tid < batch ? ((uint32_t)L << 8) | (uint32_t)tid : 0xFFFFFFFFu;
  }
  __syncthreads();
  if (tid < batch) {
    const uint32_t mk = kb[tid];
    int rank = 0;
    for (int j = 0; j < B4; j += 4) {
      const uint4 k4 = *reinterpret_cast<const uint4*>(kb + j);
      rank += (int)(k4.x < mk) + (int)(k4.y < mk) + (int)(k4.z < mk) + (int)(k4.w < mk);
    }
    rank_b[rank] = (int16_t)tid;
  }
  __syncthreads();
  paired_items(blockIdx.x, batch * p.hkv, gridDim.x, &items[0], &items[1]);
}

// Two waves per SIMD as the register budget (as the grid kernel): the
// accumulators then stay in ordinary VGPRs, where the rescale reaches them.
// PAIRS = false: grid (Hkv, B), one item per workgroup.  PAIRS = true: a 1D
// grid of W workgroups taking the items as lds_pair_items deals them (batch
// <= kPairedMaxBatch).  FP8: codes dequantised with the KV head's scales.
template <bool FP8, bool PAIRS>
__global__ void __launch_bounds__(LdsDirect<FP8>::NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
lds_direct_kernel(const SplitParams p, int batch) {
  typedef WaveAttn<kLpD, FP8> WA;
  typedef typename LdsDirect<FP8>::Pipe Pipe;
  constexpr int kLW = LdsDirect<FP8>::NW;
  constexpr int kBtOff = lds_bt_offset<FP8>();
  constexpr int TT = Pipe::TT;
  __shared__ __attribute__((aligned(16))) uint8_t smem[lds_bytes<FP8>()];
  __shared__ int64_t s_rows[kHeadsPerGroup];
  __shared__ int64_t s_orow[kHeadsPerGroup];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int items[2] = {-1, -1};
  if constexpr (PAIRS) {
    // Keys in the stages (unused until the first tile), ranks after them.
    __shared__ int16_t rank_b[kPairedMaxBatch];
    lds_pair_items(p, batch, tid, reinterpret_cast<uint32_t*>(smem), rank_b, items);
    for (int k = 0; k < 2; ++k)
      if (items[k] >= 0) items[k] = rank_b[items[k] / p.hkv] * p.hkv + items[k] % p.hkv;  // b * Hkv + kvh
    __syncthreads();  // the keys' LDS is the stages'
  } else {
    items[0] = blockIdx.y * p.hkv + blockIdx.x;
  }
  int32_t* sbt = reinterpret_cast<int32_t*>(smem + kBtOff);

  for (int k = 0; k < 2; ++k) {
    const int item = items[k];
    if (item < 0) break;
    const int b = item / p.hkv;
    const int kvh = item - b * p.hkv;
    WA A;
    A.init_lane(lane);

    // Issued while the length is in flight: the block-table row (every entry of
    // the sequence's row) and the query rows (q_len * G packed rows, 16 at most).
    for (int i = tid; i < p.max_pages; i += kLW * 64) sbt[i] = p.block_table[(int64_t)b * p.max_pages + i];
    {
      const LaneRow lq = lane_row<kLpD, false>(p, b, kvh, 0, A.n, 0, 0, 0);
      A.load_q(p.q + lq.qoff, lq.valid);
    }
    A.qk_scale = p.qk_scale_log2;
    if constexpr (FP8) A.qk_scale *= p.k_scale[kvh];
    A.reset();
    const int L = __builtin_amdgcn_readfirstlane(p.seq_lens[b]);  // uniform: tile bookkeeping stays scalar
    const LaneRow lr = lane_row<kLpD, false>(p, b, kvh, 0, A.n, L, L, 0);
    if (tid < kHeadsPerGroup) {
      s_rows[tid] = lr.row;
      s_orow[tid] = lr.ooff;
    }
    __syncthreads();

    const int ntiles = (L + TT - 1) / TT;
    const int ps = p.page_size;
    const int64_t head_off = (int64_t)kvh * p.kv.head_stride;
    Pipe P;
    P.init(smem, wave * LdsDirect<FP8>::WAVE_B, A, lane, p.kv.tok_stride);
    // Tiles wave, wave + kLW, ...; the byte offset of token tb's row of KV head
    // kvh.  (Output stores of a previous item may still be outstanding; they
    // only make the pipeline's load-count waits stricter.)
    lds_pipe_run_ns<2>(P, A, wave, kLW, ntiles, 0, L, lr.end, lr.end_min, p.k, p.v, [&](int tb) -> int64_t {
      const int page = __builtin_amdgcn_readfirstlane(sbt[tb / ps]);
      return (int64_t)page * p.kv.page_stride + (int64_t)(tb % ps) * p.kv.tok_stride + head_off;
    });
    // every load has landed: the combine below reuses the stages
    const float vsc = FP8 ? p.v_scale[kvh] : 1.0f;

    auto store = [&](int hh, int d0, f32x4 o, float lse_nat) {
      *reinterpret_cast<bf16x4*>(p.out + s_orow[hh] + d0) = to_bf16x4(o);
      if (d0 == 0 && p.lse) p.lse[s_rows[hh]] = lse_nat;
    };
    if (p.sinks)
      wg_combine<kLpD, FP8, kLW>(A, smem, wave, tid, p.rows_kv, vsc, store,
                                 [&](int hh) { return p.sinks[(int)(s_rows[hh] % p.hq)]; });
    else
      wg_combine<kLpD, FP8, kLW>(A, smem, wave, tid, p.rows_kv, vsc, store, NoSink());
    if (!PAIRS) break;
    __syncthreads();  // the stages, the staged block table and s_rows are reused by the next item
  }
}

}  // namespace

bool lds_direct_applies(int head_dim, bool fp8, int q_len, int window, int group, int page_size, int max_pages,
                        bool strided) {
  (void)fp8;  // both caches have an instance
  return head_dim == kLpD && window == 0 && q_len == 1 && group >= 1 && group <= kHeadsPerGroup &&
         page_size % 16 == 0 && max_pages >= 1 && max_pages <= kBtEntries && !strided;
}

template <bool FP8>
hipError_t launch_lds_direct_t(const SplitParams& p, int batch, int workers, hipStream_t stream) {
  const dim3 block(LdsDirect<FP8>::NW * 64);
  if (workers > 0)
    hipLaunchKernelGGL((lds_direct_kernel<FP8, true>), dim3(workers), block, 0, stream, p, batch);
  else
    hipLaunchKernelGGL((lds_direct_kernel<FP8, false>), dim3(p.hkv, batch), block, 0, stream, p, batch);
  return hipGetLastError();
}

hipError_t launch_lds_direct(const SplitParams& p, bool fp8, int batch, int workers, hipStream_t stream) {
  return fp8 ? launch_lds_direct_t<true>(p, batch, workers, stream)
             : launch_lds_direct_t<false>(p, batch, workers, stream);
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
  if (!pkd::lds_direct_applies(d.head_dim, false, 1, 0, G, d.page_size, d.max_pages_per_seq, false))
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
  p.rows_kv = G;
  p.head_groups = 1;
  p.page_size = d.page_size;
  p.max_pages = d.max_pages_per_seq;
  p.kv.head_stride = 256;
  p.kv.tok_stride = d.num_kv_heads * 256;
  p.kv.page_stride = (int64_t)d.page_size * p.kv.tok_stride;
  return pkd::launch_lds_direct(p, false, d.batch, 0, static_cast<hipStream_t>(stream)) == hipSuccess ? PKD_OK
                                                                                            : PKD_ERR_LAUNCH;
}

}  // extern "C"
