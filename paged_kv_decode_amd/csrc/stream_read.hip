// A read-only stream kernel for gfx950: the bandwidth a plain load stream gets
// from HBM with the access pattern of the decode kernels, used as the
// measured ceiling beside the decode step (not part of the decode).
//
// The buffer is `rows` rows of row_bytes.  Each row is cut into columns of
// `chunk` bytes; a column is read as one stream (chunk = 256 of 2048-byte rows
// is one KV head's rows of a bf16 cache with 8 heads of 128 dims, and
// chunk = row_bytes is a plain contiguous read).  The work space is the
// column-major sequence of 1 KB blocks (a block is one 16-byte load by each of
// a wave's 64 lanes: with pattern 0 the lanes read 1 KB of the column's bytes in
// order; with pattern 1 they read 64 bytes of each of 16 consecutive rows, lane
// l taking row l % 16, the layout of a 16x16x32 matrix-core operand, the next
// block the next 64 bytes of the same rows); workgroup w takes blocks [w K / W, (w + 1) K / W), its
// waves taking every nw-th block of that range.  A wave keeps two batches of
// U blocks in flight: while one batch is folded into a running XOR, the other
// is loading.  Each thread writes its XOR to `sink` so the loads stay live.
//
// Pattern 2 issues the row-order loads of pattern 0 as direct-to-LDS loads
// (global_load_lds_dwordx4: the 16 bytes of each lane land in LDS, never in
// registers), each wave cycling two batches of U blocks through its own LDS
// ring of 2 U KB and waiting by count for the older batch, like the register
// pipeline; it is the load path of a shared-memory staged pipeline, measured
// beside the register one.  Nothing is folded in the loop (reading the ring
// would make the compiler wait for every outstanding load first); each thread
// writes the ring word it last received to `sink`.
#include "../../include/pkd_stream.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkd {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct StreamParams {
  const uint8_t* buf;
  int64_t blocks;          // 1 KB blocks in all
  int64_t blocks_per_col;  // rows * chunk / 1024
  int64_t row_bytes;
  int32_t chunk_log2;
  int32_t pattern;         // 0: 1 KB of the column in order; 1: 64 bytes of each of 16 rows;
                           // 2: as 0, loaded straight into LDS
  uint32_t* sink;
};

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const uint8_t* a) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a));
  else return *reinterpret_cast<const u32x4*>(a);
}

template <int U, bool NT>
__global__ void __launch_bounds__(512) stream_read_kernel(const StreamParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int64_t W = gridDim.x;
  const int64_t k0 = (int64_t)blockIdx.x * p.blocks / W;
  const int64_t k1 = ((int64_t)blockIdx.x + 1) * p.blocks / W;
  const int64_t mine = k1 - k0 > wave ? (k1 - k0 - wave + nw - 1) / nw : 0;  // this wave's blocks
  const int64_t chunk = (int64_t)1 << p.chunk_log2;
  const int64_t lane_off = (int64_t)lane * 16;

  // Cursor over this wave's blocks: column col, block j of that column.
  int64_t k = k0 + wave;
  int64_t col = mine > 0 ? k / p.blocks_per_col : 0;
  int64_t j = mine > 0 ? k - col * p.blocks_per_col : 0;
  const uint8_t* first = nullptr;
  auto addr = [&](int64_t c, int64_t jj) -> const uint8_t* {
    if (p.pattern == 1) {
      const int64_t segs = chunk >> 6;  // 64-byte segments per row of the column
      const int64_t r16 = jj / segs;
      const int64_t row = r16 * 16 + (lane & 15);
      return p.buf + row * p.row_bytes + c * chunk + (jj - r16 * segs) * 64 + (lane >> 4) * 16;
    }
    const int64_t s = jj * 1024 + lane_off;
    const int64_t row = s >> p.chunk_log2;
    return p.buf + row * p.row_bytes + c * chunk + (s & (chunk - 1));
  };
  if (mine > 0) first = addr(col, j);
  int64_t issued = 0;
  // The next block's address; past this wave's last block, its first block
  // again (a cache hit, never an address outside the buffer).
  auto next = [&]() -> const uint8_t* {
    if (issued >= mine) return first;
    const uint8_t* a = addr(col, j);
    ++issued;
    j += nw;
    while (j >= p.blocks_per_col) {
      j -= p.blocks_per_col;
      ++col;
    }
    return a;
  };

  uint32_t acc = 0;
  if (mine > 0) {
    u32x4 ra[U], rb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) ra[u] = ld16<NT>(next());
    int64_t done = 0;
    while (true) {
#pragma unroll
      for (int u = 0; u < U; ++u) rb[u] = ld16<NT>(next());
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= ra[u][0] ^ ra[u][1] ^ ra[u][2] ^ ra[u][3];
      done += U;
      if (done >= mine) break;
#pragma unroll
      for (int u = 0; u < U; ++u) ra[u] = ld16<NT>(next());
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= rb[u][0] ^ rb[u][1] ^ rb[u][2] ^ rb[u][3];
      done += U;
      if (done >= mine) break;
    }
  }
  p.sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// s_waitcnt with vmcnt(n) (n < 64) and no wait on the other counters.
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int U, bool NT>
__global__ void __launch_bounds__(512) stream_lds_kernel(const StreamParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ring_all[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int64_t W = gridDim.x;
  const int64_t k0 = (int64_t)blockIdx.x * p.blocks / W;
  const int64_t k1 = ((int64_t)blockIdx.x + 1) * p.blocks / W;
  const int64_t mine = k1 - k0 > wave ? (k1 - k0 - wave + nw - 1) / nw : 0;
  const int64_t chunk = (int64_t)1 << p.chunk_log2;
  const int64_t lane_off = (int64_t)lane * 16;
  uint8_t* ring = ring_all + (size_t)wave * 2 * U * 1024;  // this wave's two batches of U blocks

  int64_t k = k0 + wave;
  int64_t col = mine > 0 ? k / p.blocks_per_col : 0;
  int64_t j = mine > 0 ? k - col * p.blocks_per_col : 0;
  auto addr = [&](int64_t c, int64_t jj) -> const uint8_t* {
    const int64_t s = jj * 1024 + lane_off;
    const int64_t row = s >> p.chunk_log2;
    return p.buf + row * p.row_bytes + c * chunk + (s & (chunk - 1));
  };
  const uint8_t* first = mine > 0 ? addr(col, j) : nullptr;
  int64_t issued = 0;
  auto next = [&]() -> const uint8_t* {
    if (issued >= mine) return first;
    const uint8_t* a = addr(col, j);
    ++issued;
    j += nw;
    while (j >= p.blocks_per_col) {
      j -= p.blocks_per_col;
      ++col;
    }
    return a;
  };
  // Lane l's 16 bytes land at ring block + 16 l.
  auto batch = [&](int half) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      __builtin_amdgcn_global_load_lds((global_void*)next(), (lds_void*)(ring + (half * U + u) * 1024), 16, 0,
                                       NT ? 2 : 0);
  };

  uint32_t got = 0;
  if (mine > 0) {
    batch(0);
    int64_t done = 0;
    while (true) {
      batch(1);
      __builtin_amdgcn_s_waitcnt(vmcnt_only(U));  // the older batch has landed
      done += U;
      if (done >= mine) break;
      batch(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_only(U));
      done += U;
      if (done >= mine) break;
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    got = reinterpret_cast<const uint32_t*>(ring)[lane];
  }
  p.sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = got;
}

template <int U>
void launch_u(const StreamParams& p, int wgs, int waves, bool nt, hipStream_t s) {
  if (p.pattern == 2) {
    const size_t lds = (size_t)waves * 2 * U * 1024;
    if (nt)
      hipLaunchKernelGGL((stream_lds_kernel<U, true>), dim3(wgs), dim3(waves * 64), lds, s, p);
    else
      hipLaunchKernelGGL((stream_lds_kernel<U, false>), dim3(wgs), dim3(waves * 64), lds, s, p);
  } else if (nt) {
    hipLaunchKernelGGL((stream_read_kernel<U, true>), dim3(wgs), dim3(waves * 64), 0, s, p);
  } else {
    hipLaunchKernelGGL((stream_read_kernel<U, false>), dim3(wgs), dim3(waves * 64), 0, s, p);
  }
}

int log2_exact(int64_t x) {
  if (x <= 0 || (x & (x - 1)) != 0) return -1;
  int l = 0;
  while ((int64_t)1 << l < x) ++l;
  return l;
}

}  // namespace
}  // namespace pkd

extern "C" {

size_t pkd_stream_read_sink_bytes(int32_t workgroups, int32_t waves) {
  if (workgroups < 1 || waves < 1 || waves > 8) return 0;
  return (size_t)workgroups * waves * 64 * sizeof(uint32_t);
}

int32_t pkd_stream_read(const void* buf, int64_t bytes, int32_t row_bytes, int32_t chunk_bytes,
                        int32_t pattern, int32_t workgroups, int32_t waves, int32_t batch_kb,
                        int32_t nontemporal, uint32_t* sink, void* stream) {
  if (!buf || !sink) return PKD_ERR_NULL_POINTER;
  if (((uintptr_t)buf & 15) != 0 || ((uintptr_t)sink & 3) != 0) return PKD_ERR_ALIGNMENT;
  const int cl = pkd::log2_exact(chunk_bytes);
  if (cl < 4 || row_bytes < chunk_bytes || row_bytes % chunk_bytes != 0 || bytes <= 0 || bytes % row_bytes != 0 ||
      bytes % 1024 != 0)
    return PKD_ERR_BAD_DIMS;
  const int64_t rows = bytes / row_bytes;
  if ((rows * chunk_bytes) % 1024 != 0 || pattern < 0 || pattern > 2) return PKD_ERR_BAD_DIMS;
  if (pattern == 1 && (chunk_bytes < 64 || rows % 16 != 0)) return PKD_ERR_BAD_DIMS;
  if (workgroups < 1 || workgroups > (1 << 20) || waves < 1 || waves > 8 || (nontemporal != 0 && nontemporal != 1))
    return PKD_ERR_BAD_DIMS;
  if (batch_kb != 4 && batch_kb != 8 && batch_kb != 16 && batch_kb != 32) return PKD_ERR_BAD_DIMS;
  if (pattern == 2 && waves * 2 * batch_kb > 128) return PKD_ERR_BAD_DIMS;  // the LDS rings
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PKD_ERR_DEVICE;
  pkd::StreamParams p{};
  p.buf = static_cast<const uint8_t*>(buf);
  p.blocks = bytes / 1024;
  p.blocks_per_col = rows * chunk_bytes / 1024;
  p.row_bytes = row_bytes;
  p.chunk_log2 = cl;
  p.pattern = pattern;
  p.sink = sink;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (batch_kb) {
    case 4: pkd::launch_u<4>(p, workgroups, waves, nontemporal != 0, s); break;
    case 8: pkd::launch_u<8>(p, workgroups, waves, nontemporal != 0, s); break;
    case 16: pkd::launch_u<16>(p, workgroups, waves, nontemporal != 0, s); break;
    default: pkd::launch_u<32>(p, workgroups, waves, nontemporal != 0, s); break;
  }
  return hipGetLastError() == hipSuccess ? PKD_OK : PKD_ERR_LAUNCH;
}

}  // extern "C"
