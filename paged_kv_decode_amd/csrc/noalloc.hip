// paged_decode_ext_noalloc: paged_decode_ext with its workspace taken from a
// fixed device array of this library instead of the caller, for callers that
// cannot allocate device memory.
//
// The array below is defined once per process and exists on every device the
// library runs on, each device holding its own copy at its own address.  Its
// name in host code is only a stand-in: the device address comes from
// hipGetSymbolAddress, queried once per device with that device current, and
// that address is what the kernels are given.  Calls on one device share the
// array; the decode never needs it cleared (partials are written before they
// are read, and the in-place merge's counters carry a per-call tag), but calls
// that overlap in time on one device (two streams) race on it.
#include "../../include/paged_kv_decode.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace {

__device__ __align__(256) uint8_t scratch[PKD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // null: not yet queried on that device

// The current device's copy of the array, or null when it cannot be found.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
  g_scratch_ptr[dev].store(ptr, std::memory_order_release);  // racing callers store the same address
  return ptr;
}

}  // namespace

extern "C" {

int32_t paged_decode_ext_noalloc(const pkd_dims* dims, const pkd_ext* ext, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                                 const float* k_scale, const float* v_scale, const float* sinks, float scale,
                                 void* out, float* lse, int32_t num_splits, void* stream) {
  if (!dims) return PKD_ERR_NULL_POINTER;
  // The workspace the mode needs (0 also for invalid dims or modes, which
  // paged_decode_ext then rejects with their own status).
  const size_t need = paged_decode_workspace_bytes_ext(dims, ext, num_splits);
  if (need > (size_t)PKD_NOALLOC_SCRATCH_BYTES) return PKD_ERR_SCRATCH_LIMIT;
  void* ws = need > 0 ? device_scratch() : nullptr;
  if (need > 0 && !ws) {
    // No device copy of the array: report argument errors first (without a
    // workspace the call enqueues nothing), else the missing device.
    const int32_t st = paged_decode_ext(dims, ext, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale,
                                        sinks, scale, out, lse, num_splits, nullptr, 0, stream);
    return st == PKD_ERR_WORKSPACE ? PKD_ERR_DEVICE : st;
  }
  return paged_decode_ext(dims, ext, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, sinks, scale,
                          out, lse, num_splits, ws, ws ? (size_t)PKD_NOALLOC_SCRATCH_BYTES : 0, stream);
}

}  // extern "C"
