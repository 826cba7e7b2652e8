// Head-dimension dispatch of the partition kernels; the kernels themselves are
// in decode_kernels.hpp, instantiated by decode_d{32,64,128,256}.hip.
#include "pkd_internal.hpp"

namespace pkd {

template <int D>
hipError_t launch_split_kv_dim(const SplitParams& p, int batch, bool fp8, bool direct, bool paged16, bool strided,
                               hipStream_t stream);
template <int D>
hipError_t launch_balanced_dim(const BalancedParams& p, bool fp8, bool strided, hipStream_t stream);

hipError_t launch_split_kv(const SplitParams& p, int batch, int head_dim, bool fp8, bool direct, bool paged16,
                           bool strided, hipStream_t stream) {
  switch (head_dim) {
    case 32: return launch_split_kv_dim<32>(p, batch, fp8, direct, paged16, strided, stream);
    case 64: return launch_split_kv_dim<64>(p, batch, fp8, direct, paged16, strided, stream);
    case 128: return launch_split_kv_dim<128>(p, batch, fp8, direct, paged16, strided, stream);
    case 256: return launch_split_kv_dim<256>(p, batch, fp8, direct, paged16, strided, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_balanced(const BalancedParams& p, int head_dim, bool fp8, bool strided, hipStream_t stream) {
  switch (head_dim) {
    case 32: return launch_balanced_dim<32>(p, fp8, strided, stream);
    case 64: return launch_balanced_dim<64>(p, fp8, strided, stream);
    case 128: return launch_balanced_dim<128>(p, fp8, strided, stream);
    case 256: return launch_balanced_dim<256>(p, fp8, strided, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkd
