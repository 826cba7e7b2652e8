// Partition-kernel instances for head dimension 32 (see decode_kernels.hpp).
#include "decode_kernels.hpp"

namespace pkd {
template hipError_t launch_split_kv_dim<32>(const SplitParams&, int, bool, bool, bool, bool, hipStream_t);
template hipError_t launch_balanced_dim<32>(const BalancedParams&, bool, bool, hipStream_t);
}  // namespace pkd
