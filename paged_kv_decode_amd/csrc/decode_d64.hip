// Partition-kernel instances for head dimension 64 (see decode_kernels.hpp).
#include "decode_kernels.hpp"

namespace pkd {
template hipError_t launch_split_kv_dim<64>(const SplitParams&, int, bool, bool, bool, bool, hipStream_t);
template hipError_t launch_balanced_dim<64>(const BalancedParams&, bool, bool, hipStream_t);
}  // namespace pkd
