// Append kernels instantiated for head_dim 128, bf16 activations.
#include "append_impl.h"

namespace qwm {
hipError_t launch_append_d128_bf16(const AppendParams& p, int heads, bool key, hipStream_t stream) {
  return append_detail::dispatch_d<128, false>(p, heads, key, stream);
}
hipError_t launch_append_d128_bf16_kv(const AppendParams& pk, const AppendParams& pv, int heads, hipStream_t stream) {
  return append_detail::dispatch_kv_d<128, false>(pk, pv, heads, stream);
}
}  // namespace qwm
