// Append kernels instantiated for head_dim 128, f32 activations.
#include "append_impl.h"

namespace qwm {
hipError_t launch_append_d128_f32(const AppendParams& p, int heads, bool key, hipStream_t stream) {
  return append_detail::dispatch_d<128, true>(p, heads, key, stream);
}
hipError_t launch_append_d128_f32_kv(const AppendParams& pk, const AppendParams& pv, int heads, hipStream_t stream) {
  return append_detail::dispatch_kv_d<128, true>(pk, pv, heads, stream);
}
}  // namespace qwm
