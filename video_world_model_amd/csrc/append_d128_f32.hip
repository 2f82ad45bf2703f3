// Append kernels instantiated for head_dim 128, f32 activations.
#include "append_impl.h"

namespace qwm {
hipError_t launch_append_d128_f32(const AppendParams& p, int heads, bool key, hipStream_t stream) {
  return append_detail::dispatch_d<128, true>(p, heads, key, stream);
}
}  // namespace qwm
