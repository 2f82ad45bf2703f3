// Append kernels instantiated for head_dim 128, bf16 activations.
#include "append_impl.h"

namespace qwm {
hipError_t launch_append_d128_bf16(const AppendParams& p, int heads, bool key, hipStream_t stream) {
  return append_detail::dispatch_d<128, false>(p, heads, key, stream);
}
}  // namespace qwm
