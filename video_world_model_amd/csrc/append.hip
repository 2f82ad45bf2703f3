// Dispatch of the quantize-append kernels (see append_impl.h).
#include "qwm_internal.h"

namespace qwm {

hipError_t launch_append_d64_bf16(const AppendParams& p, int heads, bool key, hipStream_t stream);
hipError_t launch_append_d64_f32(const AppendParams& p, int heads, bool key, hipStream_t stream);
hipError_t launch_append_d128_bf16(const AppendParams& p, int heads, bool key, hipStream_t stream);
hipError_t launch_append_d128_f32(const AppendParams& p, int heads, bool key, hipStream_t stream);
hipError_t launch_append_d64_bf16_kv(const AppendParams& pk, const AppendParams& pv, int heads, hipStream_t stream);
hipError_t launch_append_d64_f32_kv(const AppendParams& pk, const AppendParams& pv, int heads, hipStream_t stream);
hipError_t launch_append_d128_bf16_kv(const AppendParams& pk, const AppendParams& pv, int heads, hipStream_t stream);
hipError_t launch_append_d128_f32_kv(const AppendParams& pk, const AppendParams& pv, int heads, hipStream_t stream);

size_t append_lds_bytes(int Cpad, int head_dim, bool f32io, int ucols, int waves) {
  const size_t row = (size_t)(head_dim + 8) * 2;
  // codebook (bf16 rows; fp32 activations add a lo copy), start values, s, the
  // fp64 U of PSAC (ucols columns) and one row buffer per wave
  return (size_t)Cpad * row * (f32io ? 2 : 1) + (size_t)Cpad * 4 + (size_t)head_dim * 4 +
         (size_t)head_dim * ucols * 8 + (size_t)waves * head_dim * 4;
}

hipError_t launch_append(const AppendParams& p, int heads, int head_dim, bool f32io, bool key,
                         hipStream_t stream) {
  if (p.total_segs == 0) return hipSuccess;
  if (head_dim == 128) return f32io ? launch_append_d128_f32(p, heads, key, stream)
                                    : launch_append_d128_bf16(p, heads, key, stream);
  return f32io ? launch_append_d64_f32(p, heads, key, stream) : launch_append_d64_bf16(p, heads, key, stream);
}

hipError_t launch_append_kv(const AppendParams& pk, const AppendParams& pv, int heads, int head_dim, bool f32io,
                            hipStream_t stream) {
  if (pk.total_segs == 0) return hipSuccess;
  if (head_dim == 128) return f32io ? launch_append_d128_f32_kv(pk, pv, heads, stream)
                                    : launch_append_d128_bf16_kv(pk, pv, heads, stream);
  return f32io ? launch_append_d64_f32_kv(pk, pv, heads, stream) : launch_append_d64_bf16_kv(pk, pv, heads, stream);
}

}  // namespace qwm
