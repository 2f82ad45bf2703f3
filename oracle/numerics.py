"""Rounding helpers of the oracle (test infrastructure only).

The storage format fixes three roundings, each round-to-nearest-even:
  fl32  : float64 -> IEEE binary32
  fp16  : binary32 -> IEEE binary16 (subnormals kept)
  bf16  : float64 -> bfloat16 (8 significant bits, float32 exponent range)
NumPy's float64->float32 and float32->float16 casts are correctly rounded
(ties to even), so fl32 and fp16 are plain casts.  bfloat16 has no NumPy dtype;
it is computed from the binary exponent.
"""
import numpy as np


def fl32(x):
    """Round to binary32 (RNE); result as float32."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def fp16_of_f32(x32):
    """binary32 -> binary16 (RNE); result as float32 holding the fp16 value."""
    x32 = np.asarray(x32, dtype=np.float32)
    return x32.astype(np.float16).astype(np.float32)


def bf16(x):
    """float64 -> bfloat16 (RNE, no double rounding); result as float32."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    e = np.floor(np.log2(np.abs(x[nz])))
    # guard against log2 rounding at exact powers of two
    e = np.where(np.abs(x[nz]) < np.exp2(e), e - 1, e)
    e = np.where(np.abs(x[nz]) >= np.exp2(e + 1), e + 1, e)
    ulp = np.exp2(e - 7)               # 8 significant bits: ulp = 2^(e-7)
    out[nz] = np.rint(x[nz] / ulp) * ulp
    return out.astype(np.float32)


def round_storage(x, io):
    """Storage rounding of centroids: bfloat16 for bf16 I/O, binary32 for f32."""
    return fl32(x) if io == "f32" else bf16(x)
