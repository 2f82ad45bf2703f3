"""CPU oracle for the QuantWM quantize-append and dequant-attention path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct
NumPy implementation (float64 decisions, the storage format's float32 / float16
arithmetic written out literally).  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the product library never does, and
the two share no code.

Source: "QuantWM: Temporally Consistent 2-Bit KV Cache Quantization for Video
World Models" (arXiv 2609.26425) as described on the pages that report it:
 * the method section of the English news digest (QSAC and PSAC paragraphs),
 * the Hugging Face abstract (QSAC selects INT2-friendly Key centroids from
   historical Query sensitivity and residual ranges; PSAC restores Key error
   along the dominant Query subspace with low-rank projections),
 * the review page's summary (Eq. 7, E[(q^T e)^2] = e^T M e; diagonal
   approximation; top-8 principal Query directions; INT8 coefficients).
The pages give no group size, tile size, scale format or algorithm box; every
such choice is a stated reading, listed in the design notes and in the module
that implements it.

Parity status per function is stated in each module's header.
"""

from . import numerics, calibrate, codec, attention, measures, margins  # noqa: F401
