"""Oracle: compression ratio and top-1 token-selection shift.

TEST INFRASTRUCTURE ONLY (see the package header).

Compression (digest, systems paragraph; review FAQ): the ratio counts the
centres, the quantization parameters and the compensation data, against the
bf16 (or fp32) cache.  Written out, for N cached tokens, H heads, head_dim d:
  original  = 2 N H d b_in
  stored    = N H (idx_K + idx_V)            (1 byte if C <= 256 else 2)
            + 2 N H d / 4                    (2-bit codes, K and V)
            + 2 H tiles n_g 4                (fp16 zero + scale per tile-group)
            + N H r + 2 N H                  (INT8 coefficients + fp16 scale)
            + H (C_K + C_V) d b_in           (centres, stored in the I/O type)
            + H d r 4 + H d 4                (U and s in fp32)
Parity unpinned against the pages' 6.20x: that figure is for real models whose
geometry the pages do not give; the pin is the closed form against the
library's byte count.

Top-1 shift (digest, attention-analysis paragraph): the share of
(head, query) pairs whose highest-scoring historical token under the
reconstructed Keys differs from the one under the original Keys (float64
logits, ties to the lowest token index).  Parity unpinned against the pages'
53.88 % -> 10.19 % etc. (real models); pinned to 0 for zero-residual keys
and to a hand-worked four-query case with a known shift of 1/4 that a
last-maximum tie rule would get wrong (tests/test_oracle_margins.py).
"""
import math

import numpy as np


def compression_ratio(n_tokens, heads, head_dim, frame_tokens, group_tokens,
                      c_k, c_v, rank, b_in):
    tiles = (n_tokens // frame_tokens) * math.ceil(frame_tokens / group_tokens)
    ng = head_dim // 16
    idx_b = (1 if c_k <= 256 else 2) + (1 if c_v <= 256 else 2)
    orig = 2 * n_tokens * heads * head_dim * b_in
    stored = (n_tokens * heads * idx_b
              + 2 * n_tokens * heads * head_dim // 4
              + 2 * heads * tiles * ng * 4
              + (n_tokens * heads * rank + 2 * n_tokens * heads if rank > 0 else 0)
              + heads * (c_k + c_v) * head_dim * b_in
              + heads * head_dim * rank * 4 + heads * head_dim * 4)
    return orig / stored, orig, stored


def top1(q, keys):
    """argmax_t q . k_t per query (float64, first maximum)."""
    lg = np.asarray(q, np.float64) @ np.asarray(keys, np.float64).T
    return np.argmax(lg, axis=1)


def top1_shift(q, keys_orig, keys_recon):
    return float(np.mean(top1(q, keys_orig) != top1(q, keys_recon)))
