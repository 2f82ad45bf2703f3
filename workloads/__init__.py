"""Seeded synthetic workloads for the QuantWM quantize-append / dequant-attention path.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It holds the workload shapes and the random draws only: none of the method's
arithmetic (no centroid choice, no quantization, no attention) lives here.

Shapes follow the settings the QuantWM pages evaluate (480p / 720p frames,
93-frame and 1-minute histories; "QuantWM: Temporally Consistent 2-Bit KV Cache
Quantization for Video World Models", experiments section) and the single-layer
geometries chosen for them:

* K and V: x = sigma_j * N(0, 1) per head and channel, with
  sigma_j = exp(0.5 * N(0, 1)) (lognormal(0, 0.5)) and a set of outlier channels
  whose sigma is multiplied by 8.  K and V are independent draws.
* Q: q = W a + n, with W a d x 8 orthonormal basis per head (QR of a Gaussian),
  a ~ N(0, A/8 I_8), n ~ N(0, B/d I_d), where A + B = d and
  (A + 8B/d) / (A + B) = 0.70, so the top-8 directions hold 70 % of the
  expected energy (the pages report about 71 % on one LingBot-World-v2 layer).
  Historical and current queries share W and are independent draws.

Every array is drawn in float64 and rounded to the workload's I/O precision
(bfloat16 round-to-nearest-even, or float32 for the tiny case).  Values are
returned as float32 arrays; for bf16 workloads every value is exactly
representable in bfloat16.

Random streams: one numpy PCG64 generator per (config, tensor, head, frame),
seeded with SeedSequence([base_seed, config_id, tensor_id, head, frame]), so
any head or frame can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BASE_SEED = 20260925

# tensor ids of the random streams
T_KSCALE, T_VSCALE, T_K, T_V, T_QBASIS, T_QHIST, T_Q = 0, 1, 2, 3, 4, 5, 6


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    config_id: int
    heads: int
    head_dim: int
    frame_tokens: int
    frames: int          # cached frames
    n_q: int             # query chunk
    n_q_hist: int        # historical queries for the statistics
    io: str              # "bf16" or "f32"
    c_k: int
    c_v: int
    top_k: int           # QSAC candidate count
    rank: int            # PSAC rank
    group_tokens: int    # tokens sharing one (zero, scale) per 16-channel group
    n_outliers: int      # outlier channels per head
    kmeans_iters: int = 10
    description: str = ""

    @property
    def n_tokens(self) -> int:
        return self.frames * self.frame_tokens

    @property
    def n_kv_hist(self) -> int:
        # calibration window: the first frame, except the tiny case which
        # clusters all of its 128 cached tokens
        return self.n_tokens if self.name == "tiny" else self.frame_tokens


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 0, 1, 64, 64, 2, 32, 64, "f32", 16, 16, 4, 8, 16, 4,
                 description="1 head, d=64, 2 frames x 64 tokens, 32 queries, fp32"),
        Workload("matrix_game", 1, 12, 128, 880, 6, 880, 880, "bf16", 256, 256, 4, 8, 16, 3,
                 description="Matrix-Game-2-like layer: 12 heads, 880 tokens/frame, 6 frames"),
        Workload("lingbot480p", 2, 40, 128, 1560, 24, 1560, 1560, "bf16", 256, 256, 4, 8, 16, 3,
                 description="LingBot-World-v2-like 480p: 40 heads, 1560 tokens/frame, 24 frames"),
        Workload("lingbot720p", 3, 40, 128, 3600, 24, 3600, 3600, "bf16", 512, 512, 8, 8, 16, 3,
                 description="720p: 40 heads, 3600 tokens/frame, 24 frames, 512 centroids"),
        Workload("minute", 4, 40, 128, 1560, 240, 1560, 1560, "bf16", 256, 256, 4, 8, 16, 3,
                 description="1-minute: 40 heads, 1560 tokens/frame, 240 frames"),
    ]
}


def scaled(w: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(w, **kw)


def _rng(w: Workload, tensor: int, head: int, frame: int = 0, seed: int = BASE_SEED):
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([seed, w.config_id, tensor, head, frame])))


def round_bf16(x64: np.ndarray) -> np.ndarray:
    """float64 -> nearest bfloat16 value (ties to even), returned as float32."""
    x64 = np.asarray(x64, dtype=np.float64)
    m, e = np.frexp(x64)                      # x = m * 2**e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)  # keep 8 significant bits
    return r.astype(np.float32)


def _round_io(w: Workload, x64: np.ndarray) -> np.ndarray:
    return x64.astype(np.float32) if w.io == "f32" else round_bf16(x64)


def channel_scales(w: Workload, head: int, tensor: int) -> np.ndarray:
    """Per-channel lognormal(0, 0.5) scales with n_outliers channels x8."""
    rng = _rng(w, tensor, head)
    sig = np.exp(0.5 * rng.standard_normal(w.head_dim))
    out = rng.choice(w.head_dim, size=w.n_outliers, replace=False)
    sig[out] *= 8.0
    return sig


def kv_frames(w: Workload, head: int, which: str, f0: int, f1: int) -> np.ndarray:
    """K or V tokens of frames [f0, f1) for one head: [(f1-f0)*F, d] float32."""
    tsc, tdat = (T_KSCALE, T_K) if which == "k" else (T_VSCALE, T_V)
    sig = channel_scales(w, head, tsc)
    parts = []
    for f in range(f0, f1):
        z = _rng(w, tdat, head, f).standard_normal((w.frame_tokens, w.head_dim))
        parts.append(_round_io(w, z * sig[None, :]))
    return np.concatenate(parts, axis=0) if parts else np.zeros((0, w.head_dim), np.float32)


def query_energy_split(d: int, r: int = 8, frac: float = 0.70):
    """(A, B) with A + B = d and (A + r B / d) / (A + B) = frac."""
    # A + r B / d = frac d and A + B = d  ->  B (1 - r/d) = d (1 - frac)
    b = d * (1.0 - frac) / (1.0 - r / d)
    return d - b, b


def query_basis(w: Workload, head: int) -> np.ndarray:
    g = _rng(w, T_QBASIS, head).standard_normal((w.head_dim, 8))
    q, _ = np.linalg.qr(g)
    return q


def queries(w: Workload, head: int, n: int, historical: bool) -> np.ndarray:
    """n queries of one head: [n, d] float32 (values exact in the I/O precision)."""
    d = w.head_dim
    big_a, big_b = query_energy_split(d)
    basis = query_basis(w, head)
    rng = _rng(w, T_QHIST if historical else T_Q, head)
    a = rng.standard_normal((n, 8)) * math.sqrt(big_a / 8.0)
    noise = rng.standard_normal((n, d)) * math.sqrt(big_b / d)
    return _round_io(w, a @ basis.T + noise)


def _stack_heads(fn, heads, threads):
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return np.stack(list(ex.map(fn, heads)), axis=0)


def generate(w: Workload, heads=None, frames=None, threads: int = 8) -> dict:
    """All inputs of a workload for the given heads (default all) and cached frames.

    Returns float32 arrays:
      k, v      [h, frames*F, d]   cached Keys / Values (post-RoPE inputs)
      q         [h, n_q, d]        current query chunk
      q_hist    [h, n_q_hist, d]   historical queries for the statistics
      k_hist, v_hist [h, n_kv_hist, d]  calibration window (a prefix of k / v)
    """
    heads = list(range(w.heads)) if heads is None else list(heads)
    nf = w.frames if frames is None else frames
    k = _stack_heads(lambda h: kv_frames(w, h, "k", 0, nf), heads, threads)
    v = _stack_heads(lambda h: kv_frames(w, h, "v", 0, nf), heads, threads)
    q = _stack_heads(lambda h: queries(w, h, w.n_q, False), heads, threads)
    qh = _stack_heads(lambda h: queries(w, h, w.n_q_hist, True), heads, threads)
    nh = min(w.n_kv_hist, k.shape[1])
    return dict(k=k, v=v, q=q, q_hist=qh, k_hist=k[:, :nh], v_hist=v[:, :nh])


def frame_bits(job) -> np.ndarray:
    """bfloat16 bit patterns (uint16) [heads, F, d] of one frame of K or V for
    every head of a bf16 workload: job = (workload, "k" or "v", frame).  The
    same values as kv_frames, in a form that is cheap to pass between worker
    processes and to copy to a bfloat16 device tensor."""
    w, which, f = job
    x = np.stack([kv_frames(w, h, which, f, f + 1) for h in range(w.heads)])
    return (x.view(np.uint32) >> 16).astype(np.uint16)
