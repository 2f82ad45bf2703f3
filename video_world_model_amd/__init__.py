"""Python binding of libqwm, the QuantWM 2-bit KV-cache library for MI355X.

Argument marshalling only: every step of the path runs in the library's HIP
kernels (include/qwm.h is the contract).  PyTorch provides device memory and
streams.  Importing this module does not need a GPU; calling a device entry
point without the built library or without a GPU raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqwm.so")

ABI_VERSION = 3
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_ALIGN, ERR_CAPACITY, ERR_STATE, ERR_HIP = 0, -1, -2, -3, -4, -5, -6
BF16, F32 = 0, 1
UNIFORM_SENS, NO_RANGE_TERM, QVG_MODE, EXACT_ERROR, FULL_QUADRATIC = 1, 2, 3, 4, 8

EXPORTS = ["qwm_abi_version", "qwm_status_string", "qwm_layout", "qwm_footprint", "qwm_calibrate_host",
           "qwm_calib_import", "qwm_calib_import_moment", "qwm_calibrate", "qwm_cache_init", "qwm_quantize_append_k",
           "qwm_quantize_append_v", "qwm_quantize_append_kv", "qwm_attention_workspace_size", "qwm_attention",
           "qwm_attention_timed", "qwm_attention_local", "qwm_attention_epochs", "qwm_attention_logits", "qwm_top1", "qwm_dense_top1",
           "qwm_append_path_counters", "qwm_attention_noalloc"]
NOALLOC_SCRATCH_BYTES = 34078720


class QwmConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "abi_version", "num_heads", "head_dim", "frame_tokens", "max_frames", "num_centroids_k",
        "num_centroids_v", "group_channels", "group_tokens", "top_candidates", "rank", "io_dtype")] + [
        ("flags", ctypes.c_uint32), ("reserved", ctypes.c_int32)]


class QwmStrides(ctypes.Structure):
    _fields_ = [("head", ctypes.c_int64), ("token", ctypes.c_int64)]


_LAYOUT_FIELDS = ["calib_bytes", "cache_bytes", "token_capacity", "tile_capacity",
                  "mu_k", "mu_v", "sens", "u", "u64", "sgroup", "norm_kw", "norm_k", "norm_v", "head_max",
                  "mu_k16", "mu_v16", "ut16", "moment", "idx_k", "codes_k", "params_k", "coef", "coef_scale", "idx_v", "codes_v", "params_v"]


class QwmLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in _LAYOUT_FIELDS] + [
        ("idx_k_bytes", ctypes.c_uint32), ("idx_v_bytes", ctypes.c_uint32)]


class QwmCache(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("calib", ctypes.c_void_p), ("n_k", ctypes.c_int64),
                ("n_v", ctypes.c_int64), ("abi_version", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class QwmError(RuntimeError):
    def __init__(self, status, text):
        super().__init__("qwm status %d: %s" % (status, text))
        self.status = status


_lib = None


def lib():
    """The loaded libqwm (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libqwm.so is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, U64, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64, ctypes.c_float
        CFG, ST = ctypes.POINTER(QwmConfig), ctypes.POINTER(QwmStrides)
        sig = {
            "qwm_abi_version": (I32, []),
            "qwm_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "qwm_layout": (ctypes.c_int, [CFG, ctypes.POINTER(QwmLayout)]),
            "qwm_footprint": (ctypes.c_int, [CFG, I64, ctypes.POINTER(U64), ctypes.POINTER(U64), ctypes.POINTER(U64)]),
            "qwm_calibrate_host": (ctypes.c_int, [CFG, P, I64, P, P, I64, U64, I32, P, P, P, P, P]),
            "qwm_calib_import": (ctypes.c_int, [CFG, P, P, P, P, P, P]),
            "qwm_calib_import_moment": (ctypes.c_int, [CFG, P, P, P]),
            "qwm_calibrate": (ctypes.c_int, [CFG, P, P, I64, ST, P, P, I64, ST, U64, I32, P, P]),
            "qwm_cache_init": (ctypes.c_int, [CFG, P, P, ctypes.POINTER(QwmCache)]),
            "qwm_quantize_append_k": (ctypes.c_int, [CFG, ctypes.POINTER(QwmCache), P, I64, ST, P]),
            "qwm_quantize_append_v": (ctypes.c_int, [CFG, ctypes.POINTER(QwmCache), P, I64, ST, P]),
            "qwm_quantize_append_kv": (ctypes.c_int, [CFG, ctypes.POINTER(QwmCache), P, P, I64, ST, ST, P]),
            "qwm_attention_workspace_size": (ctypes.c_size_t, [CFG, I64, I64]),
            "qwm_attention": (ctypes.c_int, [CFG, ctypes.POINTER(QwmCache), P, I64, ST, F, P, ST, P, P,
                                             ctypes.c_size_t, P]),
            "qwm_attention_timed": (ctypes.c_int, [CFG, ctypes.POINTER(QwmCache), P, I64, ST, F, P, ST, P, P,
                                                   ctypes.c_size_t, P, P, P]),
            "qwm_attention_local": (ctypes.c_int, [CFG, ctypes.POINTER(QwmCache), P, I64, ST, P, P, I64, ST, ST, F,
                                                   P, ST, P, P, ctypes.c_size_t, P]),
            "qwm_attention_epochs": (ctypes.c_int, [CFG, ctypes.POINTER(QwmCache), I32, P, I64, ST, P, P, I64, ST, ST,
                                                    F, P, ST, P, P, ctypes.c_size_t, P]),
            "qwm_attention_logits": (ctypes.c_int, [CFG, ctypes.POINTER(QwmCache), P, I64, ST, F, P, P]),
            "qwm_top1": (ctypes.c_int, [CFG, ctypes.POINTER(QwmCache), P, I64, ST, P, P]),
            "qwm_dense_top1": (ctypes.c_int, [CFG, P, I64, ST, P, I64, ST, P, P]),
            "qwm_append_path_counters": (ctypes.c_int, [P]),
            "qwm_attention_noalloc": (ctypes.c_int, [CFG, ctypes.POINTER(QwmCache), P, I64, ST, F, P, ST, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status):
    if status != OK:
        raise QwmError(status, lib().qwm_status_string(status).decode())


@dataclasses.dataclass
class Config:
    heads: int
    head_dim: int
    frame_tokens: int
    max_frames: int
    c_k: int
    c_v: int
    group_tokens: int = 16
    top_k: int = 4
    rank: int = 8
    io: str = "bf16"
    flags: int = 0

    def c(self) -> QwmConfig:
        return QwmConfig(ABI_VERSION, self.heads, self.head_dim, self.frame_tokens, self.max_frames,
                         self.c_k, self.c_v, 16, self.group_tokens, self.top_k, self.rank,
                         F32 if self.io == "f32" else BF16, self.flags, 0)

    @property
    def torch_dtype(self):
        import torch
        return torch.float32 if self.io == "f32" else torch.bfloat16


def layout(cfg: Config) -> dict:
    out = QwmLayout()
    c = cfg.c()
    check(lib().qwm_layout(ctypes.byref(c), ctypes.byref(out)))
    return {n: int(getattr(out, n)) for n in _LAYOUT_FIELDS + ["idx_k_bytes", "idx_v_bytes"]}


def footprint(cfg: Config, n_tokens: int):
    """(stored, resident, original) bytes of n_tokens cached tokens."""
    s, r, o = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    c = cfg.c()
    check(lib().qwm_footprint(ctypes.byref(c), n_tokens, ctypes.byref(s), ctypes.byref(r), ctypes.byref(o)))
    return s.value, r.value, o.value


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def calibrate_host(cfg: Config, q_hist, k_hist, v_hist, seed: int, iters: int = 10) -> dict:
    """Host calibration from numpy [H, n, d] arrays (io-precision values)."""
    q, k, v = _f32(q_hist), _f32(k_hist), _f32(v_hist)
    H, d = cfg.heads, cfg.head_dim
    if q.ndim != 3 or q.shape[0] != H or q.shape[2] != d:
        raise ValueError("q_hist: shape %s, expected [%d, n, %d]" % (q.shape, H, d))
    if k.ndim != 3 or k.shape[0] != H or k.shape[2] != d or v.shape != k.shape:
        raise ValueError("k_hist / v_hist: shapes %s / %s, expected [%d, n, %d] each" % (k.shape, v.shape, H, d))
    out = dict(mu_k=np.zeros((H, cfg.c_k, d), np.float32), mu_v=np.zeros((H, cfg.c_v, d), np.float32),
               sens=np.zeros((H, d), np.float32), u=np.zeros((H, d, max(cfg.rank, 1)), np.float32),
               energy=np.zeros(H, np.float64))
    c = cfg.c()
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    check(lib().qwm_calibrate_host(ctypes.byref(c), ptr(q), q.shape[1], ptr(k), ptr(v), k.shape[1], seed, iters,
                                   ptr(out["mu_k"]), ptr(out["mu_v"]), ptr(out["sens"]), ptr(out["u"]),
                                   ptr(out["energy"])))
    out["u"] = out["u"][:, :, :cfg.rank].copy()
    return out


# ------------------------------------------------------------------ device side

def _torch():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("qwm device entry points need a GPU")
    return torch


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def strides(t) -> QwmStrides:
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError("expected a [heads, tokens, head_dim] tensor with contiguous head_dim")
    return QwmStrides(t.stride(0), t.stride(1))


def check_activation(cfg: Config, t, name: str, n_tokens=None):
    """Raises ValueError unless t is a [heads, n, head_dim] tensor of the
    config's I/O dtype on a GPU, with a contiguous head_dim axis (and, when
    given, n == n_tokens).  The library dereferences the pointer on the
    device, so a host tensor, too few heads or a narrower dtype would read
    outside the allocation."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s: expected a torch tensor" % name)
    if t.dtype != cfg.torch_dtype:
        raise ValueError("%s: dtype %s, the config's activations are %s" % (name, t.dtype, cfg.torch_dtype))
    if t.dim() != 3 or t.shape[0] != cfg.heads or t.shape[2] != cfg.head_dim:
        raise ValueError("%s: shape %s, expected [%d, n, %d]" % (name, tuple(t.shape), cfg.heads, cfg.head_dim))
    if n_tokens is not None and t.shape[1] != n_tokens:
        raise ValueError("%s: %d tokens, expected %d" % (name, t.shape[1], n_tokens))
    if t.stride(2) != 1:
        raise ValueError("%s: the head_dim axis must be contiguous" % name)
    if not t.is_cuda:
        raise ValueError("%s: the tensor is not in GPU memory" % name)


def check_device_buffer(t, name: str, dtype, shape=None, min_bytes=None):
    """Raises ValueError unless t is a contiguous GPU tensor of dtype (and of
    the given shape, or at least min_bytes long)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s: expected a torch tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s: dtype %s, expected %s" % (name, t.dtype, dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s: shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError("%s: %d bytes, at least %d needed" % (name, t.numel() * t.element_size(), min_bytes))
    if not t.is_contiguous():
        raise ValueError("%s: expected a contiguous tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s: the tensor is not in GPU memory" % name)


def _check_outputs(cfg, q, out, lse, workspace):
    import torch
    check_activation(cfg, out, "out", q.shape[1])
    check_device_buffer(lse, "lse", torch.float32, shape=(cfg.heads, q.shape[1]))
    if workspace is not None:
        check_device_buffer(workspace, "workspace", torch.uint8)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def alloc_calib(cfg: Config, device="cuda"):
    torch = _torch()
    return torch.empty(layout(cfg)["calib_bytes"], dtype=torch.uint8, device=device)


def _check_calib(cfg: Config, calib):
    import torch
    check_device_buffer(calib, "calib", torch.uint8, min_bytes=layout(cfg)["calib_bytes"])


def calib_import(cfg: Config, calib, mu_k, mu_v, sens, u):
    _check_calib(cfg, calib)
    H, d, r = cfg.heads, cfg.head_dim, cfg.rank
    for name, a, shape in (("mu_k", mu_k, (H, cfg.c_k, d)), ("mu_v", mu_v, (H, cfg.c_v, d)), ("sens", sens, (H, d))):
        if np.shape(a) != shape:
            raise ValueError("%s: shape %s, expected %s" % (name, np.shape(a), shape))
    if r and np.shape(u) != (H, d, r):
        raise ValueError("u: shape %s, expected %s" % (np.shape(u), (H, d, r)))
    c = cfg.c()
    arrs = [_f32(mu_k), _f32(mu_v), _f32(sens), _f32(u if cfg.rank else np.zeros(1))]
    check(lib().qwm_calib_import(ctypes.byref(c), _ptr(calib), *[a.ctypes.data_as(ctypes.c_void_p) for a in arrs],
                                 _stream()))


def calib_import_moment(cfg: Config, calib, m):
    """Full Query second moment [H][d][d] (float64) for FULL_QUADRATIC configs."""
    _check_calib(cfg, calib)
    c = cfg.c()
    a = np.ascontiguousarray(m, dtype=np.float64)
    if a.shape != (cfg.heads, cfg.head_dim, cfg.head_dim):
        raise ValueError("moment must be [H][d][d]")
    check(lib().qwm_calib_import_moment(ctypes.byref(c), _ptr(calib), a.ctypes.data_as(ctypes.c_void_p), _stream()))


def calibrate(cfg: Config, calib, q_hist, k_hist, v_hist, seed: int, iters: int = 10):
    """Device calibration; returns the per-head energy fraction (numpy)."""
    _check_calib(cfg, calib)
    check_activation(cfg, q_hist, "q_hist")
    check_activation(cfg, k_hist, "k_hist")
    check_activation(cfg, v_hist, "v_hist", k_hist.shape[1])
    if k_hist.stride() != v_hist.stride():
        raise ValueError("k_hist and v_hist must have the same strides")
    c = cfg.c()
    energy = np.zeros(cfg.heads, np.float64)
    sq, skv = strides(q_hist), strides(k_hist)
    check(lib().qwm_calibrate(ctypes.byref(c), _ptr(calib), _ptr(q_hist), q_hist.shape[1], ctypes.byref(sq),
                              _ptr(k_hist), _ptr(v_hist), k_hist.shape[1], ctypes.byref(skv), seed, iters,
                              energy.ctypes.data_as(ctypes.c_void_p), _stream()))
    return energy


class Cache:
    """A compressed cache: owns its device block and the host handle."""

    def __init__(self, cfg: Config, calib, device="cuda", base=None):
        """base: optional caller-provided uint8 GPU tensor of at least the
        layout's cache bytes (else one is allocated)."""
        _check_calib(cfg, calib)
        torch = _torch()
        self.cfg = cfg
        self.layout = layout(cfg)
        self.calib = calib
        if base is None:
            base = torch.empty(self.layout["cache_bytes"], dtype=torch.uint8, device=device)
        check_device_buffer(base, "base", torch.uint8, min_bytes=self.layout["cache_bytes"])
        self.base = base
        self.handle = QwmCache()
        c = cfg.c()
        check(lib().qwm_cache_init(ctypes.byref(c), _ptr(calib), _ptr(self.base), ctypes.byref(self.handle)))

    def truncate(self, n_tokens: int):
        """Drop the newest frames: both counters back to n_tokens (a whole
        number of frames, at most the current count); the next append
        overwrites the dropped tokens.  Host-side only."""
        F = self.cfg.frame_tokens
        if n_tokens < 0 or n_tokens % F or n_tokens > min(self.handle.n_k, self.handle.n_v):
            raise ValueError("truncate to %d tokens: not a whole number of frames at most the cached %d"
                             % (n_tokens, min(self.handle.n_k, self.handle.n_v)))
        self.handle.n_k = n_tokens
        self.handle.n_v = n_tokens

    def reset(self):
        """Empty the cache (counters to zero; the next appends overwrite it)."""
        c = self.cfg.c()
        check(lib().qwm_cache_init(ctypes.byref(c), _ptr(self.calib), _ptr(self.base), ctypes.byref(self.handle)))

    @property
    def n_k(self):
        return self.handle.n_k

    @property
    def n_v(self):
        return self.handle.n_v

    def arrays(self) -> dict:
        """Views of the cache fields (per head, full capacity) for inspection."""
        torch = _torch()
        L, cfg = self.layout, self.cfg
        H, N, P, ng, r = cfg.heads, L["token_capacity"], L["tile_capacity"], cfg.head_dim // 16, cfg.rank

        def view(off, count, dtype, shape):
            nbytes = count * torch.empty(0, dtype=dtype).element_size()
            return self.base[off:off + nbytes].view(dtype).view(*shape)
        it = lambda b: torch.uint8 if b == 1 else torch.int16
        out = dict(
            idx_k=view(L["idx_k"], H * N, it(L["idx_k_bytes"]), (H, N)),
            codes_k=view(L["codes_k"], H * N * ng, torch.int32, (H, N, ng)),
            params_k=view(L["params_k"], H * P * ng * 2, torch.float16, (H, P, ng, 2)),
            idx_v=view(L["idx_v"], H * N, it(L["idx_v_bytes"]), (H, N)),
            codes_v=view(L["codes_v"], H * N * ng, torch.int32, (H, N, ng)),
            params_v=view(L["params_v"], H * P * ng * 2, torch.float16, (H, P, ng, 2)))
        if r:
            out["coef"] = view(L["coef"], H * N * r, torch.int8, (H, N, r))
            out["coef_scale"] = view(L["coef_scale"], H * N, torch.float16, (H, N))
        return out


def append_k(cache: Cache, k):
    check_activation(cache.cfg, k, "k")
    c = cache.cfg.c()
    s = strides(k)
    check(lib().qwm_quantize_append_k(ctypes.byref(c), ctypes.byref(cache.handle), _ptr(k), k.shape[1],
                                      ctypes.byref(s), _stream()))


def append_v(cache: Cache, v):
    check_activation(cache.cfg, v, "v")
    c = cache.cfg.c()
    s = strides(v)
    check(lib().qwm_quantize_append_v(ctypes.byref(c), ctypes.byref(cache.handle), _ptr(v), v.shape[1],
                                      ctypes.byref(s), _stream()))


def append_kv(cache: Cache, k, v):
    """Keys and Values of the same tokens in one launch (same fields as
    append_k then append_v)."""
    if tuple(k.shape) != tuple(v.shape):
        raise ValueError("k and v: shapes %s and %s differ (the same tokens are appended)"
                         % (tuple(k.shape), tuple(v.shape)))
    check_activation(cache.cfg, k, "k")
    check_activation(cache.cfg, v, "v", k.shape[1])
    c = cache.cfg.c()
    sk, sv = strides(k), strides(v)
    check(lib().qwm_quantize_append_kv(ctypes.byref(c), ctypes.byref(cache.handle), _ptr(k), _ptr(v), k.shape[1],
                                       ctypes.byref(sk), ctypes.byref(sv), _stream()))


def workspace_bytes(cfg: Config, n_tokens: int, n_q: int) -> int:
    c = cfg.c()
    return int(lib().qwm_attention_workspace_size(ctypes.byref(c), n_tokens, n_q))


def attention(cache: Cache, q, out=None, lse=None, workspace=None, scale: float = 0.0, kernel_events=None):
    """Attention of q over the cache.  kernel_events: optional pair of
    torch.cuda.Event (already recorded once, so that they exist) that the
    library records around the main attention kernel alone."""
    cfg = cache.cfg
    check_activation(cfg, q, "q")
    torch = _torch()
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(cfg.heads, q.shape[1], dtype=torch.float32, device=q.device)
    if workspace is None:
        nb = workspace_bytes(cfg, cache.n_k, q.shape[1])
        workspace = torch.empty(nb, dtype=torch.uint8, device=q.device) if nb else None
    _check_outputs(cfg, q, out, lse, workspace)
    c = cfg.c()
    sq, so = strides(q), strides(out)
    nb = workspace.numel() if workspace is not None else 0
    if kernel_events is None:
        check(lib().qwm_attention(ctypes.byref(c), ctypes.byref(cache.handle), _ptr(q), q.shape[1],
                                  ctypes.byref(sq), scale, _ptr(out), ctypes.byref(so), _ptr(lse), _ptr(workspace),
                                  nb, _stream()))
    else:
        e0, e1 = kernel_events
        check(lib().qwm_attention_timed(ctypes.byref(c), ctypes.byref(cache.handle), _ptr(q), q.shape[1],
                                        ctypes.byref(sq), scale, _ptr(out), ctypes.byref(so), _ptr(lse),
                                        _ptr(workspace), nb, _stream(), ctypes.c_void_p(e0.cuda_event),
                                        ctypes.c_void_p(e1.cuda_event)))
    return out, lse


def attention_noalloc(cache: Cache, q, out, lse, scale: float = 0.0):
    """qwm_attention_noalloc: attention of q over the cache with the partial
    results in the library's own device array (no workspace, no allocation;
    out and lse are the caller's).  Calls that overlap on one GPU race."""
    cfg = cache.cfg
    check_activation(cfg, q, "q")
    import torch
    _check_outputs(cfg, q, out, lse, None)
    c = cfg.c()
    sq, so = strides(q), strides(out)
    check(lib().qwm_attention_noalloc(ctypes.byref(c), ctypes.byref(cache.handle), _ptr(q), q.shape[1],
                                      ctypes.byref(sq), scale, _ptr(out), ctypes.byref(so), _ptr(lse), _stream()))
    return out, lse


def attention_local(cache: Cache, q, k_loc, v_loc, out=None, lse=None, workspace=None, scale: float = 0.0):
    """Attention of the query chunk q over the compressed cache and the chunk's
    own uncompressed keys and values k_loc, v_loc [H][n_loc][d] (bf16)."""
    cfg = cache.cfg
    check_activation(cfg, q, "q")
    check_activation(cfg, k_loc, "k_loc")
    n_loc = k_loc.shape[1]
    check_activation(cfg, v_loc, "v_loc", n_loc)
    torch = _torch()
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(cfg.heads, q.shape[1], dtype=torch.float32, device=q.device)
    if workspace is None:
        nb = workspace_bytes(cfg, cache.n_k + n_loc, q.shape[1])
        workspace = torch.empty(nb, dtype=torch.uint8, device=q.device) if nb else None
    _check_outputs(cfg, q, out, lse, workspace)
    c = cfg.c()
    sq, sk, sv, so = strides(q), strides(k_loc), strides(v_loc), strides(out)
    nb = workspace.numel() if workspace is not None else 0
    check(lib().qwm_attention_local(ctypes.byref(c), ctypes.byref(cache.handle), _ptr(q), q.shape[1],
                                    ctypes.byref(sq), _ptr(k_loc), _ptr(v_loc), n_loc, ctypes.byref(sk),
                                    ctypes.byref(sv), scale, _ptr(out), ctypes.byref(so), _ptr(lse),
                                    _ptr(workspace), nb, _stream()))
    return out, lse


def attention_epochs(caches, q, k_loc=None, v_loc=None, out=None, lse=None, workspace=None, scale: float = 0.0):
    """Attention of the query chunk q over the compressed caches of successive
    calibration epochs (a list of Cache, oldest first, same Config) and,
    optionally, the chunk's own keys and values k_loc, v_loc (bf16)."""
    cfg = caches[0].cfg
    if any(c.cfg != cfg for c in caches):
        raise ValueError("every epoch's cache must have the same Config")
    check_activation(cfg, q, "q")
    n_loc = 0 if k_loc is None else k_loc.shape[1]
    if n_loc:
        check_activation(cfg, k_loc, "k_loc")
        check_activation(cfg, v_loc, "v_loc", n_loc)
    torch = _torch()
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(cfg.heads, q.shape[1], dtype=torch.float32, device=q.device)
    total = sum(c.n_k for c in caches)
    if workspace is None:
        nb = workspace_bytes(cfg, total + n_loc, q.shape[1])
        workspace = torch.empty(nb, dtype=torch.uint8, device=q.device) if nb else None
    _check_outputs(cfg, q, out, lse, workspace)
    handles = (QwmCache * len(caches))(*[c.handle for c in caches])
    c = cfg.c()
    sq, so = strides(q), strides(out)
    sk = strides(k_loc) if n_loc else QwmStrides(0, cfg.head_dim)
    sv = strides(v_loc) if n_loc else QwmStrides(0, cfg.head_dim)
    nb = workspace.numel() if workspace is not None else 0
    check(lib().qwm_attention_epochs(ctypes.byref(c), handles, len(caches), _ptr(q), q.shape[1], ctypes.byref(sq),
                                     _ptr(k_loc), _ptr(v_loc), n_loc, ctypes.byref(sk), ctypes.byref(sv), scale,
                                     _ptr(out), ctypes.byref(so), _ptr(lse), _ptr(workspace), nb, _stream()))
    return out, lse


def attention_logits(cache: Cache, q, scale: float = 0.0):
    cfg = cache.cfg
    check_activation(cfg, q, "q")
    torch = _torch()
    lg = torch.empty(cfg.heads, q.shape[1], cache.n_k, dtype=torch.float32, device=q.device)
    c = cfg.c()
    sq = strides(q)
    check(lib().qwm_attention_logits(ctypes.byref(c), ctypes.byref(cache.handle), _ptr(q), q.shape[1],
                                     ctypes.byref(sq), scale, _ptr(lg), _stream()))
    return lg


def top1(cache: Cache, q):
    cfg = cache.cfg
    check_activation(cfg, q, "q")
    torch = _torch()
    out = torch.empty(cfg.heads, q.shape[1], dtype=torch.int32, device=q.device)
    c = cfg.c()
    sq = strides(q)
    check(lib().qwm_top1(ctypes.byref(c), ctypes.byref(cache.handle), _ptr(q), q.shape[1], ctypes.byref(sq),
                         _ptr(out), _stream()))
    return out


def dense_top1(cfg: Config, q, k):
    check_activation(cfg, q, "q")
    check_activation(cfg, k, "k")
    torch = _torch()
    out = torch.empty(cfg.heads, q.shape[1], dtype=torch.int32, device=q.device)
    c = cfg.c()
    sq, sk = strides(q), strides(k)
    check(lib().qwm_dense_top1(ctypes.byref(c), _ptr(q), q.shape[1], ctypes.byref(sq), _ptr(k), k.shape[1],
                               ctypes.byref(sk), _ptr(out), _stream()))
    return out


def append_path_counters(counters):
    """Appends enqueued from now on add their path counts to counters (a GPU
    int32 tensor of 4: Key tokens settled by band rescoring, Key tokens that
    searched all centres, then the same for Values); None stops counting."""
    import torch
    if counters is not None:
        check_device_buffer(counters, "counters", torch.int32, shape=(4,))
    check(lib().qwm_append_path_counters(_ptr(counters)))
