"""C-ABI contract tests that need no GPU: the library loads, exports what
include/qwm.h declares, rejects bad arguments before any HIP call, and its
byte accounting and host calibration agree with the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

import video_world_model_amd as qwm
import workloads
from oracle import calibrate as oc
from oracle import measures

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(qwm.LIB_PATH), reason="libqwm.so not built")


def declared_functions():
    text = open(os.path.join(ROOT, "include", "qwm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qwm_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(qwm.EXPORTS)
    lib = qwm.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert lib.qwm_abi_version() == qwm.ABI_VERSION


def cfg_of(w, **kw):
    c = qwm.Config(heads=w.heads, head_dim=w.head_dim, frame_tokens=w.frame_tokens, max_frames=w.frames,
                   c_k=w.c_k, c_v=w.c_v, group_tokens=w.group_tokens, top_k=w.top_k, rank=w.rank, io=w.io)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 96, qwm.ERR_UNSUPPORTED),
    ("group_tokens", 12, qwm.ERR_UNSUPPORTED),
    ("c_k", 1024, qwm.ERR_UNSUPPORTED),
    ("c_k", 0, qwm.ERR_INVALID_ARG),
    ("rank", 33, qwm.ERR_UNSUPPORTED),
    ("top_k", 9, qwm.ERR_UNSUPPORTED),
    ("heads", 0, qwm.ERR_INVALID_ARG),
    ("flags", 16, qwm.ERR_INVALID_ARG),
    ("flags", 32, qwm.ERR_INVALID_ARG),
])
def test_config_rejections(field, value, status):
    c = cfg_of(workloads.WORKLOADS["lingbot480p"], **{field: value})
    with pytest.raises(qwm.QwmError) as e:
        qwm.layout(c)
    assert e.value.status == status


def test_lds_limit_of_the_append_working_set():
    """C = 512 with r = 32 (d = 128, bf16) does not fit one workgroup's LDS;
    r = 16 at C = 512 and r = 32 at C = 448 do."""
    w = workloads.WORKLOADS["lingbot720p"]
    for c_k, rank, ok in ((512, 16, True), (448, 32, True), (512, 32, False)):
        c = cfg_of(w, c_k=c_k, c_v=c_k, rank=rank)
        if ok:
            qwm.layout(c)
        else:
            with pytest.raises(qwm.QwmError) as e:
                qwm.layout(c)
            assert e.value.status == qwm.ERR_UNSUPPORTED


def test_layout_alignment_and_sizes():
    for name, w in workloads.WORKLOADS.items():
        L = qwm.layout(cfg_of(w))
        for f in ["mu_k", "mu_v", "sens", "u", "u64", "sgroup", "norm_kw", "norm_k", "norm_v", "head_max",
                  "mu_k16", "mu_v16", "ut16", "moment", "idx_k", "codes_k", "params_k", "coef", "coef_scale", "idx_v", "codes_v", "params_v"]:
            assert L[f] % 256 == 0
        assert L["token_capacity"] == w.n_tokens
        assert L["tile_capacity"] == w.frames * -(-w.frame_tokens // w.group_tokens)
        assert L["idx_k_bytes"] == (1 if w.c_k <= 256 else 2)
        assert L["codes_v"] - L["idx_v"] >= w.heads * w.n_tokens * L["idx_v_bytes"]
        # the full Query second moment is stored only for the full-quadratic score
        assert L["moment"] == L["calib_bytes"]
        Lf = qwm.layout(cfg_of(w, flags=qwm.FULL_QUADRATIC))
        assert Lf["moment"] == L["moment"]
        assert Lf["calib_bytes"] - Lf["moment"] >= w.heads * w.head_dim ** 2 * 8


def test_moment_import_rejections():
    L = qwm.lib()
    w = workloads.WORKLOADS["tiny"]
    m = np.zeros((1, 64, 64))
    c = cfg_of(w).c()
    # only full-quadratic configs hold a moment block
    assert L.qwm_calib_import_moment(ctypes.byref(c), _fake(), m.ctypes.data_as(ctypes.c_void_p), None) == \
        qwm.ERR_INVALID_ARG
    cf = cfg_of(w, flags=qwm.FULL_QUADRATIC).c()
    assert L.qwm_calib_import_moment(ctypes.byref(cf), _fake(), None, None) == qwm.ERR_INVALID_ARG
    assert L.qwm_calib_import_moment(ctypes.byref(cf), None, m.ctypes.data_as(ctypes.c_void_p), None) == \
        qwm.ERR_INVALID_ARG


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_footprint_equals_oracle_closed_form(name):
    w = workloads.WORKLOADS[name]
    stored, resident, original = qwm.footprint(cfg_of(w), w.n_tokens)
    b_in = 4 if w.io == "f32" else 2
    ratio, orig, st = measures.compression_ratio(w.n_tokens, w.heads, w.head_dim, w.frame_tokens,
                                                 w.group_tokens, w.c_k, w.c_v, w.rank, b_in)
    assert original == orig and stored == st
    assert resident >= stored


def _fake(addr=0x100000):
    return ctypes.c_void_p(addr)


def test_append_error_paths_move_no_counter():
    w = workloads.WORKLOADS["matrix_game"]
    c = cfg_of(w).c()
    h = qwm.QwmCache()
    L = qwm.lib()
    assert L.qwm_cache_init(ctypes.byref(c), _fake(), _fake(0x200000), ctypes.byref(h)) == 0
    st = qwm.QwmStrides(w.n_tokens * 128, 128)
    # not a whole frame
    assert L.qwm_quantize_append_k(ctypes.byref(c), ctypes.byref(h), _fake(), 100, ctypes.byref(st), None) == qwm.ERR_ALIGN
    # beyond capacity
    assert L.qwm_quantize_append_v(ctypes.byref(c), ctypes.byref(h), _fake(), w.n_tokens + w.frame_tokens,
                                   ctypes.byref(st), None) == qwm.ERR_CAPACITY
    # misaligned pointer / bad stride
    assert L.qwm_quantize_append_k(ctypes.byref(c), ctypes.byref(h), _fake(0x100002), 880, ctypes.byref(st), None) == qwm.ERR_INVALID_ARG
    bad = qwm.QwmStrides(w.n_tokens * 128, 100)
    assert L.qwm_quantize_append_k(ctypes.byref(c), ctypes.byref(h), _fake(), 880, ctypes.byref(bad), None) == qwm.ERR_INVALID_ARG
    # fused K+V append: same checks on both inputs, nothing launched on error
    assert L.qwm_quantize_append_kv(ctypes.byref(c), ctypes.byref(h), _fake(), _fake(), 100, ctypes.byref(st),
                                    ctypes.byref(st), None) == qwm.ERR_ALIGN
    assert L.qwm_quantize_append_kv(ctypes.byref(c), ctypes.byref(h), _fake(), _fake(0x100002), 880,
                                    ctypes.byref(st), ctypes.byref(st), None) == qwm.ERR_INVALID_ARG
    assert L.qwm_quantize_append_kv(ctypes.byref(c), ctypes.byref(h), _fake(), _fake(), 880, ctypes.byref(st),
                                    ctypes.byref(bad), None) == qwm.ERR_INVALID_ARG
    assert h.n_k == 0 and h.n_v == 0
    # K/V imbalance at attention and at the fused append
    h.n_k = 880
    assert L.qwm_quantize_append_kv(ctypes.byref(c), ctypes.byref(h), _fake(), _fake(), 880, ctypes.byref(st),
                                    ctypes.byref(st), None) == qwm.ERR_STATE
    out_st = qwm.QwmStrides(880 * 128, 128)
    assert L.qwm_attention(ctypes.byref(c), ctypes.byref(h), _fake(), 880, ctypes.byref(st), ctypes.c_float(0),
                           _fake(0x300000), ctypes.byref(out_st), None, None, 0, None) == qwm.ERR_STATE
    # attention with the local chunk: the same state check, then the local rows
    assert L.qwm_attention_local(ctypes.byref(c), ctypes.byref(h), _fake(), 880, ctypes.byref(st), _fake(), _fake(),
                                 880, ctypes.byref(st), ctypes.byref(st), ctypes.c_float(0), _fake(0x300000),
                                 ctypes.byref(out_st), None, None, 0, None) == qwm.ERR_STATE
    h.n_k = 0
    assert L.qwm_attention_local(ctypes.byref(c), ctypes.byref(h), _fake(), 880, ctypes.byref(st), _fake(),
                                 _fake(0x100002), 880, ctypes.byref(st), ctypes.byref(st), ctypes.c_float(0),
                                 _fake(0x300000), ctypes.byref(out_st), None, None, 0, None) == qwm.ERR_INVALID_ARG
    assert L.qwm_attention_local(ctypes.byref(c), ctypes.byref(h), _fake(), 880, ctypes.byref(st), _fake(), _fake(),
                                 -1, ctypes.byref(st), ctypes.byref(st), ctypes.c_float(0), _fake(0x300000),
                                 ctypes.byref(out_st), None, None, 0, None) == qwm.ERR_INVALID_ARG
    # fp32 activations have no local-chunk path
    wt = workloads.WORKLOADS["tiny"]
    ct = cfg_of(wt).c()
    ht = qwm.QwmCache()
    assert L.qwm_cache_init(ctypes.byref(ct), _fake(), _fake(0x200000), ctypes.byref(ht)) == 0
    stt = qwm.QwmStrides(wt.n_tokens * 64, 64)
    assert L.qwm_attention_local(ctypes.byref(ct), ctypes.byref(ht), _fake(), 32, ctypes.byref(stt), _fake(), _fake(),
                                 64, ctypes.byref(stt), ctypes.byref(stt), ctypes.c_float(0), _fake(0x300000),
                                 ctypes.byref(stt), None, None, 0, None) == qwm.ERR_UNSUPPORTED
    # calibration epochs: at least one handle, at most 64, each with n_k == n_v
    hs = (qwm.QwmCache * 65)()
    for i in range(65):
        assert L.qwm_cache_init(ctypes.byref(c), _fake(), _fake(0x200000), ctypes.byref(hs[i])) == 0
    args = (_fake(), 880, ctypes.byref(st), None, None, 0, ctypes.byref(st), ctypes.byref(st), ctypes.c_float(0),
            _fake(0x300000), ctypes.byref(out_st), None, None, 0, None)
    assert L.qwm_attention_epochs(ctypes.byref(c), hs, 0, *args) == qwm.ERR_INVALID_ARG
    assert L.qwm_attention_epochs(ctypes.byref(c), None, 1, *args) == qwm.ERR_INVALID_ARG
    assert L.qwm_attention_epochs(ctypes.byref(c), hs, 65, *args) == qwm.ERR_UNSUPPORTED
    hs[2].n_k = 880
    assert L.qwm_attention_epochs(ctypes.byref(c), hs, 3, *args) == qwm.ERR_STATE
    hs[2].n_k = 0
    hs[1].calib = None
    assert L.qwm_attention_epochs(ctypes.byref(c), hs, 3, *args) == qwm.ERR_INVALID_ARG
    assert L.qwm_attention_epochs(ctypes.byref(ct), hs, 1, _fake(), 32, ctypes.byref(stt), None, None, 0,
                                  ctypes.byref(stt), ctypes.byref(stt), ctypes.c_float(0), _fake(0x300000),
                                  ctypes.byref(stt), None, None, 0, None) == qwm.ERR_UNSUPPORTED
    # wrong abi version in the config
    c2 = cfg_of(w).c()
    c2.abi_version = 99
    assert L.qwm_layout(ctypes.byref(c2), ctypes.byref(qwm.QwmLayout())) == qwm.ERR_INVALID_ARG
    assert L.qwm_status_string(qwm.ERR_ALIGN).decode().startswith("append")


def test_host_calibration_matches_oracle_tiny():
    w = workloads.WORKLOADS["tiny"]
    d = workloads.generate(w)
    cfg = cfg_of(w)
    got = qwm.calibrate_host(cfg, d["q_hist"], d["k_hist"], d["v_hist"], seed=123, iters=10)
    ref = oc.calibrate(d["q_hist"], d["k_hist"], d["v_hist"], 16, 16, 8, "f32", seed=123, iters=10)
    assert np.array_equal(got["sens"], ref["sens"]) or np.max(np.abs(got["sens"] - ref["sens"]) / ref["sens"]) < 1e-6
    uu = got["u"][0].astype(np.float64)
    ur = ref["u"][0].astype(np.float64)
    assert np.max(np.abs(uu @ uu.T - ur @ ur.T)) < 1e-5
    assert np.max(np.abs(got["u"] - ref["u"])) < 1e-5      # same sign convention
    assert abs(got["energy"][0] - ref["energy"][0]) < 1e-9
    assert np.max(np.abs(got["mu_k"] - ref["mu_k"])) < 1e-5
    assert np.max(np.abs(got["mu_v"] - ref["mu_v"])) < 1e-5


def test_host_calibration_matches_oracle_bf16():
    w = workloads.scaled(workloads.WORKLOADS["matrix_game"], heads=2, frames=1)
    d = workloads.generate(w)
    cfg = cfg_of(w, c_k=64, c_v=64)
    got = qwm.calibrate_host(cfg, d["q_hist"], d["k_hist"], d["v_hist"], seed=5, iters=5)
    ref = oc.calibrate(d["q_hist"], d["k_hist"], d["v_hist"], 64, 64, 8, "bf16", seed=5, iters=5)
    # bf16-rounded centres agree exactly except at rare rounding-boundary / assignment ties
    for key in ("mu_k", "mu_v"):
        diff = got[key] != ref[key]
        assert diff.mean() < 1e-3, (key, diff.mean())
    for h in range(2):
        uu, ur = got["u"][h].astype(np.float64), ref["u"][h].astype(np.float64)
        assert np.max(np.abs(uu @ uu.T - ur @ ur.T)) < 1e-5
    assert np.allclose(got["energy"], ref["energy"], atol=1e-9)
