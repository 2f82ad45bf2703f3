"""The binding rejects tensors the library would read outside of, before any
GPU call (CPU only: host tensors and plain numpy arrays)."""
import numpy as np
import pytest
import torch

import video_world_model_amd as qwm

CFG = qwm.Config(heads=2, head_dim=64, frame_tokens=16, max_frames=2, c_k=8, c_v=8, io="bf16")


def _cache_stub(cfg):
    """A Cache whose handle is never used: the checks run before any call."""
    c = qwm.Cache.__new__(qwm.Cache)
    c.cfg = cfg
    c.handle = qwm.QwmCache()
    return c


@pytest.mark.parametrize("t,msg", [
    (torch.zeros(2, 16, 64, dtype=torch.float32), "dtype"),
    (torch.zeros(1, 16, 64, dtype=torch.bfloat16), "shape"),
    (torch.zeros(2, 16, 32, dtype=torch.bfloat16), "shape"),
    (torch.zeros(2, 16, dtype=torch.bfloat16), "shape"),
    (torch.zeros(2, 64, 16, dtype=torch.bfloat16).transpose(1, 2), "contiguous"),
    (torch.zeros(2, 16, 64, dtype=torch.bfloat16), "GPU memory"),
])
def test_activation_checks(t, msg):
    with pytest.raises(ValueError, match=msg):
        qwm.check_activation(CFG, t, "k")


def test_entry_points_reject_host_tensors_before_any_gpu_call():
    cache = _cache_stub(CFG)
    good_shape = torch.zeros(2, 16, 64, dtype=torch.bfloat16)
    for fn, args in [(qwm.append_k, (cache, good_shape)), (qwm.append_v, (cache, good_shape)),
                     (qwm.append_kv, (cache, good_shape, good_shape)), (qwm.attention, (cache, good_shape)),
                     (qwm.attention_local, (cache, good_shape, good_shape, good_shape)),
                     (qwm.attention_epochs, ([cache], good_shape)), (qwm.attention_logits, (cache, good_shape)),
                     (qwm.top1, (cache, good_shape)), (qwm.dense_top1, (CFG, good_shape, good_shape))]:
        with pytest.raises(ValueError, match="GPU memory"):
            fn(*args)
    # a Value block with a different token count than the Keys
    with pytest.raises(ValueError, match="differ"):
        qwm.append_kv(cache, good_shape, torch.zeros(2, 32, 64, dtype=torch.bfloat16))
    # epochs of different configs
    other = _cache_stub(qwm.Config(heads=2, head_dim=64, frame_tokens=16, max_frames=3, c_k=8, c_v=8))
    with pytest.raises(ValueError, match="same Config"):
        qwm.attention_epochs([cache, other], good_shape)


def test_buffer_checks():
    with pytest.raises(ValueError, match="dtype"):
        qwm.check_device_buffer(torch.zeros(4, dtype=torch.float16), "lse", torch.float32)
    with pytest.raises(ValueError, match="shape"):
        qwm.check_device_buffer(torch.zeros(2, 3), "lse", torch.float32, shape=(2, 4))
    with pytest.raises(ValueError, match="bytes"):
        qwm.check_device_buffer(torch.zeros(10, dtype=torch.uint8), "calib", torch.uint8, min_bytes=11)
    with pytest.raises(ValueError, match="GPU memory"):
        qwm.check_device_buffer(torch.zeros(2, 4), "lse", torch.float32, shape=(2, 4))
    # the calibration block is checked against the layout's size
    with pytest.raises(ValueError, match="bytes"):
        qwm.calib_import(CFG, torch.zeros(16, dtype=torch.uint8), np.zeros((2, 8, 64)), np.zeros((2, 8, 64)),
                         np.zeros((2, 64)), np.zeros((2, 64, 8)))


def test_host_calibration_shape_checks():
    q = np.zeros((2, 20, 64), np.float32)
    with pytest.raises(ValueError, match="q_hist"):
        qwm.calibrate_host(CFG, q[:1], q, q, seed=1)
    with pytest.raises(ValueError, match="k_hist"):
        qwm.calibrate_host(CFG, q, q, q[:, :10], seed=1)


def test_cache_truncate_host_side():
    """Truncation to whole frames only, never beyond what is cached (host
    handle only)."""
    cache = _cache_stub(CFG)
    cache.handle.n_k = cache.handle.n_v = 32  # two frames of 16 tokens
    with pytest.raises(ValueError, match="whole number of frames"):
        cache.truncate(8)
    with pytest.raises(ValueError, match="whole number of frames"):
        cache.truncate(48)
    with pytest.raises(ValueError, match="whole number of frames"):
        cache.truncate(-16)
    cache.truncate(16)
    assert (cache.handle.n_k, cache.handle.n_v) == (16, 16)
    cache.truncate(16)
    assert cache.n_k == cache.n_v == 16
    cache.truncate(0)
    assert (cache.handle.n_k, cache.handle.n_v) == (0, 0)
