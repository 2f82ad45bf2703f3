"""The allocation-free attention entry point (qwm_attention_noalloc) against
qwm_attention with a caller workspace of the same size, through the C ABI:
bit-identical outputs and lse on two calls in a row, the second with a
smaller input (fewer cached frames and fewer queries), for bf16 activations
(stream-K partial results in the library's device array) and for fp32
activations (split-KV partials)."""
import numpy as np
import pytest

import workloads
from tests import parity as P

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


@pytest.mark.parametrize("name", ["matrix_game", "tiny"])
def test_noalloc_equals_workspace_attention(name):
    import torch
    import video_world_model_amd as qwm
    w = workloads.scaled(W[name], heads=2, frames=3) if name == "matrix_game" else W[name]
    cfg = P.cfg_of(w)
    print("case noalloc %s" % name, flush=True)
    data = workloads.generate(w)
    cal = P.oracle_calibration(w, data, cfg, iters=2)
    big, _ = P.build_cache(cfg, cal, data["k"], data["v"])
    small, _ = P.build_cache(cfg, cal, data["k"][:, :w.frame_tokens], data["v"][:, :w.frame_tokens])
    ws = torch.empty(qwm.NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
    q_all = P.to_dev(data["q"], cfg)
    cases = [(big, q_all), (small, q_all[:, :max(1, w.n_q // 3)].contiguous())]
    for rep in range(2):
        for cache, q in cases:
            o_ref, l_ref = qwm.attention(cache, q, workspace=ws)
            o = torch.full_like(q, 7.0)
            lse = torch.full((cfg.heads, q.shape[1]), 7.0, dtype=torch.float32, device="cuda")
            qwm.attention_noalloc(cache, q, o, lse)
            torch.cuda.synchronize()
            assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), (name, rep, cache.n_k, q.shape[1])
    # the oracle agrees too (the small cache's first frame)
    gpu = P.gpu_fields(small, w.frame_tokens)
    stats = P.Stats()
    ko = P.check_keys_head(cfg, data["k"][0][:w.frame_tokens], cal, 0, gpu, stats)
    vo = P.check_values_head(cfg, data["v"][0][:w.frame_tokens], cal, 0, gpu, stats)
    q = cases[1][1]
    o = torch.empty_like(q)
    lse = torch.empty(cfg.heads, q.shape[1], dtype=torch.float32, device="cuda")
    qwm.attention_noalloc(small, q, o, lse)
    wo, wl = P.check_attention(cfg, cal, 0, ko, vo, data["q"][0][:q.shape[1]], o[0].float().cpu().numpy(),
                               lse[0].cpu().numpy())
    assert wo <= 1.0 and wl <= 1.0
