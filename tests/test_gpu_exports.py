"""GPU parity of the measurement exports and of the paths the main parity
cases do not reach: the timed bf16 attention kernel's own logits and top-1
exports, the dense top-1 over original keys, the device calibration entry,
the append's all-centre search (forced by a codebook of identical centres,
observed through the path counters), and guard bytes around every buffer the
library writes."""
import sys

import numpy as np
import pytest

import workloads
from tests import parity as P

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _full_matrix_game():
    import video_world_model_amd as qwm
    w = W["matrix_game"]
    cfg = P.cfg_of(w)
    data = workloads.generate(w, threads=16)
    cal = P.oracle_calibration(w, data, cfg, threads=16)
    calib = qwm.alloc_calib(cfg)
    qwm.calib_import(cfg, calib, cal["mu_k"], cal["mu_v"], cal["sens"], cal["u"])
    cache = qwm.Cache(cfg, calib)
    qwm.append_kv(cache, P.to_dev(data["k"], cfg), P.to_dev(data["v"], cfg))
    return w, cfg, data, cal, cache


def test_timed_kernel_logits_and_top1_matrix_game_all_heads():
    """The Matrix-Game-2-like workload at full size (12 heads, 5,280 cached
    tokens, 880 queries): the logits exported by the bf16 attention kernel
    (its debug variant: the same rebuild and contraction as the timed kernel)
    element by element against the oracle's tau q.k~ within 1e-3 tau ||q||
    ||k~|| and within the bound derived from the binary16 operands; its top-1
    export picks a token whose oracle logit is within that bound of the
    maximum (the same token wherever the runner-up is further away than
    twice the bound); the dense top-1 over the original keys likewise."""
    import torch
    import video_world_model_amd as qwm
    from oracle import measures
    say("case logits_top1_matrix_game: generating and calibrating (oracle)")
    w, cfg, data, cal, cache = _full_matrix_game()
    q = P.to_dev(data["q"], cfg)
    lg = qwm.attention_logits(cache, q)
    top = qwm.top1(cache, q).cpu().numpy()
    dense = qwm.dense_top1(cfg, q, P.to_dev(data["k"], cfg)).cpu().numpy()
    torch.cuda.synchronize()
    gpu = P.gpu_fields(cache, w.n_tokens)
    stats = P.Stats()
    tau = 1.0 / np.sqrt(cfg.head_dim)
    worst = worst_b = 0.0
    agree = agree_dense = sure = sure_dense = 0
    for h in range(cfg.heads):
        ko = P.check_keys_head(cfg, data["k"][h], cal, h, gpu, stats)
        vo = P.check_values_head(cfg, data["v"][h], cal, h, gpu, stats)
        _, _, kr, _ = P.oracle_attention(cfg, cal, h, ko, vo, data["q"][h][:1])
        qq = data["q"][h].astype(np.float64)
        ref = tau * qq @ kr.T
        got = lg[h].cpu().numpy()
        bound = P.logit_error_bound(cfg, cal, h, ko, qq)
        rel = 1e-3 * tau * np.linalg.norm(qq, axis=1)[:, None] * np.linalg.norm(kr, axis=1)[None, :]
        worst = max(worst, float(np.max(np.abs(got - ref) / rel)))
        worst_b = max(worst_b, float(np.max(np.abs(got - ref) / bound)))
        # top-1 over the rebuilt keys: valid everywhere, equal where certain
        rows = np.arange(w.n_q)
        best = ref.max(axis=1)
        picked = ref[rows, top[h]]
        assert np.all(best - picked <= 2 * bound.max(axis=1)), h
        srt = np.sort(ref, axis=1)
        certain = srt[:, -1] - srt[:, -2] > 2 * bound.max(axis=1)
        o_top = measures.top1(qq, kr)
        assert np.array_equal(top[h][certain], o_top[certain]), h
        agree += int(np.sum(top[h] == o_top))
        sure += int(certain.sum())
        # dense top-1: fp32 dot products of the bf16 values, error at most
        # (d + 1) 2^-24 sum_j |q_j k_j|
        k0 = data["k"][h].astype(np.float64)
        ref0 = qq @ k0.T
        b0 = (cfg.head_dim + 1) * 2.0 ** -24 * (np.abs(qq) @ np.abs(k0).T).max(axis=1)
        picked0 = ref0[rows, dense[h]]
        assert np.all(ref0.max(axis=1) - picked0 <= 2 * b0), h
        s0 = np.sort(ref0, axis=1)
        c0 = s0[:, -1] - s0[:, -2] > 2 * b0
        d_top = measures.top1(qq, k0)
        assert np.array_equal(dense[h][c0], d_top[c0]), h
        agree_dense += int(np.sum(dense[h] == d_top))
        sure_dense += int(c0.sum())
    n = cfg.heads * w.n_q
    say("  logits: worst |dl| / (1e-3 tau |q||k~|) = %.3g, / derived bound = %.3g; top-1 equal to the oracle's "
        "for %d of %d queries (%d certain); dense top-1 %d of %d (%d certain); append %s"
        % (worst, worst_b, agree, n, sure, agree_dense, n, sure_dense, dict(stats)))
    assert worst <= 1.0 and worst_b <= 1.0


def test_device_calibration_matches_host():
    """qwm_calibrate (device inputs, the entry the benchmark uses) against
    qwm_calibrate_host on the same values: bit-equal centres, s and U in the
    calibration block, for all 40 heads of the 480p-like first frame.  The
    inputs are produced by a kernel on the current stream just before the
    call, so the call must order its copies after that work."""
    import torch
    import video_world_model_amd as qwm
    w = W["lingbot480p"]
    cfg = P.cfg_of(w)
    say("case device_calibration: 40 heads")
    data = workloads.generate(w, frames=1, threads=16)
    qh, kh, vh = data["q_hist"], data["k_hist"], data["v_hist"]
    host = qwm.calibrate_host(cfg, qh, kh, vh, seed=11, iters=10)
    # device inputs written by GPU work right before the call (x * 1 on the stream)
    dq, dk, dv = [P.to_dev(np.zeros_like(a), cfg) for a in (qh, kh, vh)]
    sq, sk, sv = [P.to_dev(a, cfg) for a in (qh, kh, vh)]
    torch.cuda.synchronize()
    for dst, src in ((dq, sq), (dk, sk), (dv, sv)):
        torch.mul(src, 1.0, out=dst)
    calib = qwm.alloc_calib(cfg)
    energy = qwm.calibrate(cfg, calib, dq, dk, dv, seed=11, iters=10)
    torch.cuda.synchronize()
    L = qwm.layout(cfg)
    raw = calib.cpu().numpy()
    H, d, r = cfg.heads, cfg.head_dim, cfg.rank

    def field(off, count, dt):
        return raw[off:off + count * np.dtype(dt).itemsize].view(dt)
    mu_k = (field(L["mu_k"], H * cfg.c_k * d, np.uint16).astype(np.uint32) << 16).view(np.float32)
    mu_v = (field(L["mu_v"], H * cfg.c_v * d, np.uint16).astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(mu_k.reshape(H, cfg.c_k, d), host["mu_k"])
    assert np.array_equal(mu_v.reshape(H, cfg.c_v, d), host["mu_v"])
    assert np.array_equal(field(L["sens"], H * d, np.float32).reshape(H, d), host["sens"])
    assert np.array_equal(field(L["u"], H * d * r, np.float32).reshape(H, d, r), host["u"])
    assert np.array_equal(energy, host["energy"])
    assert float(np.abs(mu_k).max()) > 0 and float(host["sens"].min()) > 0   # not an all-zero block
    say("  device calibration equals the host calibration bit for bit (energy mean %.4f)" % energy.mean())


def test_all_centre_search_and_path_counters():
    """A codebook whose first ten centres are copies of one row, and tokens
    placed next to that row: the screen's tracked list (K_c + 3 entries for
    Keys, 3 for Values) cannot hold every equally near centre, so the append
    must search all centres for those tokens.  The path counters show that it
    did (Keys and Values); every decision matches the oracle, which takes the
    lowest index among the exact ties."""
    import torch
    import video_world_model_amd as qwm
    w = workloads.scaled(W["matrix_game"], heads=2, frames=2)
    cfg = P.cfg_of(w)
    say("case all_centre_search")
    data = workloads.generate(w)
    cal = P.oracle_calibration(w, data, cfg, iters=2)
    for key in ("mu_k", "mu_v"):
        cal[key] = cal[key].copy()
        cal[key][:, 1:10] = cal[key][:, 0:1]
    rng = np.random.default_rng(21)
    k, v = data["k"].copy(), data["v"].copy()
    n = k.shape[1]
    near = rng.random(n) < 0.3
    for h in range(cfg.heads):
        for x, mu in ((k, cal["mu_k"]), (v, cal["mu_v"])):
            noise = rng.standard_normal((int(near.sum()), cfg.head_dim)) * 1e-2
            x[h, near] = workloads.round_bf16(mu[h][0][None, :].astype(np.float64) + noise)
    counters = torch.zeros(4, dtype=torch.int32, device="cuda")
    qwm.append_path_counters(counters)
    try:
        cache, _ = P.build_cache(cfg, cal, k, v)
    finally:
        qwm.append_path_counters(None)
    cnt = counters.cpu().numpy().tolist()
    gpu = P.gpu_fields(cache, n)
    stats = P.Stats()
    for h in range(cfg.heads):
        ko = P.check_keys_head(cfg, k[h], cal, h, gpu, stats)
        P.check_values_head(cfg, v[h], cal, h, gpu, stats)
        assert np.all(ko["idx"][near] < 10)
    say("  path counters (Key band, Key search, Value band, Value search) = %s; %s" % (cnt, dict(stats)))
    assert cnt[1] > 0 and cnt[3] > 0
    assert stats.get("k_adopted", 0) == 0 and stats.get("v_adopted", 0) == 0
    # nothing of the copies above index 0 is ever chosen (exact ties, lowest index)
    assert not np.any((gpu["idx_k"] >= 1) & (gpu["idx_k"] < 10))
    assert not np.any((gpu["idx_v"] >= 1) & (gpu["idx_v"] < 10))


def test_guard_bytes_around_every_written_buffer():
    """Cache block, attention output, lse and workspace each sit inside a
    larger buffer filled with a pattern; after the fused append of two of
    three frames, attention and attention with the local chunk, the pattern
    is intact outside each buffer, and every cache field is untouched past
    the appended tokens and tiles."""
    import torch
    import video_world_model_amd as qwm
    w = workloads.scaled(W["matrix_game"], heads=2, frames=2)
    cfg = P.cfg_of(w, max_frames=3)
    say("case guard_bytes")
    data = workloads.generate(w)
    cal = P.oracle_calibration(w, data, cfg, iters=2)
    calib = qwm.alloc_calib(cfg)
    qwm.calib_import(cfg, calib, cal["mu_k"], cal["mu_v"], cal["sens"], cal["u"])
    G = 4096
    L = qwm.layout(cfg)
    pat = 0xA5
    big = torch.full((L["cache_bytes"] + 2 * G,), pat, dtype=torch.uint8, device="cuda")
    cache = qwm.Cache(cfg, calib, base=big[G:G + L["cache_bytes"]])
    kd, vd = P.to_dev(data["k"], cfg), P.to_dev(data["v"], cfg)
    qwm.append_kv(cache, kd, vd)
    n_q = w.n_q
    H, d = cfg.heads, cfg.head_dim
    out_big = torch.full((H, n_q + 16, d), 123.0, dtype=torch.bfloat16, device="cuda")
    out = out_big[:, 8:8 + n_q]
    lse_big = torch.full((H * n_q + 128,), 77.0, dtype=torch.float32, device="cuda")
    lse = lse_big[64:64 + H * n_q].view(H, n_q)
    nb = qwm.workspace_bytes(cfg, w.n_tokens + w.frame_tokens, n_q)
    ws_big = torch.full((nb + 2 * G,), pat, dtype=torch.uint8, device="cuda")
    ws = ws_big[G:G + nb]
    q = P.to_dev(data["q"], cfg)
    qwm.attention(cache, q, out=out, lse=lse, workspace=ws)
    kl = P.to_dev(np.stack([workloads.kv_frames(w, h, "k", 2, 3) for h in range(H)]), cfg)
    vl = P.to_dev(np.stack([workloads.kv_frames(w, h, "v", 2, 3) for h in range(H)]), cfg)
    qwm.attention_local(cache, q, kl, vl, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    assert bool((big[:G] == pat).all()) and bool((big[G + L["cache_bytes"]:] == pat).all()), "cache guard"
    assert bool((out_big[:, :8].float() == 123.0).all()) and bool((out_big[:, 8 + n_q:].float() == 123.0).all()), \
        "output guard"
    assert bool((lse_big[:64] == 77.0).all()) and bool((lse_big[64 + H * n_q:] == 77.0).all()), "lse guard"
    assert bool((ws_big[:G] == pat).all()) and bool((ws_big[G + nb:] == pat).all()), "workspace guard"
    n = w.n_tokens
    tiles = 2 * -(-w.frame_tokens // w.group_tokens)
    arr = cache.arrays()
    for name, a in arr.items():
        tail = a[:, tiles:] if name.startswith("params") else a[:, n:]
        assert bool((tail.contiguous().view(torch.uint8) == pat).all()), name
    # the outputs are complete (no pattern left inside them)
    assert bool(torch.isfinite(out.float()).all()) and not bool((out.float() == 123.0).all())
    assert bool(torch.isfinite(lse).all())
    say("  guards intact around cache, output, lse and workspace")
