"""GPU parity: the HIP path through the C-ABI against the CPU oracle on seeded
inputs (tie-following bit-exactness for indices, codes, tile parameters and
INT8 coefficients; attention outputs within 2e-2 max-abs beyond the bf16
output's own rounding; lse within the bound derived from the kernel's binary16
operands (tests/parity.py); logits within 1e-3 * tau * ||q|| * ||k~|| and
within the derived per-element bound)."""
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


def case_data(w, heads=None):
    return workloads.generate(w, heads=heads)


CASES = {
    "tiny": (W["tiny"], {}, 10),
    "mg_2h_2f": (workloads.scaled(W["matrix_game"], heads=2, frames=2), {}, 3),
    "lb480_ragged_2h_2f": (workloads.scaled(W["lingbot480p"], heads=2, frames=2), {}, 3),
    "lb720_1h_1f_c512_k8": (workloads.scaled(W["lingbot720p"], heads=1, frames=1), {}, 2),
}


def run_case(w, overrides, iters, attn=True, logits=False, frames_per_call=None, seed=7, q_rows=None):
    cfg = P.cfg_of(w, **overrides)
    say("case %s heads=%d F=%d frames=%d C=%d/%d Kc=%d r=%d T=%d io=%s flags=%d" % (
        w.name, cfg.heads, cfg.frame_tokens, cfg.max_frames, cfg.c_k, cfg.c_v, cfg.top_k, cfg.rank,
        cfg.group_tokens, cfg.io, cfg.flags))
    data = case_data(w)
    cal = P.oracle_calibration(w, data, cfg, seed=seed, iters=iters)
    cache, calib = P.build_cache(cfg, cal, data["k"], data["v"], frames_per_call)
    n = data["k"].shape[1]
    assert cache.n_k == n and cache.n_v == n
    gpu = P.gpu_fields(cache, n)
    stats = P.Stats()
    outs = []
    for h in range(cfg.heads):
        ko = P.check_keys_head(cfg, data["k"][h], cal, h, gpu, stats)
        vo = P.check_values_head(cfg, data["v"][h], cal, h, gpu, stats)
        outs.append((ko, vo))
    say("  append parity ok: %s" % dict(stats))
    res = dict(cfg=cfg, data=data, cal=cal, cache=cache, gpu=gpu, outs=outs, stats=stats)
    if attn:
        import video_world_model_amd as qwm
        q = P.to_dev(data["q"], cfg)
        o, lse = qwm.attention(cache, q)
        o = o.float().cpu().numpy()
        lse = lse.cpu().numpy()
        worst_o, worst_l = 0.0, 0.0
        rep = {}
        for h in range(cfg.heads):
            ko, vo = outs[h]
            rows = slice(None) if q_rows is None else q_rows
            wo, wl = P.check_attention(cfg, cal, h, ko, vo, data["q"][h][rows], o[h][rows], lse[h][rows], rep)
            worst_o, worst_l = max(worst_o, wo), max(worst_l, wl)
        say("  attention max(|dO| - half ulp)/tol=%.3g max|dlse|/bound=%.3g %s" % (worst_o, worst_l, rep))
        assert worst_o <= 1.0 and worst_l <= 1.0
        res["o"], res["lse"] = o, lse
    if logits:
        import video_world_model_amd as qwm
        q = P.to_dev(data["q"], cfg)
        lg = qwm.attention_logits(cache, q).cpu().numpy()
        tau = 1.0 / np.sqrt(cfg.head_dim)
        worst = worst_b = 0.0
        for h in range(cfg.heads):
            ko, vo = outs[h]
            _, _, kr, _ = P.oracle_attention(cfg, cal, h, ko, vo, data["q"][h][:1])
            qq = data["q"][h].astype(np.float64)
            ref = tau * qq @ kr.T
            scale = 1e-3 * tau * np.linalg.norm(qq, axis=1)[:, None] * np.linalg.norm(kr, axis=1)[None, :]
            worst = max(worst, float(np.max(np.abs(lg[h] - ref) / scale)))
            if cfg.io == "bf16":
                worst_b = max(worst_b, float(np.max(np.abs(lg[h] - ref) / P.logit_error_bound(cfg, cal, h, ko, qq))))
        say("  logits worst |dl| / (1e-3 tau |q||k~|) = %.3g, / derived bound = %.3g" % (worst, worst_b))
        assert worst <= 1.0 and worst_b <= 1.0
        top = qwm.top1(cache, q).cpu().numpy()
        for h in range(cfg.heads):
            ko, vo = outs[h]
            _, _, kr, _ = P.oracle_attention(cfg, cal, h, ko, vo, data["q"][h][:1])
            qq = data["q"][h].astype(np.float64)
            lgt = qq @ kr.T
            best = lgt.max(axis=1)
            picked = lgt[np.arange(len(qq)), top[h]]
            tol = 1e-3 * np.linalg.norm(qq, axis=1) * np.linalg.norm(kr, axis=1).max()
            assert np.all(best - picked <= tol)
    return res


@pytest.mark.parametrize("name", list(CASES))
def test_parity_cases(name):
    w, ov, iters = CASES[name]
    run_case(w, ov, iters, logits=name in ("tiny", "mg_2h_2f"))


SMALL = workloads.scaled(W["matrix_game"], heads=2, frames=2)


@pytest.mark.parametrize("label,ov", [
    ("qvg_mode", dict(flags=3)),
    ("no_range", dict(flags=2)),
    ("uniform_sens", dict(flags=1)),
    ("rank0", dict(rank=0)),
    ("rank16", dict(rank=16)),
    ("rank5", dict(rank=5)),
    ("rank20", dict(rank=20)),
    ("T1", dict(group_tokens=1)),
    ("T2", dict(group_tokens=2)),
    ("T4", dict(group_tokens=4)),
    ("T8", dict(group_tokens=8)),
    ("T32", dict(group_tokens=32)),
    ("C40", dict(c_k=40, c_v=40)),
    ("C3_lt_Kc", dict(c_k=3, c_v=3)),
    ("Kc2", dict(top_k=2)),
    ("Kc8", dict(top_k=8)),
    ("Kc0", dict(top_k=0)),
    ("exact_error", dict(flags=4)),
    ("full_quadratic", dict(flags=8)),
    ("full_quadratic_uniform", dict(flags=9)),
    ("full_quadratic_Kc8", dict(flags=8, top_k=8)),
])
def test_parity_variants(label, ov):
    run_case(SMALL, ov, iters=3)


def test_parity_rank32_logits_and_top1():
    """r = 32: two PSAC k-steps in both attention kernels (softmax, logits and
    top-1 exports) and the two-pass projection of the append."""
    run_case(SMALL, dict(rank=32), iters=3, logits=True)


def test_parity_rank32_f32_d64():
    """r = 32 with fp32 activations and head_dim 64 (the generic kernel)."""
    run_case(W["tiny"], dict(rank=32), iters=10, logits=True)


def test_local_chunk_rank32():
    """The multi-part kernel with two PSAC k-steps: cache + local chunk."""
    import video_world_model_amd as qwm
    w = workloads.scaled(W["matrix_game"], heads=2, frames=2)
    cfg = P.cfg_of(w, rank=32)
    say("case local_chunk rank32")
    data = case_data(w)
    cal = P.oracle_calibration(w, data, cfg, iters=3)
    cache, _ = P.build_cache(cfg, cal, data["k"], data["v"])
    gpu = P.gpu_fields(cache, cache.n_k)
    stats = P.Stats()
    outs = [(P.check_keys_head(cfg, data["k"][h], cal, h, gpu, stats),
             P.check_values_head(cfg, data["v"][h], cal, h, gpu, stats)) for h in range(cfg.heads)]
    k_loc = np.stack([workloads.kv_frames(w, h, "k", w.frames, w.frames + 1)[:300] for h in range(cfg.heads)])
    v_loc = np.stack([workloads.kv_frames(w, h, "v", w.frames, w.frames + 1)[:300] for h in range(cfg.heads)])
    q = P.to_dev(data["q"], cfg)
    o, lse = qwm.attention_local(cache, q, P.to_dev(k_loc, cfg), P.to_dev(v_loc, cfg))
    wo, wl = check_local(cfg, cal, outs, data["q"], k_loc, v_loc, o.float().cpu().numpy(), lse.cpu().numpy(),
                         range(cfg.heads))
    say("  local chunk r=32: %.3g %.3g" % (wo, wl))
    assert wo <= 1.0 and wl <= 1.0


@pytest.mark.parametrize("flags", [4, 8])
def test_parity_stage2_variants_f32_d64(flags):
    """The exact-error scores on the fp32, head_dim 64 instantiation."""
    run_case(W["tiny"], dict(flags=flags), iters=10)


def test_parity_head_dim_64_bf16():
    w = workloads.scaled(W["matrix_game"], heads=2, frames=2, head_dim=64, n_outliers=2)
    run_case(w, {}, iters=3)


def test_parity_f32_head_dim_128():
    w = workloads.scaled(W["matrix_game"], heads=1, frames=2, io="f32")
    run_case(w, dict(c_k=64, c_v=64), iters=3)


def test_frame_by_frame_equals_bulk():
    import torch
    w = workloads.scaled(W["lingbot480p"], heads=2, frames=3)
    cfg = P.cfg_of(w)
    say("case frame_by_frame_equals_bulk")
    data = case_data(w)
    cal = P.oracle_calibration(w, data, cfg, iters=2)
    c1, _ = P.build_cache(cfg, cal, data["k"], data["v"])
    c2, _ = P.build_cache(cfg, cal, data["k"], data["v"], frames_per_call=1)
    a1, a2 = c1.arrays(), c2.arrays()
    for key in a1:
        assert torch.equal(a1[key], a2[key]), key


def test_split_kv_matches_single_and_empty_cache():
    import torch
    import video_world_model_amd as qwm
    w = workloads.scaled(W["lingbot480p"], heads=2, frames=4)
    cfg = P.cfg_of(w)
    say("case split_kv")
    data = case_data(w)
    cal = P.oracle_calibration(w, data, cfg, iters=2)
    cache, _ = P.build_cache(cfg, cal, data["k"], data["v"])
    q = P.to_dev(data["q"][:, :200], cfg)
    assert qwm.workspace_bytes(cfg, cache.n_k, 200) > 0
    o_split, l_split = qwm.attention(cache, q)
    o_one, l_one = qwm.attention(cache, q, workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    # different fp32 summation orders may land on either side of a bf16
    # rounding boundary: allow one bf16 ulp of |o|
    ref = o_one.float().cpu().numpy()
    diff = np.abs(o_split.float().cpu().numpy() - ref)
    assert np.all(diff <= 4 * P.bf16_half_ulp(ref) + 1e-3)
    # the sum of probabilities is taken over the fp16-rounded values that enter
    # P V, each within 2^-11 relative of the exact one, and every split rounds
    # at its own running max: each lse is within log(1 + 2^-11) of the exact
    # one, so the two differ by at most about 2^-10
    assert float((l_split - l_one).abs().max()) <= 2.0 ** -10
    # empty cache: zero output, lse = -inf
    empty = qwm.Cache(cfg, cache.calib)
    o0, l0 = qwm.attention(empty, q)
    assert float(o0.float().abs().max()) == 0.0 and bool(torch.all(torch.isneginf(l0)))


def test_fused_kv_append_equals_separate():
    import torch
    import video_world_model_amd as qwm
    w = workloads.scaled(W["lingbot480p"], heads=2, frames=3)
    cfg = P.cfg_of(w)
    say("case fused_kv_append")
    data = case_data(w)
    cal = P.oracle_calibration(w, data, cfg, iters=2)
    c1, calib = P.build_cache(cfg, cal, data["k"], data["v"])
    c2 = qwm.Cache(cfg, calib)
    kd, vd = P.to_dev(data["k"], cfg), P.to_dev(data["v"], cfg)
    F = cfg.frame_tokens
    qwm.append_kv(c2, kd[:, :F], vd[:, :F])          # one frame, then the rest
    qwm.append_kv(c2, kd[:, F:], vd[:, F:])
    torch.cuda.synchronize()
    assert c2.n_k == c1.n_k and c2.n_v == c1.n_v
    a1, a2 = c1.arrays(), c2.arrays()
    for key in a1:
        assert torch.equal(a1[key], a2[key]), key


def test_full_size_480p_sampled():
    """The 480p-like workload at full size (40 heads, 24 frames of 1560
    tokens, 1560 queries) in the launch configuration the bench times: one
    fused K+V append of all frames, then attention with the default workspace
    (stream-K).  Heads 0 and 39 are checked against the oracle: every append
    decision with tie following, and attention for 64 sampled queries."""
    import video_world_model_amd as qwm
    w = W["lingbot480p"]
    cfg = P.cfg_of(w)
    say("case full_size_480p: generating and calibrating (oracle)")
    data = workloads.generate(w, threads=16)
    cal = P.oracle_calibration(w, data, cfg, iters=1, threads=16)
    calib = qwm.alloc_calib(cfg)
    qwm.calib_import(cfg, calib, cal["mu_k"], cal["mu_v"], cal["sens"], cal["u"])
    cache = qwm.Cache(cfg, calib)
    qwm.append_kv(cache, P.to_dev(data["k"], cfg), P.to_dev(data["v"], cfg))
    o, lse = qwm.attention(cache, P.to_dev(data["q"], cfg))
    n = data["k"].shape[1]
    assert cache.n_k == n == w.n_tokens
    gpu = P.gpu_fields(cache, n)
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    rows = np.sort(np.random.default_rng(5).choice(w.n_q, 64, replace=False))
    # the timed kernel's logits for the sampled queries
    lg = qwm.attention_logits(cache, P.to_dev(data["q"][:, rows], cfg))
    stats = P.Stats()
    rep = {}
    tau = 1.0 / np.sqrt(cfg.head_dim)
    for h in (0, 39):
        say("  head %d: append parity" % h)
        ko = P.check_keys_head(cfg, data["k"][h], cal, h, gpu, stats)
        vo = P.check_values_head(cfg, data["v"][h], cal, h, gpu, stats)
        wo, wl = P.check_attention(cfg, cal, h, ko, vo, data["q"][h][rows], o[h][rows], lse[h][rows], rep)
        say("  head %d: attention max(|dO| - half ulp)/tol=%.3g max|dlse|/bound=%.3g" % (h, wo, wl))
        assert wo <= 1.0 and wl <= 1.0
        _, _, kr, _ = P.oracle_attention(cfg, cal, h, ko, vo, data["q"][h][:1])
        qq = data["q"][h][rows].astype(np.float64)
        dl = np.abs(lg[h].cpu().numpy() - tau * qq @ kr.T)
        rel = 1e-3 * tau * np.linalg.norm(qq, axis=1)[:, None] * np.linalg.norm(kr, axis=1)[None, :]
        wr, wb = float(np.max(dl / rel)), float(np.max(dl / P.logit_error_bound(cfg, cal, h, ko, qq)))
        say("  head %d: logits worst |dl| / (1e-3 tau |q||k~|) = %.3g, / derived bound = %.3g" % (h, wr, wb))
        assert wr <= 1.0 and wb <= 1.0
    say("  append parity ok: %s; absolute errors %s" % (dict(stats), rep))


def test_full_size_matrix_game_all_heads():
    """The Matrix-Game-2-like workload the default bench line times, at full
    size (12 heads, 6 frames of 880 tokens, 880 queries) and in its launch
    configuration: one fused K+V append of all frames, then attention with
    the stream-K workspace, captured in a HIP graph and replayed.  Every head,
    every append decision (tie following) and every query's output and lse
    are checked against the oracle; so is the generation step with the next
    frame as the local chunk."""
    import torch
    import video_world_model_amd as qwm
    w = W["matrix_game"]
    cfg = P.cfg_of(w)
    say("case full_size_matrix_game: generating and calibrating (oracle)")
    data = workloads.generate(w, threads=16)
    cal = P.oracle_calibration(w, data, cfg, threads=16)
    calib = qwm.alloc_calib(cfg)
    qwm.calib_import(cfg, calib, cal["mu_k"], cal["mu_v"], cal["sens"], cal["u"])
    cache = qwm.Cache(cfg, calib)
    kd, vd, qd = P.to_dev(data["k"], cfg), P.to_dev(data["v"], cfg), P.to_dev(data["q"], cfg)
    out = torch.empty_like(qd)
    lse = torch.empty(cfg.heads, w.n_q, dtype=torch.float32, device="cuda")
    ws = torch.empty(qwm.workspace_bytes(cfg, w.n_tokens, w.n_q), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):  # warm-up outside the capture
        cache.reset()
        qwm.append_kv(cache, kd, vd)
        qwm.attention(cache, qd, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cache.reset()
        qwm.append_kv(cache, kd, vd)
        qwm.attention(cache, qd, out=out, lse=lse, workspace=ws)
    out.zero_()
    g.replay()
    torch.cuda.synchronize()
    n = w.n_tokens
    assert cache.n_k == n
    gpu = P.gpu_fields(cache, n)
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    stats = P.Stats()
    outs = []
    worst_o = worst_l = 0.0
    rep = {}
    for h in range(cfg.heads):
        ko = P.check_keys_head(cfg, data["k"][h], cal, h, gpu, stats)
        vo = P.check_values_head(cfg, data["v"][h], cal, h, gpu, stats)
        outs.append((ko, vo))
        wo, wl = P.check_attention(cfg, cal, h, ko, vo, data["q"][h], o[h], l[h], rep)
        worst_o, worst_l = max(worst_o, wo), max(worst_l, wl)
    say("  append parity ok: %s; attention max(|dO| - half ulp)/tol=%.3g max|dlse|/bound=%.3g; absolute %s"
        % (dict(stats), worst_o, worst_l, rep))
    assert worst_o <= 1.0 and worst_l <= 1.0
    k_loc = np.stack([workloads.kv_frames(w, h, "k", w.frames, w.frames + 1) for h in range(cfg.heads)])
    v_loc = np.stack([workloads.kv_frames(w, h, "v", w.frames, w.frames + 1) for h in range(cfg.heads)])
    o2, l2 = qwm.attention_local(cache, qd, P.to_dev(k_loc, cfg), P.to_dev(v_loc, cfg))
    wo, wl = check_local(cfg, cal, outs, data["q"], k_loc, v_loc, o2.float().cpu().numpy(), l2.cpu().numpy(),
                         range(cfg.heads))
    say("  generation step with the local chunk: %.3g %.3g" % (wo, wl))
    assert wo <= 1.0 and wl <= 1.0


def check_local(cfg, cal, outs, q, k_loc, v_loc, o, lse, heads):
    """Attention over cache + local chunk against the oracle: worst output and
    lse errors over their bounds (2e-2 beyond the bf16 output rounding; the
    lse bound derived from both key sets' operands)."""
    worst_o, worst_l = 0.0, 0.0
    for h in heads:
        qq = q[h].astype(np.float64)
        parts = []
        if outs is not None:
            ko, vo = outs[h]
            _, _, kr, vr = P.oracle_attention(cfg, cal, h, ko, vo, q[h][:1])
            parts.append((kr, vr, P.logit_error_bound(cfg, cal, h, ko, qq)))
        kl, vl = k_loc[h].astype(np.float64), v_loc[h].astype(np.float64)
        parts.append((kl, vl, P.local_logit_error_bound(qq, kl)))
        wo, wl = P.check_parts(qq, parts, o[h], lse[h])
        worst_o, worst_l = max(worst_o, wo), max(worst_l, wl)
    return worst_o, worst_l


@pytest.mark.parametrize("n_loc", [880, 100])
def test_local_chunk_attention(n_loc):
    """One generation step: the query chunk over the compressed cache (2
    frames) and the chunk's own bf16 keys and values (the next frame, whole or
    a ragged prefix), with stream-K pieces that straddle the two key sets."""
    import video_world_model_amd as qwm
    w = workloads.scaled(W["matrix_game"], heads=2, frames=2)
    cfg = P.cfg_of(w)
    say("case local_chunk n_loc=%d" % n_loc)
    data = case_data(w)
    cal = P.oracle_calibration(w, data, cfg, iters=3)
    cache, _ = P.build_cache(cfg, cal, data["k"], data["v"])
    gpu = P.gpu_fields(cache, cache.n_k)
    stats = P.Stats()
    outs = [(P.check_keys_head(cfg, data["k"][h], cal, h, gpu, stats),
             P.check_values_head(cfg, data["v"][h], cal, h, gpu, stats)) for h in range(cfg.heads)]
    k_loc = np.stack([workloads.kv_frames(w, h, "k", w.frames, w.frames + 1)[:n_loc] for h in range(cfg.heads)])
    v_loc = np.stack([workloads.kv_frames(w, h, "v", w.frames, w.frames + 1)[:n_loc] for h in range(cfg.heads)])
    q = P.to_dev(data["q"], cfg)
    o, lse = qwm.attention_local(cache, q, P.to_dev(k_loc, cfg), P.to_dev(v_loc, cfg))
    wo, wl = check_local(cfg, cal, outs, data["q"], k_loc, v_loc, o.float().cpu().numpy(), lse.cpu().numpy(),
                         range(cfg.heads))
    say("  local chunk: max(|dO| - half ulp)/tol=%.3g max|dlse|/bound=%.3g" % (wo, wl))
    assert wo <= 1.0 and wl <= 1.0


def test_local_chunk_edge_cases():
    """Empty cache (local keys alone); no local keys (the cache-only kernel,
    bit for bit); one ragged local tile over an empty cache."""
    import torch
    import video_world_model_amd as qwm
    w = workloads.scaled(W["matrix_game"], heads=2, frames=1)
    cfg = P.cfg_of(w)
    say("case local_chunk_edges")
    data = case_data(w)
    cal = P.oracle_calibration(w, data, cfg, iters=2)
    cache, calib = P.build_cache(cfg, cal, data["k"], data["v"])
    q = P.to_dev(data["q"][:, :300], cfg)
    k_loc = np.stack([workloads.kv_frames(w, h, "k", 1, 2) for h in range(cfg.heads)])
    v_loc = np.stack([workloads.kv_frames(w, h, "v", 1, 2) for h in range(cfg.heads)])
    kd, vd = P.to_dev(k_loc, cfg), P.to_dev(v_loc, cfg)
    # no local keys: identical to qwm.attention
    o_a, l_a = qwm.attention(cache, q)
    o_b, l_b = qwm.attention_local(cache, q, kd[:, :0], vd[:, :0])
    assert torch.equal(o_a, o_b) and torch.equal(l_a, l_b)
    # empty cache: attention over the local chunk alone
    empty = qwm.Cache(cfg, calib)
    for n in (880, 37):
        o, lse = qwm.attention_local(empty, q, kd[:, :n].contiguous(), vd[:, :n].contiguous())
        wo, wl = check_local(cfg, cal, None, data["q"][:, :300], k_loc[:, :n], v_loc[:, :n],
                             o.float().cpu().numpy(), lse.cpu().numpy(), range(cfg.heads))
        say("  empty cache, n_loc=%d: %.3g %.3g" % (n, wo, wl))
        assert wo <= 1.0 and wl <= 1.0


def test_graph_replay_equals_eager():
    """One step (reset, fused append, attention with its merge pass) captured
    into a HIP graph and replayed three times, with other work and
    synchronisations between the replays: every replay reproduces the eager
    cache fields and outputs bit for bit."""
    import torch
    import video_world_model_amd as qwm
    w = workloads.scaled(W["matrix_game"], heads=2, frames=2)
    cfg = P.cfg_of(w)
    say("case graph_replay")
    data = case_data(w)
    cal = P.oracle_calibration(w, data, cfg, iters=2)
    cache, calib = P.build_cache(cfg, cal, data["k"], data["v"])
    q = P.to_dev(data["q"], cfg)
    o_e, l_e = qwm.attention(cache, q)
    fields_e = {k: v.clone() for k, v in cache.arrays().items()}
    kd, vd = P.to_dev(data["k"], cfg), P.to_dev(data["v"], cfg)
    c2 = qwm.Cache(cfg, calib)
    o_g, l_g = torch.empty_like(o_e), torch.empty_like(l_e)
    ws = torch.empty(max(qwm.workspace_bytes(cfg, data["k"].shape[1], q.shape[1]), 1), dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        c2.reset()
        qwm.append_kv(c2, kd, vd)
        qwm.attention(c2, q, out=o_g, lse=l_g, workspace=ws)
    q_other = P.to_dev(data["q"][:, :100], cfg)
    for rep in range(3):
        o_g.zero_()
        l_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(l_g, l_e), "replay %d" % rep
        for name, ref in fields_e.items():
            assert torch.equal(c2.arrays()[name], ref), (rep, name)
        # other eager work between the replays
        qwm.attention(cache, q_other)
        torch.cuda.synchronize()


def _epoch_cache(cfg, cal, k, v):
    """A cache bound to its own calibration, holding k, v (possibly no frames)."""
    import torch
    import video_world_model_amd as qwm
    if k.shape[1]:
        return P.build_cache(cfg, cal, k, v)[0]
    calib = qwm.alloc_calib(cfg)
    qwm.calib_import(cfg, calib, cal["mu_k"], cal["mu_v"], cal["sens"], cal["u"])
    torch.cuda.synchronize()
    return qwm.Cache(cfg, calib)


@pytest.mark.parametrize("with_local", [True, False])
def test_epochs_attention(with_local):
    """Attention over three calibration epochs of one rollout (2, 0 and 1
    frames, each encoded with a calibration of its own: the first from the
    history window, the later ones from the last frame before them) and,
    optionally, the chunk's own keys: one softmax against the oracle, each
    epoch's tokens rebuilt with its own centres and U.  Stream-K pieces start
    inside and cross the epoch boundaries."""
    import video_world_model_amd as qwm
    from oracle import attention as oa
    w = workloads.scaled(W["matrix_game"], heads=2, frames=3)
    cfg = P.cfg_of(w)
    F = w.frame_tokens
    say("case epochs_attention local=%s" % with_local)
    data = case_data(w)
    spans = [(0, 2), (2, 2), (2, 3)]
    caches, rebuilt = [], [[] for _ in range(cfg.heads)]
    qq = [data["q"][h].astype(np.float64) for h in range(cfg.heads)]
    for e, (a, b) in enumerate(spans):
        if e == 0:
            hist = data
        else:
            hist = dict(q_hist=data["q"], k_hist=data["k"][:, (a - 1) * F:a * F],
                        v_hist=data["v"][:, (a - 1) * F:a * F])
        cal = P.oracle_calibration(w, hist, cfg, seed=7 + e, iters=3)
        k_e, v_e = data["k"][:, a * F:b * F], data["v"][:, a * F:b * F]
        cache = _epoch_cache(cfg, cal, k_e, v_e)
        caches.append(cache)
        n = k_e.shape[1]
        if n == 0:
            for h in range(cfg.heads):
                rebuilt[h].append((np.zeros((0, cfg.head_dim)), np.zeros((0, cfg.head_dim)),
                                   np.zeros((w.n_q, 0))))
            continue
        gpu = P.gpu_fields(cache, n)
        stats = P.Stats()
        for h in range(cfg.heads):
            ko = P.check_keys_head(cfg, k_e[h], cal, h, gpu, stats)
            vo = P.check_values_head(cfg, v_e[h], cal, h, gpu, stats)
            _, _, kr, vr = P.oracle_attention(cfg, cal, h, ko, vo, data["q"][h][:1])
            rebuilt[h].append((kr, vr, P.logit_error_bound(cfg, cal, h, ko, qq[h])))
        say("  epoch %d append parity ok: %s" % (e, dict(stats)))
    q = P.to_dev(data["q"], cfg)
    if with_local:
        k_loc = np.stack([workloads.kv_frames(w, h, "k", 3, 4)[:500] for h in range(cfg.heads)])
        v_loc = np.stack([workloads.kv_frames(w, h, "v", 3, 4)[:500] for h in range(cfg.heads)])
        o, lse = qwm.attention_epochs(caches, q, P.to_dev(k_loc, cfg), P.to_dev(v_loc, cfg))
    else:
        k_loc = v_loc = np.zeros((cfg.heads, 0, cfg.head_dim))
        o, lse = qwm.attention_epochs(caches, q)
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    worst_o, worst_l = 0.0, 0.0
    for h in range(cfg.heads):
        # the oracle's one softmax over every epoch and the local keys ...
        oo, ll = oa.attention_over_epochs(data["q"][h], [(kr, vr) for kr, vr, _ in rebuilt[h]],
                                          k_loc[h].astype(np.float64), v_loc[h].astype(np.float64))
        kl = k_loc[h].astype(np.float64)
        parts = rebuilt[h] + [(kl, v_loc[h].astype(np.float64), P.local_logit_error_bound(qq[h], kl))]
        wo, wl = P.check_parts(qq[h], parts, o[h], lse[h])
        # ... is the softmax over the concatenated key sets that check_parts takes
        _, ll2 = oa.softmax_attention(qq[h], np.concatenate([k for k, _, _ in parts]),
                                      np.concatenate([v for _, v, _ in parts]))
        assert np.allclose(ll, ll2, rtol=0, atol=1e-9)
        worst_o, worst_l = max(worst_o, wo), max(worst_l, wl)
    say("  epochs: max(|dO| - half ulp)/tol=%.3g max|dlse|/bound=%.3g" % (worst_o, worst_l))
    assert worst_o <= 1.0 and worst_l <= 1.0


def test_epochs_single_equals_local():
    """One epoch: qwm_attention_epochs is qwm_attention_local, bit for bit."""
    import torch
    import video_world_model_amd as qwm
    w = workloads.scaled(W["matrix_game"], heads=2, frames=1)
    cfg = P.cfg_of(w)
    say("case epochs_single_equals_local")
    data = case_data(w)
    cal = P.oracle_calibration(w, data, cfg, iters=2)
    cache, _ = P.build_cache(cfg, cal, data["k"], data["v"])
    q = P.to_dev(data["q"][:, :300], cfg)
    kd = P.to_dev(np.stack([workloads.kv_frames(w, h, "k", 1, 2) for h in range(cfg.heads)]), cfg)
    vd = P.to_dev(np.stack([workloads.kv_frames(w, h, "v", 1, 2) for h in range(cfg.heads)]), cfg)
    o_a, l_a = qwm.attention_local(cache, q, kd, vd)
    o_b, l_b = qwm.attention_epochs([cache], q, kd, vd)
    assert torch.equal(o_a, o_b) and torch.equal(l_a, l_b)
    o_c, l_c = qwm.attention(cache, q)
    o_d, l_d = qwm.attention_epochs([cache], q)
    assert torch.equal(o_c, o_d) and torch.equal(l_c, l_d)


def test_epochs_edge_cases():
    """Sixteen epochs (the most one call takes; one frame each, several empty),
    and epochs that are all empty with and without local keys."""
    import torch
    import video_world_model_amd as qwm
    from oracle import attention as oa
    w = workloads.scaled(W["matrix_game"], heads=1, frames=4)
    cfg = P.cfg_of(w, max_frames=1)
    F = w.frame_tokens
    say("case epochs_edges")
    data = case_data(w)
    cal = P.oracle_calibration(w, data, cfg, iters=2)
    caches, rebuilt = [], []
    frames = [0, None, 1, None, None, 2, None, None, None, None, 3, None, None, None, None, None]
    for f in frames:
        if f is None:
            caches.append(_epoch_cache(cfg, cal, data["k"][:, :0], data["v"][:, :0]))
            continue
        k_e, v_e = data["k"][:, f * F:(f + 1) * F], data["v"][:, f * F:(f + 1) * F]
        cache = _epoch_cache(cfg, cal, k_e, v_e)
        caches.append(cache)
        gpu = P.gpu_fields(cache, F)
        stats = P.Stats()
        ko = P.check_keys_head(cfg, k_e[0], cal, 0, gpu, stats)
        vo = P.check_values_head(cfg, v_e[0], cal, 0, gpu, stats)
        _, _, kr, vr = P.oracle_attention(cfg, cal, 0, ko, vo, data["q"][0][:1])
        rebuilt.append((kr, vr, P.logit_error_bound(cfg, cal, 0, ko, data["q"][0][:200].astype(np.float64))))
    assert len(caches) == 16
    q = P.to_dev(data["q"][:, :200], cfg)
    o, lse = qwm.attention_epochs(caches, q)
    wo, wl = P.check_parts(data["q"][0][:200].astype(np.float64), rebuilt, o[0].float().cpu().numpy(),
                           lse[0].cpu().numpy())
    say("  16 epochs: %.3g %.3g" % (wo, wl))
    assert wo <= 1.0 and wl <= 1.0
    # every epoch empty: no keys (zeros, lse = -inf), or the local keys alone
    empties = [c for c in caches if c.n_k == 0][:3]
    o0, l0 = qwm.attention_epochs(empties, q)
    assert float(o0.float().abs().max()) == 0.0 and bool(torch.isinf(l0).all())
    k_loc = workloads.kv_frames(w, 0, "k", 4, 5)[None, :77]
    v_loc = workloads.kv_frames(w, 0, "v", 4, 5)[None, :77]
    o1, l1 = qwm.attention_epochs(empties, q, P.to_dev(k_loc, cfg), P.to_dev(v_loc, cfg))
    wo, wl = check_local(cfg, cal, None, data["q"][:, :200], k_loc, v_loc, o1.float().cpu().numpy(),
                         l1.cpu().numpy(), [0])
    say("  empty epochs + local: %.3g %.3g" % (wo, wl))
    assert wo <= 1.0 and wl <= 1.0



def test_epochs_most_parts():
    """Sixty-four epochs, the most one call takes (one frame in four of them,
    the others empty), against the oracle."""
    import video_world_model_amd as qwm
    w = workloads.scaled(W["matrix_game"], heads=1, frames=4)
    cfg = P.cfg_of(w, max_frames=1)
    F = w.frame_tokens
    say("case epochs_64")
    data = case_data(w)
    cal = P.oracle_calibration(w, data, cfg, iters=2)
    where = {0: 0, 17: 1, 40: 2, 63: 3}
    caches, rebuilt = [], []
    for e in range(64):
        f = where.get(e)
        if f is None:
            caches.append(_epoch_cache(cfg, cal, data["k"][:, :0], data["v"][:, :0]))
            continue
        k_e, v_e = data["k"][:, f * F:(f + 1) * F], data["v"][:, f * F:(f + 1) * F]
        cache = _epoch_cache(cfg, cal, k_e, v_e)
        caches.append(cache)
        gpu = P.gpu_fields(cache, F)
        stats = P.Stats()
        ko = P.check_keys_head(cfg, k_e[0], cal, 0, gpu, stats)
        vo = P.check_values_head(cfg, v_e[0], cal, 0, gpu, stats)
        _, _, kr, vr = P.oracle_attention(cfg, cal, 0, ko, vo, data["q"][0][:1])
        rebuilt.append((kr, vr, P.logit_error_bound(cfg, cal, 0, ko, data["q"][0][:200].astype(np.float64))))
    q = P.to_dev(data["q"][:, :200], cfg)
    o, lse = qwm.attention_epochs(caches, q)
    wo, wl = P.check_parts(data["q"][0][:200].astype(np.float64), rebuilt, o[0].float().cpu().numpy(),
                           lse[0].cpu().numpy())
    say("  64 epochs: %.3g %.3g" % (wo, wl))
    assert wo <= 1.0 and wl <= 1.0

def test_degenerate_inputs_zero_residual_and_tied_centres():
    """Keys and Values that sit exactly on their centres (zero residual: every
    tile scale 0, every code 0, every PSAC scale 0) mixed with ordinary tokens,
    and a codebook with a duplicated centre (exact score ties, taken to the
    lower index by both appends).  Append parity with tie following; where the residual is
    zero the rebuilt keys equal the inputs, so attention over those tokens is
    plain softmax attention over the bf16 keys."""
    import torch
    import video_world_model_amd as qwm
    from oracle import attention as oa
    w = workloads.scaled(W["matrix_game"], heads=2, frames=2)
    cfg = P.cfg_of(w)
    say("case degenerate_inputs")
    data = case_data(w)
    cal = P.oracle_calibration(w, data, cfg, iters=2)
    for key in ("mu_k", "mu_v"):  # centre 1 repeats centre 0
        cal[key] = cal[key].copy()
        cal[key][:, 1] = cal[key][:, 0]
    rng = np.random.default_rng(3)
    k, v = data["k"].copy(), data["v"].copy()
    n = k.shape[1]
    on = rng.random(n) < 0.75  # tokens placed on a centre (the first frame: all of them)
    on[:w.frame_tokens] = True
    for h in range(cfg.heads):
        ck = rng.integers(0, cfg.c_k, n)
        cv = rng.integers(0, cfg.c_v, n)
        k[h, on] = cal["mu_k"][h][ck[on]]
        v[h, on] = cal["mu_v"][h][cv[on]]
    cache, _ = P.build_cache(cfg, cal, k, v)
    gpu = P.gpu_fields(cache, n)
    stats = P.Stats()
    q = P.to_dev(data["q"], cfg)
    o, lse = qwm.attention(cache, q)
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    F, T = w.frame_tokens, w.group_tokens
    for h in range(cfg.heads):
        ko = P.check_keys_head(cfg, k[h], cal, h, gpu, stats)
        vo = P.check_values_head(cfg, v[h], cal, h, gpu, stats)
        # the first frame lies on centres: zero scales and codes in all its tiles
        tiles0 = -(-F // T)
        assert np.all(gpu["s_k"][h][:tiles0] == 0) and np.all(gpu["s_v"][h][:tiles0] == 0)
        assert np.all(gpu["codes_k"][h][:F] == 0) and np.all(gpu["coef_scale"][h][:F] == 0)
        wo, wl = P.check_attention(cfg, cal, h, ko, vo, data["q"][h], o[h], lse[h])
        assert wo <= 1.0 and wl <= 1.0
        # rebuilt keys and values of the first frame equal the inputs
        _, _, kr, vr = P.oracle_attention(cfg, cal, h, ko, vo, data["q"][h][:1])
        assert np.array_equal(kr[:F], k[h][:F].astype(np.float64))
        assert np.array_equal(vr[:F], v[h][:F].astype(np.float64))
    # a duplicated centre is never chosen over its first copy (exact ties go
    # to the lower index)
    assert not np.any(gpu["idx_v"] == 1) and not np.any(gpu["idx_k"] == 1)
    say("  degenerate inputs ok: %s" % dict(stats))
