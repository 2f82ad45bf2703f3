"""Full-size parity at the two largest workloads, in the launch configuration
bench.py times, on sampled heads and queries.

Heads are independent in every kernel (each workgroup reads and writes one
head's slices), so the unchecked heads carry copies of head 0's inputs and
calibration: the grid, the capacities and every offset are those of the full
workload, and the checked heads hold the seeded workload's own data.
  * 720p (40 heads, 24 frames of 3,600 tokens, 512 centres, K_c = 8): one fused
    K+V append of all frames, attention with the stream-K workspace.  Head 39
    is checked token by token (every append decision with tie following, 64
    sampled queries' outputs and lse); head 0 on its first and last frames.
  * 1-minute (40 heads, 240 frames of 1,560 tokens): frame-by-frame appends of
    frames 0..238, then the generation step the benchmark times, captured in
    a HIP graph and replayed twice: append of frame 239 and attention of the
    1,560-query chunk over all 374,400 cached tokens.  Head 0 is checked
    token by token and on 32 sampled queries; head 39 on frames 0, 1, 238
    and 239."""
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import workloads
from oracle import codec
from tests import parity as P

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def head_inputs(w, h, frames):
    k = workloads.kv_frames(w, h, "k", 0, frames)
    v = workloads.kv_frames(w, h, "v", 0, frames)
    q = workloads.queries(w, h, w.n_q, historical=False)
    qh = workloads.queries(w, h, w.n_q_hist, historical=True)
    return k, v, q, qh


def calibration_two_heads(w, cfg, ins, heads):
    """Oracle calibration of the checked heads (1 Lloyd round, the window is
    the first frame); the other heads take head 0's."""
    cals = {}
    for h in heads:
        k, v, q, qh = ins[h]
        F = w.frame_tokens
        d = dict(q_hist=qh[None], k_hist=k[None, :F], v_hist=v[None, :F])
        cals[h] = P.oracle_calibration(w, d, cfg, seed=7 + 2 * h, iters=1)
    full = {}
    for key in ("mu_k", "mu_v", "sens", "u"):
        arr = np.concatenate([cals[heads[0]][key]] * w.heads)
        for h in heads:
            arr[h] = cals[h][key][0]
        full[key] = arr
    return full


def head_view(cal, h):
    return {key: cal[key][h:h + 1] for key in ("mu_k", "mu_v", "sens", "u")}


def check_frames(cfg, cal, h, k, v, gpu, frames, stats, threads=16):
    """Append parity of one head on whole frames (every decision, tie
    following), through the single-frame view of the library's fields."""
    F = cfg.frame_tokens
    tpf = -(-F // cfg.group_tokens)
    calh = head_view(cal, h)

    def one(f):
        sub = {}
        for key in ("idx_k", "idx_v", "codes_k", "codes_v", "coef", "coef_scale"):
            if key in gpu:
                sub[key] = gpu[key][h:h + 1, f * F:(f + 1) * F]
        for key in ("z_k", "s_k", "z_v", "s_v"):
            sub[key] = gpu[key][h:h + 1, f * tpf:(f + 1) * tpf]
        st = P.Stats()
        ko = P.check_keys_head(cfg, k[f * F:(f + 1) * F], calh, 0, sub, st)
        vo = P.check_values_head(cfg, v[f * F:(f + 1) * F], calh, 0, sub, st)
        return f, ko, vo, st
    outs = {}
    with ThreadPoolExecutor(threads) as ex:
        for f, ko, vo, st in ex.map(one, frames):
            outs[f] = (ko, vo)
            for key, val in st.items():
                stats.add(key, val)
    return outs


def concat_outs(outs, frames, cfg):
    """Oracle outputs of whole frames joined into one head's token axis."""
    ko = {key: np.concatenate([outs[f][0][key] for f in frames]) for key in ("idx", "codes", "coef", "coef_scale")}
    ko["z"] = np.concatenate([outs[f][0]["z"] for f in frames])
    ko["s"] = np.concatenate([outs[f][0]["s"] for f in frames])
    vo = {key: np.concatenate([outs[f][1][key] for f in frames]) for key in ("idx", "codes", "z", "s")}
    return ko, vo


def device_inputs(w, cfg, ins, heads, frames):
    """[H, n, d] device tensors: the checked heads' own data, head 0's copy
    elsewhere."""
    import torch
    n = frames * w.frame_tokens
    out = []
    for idx in range(4):
        rows = ins[heads[0]][idx]
        t = P.to_dev(rows[None], cfg).expand(w.heads, -1, -1).contiguous()
        for h in heads[1:]:
            t[h] = P.to_dev(ins[h][idx], cfg)
        out.append(t)
    torch.cuda.synchronize()
    assert out[0].shape[1] == n
    return out


def test_full_size_720p_sampled():
    import video_world_model_amd as qwm
    w = W["lingbot720p"]
    cfg = P.cfg_of(w)
    heads = [0, 39]
    say("case full_size_720p: generating heads %s and calibrating (oracle)" % heads)
    ins = {h: head_inputs(w, h, w.frames) for h in heads}
    cal = calibration_two_heads(w, cfg, ins, heads)
    kd, vd, qd, _ = device_inputs(w, cfg, ins, heads, w.frames)
    calib = qwm.alloc_calib(cfg)
    qwm.calib_import(cfg, calib, cal["mu_k"], cal["mu_v"], cal["sens"], cal["u"])
    cache = qwm.Cache(cfg, calib)
    qwm.append_kv(cache, kd, vd)
    o, lse = qwm.attention(cache, qd)
    n = w.n_tokens
    gpu = P.gpu_fields(cache, n)
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    stats = P.Stats()
    say("  head 39: every frame; head 0: frames 0 and 23")
    outs39 = check_frames(cfg, cal, 39, ins[39][0], ins[39][1], gpu, range(w.frames), stats)
    check_frames(cfg, cal, 0, ins[0][0], ins[0][1], gpu, [0, w.frames - 1], stats)
    ko, vo = concat_outs(outs39, range(w.frames), cfg)
    rows = np.sort(np.random.default_rng(9).choice(w.n_q, 64, replace=False))
    rep = {}
    wo, wl = P.check_attention(cfg, cal, 39, ko, vo, ins[39][2][rows], o[39][rows], lse[39][rows], rep)
    say("  append parity %s; head 39 attention max(|dO| - half ulp)/tol=%.3g max|dlse|/bound=%.3g %s"
        % (dict(stats), wo, wl, rep))
    assert wo <= 1.0 and wl <= 1.0


def test_full_size_minute_sampled():
    import torch
    import video_world_model_amd as qwm
    w = W["minute"]
    cfg = P.cfg_of(w)
    heads = [0, 39]
    F, nf = w.frame_tokens, w.frames
    say("case full_size_minute: generating heads %s and calibrating (oracle)" % heads)
    ins = {h: head_inputs(w, h, nf) for h in heads}
    cal = calibration_two_heads(w, cfg, ins, heads)
    kd, vd, qd, _ = device_inputs(w, cfg, ins, heads, nf)
    calib = qwm.alloc_calib(cfg)
    qwm.calib_import(cfg, calib, cal["mu_k"], cal["mu_v"], cal["sens"], cal["u"])
    cache = qwm.Cache(cfg, calib)
    for f in range(nf - 1):
        qwm.append_kv(cache, kd[:, f * F:(f + 1) * F], vd[:, f * F:(f + 1) * F])
    out = torch.empty_like(qd)
    lse = torch.empty(cfg.heads, w.n_q, dtype=torch.float32, device="cuda")
    ws = torch.empty(qwm.workspace_bytes(cfg, w.n_tokens, w.n_q), dtype=torch.uint8, device="cuda")
    k_last, v_last = kd[:, (nf - 1) * F:].contiguous(), vd[:, (nf - 1) * F:].contiguous()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    n_before = cache.n_k
    with torch.cuda.graph(g):
        qwm.append_kv(cache, k_last, v_last)
        qwm.attention(cache, qd, out=out, lse=lse, workspace=ws)
    assert cache.n_k == w.n_tokens
    for _ in range(2):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
    assert n_before == (nf - 1) * F
    gpu = P.gpu_fields(cache, w.n_tokens)
    o, l = out.float().cpu().numpy(), lse.cpu().numpy()
    stats = P.Stats()
    say("  head 0: all %d frames (oracle append); head 39: frames 0, 1, %d, %d" % (nf, nf - 2, nf - 1))
    outs0 = check_frames(cfg, cal, 0, ins[0][0], ins[0][1], gpu, range(nf), stats)
    check_frames(cfg, cal, 39, ins[39][0], ins[39][1], gpu, [0, 1, nf - 2, nf - 1], stats)
    ko, vo = concat_outs(outs0, range(nf), cfg)
    rows = np.sort(np.random.default_rng(10).choice(w.n_q, 32, replace=False))
    rep = {}
    wo, wl = P.check_attention(cfg, cal, 0, ko, vo, ins[0][2][rows], o[0][rows], l[0][rows], rep)
    say("  append parity %s; head 0 attention max(|dO| - half ulp)/tol=%.3g max|dlse|/bound=%.3g %s"
        % (dict(stats), wo, wl, rep))
    assert wo <= 1.0 and wl <= 1.0
