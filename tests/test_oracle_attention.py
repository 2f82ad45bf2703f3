"""Pins of the oracle's reconstruction + attention and measures (CPU only)."""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as oa
from oracle import calibrate as oc
from oracle import codec, measures


@pytest.fixture(scope="module")
def tiny():
    w = workloads.WORKLOADS["tiny"]
    d = workloads.generate(w)
    cal = oc.calibrate(d["q_hist"], d["k_hist"], d["v_hist"], 16, 16, 8, "f32", seed=11)
    return w, d, cal


def _zero_residual_keys(mu, n, seed):
    """Keys drawn exactly on the centres: rho = 0, e = 0."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, mu.shape[0], n)
    return mu[idx].copy(), idx


def test_zero_residual_reduces_to_textbook_attention(tiny):
    w, d, cal = tiny
    mu_k, mu_v, u = cal["mu_k"][0], cal["mu_v"][0], cal["u"][0]
    k, _ = _zero_residual_keys(mu_k, 128, 1)
    v, _ = _zero_residual_keys(mu_v, 128, 2)
    ko = codec.append_keys(k, mu_k, cal["sens"][0], u, 64, 16, 4, 0)
    vo = codec.append_values(v, mu_v, 64, 16)
    assert np.all(ko["codes"] == 0) and np.all(ko["s"] == 0) and np.all(ko["coef"] == 0)
    kr = oa.reconstruct_keys(ko["idx"], ko["codes"], ko["z"], ko["s"], ko["coef"],
                             ko["coef_scale"], mu_k, u, 64, 16)
    vr = oa.reconstruct_values(vo["idx"], vo["codes"], vo["z"], vo["s"], mu_v, 64, 16)
    assert np.array_equal(kr, k.astype(np.float64)) and np.array_equal(vr, v.astype(np.float64))
    q = d["q"][0]
    o, lse = oa.softmax_attention(q, kr, vr)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64))[None],
        torch.from_numpy(k.astype(np.float64))[None],
        torch.from_numpy(v.astype(np.float64))[None])[0].numpy()
    assert np.max(np.abs(o - ref)) < 1e-12
    assert measures.top1_shift(q, k, kr) == 0.0


def test_constant_values_give_that_value():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((5, 16))
    k = rng.standard_normal((40, 16))
    vconst = rng.standard_normal(16)
    o, _ = oa.softmax_attention(q, k, np.tile(vconst, (40, 1)))
    assert np.max(np.abs(o - vconst)) < 1e-12


def test_softmax_rows_sum_to_one_and_lse():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((6, 16)) * 4
    k = rng.standard_normal((50, 16)) * 4
    lg = oa.logits(q, k)
    _, lse = oa.softmax_attention(q, k, np.eye(50, 16))
    p = np.exp(lg - lse[:, None])
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12)
    for i in range(6):
        assert abs(lse[i] - math.log(sum(math.exp(x) for x in lg[i]))) < 1e-12


def test_split_lse_merge_equals_unsplit():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((7, 32))
    k = rng.standard_normal((300, 32)) * 2
    v = rng.standard_normal((300, 32))
    o, lse = oa.softmax_attention(q, k, v)
    parts = [oa.softmax_attention(q, k[a:a + 77], v[a:a + 77]) for a in range(0, 300, 77)]
    om, lm = oa.merge_partials(parts)
    assert np.max(np.abs(om - o)) < 1e-12 and np.max(np.abs(lm - lse)) < 1e-12


def test_bruteforce_attention_tiny(tiny):
    """Invariant (d) for attention: per-query scalar loops (math.exp) on the
    tiny case equal the vectorised oracle."""
    w, d, cal = tiny
    ko = codec.append_keys(d["k"][0], cal["mu_k"][0], cal["sens"][0], cal["u"][0], 64, 16, 4, 0)
    vo = codec.append_values(d["v"][0], cal["mu_v"][0], 64, 16)
    kr = oa.reconstruct_keys(ko["idx"], ko["codes"], ko["z"], ko["s"], ko["coef"],
                             ko["coef_scale"], cal["mu_k"][0], cal["u"][0], 64, 16)
    vr = oa.reconstruct_values(vo["idx"], vo["codes"], vo["z"], vo["s"], cal["mu_v"][0], 64, 16)
    q = d["q"][0].astype(np.float64)
    o, lse = oa.softmax_attention(q, kr, vr)
    for i in range(0, q.shape[0], 4):
        lg = [sum(q[i, j] * kr[t, j] for j in range(64)) / 8.0 for t in range(128)]
        m = max(lg)
        ex = [math.exp(x - m) for x in lg]
        tot = sum(ex)
        for j in range(0, 64, 9):
            oj = sum(ex[t] * vr[t, j] for t in range(128)) / tot
            assert abs(oj - o[i, j]) < 1e-10
        assert abs(m + math.log(tot) - lse[i]) < 1e-10


def test_local_chunk_bruteforce():
    """One softmax over cache and local keys, by per-query loops."""
    rng = np.random.default_rng(21)
    q = rng.standard_normal((3, 8))
    kc, vc = rng.standard_normal((5, 8)), rng.standard_normal((5, 8))
    kl, vl = rng.standard_normal((4, 8)), rng.standard_normal((4, 8))
    o, lse = oa.attention_with_local(q, kc, vc, kl, vl)
    for i in range(3):
        keys = list(kc) + list(kl)
        vals = list(vc) + list(vl)
        ls = [sum(q[i, j] * kk[j] for j in range(8)) / math.sqrt(8) for kk in keys]
        m = max(ls)
        ws = [math.exp(x - m) for x in ls]
        tot = sum(ws)
        for j in range(8):
            ref = sum(wt * vv[j] for wt, vv in zip(ws, vals)) / tot
            assert abs(o[i, j] - ref) < 1e-12
        assert abs(lse[i] - (m + math.log(tot))) < 1e-12


def test_local_chunk_without_cache_is_sdpa():
    rng = np.random.default_rng(22)
    q = rng.standard_normal((6, 16))
    kl, vl = rng.standard_normal((9, 16)), rng.standard_normal((9, 16))
    o, _ = oa.attention_with_local(q, np.zeros((0, 16)), np.zeros((0, 16)), kl, vl)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(kl)[None], torch.from_numpy(vl)[None])[0].numpy()
    assert np.max(np.abs(o - ref)) < 1e-12
    o0, l0 = oa.attention_with_local(q, np.zeros((0, 16)), np.zeros((0, 16)), np.zeros((0, 16)), np.zeros((0, 16)))
    assert np.all(o0 == 0) and np.all(l0 == -np.inf)


def test_local_chunk_repeating_the_cache():
    """Every key twice: the same weights, so o is unchanged and lse gains log 2."""
    rng = np.random.default_rng(23)
    q = rng.standard_normal((4, 16))
    k, v = rng.standard_normal((7, 16)), rng.standard_normal((7, 16))
    o1, l1 = oa.attention_with_local(q, k, v, np.zeros((0, 16)), np.zeros((0, 16)))
    o2, l2 = oa.attention_with_local(q, k, v, k, v)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs(l2 - l1 - math.log(2.0))) < 1e-12


def test_reconstruction_uses_frame_tiles():
    """Token t of a 1560-token frame uses tile (t // 1560) * 98 + (t % 1560) // 16."""
    assert oa.tile_index(1559, 1560, 16) == 97
    assert oa.tile_index(1560, 1560, 16) == 98
    assert oa.tile_index(3119, 1560, 16) == 195


def test_compression_closed_form_by_hand():
    """The closed form, evaluated by hand for a small case:
    N=32 tokens, H=1, d=16, F=16, T=16, C_K=C_V=4, r=2, bf16.
    original 2*32*16*2 = 2048 B; stored: idx 64 + codes 2*32*16/4 = 256 +
    params 2*2*1*4 = 16 + coef 32*2 = 64 + coef scale 64 + centres 2*4*16*2 = 256
    + U 16*2*4 = 128 + s 64 = 912 B."""
    ratio, orig, stored = measures.compression_ratio(32, 1, 16, 16, 16, 4, 4, 2, 2)
    assert orig == 2048 and stored == 912


def test_compression_large_configs_exceed_six():
    for name in ("lingbot480p", "lingbot720p", "minute"):
        w = workloads.WORKLOADS[name]
        ratio, _, _ = measures.compression_ratio(w.n_tokens, w.heads, w.head_dim, w.frame_tokens,
                                                 w.group_tokens, w.c_k, w.c_v, w.rank, 2)
        assert ratio > 6.0, (name, ratio)


def test_epochs_bruteforce_and_merge():
    """One softmax over several epochs' keys and the local chunk: per-query
    loops, and the log-sum-exp merge of each epoch's own attention."""
    rng = np.random.default_rng(33)
    q = rng.standard_normal((3, 8))
    eps = [(rng.standard_normal((n, 8)), rng.standard_normal((n, 8))) for n in (5, 0, 3)]
    kl, vl = rng.standard_normal((2, 8)), rng.standard_normal((2, 8))
    o, lse = oa.attention_over_epochs(q, eps, kl, vl)
    keys = [k for e in eps for k in e[0]] + list(kl)
    vals = [v for e in eps for v in e[1]] + list(vl)
    for i in range(3):
        ls = [sum(q[i, j] * kk[j] for j in range(8)) / math.sqrt(8) for kk in keys]
        m = max(ls)
        ws = [math.exp(x - m) for x in ls]
        tot = sum(ws)
        for j in range(8):
            assert abs(o[i, j] - sum(wt * vv[j] for wt, vv in zip(ws, vals)) / tot) < 1e-12
        assert abs(lse[i] - (m + math.log(tot))) < 1e-12
    parts = [oa.softmax_attention(q, k, v) for k, v in eps if len(k)] + [oa.softmax_attention(q, kl, vl)]
    om, lm = oa.merge_partials(parts)
    assert np.allclose(o, om, rtol=0, atol=1e-12) and np.allclose(lse, lm, rtol=0, atol=1e-12)
    # one epoch and no local keys: plain attention
    o1, l1 = oa.attention_over_epochs(q, eps[:1])
    o2, l2 = oa.softmax_attention(q, *eps[0])
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
