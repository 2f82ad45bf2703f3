"""Pins of the oracle's quantize-append (CPU only)."""
import json
import os

import numpy as np
import pytest

import workloads
from oracle import calibrate as oc
from oracle import codec
from oracle import attention as oa
from oracle.numerics import bf16, fl32, fp16_of_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def tiny():
    w = workloads.WORKLOADS["tiny"]
    d = workloads.generate(w)
    cal = oc.calibrate(d["q_hist"], d["k_hist"], d["v_hist"], 16, 16, 8, "f32", seed=11)
    return w, d, cal


def test_bf16_rounding_against_bit_rounding():
    """bfloat16 RNE from float64 equals rounding the float32 pattern when the
    float32 step is exact, and handles ties to even."""
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 3.14159, 1e-3, 65504.0])
    got = bf16(x)
    assert got[1] == 1.0                     # tie -> even (1.0)
    assert got[2] == 1.0 + 2**-6            # tie -> even (1 + 2^-6)
    b = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    rnd = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    assert np.array_equal(got.view(np.uint32), rnd.astype(np.uint32))


def test_int2_golden_example():
    g = json.load(open(os.path.join(GOLDEN, "int2_worked.json")))
    rho = np.array(g["rho"], np.float32)[None, :]
    z, s = codec.int2_params(rho)
    assert (z, s) == (g["z"], g["s"])
    codes = codec.int2_encode(rho, z, s)
    assert codes[0].tolist() == g["codes"]
    assert codec.int2_decode(codes, z, s)[0].tolist() == g["rho_hat"]
    assert int(codec.pack_codes(codes)[0, 0]) == int(g["packed_hex"], 16)
    assert np.array_equal(codec.unpack_codes(codec.pack_codes(codes), 16), codes)


def test_int8_golden_example():
    g = json.load(open(os.path.join(GOLDEN, "int8_worked.json")))
    c = np.array(g["c"])
    r = len(c)
    u = np.eye(r)                      # e = c along an orthonormal basis
    n, sigma, _ = codec.psac(c[None, :], np.zeros((1, r)), np.zeros((1, r)), u)
    assert float(sigma[0]) == g["sigma"]
    assert n[0].tolist() == g["n"]


def test_invariant_a_qvg_mode_is_nearest(tiny):
    w, d, cal = tiny
    k = d["k"][0]
    mu = cal["mu_k"][0]
    idx, _ = codec.select_keys(k, mu, cal["sens"][0], 4, codec.QVG_MODE)
    for t in range(k.shape[0]):
        best, bd = -1, np.inf
        for c in range(mu.shape[0]):
            dd = sum((float(k[t, j]) - float(mu[c, j])) ** 2 for j in range(k.shape[1]))
            if dd < bd:
                best, bd = c, dd
        assert idx[t] == best


def test_no_range_term_is_weighted_nearest(tiny):
    w, d, cal = tiny
    k, mu, s = d["k"][0], cal["mu_k"][0], cal["sens"][0].astype(np.float64)
    idx, _ = codec.select_keys(k, mu, s, 4, codec.NO_RANGE_TERM)
    for t in range(0, k.shape[0], 7):
        dd = [sum(s[j] * (float(k[t, j]) - float(mu[c, j])) ** 2 for j in range(64)) for c in range(16)]
        assert idx[t] == int(np.argmin(dd))


def test_invariant_d_all_candidates_is_global_argmin(tiny):
    """K_c = C: QSAC's choice is the brute-force argmin of P over all centres
    (ties: smaller D, lower index)."""
    w, d, cal = tiny
    k, mu, s = d["k"][0], cal["mu_k"][0], cal["sens"][0].astype(np.float64)
    sg = [sum(s[16 * g:16 * g + 16]) for g in range(4)]
    idx, _ = codec.select_keys(k, mu, s, 16, 0)
    for t in range(0, k.shape[0], 5):
        best = None
        for c in range(16):
            rho = [float(np.float32(float(k[t, j]) - float(mu[c, j]))) for j in range(64)]
            p = sum(sg[g] * (max(rho[16 * g:16 * g + 16]) - min(rho[16 * g:16 * g + 16])) ** 2
                    for g in range(4)) / 108.0
            dd = sum(s[j] * (float(k[t, j]) - float(mu[c, j])) ** 2 for j in range(64))
            key = (p, dd, c)
            if best is None or key < best:
                best = key
        assert idx[t] == best[2]


def test_qsac_lowers_weighted_int2_error():
    """Statistical sanity (not parity): the sensitivity-weighted INT2 error
    of QSAC is no larger on average than nearest-centre assignment."""
    w = workloads.scaled(workloads.WORKLOADS["matrix_game"], heads=1, frames=2)
    d = workloads.generate(w)
    cal = oc.calibrate(d["q_hist"], d["k_hist"], d["v_hist"], 64, 64, 8, "bf16", seed=3, iters=4)
    k = d["k"][0]
    s = cal["sens"][0].astype(np.float64)
    errs = {}
    for name, flags in (("qsac", 0), ("qvg", codec.QVG_MODE)):
        out = codec.append_keys(k, cal["mu_k"][0], cal["sens"][0], cal["u"][0][:, :0],
                                w.frame_tokens, 16, 4, flags)
        e = out["rho"].astype(np.float64) - out["rho_hat"].astype(np.float64)
        errs[name] = np.mean((e * e) @ s)
    assert errs["qsac"] <= errs["qvg"]


def _ulp32(x):
    x = np.abs(np.asarray(x, np.float32))
    return (np.nextafter(x, np.float32(np.inf)) - x).astype(np.float64)


@pytest.mark.parametrize("fp32_params", [False, True])
def test_invariant_b_int2_error_bound(tiny, fp32_params):
    w, d, cal = tiny
    flags = codec.FP32_PARAMS_TEST if fp32_params else 0
    out = codec.append_keys(d["k"][0], cal["mu_k"][0], cal["sens"][0], cal["u"][0],
                            64, 16, 4, flags)
    rho, rho_hat = out["rho"], out["rho_hat"]
    for p, (a, b) in enumerate(codec.frame_tiles(128, 64, 16)):
        for g in range(4):
            blk = rho[a:b, 16 * g:16 * g + 16].astype(np.float64)
            hat = rho_hat[a:b, 16 * g:16 * g + 16].astype(np.float64)
            m, mx = blk.min(), blk.max()
            rng = mx - m
            err = np.abs(blk - hat)
            slack = 2 * _ulp32(blk)
            if fp32_params:
                bound = rng / 6 * (1 + 2**-20) + slack
            else:
                z, s = out["z"][p, g], out["s"][p, g]
                bound = rng / 6 + abs(z - m) + 1.5 * abs(s - rng / 3) + slack
            assert np.all(err <= bound)
            codes = out["codes"][a:b, 16 * g:16 * g + 16]
            assert codes.max() <= 3
            # idempotence: re-quantizing the decoded values gives the codes back
            z, s = out["z"][p, g], out["s"][p, g]
            assert np.array_equal(codec.int2_encode(hat.astype(np.float32), z, s), codes)
            if fp32_params and rng > 0:
                assert codes[blk == m].max() == 0 and codes[blk == mx].min() == 3


def test_invariant_c_rank0_is_qvg_reconstruction(tiny):
    w, d, cal = tiny
    k = d["k"][0]
    u0 = np.zeros((64, 0), np.float32)
    out = codec.append_keys(k, cal["mu_k"][0], cal["sens"][0], u0, 64, 16, 4, 0)
    rec = oa.reconstruct_keys(out["idx"], out["codes"], out["z"], out["s"], out["coef"],
                              out["coef_scale"], cal["mu_k"][0], u0, 64, 16)
    expect = cal["mu_k"][0][out["idx"]].astype(np.float64) + out["rho_hat"].astype(np.float64)
    assert np.array_equal(rec, expect)


def test_invariant_c_full_rank_removes_error(tiny):
    """U a full orthonormal basis: ||k - k~|| = ||c - c_hat|| <= sqrt(d) sigma/2."""
    w, d, cal = tiny
    k = d["k"][0]
    rng = np.random.default_rng(5)
    u = fl32(np.linalg.qr(rng.standard_normal((64, 64)))[0])
    out = codec.append_keys(k, cal["mu_k"][0], cal["sens"][0], u, 64, 16, 4, 0)
    rec = oa.reconstruct_keys(out["idx"], out["codes"], out["z"], out["s"], out["coef"],
                              out["coef_scale"], cal["mu_k"][0], u, 64, 16)
    err = np.linalg.norm(k.astype(np.float64) - rec, axis=1)
    sig = out["coef_scale"].astype(np.float64)
    # U is orthonormal only to float32 rounding: allow that slack
    e_norm = np.linalg.norm(k.astype(np.float64) - cal["mu_k"][0][out["idx"]] - out["rho_hat"], axis=1)
    assert np.all(err <= np.sqrt(64) * sig / 2 + 1e-5 * e_norm + 1e-12)
    qvg_err = e_norm
    assert np.mean(err) < 0.2 * np.mean(qvg_err)


def test_psac_projection_bound_any_rank(tiny):
    """|U^T (k - k~)|_inf <= sigma/2 (+ float32 U slack), since U^T U = I."""
    w, d, cal = tiny
    k = d["k"][0]
    u = cal["u"][0]
    out = codec.append_keys(k, cal["mu_k"][0], cal["sens"][0], u, 64, 16, 4, 0)
    rec = oa.reconstruct_keys(out["idx"], out["codes"], out["z"], out["s"], out["coef"],
                              out["coef_scale"], cal["mu_k"][0], u, 64, 16)
    proj = np.abs((k.astype(np.float64) - rec) @ u.astype(np.float64)).max(axis=1)
    e_norm = np.linalg.norm(k.astype(np.float64) - cal["mu_k"][0][out["idx"]] - out["rho_hat"], axis=1)
    assert np.all(proj <= out["coef_scale"] / 2 + 1e-5 * e_norm)
    # and for q in span(U): |q.k~ - q.k| <= ||U^T q||_1 sigma / 2 (+ slack)
    qc = rng_q = np.random.default_rng(2).standard_normal(8)
    q = u.astype(np.float64) @ qc
    diff = np.abs((rec - k.astype(np.float64)) @ q)
    assert np.all(diff <= np.abs(u.astype(np.float64).T @ q).sum() * out["coef_scale"] / 2
                  + 1e-5 * e_norm * np.abs(q).sum())


def test_values_nearest_and_int2(tiny):
    w, d, cal = tiny
    v, mu = d["v"][0], cal["mu_v"][0]
    out = codec.append_values(v, mu, 64, 16)
    for t in range(0, v.shape[0], 3):
        dd = [sum((float(v[t, j]) - float(mu[c, j])) ** 2 for j in range(64)) for c in range(16)]
        assert out["idx"][t] == int(np.argmin(dd))
    assert np.array_equal(out["rho"], fl32(v.astype(np.float64) - mu[out["idx"]]))


def test_frame_tiles_ragged():
    t = codec.frame_tiles(2 * 1560, 1560, 16)
    assert len(t) == 2 * 98
    assert t[97] == (1552, 1560) and t[98] == (1560, 1576)


def test_fp16_of_f32_rne():
    # 1 + 2^-11 is the midpoint between 1 and 1 + 2^-10 in binary16 -> even (1)
    assert fp16_of_f32(np.float32(1 + 2**-11)) == 1.0
    assert fp16_of_f32(np.float32(1 + 3 * 2**-11)) == 1 + 2**-9


# ---- stage-2 ablation scores (exact INT2 error; diagonal and full Eq. 7 forms)

def test_stage2_variant_golden_example():
    g = json.load(open(os.path.join(GOLDEN, "stage2_exact_error.json")))
    rho = np.array(json.load(open(os.path.join(GOLDEN, "int2_worked.json")))["rho"], np.float32)[None, :]
    e = codec.token_int2_error(rho)
    assert e[0].tolist() == g["e"]
    assert codec.exact_error_score(rho, np.array(g["weights"], np.float64))[0] == g["diagonal_score"]
    m = np.eye(16) + np.ones((16, 16))
    assert codec.quadratic_error_score(rho, m)[0] == g["full_score_identity_plus_ones"]
    assert abs(codec.range_score(rho, [16.0])[0] - g["range_score_uniform"]) < 1e-15


def test_token_error_equals_one_token_tiles(tiny):
    """The per-token error is the tile path's error with one-token tiles."""
    w, d, cal = tiny
    rho = codec.residual(d["k"][0], cal["mu_k"][0][np.arange(128) % 16])
    _, _, _, rho_hat = codec.quantize_residuals(rho, 1, 1)
    assert np.array_equal(codec.token_int2_error(rho), rho.astype(np.float64) - rho_hat.astype(np.float64))


def test_full_quadratic_is_mean_squared_logit_perturbation():
    """Eq. 7 by brute force: e^T M e equals the mean over the historical
    queries of (q . e)^2 when M is their second moment."""
    rng = np.random.default_rng(4)
    q = rng.standard_normal((300, 64)) * np.exp(rng.standard_normal(64))
    rho = (rng.standard_normal((20, 64)) * 0.3).astype(np.float32)
    m = oc.second_moment(q)
    e = codec.token_int2_error(rho)
    brute = np.mean((q @ e.T) ** 2, axis=0)
    got = codec.quadratic_error_score(rho, m)
    assert np.allclose(got, brute, rtol=1e-12, atol=0)


def test_full_quadratic_with_diagonal_moment_is_diagonal_form(tiny):
    w, d, cal = tiny
    s = cal["sens"][0].astype(np.float64)
    k, mu = d["k"][0], cal["mu_k"][0]
    a, ia = codec.select_keys(k, mu, s, 4, codec.EXACT_ERROR)
    b, ib = codec.select_keys(k, mu, s, 4, codec.FULL_QUADRATIC, moment=np.diag(s))
    assert np.array_equal(a, b)
    assert np.allclose(ia["P"], ib["P"], rtol=1e-12, atol=0)
    # with UNIFORM_SENS the full form uses M = I: the diagonal form with s = 1
    a, _ = codec.select_keys(k, mu, s, 4, codec.EXACT_ERROR | codec.UNIFORM_SENS)
    b, _ = codec.select_keys(k, mu, s, 4, codec.FULL_QUADRATIC | codec.UNIFORM_SENS, moment=np.zeros((64, 64)))
    assert np.array_equal(a, b)


def _one_token_error_py(x, m):
    """rho = fl32(x - m) and its INT2 error with the token's own parameters per
    group of 16, one channel at a time with the scalar step-3 functions."""
    d = len(x)
    rho = np.array([np.float32(float(x[j]) - float(m[j])) for j in range(d)], np.float32)
    e = []
    for g in range(d // 16):
        blk = rho[16 * g:16 * g + 16]
        z, s = codec.int2_params(blk)
        rh = codec.int2_decode(codec.int2_encode(blk, z, s), z, s)
        e += [float(blk[j]) - float(rh[j]) for j in range(16)]
    return e


@pytest.mark.parametrize("mode", ["exact", "full"])
def test_invariant_d_stage2_variants_global_argmin(tiny, mode):
    """K_c = C: the variant's choice is the brute-force argmin over all centres
    of its score (full form: the mean squared logit perturbation over the
    historical queries), ties to smaller D then lower index."""
    w, d, cal = tiny
    k, mu, s = d["k"][0], cal["mu_k"][0], cal["sens"][0].astype(np.float64)
    qh = d["q_hist"][0].astype(np.float64)
    m = oc.second_moment(qh)
    flags = codec.EXACT_ERROR if mode == "exact" else codec.FULL_QUADRATIC
    idx, _ = codec.select_keys(k, mu, s, 16, flags, moment=m)
    for t in range(0, k.shape[0], 7):
        best = None
        for c in range(16):
            e = _one_token_error_py(k[t], mu[c])
            if mode == "exact":
                p = sum(s[j] * e[j] ** 2 for j in range(64))
            else:
                p = float(np.mean((qh @ np.array(e)) ** 2))
            dd = sum(s[j] * (float(k[t, j]) - float(mu[c, j])) ** 2 for j in range(64))
            key = (p, dd, c)
            if best is None or key[0] < best[0] * (1 - 1e-9) or (abs(key[0] - best[0]) <= 1e-9 * best[0] and key[1:] < best[1:]):
                best = key
        assert idx[t] == best[2], (t, idx[t], best)


def test_epoch_keys_keep_their_own_calibration():
    """Two calibration epochs of one rollout: each epoch's Keys, encoded and
    rebuilt with its own centres and U, obey the PSAC bound
    |U^T (k - k~)| <= sigma/2 along that epoch's U; the other epoch's U does
    not (the rebuilt keys are tied to the calibration they were encoded with)."""
    w = workloads.scaled(workloads.WORKLOADS["matrix_game"], heads=1, frames=2)
    d = workloads.generate(w)
    F = w.frame_tokens
    k = d["k"][0]
    cal0 = oc.calibrate(d["q_hist"], d["k_hist"], d["v_hist"], 32, 32, 8, "bf16", seed=1, iters=2)
    # the second epoch recalibrates from the first epoch's last frame and the
    # chunk's queries
    cal1 = oc.calibrate(d["q"], d["k"][:, :F], d["v"][:, :F], 32, 32, 8, "bf16", seed=2, iters=2)
    worst_own, worst_other = 0.0, 0.0
    for e, (cal, other) in enumerate(((cal0, cal1), (cal1, cal0))):
        ke = k[e * F:(e + 1) * F]
        out = codec.append_keys(ke, cal["mu_k"][0], cal["sens"][0], cal["u"][0], F, 16, 4, 0)
        kr = oa.reconstruct_keys(out["idx"], out["codes"], out["z"], out["s"], out["coef"], out["coef_scale"],
                                 cal["mu_k"][0], cal["u"][0], F, 16)
        err = ke.astype(np.float64) - kr
        sig = out["coef_scale"].astype(np.float64)[:, None]
        own = np.abs(err @ cal["u"][0].astype(np.float64)) - sig / 2
        oth = np.abs(err @ other["u"][0].astype(np.float64)) - sig / 2
        worst_own = max(worst_own, float(own.max()))
        worst_other = max(worst_other, float(oth.max()))
    assert worst_own <= 1e-4
    assert worst_other > 1e-2


def test_qsac_hand_worked_candidates_and_choice():
    """Stage 1 and stage 2 on a hand-worked example whose distances and
    range scores are exact binary fractions: the candidate lists (K_c
    smallest D, the lower index first at a tie) and the final choice for
    K_c = 1..5, with per-channel and with uniform sensitivities."""
    g = json.load(open(os.path.join(GOLDEN, "qsac_worked.json")))
    d = g["d"]
    mu = np.zeros((len(g["centres"]), d), np.float32)
    for c, row in g["centres"].items():
        for j, val in row.items():
            mu[int(c), int(j)] = val
    k = np.zeros((1, d), np.float32)
    s = np.array(g["sens"], np.float32)
    _, info = codec.select_keys(k, mu, s, 5, 0)
    assert info["D"][0].tolist() == g["D"]
    assert (info["P"][0] * 108).tolist() == [g["P_times_108"][c] for c in info["cand"][0]]
    for case in g["cases"]:
        flags = codec.UNIFORM_SENS if case["uniform"] else 0
        idx, info = codec.select_keys(k, mu, s, case["top_k"], flags)
        assert info["cand"][0].tolist() == case["cand"], case
        assert int(idx[0]) == case["choice"], case
    # argmin modes take the nearest centre whatever K_c is
    for flags in (codec.NO_RANGE_TERM,):
        idx, _ = codec.select_keys(k, mu, s, 4, flags)
        assert int(idx[0]) == 0
    idx, _ = codec.select_keys(k, mu, s, 0, 0)
    assert int(idx[0]) == 0


@pytest.mark.parametrize("top_k", [2, 4, 8])
def test_candidate_sets_equal_bruteforce_sort(tiny, top_k):
    """K_c < C: the candidate set of every token is the first K_c entries of a
    brute-force sort of (D, c) computed with scalar loops, and the choice is
    the brute-force minimum of (P, D, c) over those candidates only."""
    w, d, cal = tiny
    k, mu, s = d["k"][0], cal["mu_k"][0], cal["sens"][0].astype(np.float64)
    n_c = mu.shape[0]
    assert top_k < n_c
    sg = [sum(s[16 * g:16 * g + 16]) for g in range(4)]
    idx, info = codec.select_keys(k, mu, s, top_k, 0)
    for t in range(0, k.shape[0], 3):
        dd = [sum(s[j] * (float(k[t, j]) - float(mu[c, j])) ** 2 for j in range(64)) for c in range(n_c)]
        order = sorted(range(n_c), key=lambda c: (dd[c], c))
        assert info["cand"][t].tolist() == order[:top_k]
        best = None
        for c in order[:top_k]:
            rho = [float(np.float32(float(k[t, j]) - float(mu[c, j]))) for j in range(64)]
            p = sum(sg[g] * (max(rho[16 * g:16 * g + 16]) - min(rho[16 * g:16 * g + 16])) ** 2
                    for g in range(4)) / 108.0
            key = (p, dd[c], c)
            if best is None or key < best:
                best = key
        assert idx[t] == best[2]
