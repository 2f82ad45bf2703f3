"""Oracle: quantize-append of Keys (QSAC + INT2 + PSAC) and Values (QVG + INT2).

TEST INFRASTRUCTURE ONLY (see the package header).

This is a heuristic encoding, not a closed form, so the oracle takes the
method's steps in the pages' order (English digest, QSAC and PSAC paragraphs;
review summary):

 1. QSAC stage 1 -- screen candidate centres with a Query-sensitivity-weighted
    distance  D_c = sum_j s_j (k_j - mu_cj)^2  over all C centres, keep the K_c
    smallest (ties: lower c).  s = diag(M) (diagonal of Eq. 7).
 2. QSAC stage 2 -- for each candidate, estimate the attention perturbation of
    INT2-quantizing its residual from each residual group's dynamic range and
    that group's sensitivity:  P_c = sum_g S_g range_g^2 / 108,
    S_g = sum_{j in g} s_j, range_g = max - min of rho = fl32(k - mu_c) over the
    token's 16 channels of group g; choose argmin P (ties: smaller D, lower c).
    [reading: uniform-noise model, E[e^2] = Delta^2/12 with Delta = range/3,
    combined through diagonal Eq. 7.]
 3. INT2 residual -- per (16 channels x tile of T tokens of one frame):
    m = min, Mx = max of rho; z = fp16(m); s = fp16(fl32(fl32(Mx - m)/3));
    thresholds t_i = fl32(z + (i - 1/2) s), code = #{i : rho >= t_i};
    rho_hat = fl32(z + code s); s = 0 gives code 0.
 4. PSAC -- e = k - (mu_c + rho_hat) (float64), c = U^T e, c32 = fl32(c),
    sigma = fp16(fl32(max|c32| / 127)), n = clamp(rne(fl32(c32/sigma)), +-127)
    (INT8, per-token float16 scale).  sigma = 0 gives n = 0.
 5. Values -- nearest Euclidean centre (ties: lower c), INT2 as in step 3, no
    compensation (QVG scheme).

Flags: UNIFORM_SENS (s = 1), NO_RANGE_TERM (argmin D), QVG_MODE = both, and the
oracle-only FP32_PARAMS_TEST (z, s kept in float32) used by the INT2 pin.

Stage-2 ablation variants (review summary: Eq. 7 and Table 10, where the full
quadratic form is compared with the diagonal approximation):
 * EXACT_ERROR -- instead of the range model, the candidate's actual INT2 error
   e = rho - Q(rho), where Q quantizes each of the token's own 16-channel groups
   with that group's parameters (the step-3 arithmetic with a one-token tile;
   the shared tile's parameters are unknown while its tokens choose), scored
   by the diagonal form  P_c = sum_j s_j e_j^2.
 * FULL_QUADRATIC -- the same error scored by the full form of Eq. 7,
   P_c = e^T M e, with M the Query second moment (with UNIFORM_SENS, M = I).
   Reading: the variant changes stage 2 only; stage 1 stays the diagonal
   screen, which the pages name as the screening distance.

Pins (tests/test_oracle_codec.py): invariant (a) QVG_MODE = brute-force nearest
centre; invariant (b) |rho - rho_hat| <= range/6 + rounding slack; invariant
(c) rank 0 = QVG reconstruction, rank d removes the Key error up to INT8
rounding; invariant (d) K_c = C equals a brute-force global argmin of P;
INT2 idempotence; a hand-worked INT2/INT8 example under tests/golden; a
hand-worked QSAC example (tests/golden/qsac_worked.json: candidate lists and
choices for K_c = 1..5, per-channel and uniform sensitivities); for K_c < C,
candidate sets equal to a brute-force sort of (D, c) and the choice the
brute-force minimum of (P, D, c) among them.
"""
import math

import numpy as np

from .numerics import fl32, fp16_of_f32

UNIFORM_SENS = 1
NO_RANGE_TERM = 2
QVG_MODE = UNIFORM_SENS | NO_RANGE_TERM
EXACT_ERROR = 4
FULL_QUADRATIC = 8
FP32_PARAMS_TEST = 16

GROUP = 16


def group_sums(s):
    """S_g = sum of s_j over the 16 channels of group g (float64)."""
    s = np.asarray(s, dtype=np.float64)
    return s.reshape(-1, GROUP).sum(axis=1)


def weighted_sq_distances(x, mu, s):
    """D[t, c] = sum_j s_j (x_tj - mu_cj)^2 in float64, direct form."""
    x = np.asarray(x, dtype=np.float64)
    mu = np.asarray(mu, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    out = np.empty((x.shape[0], mu.shape[0]), dtype=np.float64)
    step = max(1, 4_000_000 // max(1, mu.size))
    for a in range(0, x.shape[0], step):
        diff = x[a:a + step, None, :] - mu[None, :, :]
        out[a:a + step] = np.einsum("ncd,ncd,d->nc", diff, diff, s)
    return out


def residual(x, mu_rows):
    """rho = fl32(x - mu) for bf16/f32 inputs (float32 result)."""
    return fl32(np.asarray(x, np.float64) - np.asarray(mu_rows, np.float64))


def range_score(rho, s_group):
    """P = sum_g S_g range_g^2 / 108 for residual rows rho [..., d] (float64)."""
    r = np.asarray(rho, dtype=np.float64)
    g = r.reshape(r.shape[:-1] + (-1, GROUP))
    rng = g.max(axis=-1) - g.min(axis=-1)
    return (rng * rng) @ np.asarray(s_group, np.float64) / 108.0


def token_int2_error(rho):
    """e = rho - Q(rho) in float64, Q quantizing each 16-channel group of each
    row with the row's own parameters: step 3 with a one-token tile, written
    out over all (row, group) pairs at once."""
    r = np.asarray(rho, dtype=np.float32)
    n, d = r.shape
    g = r.reshape(n, d // GROUP, GROUP)
    m = g.min(axis=2)
    mx = g.max(axis=2)
    width = fl32(mx.astype(np.float64) - m.astype(np.float64))
    step = fl32(width.astype(np.float64) / 3.0)
    z = fp16_of_f32(m).astype(np.float64)[..., None]
    s = fp16_of_f32(step).astype(np.float64)[..., None]
    code = np.zeros(g.shape, dtype=np.float64)
    for i in (1, 2, 3):
        code += g >= fl32(z + (i - 0.5) * s)
    code = np.where(s == 0, 0.0, code)
    rhat = fl32(z + code * s)
    return (g.astype(np.float64) - rhat.astype(np.float64)).reshape(n, d)


def exact_error_score(rho, s):
    """P = sum_j s_j e_j^2 with e the one-token INT2 error (float64)."""
    e = token_int2_error(rho)
    return (e * e) @ np.asarray(s, np.float64)


def quadratic_error_score(rho, m):
    """P = e^T M e with e the one-token INT2 error (Eq. 7, full form)."""
    e = token_int2_error(rho)
    return np.einsum("ti,ij,tj->t", e, np.asarray(m, np.float64), e)


def select_keys(k, mu, sens, top_k, flags, moment=None):
    """QSAC centre choice for each Key row.  Returns (idx, info) where info
    holds D [n, C], the candidate lists and their P scores.  moment: the
    Query second moment M [d, d], needed by FULL_QUADRATIC."""
    n, d = k.shape
    c_count = mu.shape[0]
    s = np.ones(d) if flags & UNIFORM_SENS else np.asarray(sens, np.float64)
    if flags & FULL_QUADRATIC:
        m_full = np.eye(d) if flags & UNIFORM_SENS else np.asarray(moment, np.float64)
    s_group = group_sums(s)
    dist = weighted_sq_distances(k, mu, s)
    info = dict(D=dist, s=s, s_group=s_group)
    if (flags & NO_RANGE_TERM) or top_k == 0:
        idx = np.argmin(dist, axis=1)                 # first min -> lower c
        info["cand"] = None
        return idx.astype(np.int64), info
    kc = min(top_k, c_count)
    order = np.argsort(dist, axis=1, kind="stable")   # equal D keep c order
    cand = order[:, :kc]
    pscore = np.empty((n, kc))
    for j in range(kc):
        rho = residual(k, mu[cand[:, j]])
        if flags & FULL_QUADRATIC:
            pscore[:, j] = quadratic_error_score(rho, m_full)
        elif flags & EXACT_ERROR:
            pscore[:, j] = exact_error_score(rho, s)
        else:
            pscore[:, j] = range_score(rho, s_group)
    idx = np.empty(n, dtype=np.int64)
    for t in range(n):
        best = min(range(kc), key=lambda j: (pscore[t, j], dist[t, cand[t, j]], cand[t, j]))
        idx[t] = cand[t, best]
    info["cand"] = cand
    info["P"] = pscore
    return idx, info


def select_values(v, mu):
    """QVG centre choice: nearest Euclidean centre, ties to the lower index."""
    dist = weighted_sq_distances(v, mu, np.ones(v.shape[1]))
    return np.argmin(dist, axis=1).astype(np.int64), dict(D=dist)


def frame_tiles(n_tokens, frame_tokens, group_tokens):
    """Token ranges [a, b) of the parameter tiles of a block of whole frames,
    in storage order (frame-major, then tile within the frame)."""
    if n_tokens % frame_tokens:
        raise ValueError("appends are whole frames")
    tiles = []
    for f in range(n_tokens // frame_tokens):
        base = f * frame_tokens
        for a in range(0, frame_tokens, group_tokens):
            tiles.append((base + a, base + min(a + group_tokens, frame_tokens)))
    return tiles


def int2_params(rho_tile, fp32_params=False):
    """(z, s) of one tile-group of residuals (float32 values)."""
    m = np.float32(np.min(rho_tile))
    mx = np.float32(np.max(rho_tile))
    width = fl32(np.float64(mx) - np.float64(m))
    step = fl32(np.float64(width) / 3.0)
    if fp32_params:
        return np.float32(m), np.float32(step)
    return np.float32(fp16_of_f32(m)), np.float32(fp16_of_f32(step))


def int2_encode(rho, z, s):
    """codes in {0..3}: number of thresholds t_i = fl32(z + (i-1/2)s) <= rho."""
    rho = np.asarray(rho, dtype=np.float32)
    if s == 0:
        return np.zeros(rho.shape, dtype=np.uint8)
    code = np.zeros(rho.shape, dtype=np.uint8)
    for i in (1, 2, 3):
        t = fl32(np.float64(z) + (i - 0.5) * np.float64(s))
        code += (rho >= t).astype(np.uint8)
    return code


def int2_decode(code, z, s):
    """rho_hat = fl32(z + code * s)."""
    return fl32(np.float64(z) + np.asarray(code, np.float64) * np.float64(s))


def quantize_residuals(rho, frame_tokens, group_tokens, fp32_params=False):
    """INT2 codes of residual rows rho [n, d] (whole frames).  Returns
    codes [n, d] uint8, z and s [tiles, d/16] float32, rho_hat [n, d] float32."""
    n, d = rho.shape
    tiles = frame_tiles(n, frame_tokens, group_tokens)
    codes = np.zeros((n, d), dtype=np.uint8)
    rho_hat = np.zeros((n, d), dtype=np.float32)
    zs = np.zeros((len(tiles), d // GROUP), dtype=np.float32)
    ss = np.zeros_like(zs)
    for p, (a, b) in enumerate(tiles):
        for g in range(d // GROUP):
            blk = rho[a:b, g * GROUP:(g + 1) * GROUP]
            z, s = int2_params(blk, fp32_params)
            zs[p, g], ss[p, g] = z, s
            c = int2_encode(blk, z, s)
            codes[a:b, g * GROUP:(g + 1) * GROUP] = c
            rho_hat[a:b, g * GROUP:(g + 1) * GROUP] = int2_decode(c, z, s)
    return codes, zs, ss, rho_hat


def pack_codes(codes):
    """Pack [n, d] codes 16 per 32-bit word: word (t, g) holds channel 16g+i in
    bits [2i, 2i+1]."""
    n, d = codes.shape
    c = codes.reshape(n, d // GROUP, GROUP).astype(np.uint32)
    shifts = (2 * np.arange(GROUP, dtype=np.uint32))[None, None, :]
    return np.bitwise_or.reduce(c << shifts, axis=2).astype(np.uint32)


def unpack_codes(words, d):
    w = np.asarray(words, dtype=np.uint32)
    shifts = (2 * np.arange(GROUP, dtype=np.uint32))[None, None, :]
    c = (w[:, :, None] >> shifts) & 3
    return c.reshape(w.shape[0], d).astype(np.uint8)


def psac(k, mu_rows, rho_hat, u):
    """INT8 low-rank compensation of the remaining Key error along U."""
    r = u.shape[1]
    n = k.shape[0]
    if r == 0:
        return np.zeros((n, 0), np.int8), np.zeros(n, np.float32), np.zeros((n, 0))
    e = np.asarray(k, np.float64) - (np.asarray(mu_rows, np.float64) + np.asarray(rho_hat, np.float64))
    c = e @ np.asarray(u, np.float64)
    psac.last_abs_scale = np.abs(e) @ np.abs(np.asarray(u, np.float64))
    c32 = fl32(c)
    a = np.max(np.abs(c32), axis=1)
    sigma = fp16_of_f32(fl32(a.astype(np.float64) / 127.0))
    q = np.zeros((n, r), dtype=np.int8)
    nz = sigma > 0
    ratio = fl32(c32[nz].astype(np.float64) / sigma[nz, None].astype(np.float64))
    q[nz] = np.clip(np.rint(ratio), -127, 127).astype(np.int8)
    return q, sigma.astype(np.float32), c


def append_keys(k_new, mu_k, sens, u, frame_tokens, group_tokens, top_k, flags,
                idx_override=None, moment=None):
    """Quantize-append of a block of whole frames of Keys for one head.

    idx_override: optional {token: centre} dict of decisions to adopt (used by
    the tie-following checker); everything downstream is recomputed.
    moment: Query second moment M (FULL_QUADRATIC only)."""
    k_new = np.asarray(k_new, dtype=np.float32)
    idx, info = select_keys(k_new, mu_k, sens, top_k, flags, moment)
    if idx_override:
        for t, cidx in idx_override.items():
            idx[t] = cidx
    rho = residual(k_new, mu_k[idx])
    codes, zs, ss, rho_hat = quantize_residuals(
        rho, frame_tokens, group_tokens, bool(flags & FP32_PARAMS_TEST))
    coef, coef_scale, c_exact = psac(k_new, mu_k[idx], rho_hat, u)
    c_abs = psac.last_abs_scale if u.shape[1] > 0 else np.zeros((k_new.shape[0], 0))
    return dict(idx=idx, codes=codes, z=zs, s=ss, coef=coef, coef_scale=coef_scale,
                rho=rho, rho_hat=rho_hat, c=c_exact, c_abs=c_abs, info=info)


def append_values(v_new, mu_v, frame_tokens, group_tokens, idx_override=None):
    """Quantize-append of a block of whole frames of Values for one head."""
    v_new = np.asarray(v_new, dtype=np.float32)
    idx, info = select_values(v_new, mu_v)
    if idx_override:
        for t, cidx in idx_override.items():
            idx[t] = cidx
    rho = residual(v_new, mu_v[idx])
    codes, zs, ss, rho_hat = quantize_residuals(rho, frame_tokens, group_tokens)
    return dict(idx=idx, codes=codes, z=zs, s=ss, rho=rho, rho_hat=rho_hat, info=info)


def tiles_per_frame(frame_tokens, group_tokens):
    return math.ceil(frame_tokens / group_tokens)
