"""Oracle: decision margins for tie-following parity.

TEST INFRASTRUCTURE ONLY (see the package header).

Every discrete decision of the append path gets a relative margin, computed in
float64.  A decision whose margin is below TIE (1e-6) is a documented tie: a
faithful implementation in other arithmetic may take either side, and the
checker then adopts the implementation's choice and recomputes everything
downstream before demanding bit-exactness again.

Kinds
  cand   : |D_(Kc) - D_(Kc+1)| / max    (QSAC candidate-set boundary)
  choice : |P_(1) - P_(2)| / max         (QSAC final choice; D for argmin modes)
  c32    : distance of c to the nearest binary32 rounding midpoint, divided by
           sum_j |U_ji e_j| (the scale of a float64 summation-order error).
           The projection is float64 on both sides, so c32 is the only PSAC
           decision that can differ; its tie threshold is PSAC_TIE (1e-12,
           about 100x the float64 error bound of a 128-term sum).
  sigma  : distance of fl32(a/127) to the nearest binary16 midpoint / sigma
  int8   : |c32/sigma - (n + 1/2)| sigma / a for the nearest half-integer
           (sigma and int8 are reported only: they are exact functions of c32)

Pins (tests/test_oracle_margins.py): values placed exactly on and at known
distances from binary32 and binary16 rounding midpoints, half-integer INT8
ratios, exact and near ties of D and P with binary-exact gaps.
"""
import numpy as np

TIE = 1e-6
PSAC_TIE = 1e-12


def _rel(a, b):
    den = np.maximum(np.abs(a), np.abs(b))
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.abs(a - b) / den
    return np.where(den == 0, 0.0, out)


def argmin_margin(dist):
    """Relative gap between the two smallest entries of each row."""
    if dist.shape[1] < 2:
        return np.full(dist.shape[0], np.inf)
    part = np.partition(dist, 1, axis=1)
    return _rel(part[:, 0], part[:, 1])


def key_margins(info, top_k, flags, no_range_flag=2):
    """Per-token min margin over the QSAC decisions (cand, choice)."""
    dist = info["D"]
    n, c_count = dist.shape
    if info.get("cand") is None:
        m = argmin_margin(dist)
        return dict(cand=np.full(n, np.inf), choice=m)
    kc = info["cand"].shape[1]
    srt = np.sort(dist, axis=1)
    cand = _rel(srt[:, kc - 1], srt[:, kc]) if kc < c_count else np.full(n, np.inf)
    p = info["P"]
    if kc < 2:
        choice = np.full(n, np.inf)
    else:
        ps = np.sort(p, axis=1)
        choice = _rel(ps[:, 0], ps[:, 1])
    return dict(cand=cand, choice=choice)


def _midpoint_dist_f32(c):
    """Distance of each float64 value to the nearest binary32 rounding midpoint."""
    c = np.asarray(c, np.float64)
    c32 = c.astype(np.float32)
    up = np.nextafter(c32, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(c32, np.float32(-np.inf)).astype(np.float64)
    mid_up = (c32.astype(np.float64) + up) / 2
    mid_dn = (c32.astype(np.float64) + dn) / 2
    return np.minimum(np.abs(c - mid_up), np.abs(c - mid_dn))


def _midpoint_margin_f16(y32):
    y = np.asarray(y32, np.float64)
    h = y.astype(np.float16)
    nxt = np.nextafter(h, np.float16(np.inf))
    ulp = np.abs(nxt.astype(np.float64) - h.astype(np.float64))
    dist = np.abs(np.abs(y - h.astype(np.float64)) - ulp / 2)
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(h == 0, np.inf, dist / np.abs(h.astype(np.float64)))


def psac_margins(c_exact, coef_scale, abs_scale):
    """Per-token minimum margins of the PSAC roundings (c32, sigma, int8).
    abs_scale [n, r] = sum_j |U_ji e_j| of each coefficient."""
    n = c_exact.shape[0]
    if c_exact.shape[1] == 0:
        inf = np.full(n, np.inf)
        return dict(c32=inf, sigma=inf, int8=inf)
    with np.errstate(invalid="ignore", divide="ignore"):
        c32m = np.where(abs_scale > 0, _midpoint_dist_f32(c_exact) / abs_scale, np.inf).min(axis=1)
    c32 = c_exact.astype(np.float32)
    a = np.abs(c32).max(axis=1).astype(np.float64)
    y = (a / 127.0).astype(np.float32)
    sig = _midpoint_margin_f16(y)
    sg = np.asarray(coef_scale, np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        x = (c32.astype(np.float64) / sg[:, None]).astype(np.float32).astype(np.float64)
        frac = np.abs(x - (np.floor(x) + 0.5))
        i8 = np.where(sg[:, None] > 0, frac * sg[:, None] / a[:, None], np.inf).min(axis=1)
    return dict(c32=c32m, sigma=sig, int8=i8)
