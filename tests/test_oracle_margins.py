"""Pins of the oracle's top-1 measure and of the decision margins that the
tie-following parity checker uses (CPU only)."""
import numpy as np

from oracle import margins, measures


def test_top1_shift_constructed_case():
    """Four queries over three keys, worked by hand.  Original logits
    q0: (2, 0, 1) -> 0; q1: (0, 2, 1) -> 1; q2: (2, 2, 2) -> 0 (three-way tie,
    lowest index); q3: (2, -2, 0) -> 0.  Rebuilt keys k1 = (0, 3),
    k2 = (1.5, 1.5): q0: (2, 0, 1.5) -> 0; q1: (0, 3, 1.5) -> 1;
    q2: (2, 3, 3) -> 1 (tie, lowest index); q3: (2, -3, 0) -> 0.  One of four
    selections moves: shift 0.25.  A last-maximum tie rule would report 0."""
    q = np.array([[1, 0], [0, 1], [1, 1], [1, -1]], np.float64)
    k_orig = np.array([[2, 0], [0, 2], [1, 1]], np.float64)
    k_rec = np.array([[2, 0], [0, 3], [1.5, 1.5]], np.float64)
    assert measures.top1(q, k_orig).tolist() == [0, 1, 0, 0]
    assert measures.top1(q, k_rec).tolist() == [0, 1, 1, 0]
    assert measures.top1_shift(q, k_orig, k_rec) == 0.25
    assert measures.top1_shift(q, k_orig, k_orig) == 0.0
    # swapping the two rebuilt keys that win moves three selections
    assert measures.top1_shift(q, k_orig, k_rec[[0, 2, 1]]) == 0.5


def test_argmin_margin_values():
    e = 2.0 ** -30
    dist = np.array([[1.0, 1.0 + e, 5.0], [3.0, 1.0, 2.0], [2.0, 2.0, 7.0]])
    m = margins.argmin_margin(dist)
    assert m[0] == e / (1.0 + e)
    assert m[1] == 0.5
    assert m[2] == 0.0
    assert m[0] < margins.TIE and m[1] > margins.TIE and m[2] < margins.TIE
    assert np.all(np.isinf(margins.argmin_margin(np.ones((2, 1)))))


def test_key_margins_candidate_boundary_and_choice():
    """cand: gap between the K_c-th and (K_c+1)-th smallest D; choice: gap
    between the two smallest P among the candidates."""
    e = 2.0 ** -29
    info = dict(D=np.array([[1.0, 2.0, 2.0 + e, 9.0], [4.0, 1.0, 3.0, 2.0]]),
                cand=np.array([[0, 1], [1, 3]]), P=np.array([[3.0, 3.5], [1.0, 1.0]]))
    m = margins.key_margins(info, 2, 0)
    assert m["cand"][0] == e / (2.0 + e) and m["cand"][0] < margins.TIE
    assert m["cand"][1] == (3.0 - 2.0) / 3.0
    assert m["choice"][0] == 0.5 / 3.5 and m["choice"][1] == 0.0
    # argmin modes: only the choice among all D
    m0 = margins.key_margins(dict(D=info["D"], cand=None), 0, 2)
    assert np.all(np.isinf(m0["cand"])) and m0["choice"][1] == 0.5


def test_f32_midpoint_distance():
    c = np.array([1 + 2.0 ** -24, 1 + 2.0 ** -24 + 2.0 ** -40, 1.0, -(1 + 2.0 ** -24), 3 * 2.0 ** -30])
    dist = margins._midpoint_dist_f32(c)
    assert dist[0] == 0.0 and dist[3] == 0.0          # exactly on a rounding midpoint
    assert dist[1] == 2.0 ** -40
    assert dist[2] == 2.0 ** -25                        # midpoint below 1 is 1 - 2^-25
    assert dist[4] == 2.0 ** -53                        # 3 * 2^-30 is exact; ulp there is 2^-52


def test_psac_margins_on_and_off_midpoints():
    """c32: c on a binary32 midpoint; sigma: max|c|/127 on a binary16 midpoint
    (127 (1 + 2^-11) / 127 = 1 + 2^-11, halfway between 1 and 1 + 2^-10);
    int8: c / sigma a half-integer (0.00390625 / 2^-7 = 0.5)."""
    c = np.array([[1 + 2.0 ** -24, 0.5], [127 * (1 + 2.0 ** -11), 3.0],
                  [0.9921875, 0.00390625], [0.9921875, 0.375]])
    c32 = c.astype(np.float32)
    a = np.abs(c32).max(axis=1).astype(np.float64)
    sigma = (a / 127.0).astype(np.float32).astype(np.float16).astype(np.float32)
    m = margins.psac_margins(c, sigma, np.ones_like(c))
    assert m["c32"][0] == 0.0 and m["c32"][0] < margins.PSAC_TIE
    assert m["c32"][2] > margins.PSAC_TIE
    assert m["sigma"][1] == 0.0
    assert m["sigma"][2] > margins.TIE                # 2^-7 is exact in binary16
    assert m["int8"][2] == 0.0
    # 0.375 / 2^-7 = 48: the nearest half-integer is 0.5 away, margin 0.5 sigma / a
    assert abs(m["int8"][3] - 0.5 * 2.0 ** -7 / 0.9921875) < 1e-15
