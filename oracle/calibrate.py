"""Oracle: historical-Query statistics and centroids (calibration step).

TEST INFRASTRUCTURE ONLY (see the package header).

What the pages fix
 * Both components use statistics of already-generated Queries only: the
   method is training-free and causal (English digest, method section; review
   FAQ "strictly causal").
 * The expected squared logit perturbation of a Key error e is
   E[(q^T e)^2] = e^T M e with M the Query second moment (review summary,
   Eq. 7).  QSAC uses the diagonal of M (review: "diagonal approximation").
 * PSAC uses the top-8 principal Query directions; on one LingBot-World-v2
   layer they hold about 71 % of the Query energy (digest, PSAC paragraph;
   review, Fig. 4).
 * Keys are assigned to cluster centres kept at higher precision (QVG scheme,
   digest QSAC paragraph).

Readings (the pages are silent)
 * M is the uncentred second moment (1/n) sum q q^T of the given historical
   queries, per head, in float64.  s = diag(M) and U are stored in float32.
 * U = eigenvectors of the r largest eigenvalues, descending; each column's
   largest-magnitude entry (lowest index on ties) is made positive.
   energy(r) = sum of the r largest eigenvalues / trace(M).
 * Centroids are plain Lloyd k-means (Euclidean, float64), seeded Forgy
   initialisation from a SplitMix64-driven partial Fisher-Yates shuffle,
   `iters` assignment+update rounds, assignment ties to the lowest index,
   empty clusters keep their previous centre.  The stream of head h starts at
   seed + 2h for Keys and seed + 2h + 1 for Values.  Centroids are then stored
   rounded to the I/O precision (bfloat16, or float32 for float32 I/O).
 * Centroids and statistics are frozen for the life of a cache.

Pins (tests/test_oracle_calibrate.py): Eq. 7 identity on random e; LAPACK eigh
against an independent subspace iteration; generator energy ~0.70; k-means
objective non-increasing, zero with C = n distinct points, assignments equal a
brute-force nearest search; SplitMix64 against its published seed-0 outputs;
the Forgy indices against a list worked out by hand from those outputs
(tests/golden/forgy_seed0.json).
"""
import numpy as np

from .numerics import fl32, round_storage

MASK64 = (1 << 64) - 1


def second_moment(q_hist):
    """M = (1/n) sum_i q_i q_i^T, float64 [d, d] (Eq. 7's matrix)."""
    q = np.asarray(q_hist, dtype=np.float64)
    return (q.T @ q) / q.shape[0]


def principal_directions(m, r):
    """Top-r eigenvectors of M (descending), sign-normalised, and energy(r)."""
    w, vecs = np.linalg.eigh(m)
    order = np.argsort(-w, kind="stable")
    w, vecs = w[order], vecs[:, order]
    u = vecs[:, :r].copy()
    for i in range(r):
        j = int(np.argmax(np.abs(u[:, i])))      # first max -> lowest index
        if u[j, i] < 0:
            u[:, i] = -u[:, i]
    energy = float(np.sum(w[:r]) / np.trace(m)) if r > 0 else 0.0
    return u, energy, w


class SplitMix64:
    """SplitMix64 (Steele, Lea, Flood 2014): a 64-bit counter hashed per step."""

    def __init__(self, seed):
        self.state = seed & MASK64

    def next(self):
        self.state = (self.state + 0x9E3779B97F4A7C15) & MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        return z ^ (z >> 31)


def forgy_indices(n, c, seed):
    """C distinct sample indices: the first C slots of a partial Fisher-Yates
    shuffle of 0..n-1, with swap partner i + (next() mod (n - i))."""
    if c > n:
        raise ValueError("more centroids than points")
    perm = list(range(n))
    rng = SplitMix64(seed)
    for i in range(c):
        j = i + rng.next() % (n - i)
        perm[i], perm[j] = perm[j], perm[i]
    return np.array(perm[:c], dtype=np.int64)


def sq_distances(x, mu):
    """Direct-form squared Euclidean distances sum_j (x_j - mu_j)^2, [n, C]."""
    out = np.empty((x.shape[0], mu.shape[0]), dtype=np.float64)
    step = max(1, 2_000_000 // max(1, mu.size))
    for a in range(0, x.shape[0], step):
        diff = x[a:a + step, None, :] - mu[None, :, :]
        out[a:a + step] = np.einsum("ncd,ncd->nc", diff, diff)
    return out


def kmeans(x, c, iters, seed, history=False):
    """Lloyd's algorithm in float64.  Returns (centroids fp64 [C, d], assign)
    and, with history=True, the objective after every assignment step."""
    x = np.asarray(x, dtype=np.float64)
    mu = x[forgy_indices(x.shape[0], c, seed)].copy()
    objective = []
    assign = None
    for _ in range(iters):
        dist = sq_distances(x, mu)
        assign = np.argmin(dist, axis=1)         # ties -> lowest index
        objective.append(float(dist[np.arange(x.shape[0]), assign].sum()))
        for ci in range(c):
            members = x[assign == ci]
            if members.shape[0] > 0:             # empty cluster keeps its centre
                mu[ci] = members.mean(axis=0)
    if history:
        return mu, assign, objective
    return mu, assign


def calibrate(q_hist, k_hist, v_hist, c_k, c_v, rank, io, seed, iters=10):
    """Per-head calibration.  Inputs are [H, n, d].  Returns a dict of the
    stored fields: mu_k [H,C_K,d], mu_v [H,C_V,d] (float32 holding the storage
    precision), sens [H,d] float32, u [H,d,r] float32, energy [H] float64,
    and moment [H,d,d] float64 (the full M, for the full-quadratic stage-2
    variant)."""
    h_count, _, d = np.shape(q_hist)
    out = dict(mu_k=[], mu_v=[], sens=[], u=[], energy=[], moment=[])
    for h in range(h_count):
        m = second_moment(q_hist[h])
        u, energy, _ = principal_directions(m, rank)
        mk, _ = kmeans(k_hist[h], c_k, iters, seed + 2 * h)
        mv, _ = kmeans(v_hist[h], c_v, iters, seed + 2 * h + 1)
        out["mu_k"].append(round_storage(mk, io))
        out["mu_v"].append(round_storage(mv, io))
        out["sens"].append(fl32(np.diag(m)))
        out["u"].append(fl32(u).reshape(d, rank))
        out["energy"].append(energy)
        out["moment"].append(m)
    return {key: np.stack(val) if key != "energy" else np.array(val)
            for key, val in out.items()}
