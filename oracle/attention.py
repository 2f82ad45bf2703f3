"""Oracle: cache reconstruction and attention over the compressed cache.

TEST INFRASTRUCTURE ONLY (see the package header).

What the pages fix
 * The attention logits are the dot products of the current Query with the
   historical Keys, QK^T (abstract, final page).
 * PSAC compensates the Key during cache reconstruction (digest, PSAC
   paragraph); the review phrases it as a low-rank correction to the attention
   logits -- the same quantity, since q.(k_hat + U c_hat) = q.k_hat + (U^T q).c_hat.
 * Each Key is rebuilt as its centre plus the dequantized residual (QVG scheme).

Definition (written out, float64):
   k~_t = mu_K[idx_t] + rho_hat_t + U c_hat_t,  c_hat = n * sigma
   v~_t = mu_V[idx_t] + rho_hat^V_t
   l_t  = tau * q . k~_t   (tau = 1/sqrt(d) unless given)
   o    = sum_t softmax(l)_t v~_t,   lse = log sum_t exp(l_t)
Every cached token is visible (all of them lie in the past; no mask).

Readings: softmax scale 1/sqrt(d); inputs are the post-positional-encoding
Q/K that enter the dot product; the current chunk's own K/V are not part of
the compressed cache (lse is returned so a caller can merge them).

One generation step (attention_with_local): the chunk's queries attend to the
rebuilt cache and to the chunk's own uncompressed keys and values (the pages
describe generation that reads the growing cache of historical frames while
the current frames are produced: digest, opening paragraph).  Reading: every
key of the chunk is visible to every query of the chunk (the chunk is one
block; no mask inside it).

Calibration epochs (attention_over_epochs): over a long rollout the caller
may calibrate again from recent content (the statistics come from content
already generated: digest, method section; 1-minute generation: digest,
experiments paragraph) and encode the frames that follow with the new
calibration.  Reading: every stored token keeps the calibration it was
encoded with, so the epochs' tokens are rebuilt each with their own centres
and U, and one softmax runs over all of them (and the chunk's own keys).

Pins (tests/test_oracle_attention.py): zero-residual keys reduce to textbook
softmax attention (PyTorch CPU scaled_dot_product_attention in float64);
constant V gives o = v; softmax rows sum to one; a split-KV log-sum-exp merge
equals the unsplit result; brute-force per-query loops on the tiny case.
attention_with_local: brute-force loops over both key sets; an empty cache
gives PyTorch's scaled_dot_product_attention over the local keys; local keys
that repeat the cache's keys leave o unchanged and raise lse by log 2.
attention_over_epochs: the log-sum-exp merge of each epoch's own attention;
brute-force loops; each epoch's rebuilt keys obey the PSAC bound along that
epoch's U (tests/test_oracle_codec.py).
"""
import numpy as np

from .numerics import fl32

GROUP = 16


def tile_index(t, frame_tokens, group_tokens):
    """Parameter-tile index of cached token t: frame * tiles_per_frame + tile."""
    tpf = -(-frame_tokens // group_tokens)
    f = t // frame_tokens
    return f * tpf + (t % frame_tokens) // group_tokens


def dequant_residual(codes, z, s, frame_tokens, group_tokens):
    """rho_hat [n, d] = fl32(z + code * s) using each token's tile params."""
    n, d = codes.shape
    p = tile_index(np.arange(n), frame_tokens, group_tokens)
    zz = np.repeat(z[p], GROUP, axis=1)
    ss = np.repeat(s[p], GROUP, axis=1)
    return fl32(zz.astype(np.float64) + codes.astype(np.float64) * ss.astype(np.float64))


def reconstruct_keys(idx, codes, z, s, coef, coef_scale, mu_k, u, frame_tokens, group_tokens):
    rho_hat = dequant_residual(codes, z, s, frame_tokens, group_tokens)
    k = np.asarray(mu_k, np.float64)[idx] + rho_hat.astype(np.float64)
    if u.shape[1] > 0:
        c_hat = coef.astype(np.float64) * np.asarray(coef_scale, np.float64)[:, None]
        k = k + c_hat @ np.asarray(u, np.float64).T
    return k


def reconstruct_values(idx, codes, z, s, mu_v, frame_tokens, group_tokens):
    rho_hat = dequant_residual(codes, z, s, frame_tokens, group_tokens)
    return np.asarray(mu_v, np.float64)[idx] + rho_hat.astype(np.float64)


def logits(q, keys, scale=None):
    q = np.asarray(q, np.float64)
    tau = 1.0 / np.sqrt(q.shape[1]) if scale is None else scale
    return tau * (q @ np.asarray(keys, np.float64).T)


def softmax_attention(q, keys, values, scale=None):
    """o [n_q, d] and lse [n_q] in float64."""
    lg = logits(q, keys, scale)
    m = lg.max(axis=1, keepdims=True)
    p = np.exp(lg - m)
    l_sum = p.sum(axis=1, keepdims=True)
    o = (p @ np.asarray(values, np.float64)) / l_sum
    return o, (m + np.log(l_sum))[:, 0]


def merge_partials(parts):
    """Combine (o_i, lse_i) over disjoint key sets by log-sum-exp weights."""
    lses = np.stack([p[1] for p in parts])
    top = lses.max(axis=0)
    w = np.exp(lses - top)
    lse = top + np.log(w.sum(axis=0))
    o = sum(np.exp(p[1] - lse)[:, None] * p[0] for p in parts)
    return o, lse


def attention_with_local(q, keys, values, k_loc, v_loc, scale=None):
    """o [n_q, d] and lse [n_q] (float64) of one softmax over the rebuilt cache
    keys/values and the chunk's own keys/values, all visible.  No keys at all
    gives o = 0 and lse = -inf."""
    q = np.asarray(q, np.float64)
    d = q.shape[1]
    k = np.concatenate([np.asarray(keys, np.float64).reshape(-1, d), np.asarray(k_loc, np.float64).reshape(-1, d)])
    v = np.concatenate([np.asarray(values, np.float64).reshape(-1, d), np.asarray(v_loc, np.float64).reshape(-1, d)])
    if k.shape[0] == 0:
        return np.zeros_like(q), np.full(q.shape[0], -np.inf)
    return softmax_attention(q, k, v, scale)


def attention_over_epochs(q, epochs, k_loc=None, v_loc=None, scale=None):
    """o [n_q, d] and lse [n_q] (float64) of one softmax over the rebuilt keys
    and values of every epoch (a list of (keys, values), each rebuilt with its
    own calibration) and the chunk's own keys and values (optional)."""
    d = np.shape(q)[1]
    keys = [np.asarray(k, np.float64).reshape(-1, d) for k, _ in epochs]
    values = [np.asarray(v, np.float64).reshape(-1, d) for _, v in epochs]
    kl = np.zeros((0, d)) if k_loc is None else k_loc
    vl = np.zeros((0, d)) if v_loc is None else v_loc
    return attention_with_local(q, np.concatenate(keys), np.concatenate(values), kl, vl, scale)
