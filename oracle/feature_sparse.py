"""Sparse Feature Attention (SFA) -- oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Scaling Attention via Feature Sparsity", sec. 2: every query and key
vector is replaced by its k-sparse code -- the k channels of largest
magnitude keep their values, the others become zero -- and a score is
computed only over the channels active in both the query and the key.  The
softmax and the value product stay those of exact attention.

Readings: ties in magnitude go to the lower channel; the scaled score
sigma * sum over the intersection; causal prefill attention (key s visible
to query t when s <= t), values dense.
"""
from __future__ import annotations

import numpy as np


def sparsify(x: np.ndarray, k: int) -> np.ndarray:
    """k-sparse code of every row of x[..., d]: the k largest |x_c| (ties to
    the lower channel) keep their value, every other channel is 0."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    flat = x.reshape(-1, d)
    out = np.zeros_like(flat)
    ch = np.arange(d)
    for r in range(flat.shape[0]):
        order = np.lexsort((ch, -np.abs(flat[r])))
        keep = order[:k]
        out[r, keep] = flat[r, keep]
    return out.reshape(x.shape)


def intersection_score(q_row: np.ndarray, k_row: np.ndarray, kf: int) -> float:
    """The score as the pages define it: a sum over the channels active in both codes."""
    aq = set(np.lexsort((np.arange(q_row.size), -np.abs(q_row)))[:kf].tolist())
    ak = set(np.lexsort((np.arange(k_row.size), -np.abs(k_row)))[:kf].tolist())
    return float(sum(float(q_row[c]) * float(k_row[c]) for c in sorted(aq & ak)))


def sfa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, kf: int, sm_scale: float,
                  causal: bool = True):
    """q [B, Hq, S, d], k, v [B, Hkv, S, d] -> (out [B, Hq, S, d], lse [B, Hq, S]) in fp64.

    Scores of the k-sparse codes: the dot product of the zero-filled codes,
    which is the sum over the channels active in both."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    grp = Hq // Hkv
    qs, ks = sparsify(q, kf), sparsify(k, kf)
    out = np.zeros_like(q)
    lse = np.zeros((B, Hq, S))
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            s = sm_scale * (qs[b, h] @ ks[b, g].T)
            if causal:
                s = np.where(np.tril(np.ones((S, S), bool)), s, -np.inf)
            mx = s.max(axis=1, keepdims=True)
            p = np.exp(s - mx)
            den = p.sum(axis=1, keepdims=True)
            out[b, h] = (p @ v[b, g]) / den
            lse[b, h] = mx[:, 0] + np.log(den[:, 0])
    return out, lse
