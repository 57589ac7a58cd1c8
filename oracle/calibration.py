"""Offline calibration of the dominant rotary pairs -- oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"FASA: Frequency-aware Sparse Attention", sec. 2.A: a small fixed set of
dominant frequency chunks reproduces a head's context selection; sec. 2.B
item 1: that set comes from a one-time offline calibration.  The pages give
no criterion.  Reading taken here:

* a pair's partial score of key t for query q is q_i k_{t,i} + q_{i+P} k_{t,i+P}
  (pair i = channels i and i + P, P = d/2), the full score is sum_c q_c k_{t,c};
* for every calibration query, the pair's overlap is the number of keys its
  partial-score top-k shares with the full-score top-k (top-k by score
  descending, then key index ascending);
* a KV head's count of pair i sums the overlaps over its query heads and
  calibration queries; the dominant set is the n_dom pairs with the largest
  counts (ties to the lower pair), listed in ascending order.

Every score is the plain fp64 definition above (one matrix product for the
full scores, one sum of two products for a pair).  A fast path that scores in
lower precision may order near-tied keys differently; comparing it with this
definition is the test's business (it bounds that path's rounding), not the
oracle's.
"""
from __future__ import annotations

import numpy as np


def calibration_scores(q: np.ndarray, k: np.ndarray):
    """q [d], k [L, d] -> (full [L], pairs [P, L]), fp64."""
    d = q.shape[-1]
    P = d // 2
    qd = np.asarray(q, np.float64)
    kd = np.asarray(k, np.float64)
    full = kd @ qd
    pairs = (kd[:, :P] * qd[None, :P] + kd[:, P:] * qd[None, P:]).T
    return full, pairs


def topk_set(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k best entries by (score descending, index ascending)."""
    idx = np.arange(scores.shape[0])
    order = np.lexsort((idx, -np.asarray(scores, np.float64)))
    return np.sort(order[:k])


def overlap_counts(q: np.ndarray, k: np.ndarray, k_cal: int) -> np.ndarray:
    """q [Hq, M, d], k [Hkv, L, d] -> counts [Hkv, P] (int64)."""
    Hq, M, d = q.shape
    Hkv = k.shape[0]
    P = d // 2
    grp = Hq // Hkv
    counts = np.zeros((Hkv, P), np.int64)
    for h in range(Hq):
        g = h // grp
        for m in range(M):
            full, pairs = calibration_scores(q[h, m], k[g])
            F = set(topk_set(full, k_cal).tolist())
            for i in range(P):
                counts[g, i] += len(F.intersection(topk_set(pairs[i], k_cal).tolist()))
    return counts


def dominant_from_counts(counts: np.ndarray, n_dom: int) -> np.ndarray:
    """counts [Hkv, P] -> the n_dom pairs with the largest counts per KV head
    (ties to the lower pair), ascending."""
    P = counts.shape[1]
    dom = np.empty((counts.shape[0], n_dom), np.int32)
    for g in range(counts.shape[0]):
        order = np.lexsort((np.arange(P), -counts[g]))
        dom[g] = np.sort(order[:n_dom])
    return dom


def calibrate_dominant(q: np.ndarray, k: np.ndarray, k_cal: int, n_dom: int):
    """-> (counts [Hkv, P], dominant pairs [Hkv, n_dom] ascending)."""
    counts = overlap_counts(q, k, k_cal)
    return counts, dominant_from_counts(counts, n_dom)
