"""Pins of the calibration oracle (dominant rotary pairs).

"FASA: Frequency-aware Sparse Attention", sec. 2.A (a small fixed set of
dominant frequency chunks reproduces a head's context selection) and sec.
2.B item 1 (one-time offline calibration).  The pages give no criterion and
no worked example; the oracle's reading is pinned by a hand-worked case, by
recovery of planted dominant pairs, and by exact invariances.
"""
import json
import os

import numpy as np
import pytest

from oracle import calibration as C
from synth import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden", "calibration_tiny.json")


def test_hand_worked_case():
    g = json.load(open(GOLD))
    q = np.array(g["q"], np.float64)
    k = np.array(g["k"], np.float64)
    full, pairs = C.calibration_scores(q[0, 0], k[0])
    assert full.tolist() == g["full_scores"]
    assert C.topk_set(full, g["k_cal"]).tolist() == g["full_topk"]
    for i, want in enumerate(g["pair_topk"]):
        assert C.topk_set(pairs[i], g["k_cal"]).tolist() == want
    for n_dom, want in g["dominant"].items():
        counts, dom = C.calibrate_dominant(q, k, g["k_cal"], int(n_dom))
        assert counts.tolist() == g["counts"]
        assert dom.tolist() == want


def test_recovers_planted_pairs():
    cfg = W.CalibConfig("pin", 4, 2, 4, 512, 64, n_dom=4, k_cal=16)
    q, k, planted = W.calibration_inputs_host(cfg)
    counts, dom = C.calibrate_dominant(q, k, cfg.k_cal, cfg.n_dom)
    assert np.array_equal(dom, planted)
    # every planted pair is clearly ahead of every other pair
    for g in range(cfg.Hkv):
        rest = np.setdiff1d(np.arange(cfg.d // 2), planted[g])
        assert counts[g, planted[g]].min() > 2 * counts[g, rest].max()


def _integer_case(seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(-8, 9, size=(4, 3, 16)).astype(np.float64)   # Hq 4, M 3, d 16
    k = rng.integers(-8, 9, size=(2, 40, 16)).astype(np.float64)  # Hkv 2, L 40
    return q, k


def test_pair_permutation_equivariance():
    # integer inputs: every score is exact in fp32 whatever the summation order
    q, k = _integer_case(1)
    P = 8
    perm = np.array([5, 2, 7, 0, 3, 6, 1, 4])
    ch = np.concatenate([perm, perm + P])
    c0 = C.overlap_counts(q, k, 6)
    c1 = C.overlap_counts(q[..., ch], k[..., ch], 6)
    assert np.array_equal(c1, c0[:, perm])


def test_positive_scale_invariance():
    q, k = _integer_case(2)
    assert np.array_equal(C.overlap_counts(q, k, 5), C.overlap_counts(4.0 * q, k, 5))


def test_single_pair_carries_everything():
    # only pair 3 is non-zero in the keys: its partial scores equal the full
    # scores, so its overlap is k_cal for every query; every other pair scores
    # all keys 0 and keeps the k_cal lowest indices
    rng = np.random.default_rng(3)
    d, P, L, kk = 16, 8, 30, 4
    q = rng.normal(size=(2, 5, d))
    k = np.zeros((1, L, d))
    k[0, :, 3] = rng.normal(size=L)
    k[0, :, 3 + P] = rng.normal(size=L)
    counts = C.overlap_counts(q, k, kk)
    assert counts[0, 3] == 2 * 5 * kk
    low = set(range(kk))
    want = 0
    for h in range(2):
        for m in range(5):
            full, _ = C.calibration_scores(q[h, m], k[0])
            want += len(low & set(C.topk_set(full, kk).tolist()))
    assert all(counts[0, i] == want for i in range(P) if i != 3)
