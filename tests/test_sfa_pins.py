"""Pins of the Sparse Feature Attention oracle.

"Scaling Attention via Feature Sparsity", sec. 2: k-sparse query and key
codes (the k channels of largest magnitude keep their values) and scores
computed over the channels active in both.  Pinned by a hand-worked code,
by the literal intersection sum, by the dense special case k = d (torch's
attention routine) and by GQA consistency.
"""
import numpy as np
import pytest
import torch

from oracle import feature_sparse as F


def test_hand_worked_code():
    x = np.array([1.0, -3.0, 2.0, 3.0, 0.5, -2.0])
    # |x| = 1 3 2 3 0.5 2: channels 1 and 3 (3), then the tie at 2 goes to channel 2
    assert F.sparsify(x[None], 3)[0].tolist() == [0.0, -3.0, 2.0, 3.0, 0.0, 0.0]
    assert F.sparsify(x[None], 1)[0].tolist() == [0.0, -3.0, 0.0, 0.0, 0.0, 0.0]
    assert F.sparsify(x[None], 6)[0].tolist() == x.tolist()


def test_dense_code_dot_is_the_intersection_sum():
    rng = np.random.default_rng(5)
    for kf in (1, 3, 8, 16):
        q = rng.normal(size=(20, 32))
        k = rng.normal(size=(20, 32))
        qs, ks = F.sparsify(q, kf), F.sparsify(k, kf)
        for i in range(20):
            lit = F.intersection_score(q[i], k[i], kf)
            assert abs(float(qs[i] @ ks[i]) - lit) <= 1e-12 * (1 + abs(lit))
            # the active sets have k channels each
            assert np.count_nonzero(qs[i]) == kf


def test_full_code_is_dense_attention():
    rng = np.random.default_rng(6)
    q = rng.normal(size=(1, 2, 24, 16))
    k = rng.normal(size=(1, 2, 24, 16))
    v = rng.normal(size=(1, 2, 24, 16))
    out, _ = F.sfa_attention(q, k, v, 16, 0.25, causal=True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True, scale=0.25)
    assert np.abs(out - ref.numpy()).max() < 1e-12


def test_gqa_matches_repeated_heads():
    rng = np.random.default_rng(7)
    q = rng.normal(size=(1, 4, 10, 8))
    k = rng.normal(size=(1, 2, 10, 8))
    v = rng.normal(size=(1, 2, 10, 8))
    out, lse = F.sfa_attention(q, k, v, 3, 0.5)
    out2, lse2 = F.sfa_attention(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), 3, 0.5)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
