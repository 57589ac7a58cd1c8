"""The seeded generator and the stored oracle regression values (CPU)."""
import json
import os

import numpy as np

import synth
from synth import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))


def test_splitmix64_known_answer():
    # SplitMix64 started at state 0 (published reference sequence)
    w = synth.splitmix_words(0, 0, np.array([0], dtype=np.uint64), 3)
    assert [int(x[0]) for x in w] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_irwin_hall_moments_and_range():
    z = synth.gaussian_f32(3, 1, np.arange(1 << 20, dtype=np.uint64)).astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    assert np.all(np.abs(z) <= 6.0)
    # counter-based: any slice regenerates identically
    assert np.array_equal(z[1000:1010], synth.gaussian_f32(3, 1, np.arange(1000, 1010, dtype=np.uint64)))


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.0, 3.0e38, np.inf], dtype=np.float32)
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties to even (1.0)
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to even (1 + 2^-6)
    got = synth.round_to_bf16(x)
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == np.float32(1.015625)
    assert got[3] == -2.0 and np.isinf(got[5])


def test_keep_budget_matches_oracle_rule():
    from oracle import sparse_attention as sa
    for cfg in (W.C1, W.C2, W.C3):
        ours = W.keep_budget(cfg).tolist()
        ref = sa.keep_budget(cfg.N, keep_const=cfg.keep_const, keep_percent=cfg.keep_percent)
        assert ours == ref


def test_dominant_sets_and_needles():
    dom = W.dominant_pairs(W.C4)
    assert dom.shape == (8, 16) and np.all(np.diff(dom, axis=1) > 0) and dom.max() < 64
    lens = W.cache_lengths(W.C4.with_(B=3, ragged=100))
    nd = W.decode_needles(W.C4.with_(B=3, ragged=100), lens)
    assert len(nd) == 3 * 32 * 4
    for b, h, p in nd:
        assert 0 <= p <= lens[b] - 2


def test_golden_c1_oracle_regression():
    import importlib.util
    spec = importlib.util.spec_from_file_location("mk", os.path.join(HERE, "golden", "make_golden.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    now = mk.c1_values()
    with open(os.path.join(HERE, "golden", "c1_oracle.json")) as f:
        stored = json.load(f)
    assert now["selected_blocks"] == stored["selected_blocks"]
    for a, b in zip(now["block_scores_lower"], stored["block_scores_lower"]):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12)
    for t in stored["out_rows"]:
        assert np.allclose(now["out_rows"][t], stored["out_rows"][t], atol=1e-12)
        assert abs(now["lse_rows"][t] - stored["lse_rows"][t]) < 1e-12
