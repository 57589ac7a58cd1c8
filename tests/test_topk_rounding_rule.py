"""CPU checks of the rule that compares a low-precision top-k with the fp64
oracle's (tests/parity_utils.py: topk_status, overlap_range,
calibration_count_bounds).

The rule says which entries every admissible top-k keeps, which it may keep,
and how far an overlap of two such selections can move.  It is pinned here
by exhaustive enumeration on small cases, by sampling scores inside the
stated rounding intervals, and by an fp32 calibration in the channel order
of the GPU kernel, whose counts must fall inside the bounds while a
calibration with a planted mistake must not.
"""
import itertools

import numpy as np

from oracle import calibration as C
from synth import workloads as W
from tests.parity_utils import calibration_count_bounds, overlap_range, topk_status


def _topk(v, k):
    return set(C.topk_set(v, k).tolist())


def test_exact_scores_leave_nothing_ambiguous():
    rng = np.random.default_rng(0)
    for _ in range(50):
        n = int(rng.integers(1, 40))
        k = int(rng.integers(1, n + 1))
        s = rng.integers(-3, 4, size=n).astype(np.float64)  # many exact ties
        sure_in, amb = topk_status(s, np.zeros(n), k)
        assert not amb.any()
        assert set(np.nonzero(sure_in)[0].tolist()) == _topk(s, k)


def test_sampled_scores_stay_inside_the_rule():
    rng = np.random.default_rng(1)
    for _ in range(40):
        n = int(rng.integers(5, 60))
        k = int(rng.integers(1, n))
        s = np.round(rng.normal(size=n) * 4) / 4          # ties on a grid
        tol = rng.choice([0.0, 0.05, 0.2], size=n)
        sure_in, amb = topk_status(s, tol, k)
        s2 = np.round(rng.normal(size=n) * 4) / 4
        t2 = rng.choice([0.0, 0.1], size=n)
        p_in, p_amb = topk_status(s2, t2, k)
        lo, hi = overlap_range(sure_in, amb, k, p_in, p_amb, k)
        for _ in range(60):
            v = s + tol * rng.choice([-1.0, 0.0, 1.0, rng.uniform(-1, 1)], size=n)
            v2 = s2 + t2 * rng.choice([-1.0, 0.0, 1.0], size=n)
            F, Pk = _topk(v, k), _topk(v2, k)
            assert set(np.nonzero(sure_in)[0].tolist()) <= F <= set(np.nonzero(sure_in | amb)[0].tolist())
            assert lo <= len(F & Pk) <= hi


def test_overlap_range_is_exact_on_small_cases():
    rng = np.random.default_rng(2)
    for _ in range(200):
        n = int(rng.integers(2, 9))
        cat_f = rng.integers(0, 3, size=n)   # 0 in, 1 ambiguous, 2 out
        cat_p = rng.integers(0, 3, size=n)
        f_in, f_amb = cat_f == 0, cat_f == 1
        p_in, p_amb = cat_p == 0, cat_p == 1
        kf = int(f_in.sum()) + int(rng.integers(0, f_amb.sum() + 1))
        kp = int(p_in.sum()) + int(rng.integers(0, p_amb.sum() + 1))
        lo, hi = overlap_range(f_in, f_amb, kf, p_in, p_amb, kp)
        fa, pa = np.nonzero(f_amb)[0], np.nonzero(p_amb)[0]
        seen = set()
        for X in itertools.combinations(fa.tolist(), kf - int(f_in.sum())):
            F = set(np.nonzero(f_in)[0].tolist()) | set(X)
            for Y in itertools.combinations(pa.tolist(), kp - int(p_in.sum())):
                Pk = set(np.nonzero(p_in)[0].tolist()) | set(Y)
                seen.add(len(F & Pk))
        assert (lo, hi) == (min(seen), max(seen))


def _fp32_counts(q, k, k_cal, mistake=None):
    """Calibration counts with fp32 scores in the GPU kernel's order: the
    products (exact for bf16 values) summed channel by channel, a pair score
    one rounding of its two products.  ``mistake`` plants an error."""
    Hq, M, d = q.shape
    Hkv = k.shape[0]
    P = d // 2
    grp = Hq // Hkv
    counts = np.zeros((Hkv, P), np.int64)
    for h in range(Hq):
        g = h // grp
        for m in range(M):
            prod = q[h, m].astype(np.float32)[None, :] * k[g].astype(np.float32)
            full = np.zeros(k.shape[1], np.float32)
            chans = range(d - 1) if mistake == "drop-channel" else range(d)
            for c in chans:
                full = full + prod[:, c]
            if mistake == "interleaved":
                pairs = (prod[:, 0::2] + prod[:, 1::2]).T
            else:
                pairs = (prod[:, :P] + prod[:, P:]).T
            F = _topk(full, k_cal)
            for i in range(P):
                counts[g, i] += len(F & _topk(pairs[i], k_cal))
    return counts


def test_fp32_calibration_lies_within_the_bounds():
    cfg = W.CalibConfig("rule", 4, 2, 3, 700, 64, n_dom=4, k_cal=24, seed=21)
    q, k, _ = W.calibration_inputs_host(cfg)
    lo, hi, _n = calibration_count_bounds(q, k, cfg.k_cal)
    ref = C.overlap_counts(q, k, cfg.k_cal)
    assert np.all((lo <= ref) & (ref <= hi))
    got = _fp32_counts(q, k, cfg.k_cal)
    assert np.all((lo <= got) & (got <= hi))
    for mistake in ("drop-channel", "interleaved"):
        bad = _fp32_counts(q, k, cfg.k_cal, mistake)
        assert not np.all((lo <= bad) & (bad <= hi)), mistake
