"""GPU parity of the offline calibration of the dominant rotary pairs.

"FASA: Frequency-aware Sparse Attention", sec. 2.A and sec. 2.B item 1; the
criterion is the one the oracle states (oracle/calibration.py), whose scores
are plain fp64.  The GPU scores in fp32 (a running sum of exact bf16
products; a pair score one rounding of two products), so near the k-th and
(k+1)-th key its top-k may differ from the oracle's.  The test bounds that:
from the oracle's scores and the fp32 rounding bound, every key of every
selection is sure-in, sure-out or ambiguous, and each per-query, per-pair
overlap lies in a range that collapses to the oracle's value wherever no
boundary is ambiguous (tests/parity_utils.calibration_count_bounds).  The
GPU's per-pair counts must lie in the summed ranges (equal to the oracle's
where every range is one value), and its dominant set must be the top n_dom
of its own counts (integer work, bit for bit).
"""
import numpy as np
import pytest
import torch

from oracle import calibration as C
from synth import workloads as W
from tests.parity_utils import calibration_count_bounds, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import long_context_sparse_apply_amd as m
    return m


def _run(sa, q, k, k_cal, n_dom):
    qt = torch.from_numpy(np.ascontiguousarray(q, np.float32)).to(DEV).to(torch.bfloat16)
    kt = torch.from_numpy(np.ascontiguousarray(k, np.float32)).to(DEV).to(torch.bfloat16)
    Hq, M, d = q.shape
    Hkv, L = k.shape[:2]
    ws = torch.empty(sa.calibrate_workspace_bytes(Hq, Hkv, M, L, d, k_cal), dtype=torch.uint8,
                     device=DEV)
    dom = torch.full((Hkv, n_dom), -7, dtype=torch.int32, device=DEV)
    counts = torch.full((Hkv, d // 2), -7, dtype=torch.int32, device=DEV)
    sa.sa_calibrate_dominant(qt, kt, dom, counts, ws, k_cal=k_cal)
    torch.cuda.synchronize()
    return dom.cpu().numpy(), counts.cpu().numpy()


CASES = [
    # name, config, k_cal, n_dom
    ("small-planted", W.CAL_SMALL, 64, 16),
    ("d64-short-rows", W.CalibConfig("d64", 2, 2, 3, 1000, 64, n_dom=5, k_cal=8, seed=11), 7, 5),
    ("gqa4-long-ragged", W.CalibConfig("g4", 4, 1, 2, 5000, 128, n_dom=8, k_cal=600, seed=12), 300, 32),
    ("all-keys-all-pairs", W.CalibConfig("all", 2, 1, 2, 300, 64, n_dom=4, k_cal=8, seed=13), 300, 32),
]


@pytest.mark.parametrize("name,cfg,k_cal,n_dom", CASES, ids=[c[0] for c in CASES])
def test_calibration_parity(sa, name, cfg, k_cal, n_dom):
    say(f"case: calibration {name}")
    q, k, planted = W.calibration_inputs_host(cfg)
    dom, counts = _run(sa, q, k, k_cal, n_dom)
    ref_counts, ref_dom = C.calibrate_dominant(q, k, k_cal, n_dom)
    lo, hi, n_amb = calibration_count_bounds(q, k, k_cal)
    assert np.all((lo <= ref_counts) & (ref_counts <= hi))
    inside = (lo <= counts) & (counts <= hi)
    assert inside.all(), (np.argwhere(~inside)[:5], counts[~inside][:5], lo[~inside][:5],
                          hi[~inside][:5])
    exact = lo == hi
    assert np.array_equal(counts[exact], ref_counts[exact])
    # the dominant set is the top n_dom of the GPU's own counts
    assert np.array_equal(dom, C.dominant_from_counts(counts.astype(np.int64), n_dom))
    # where the oracle's ranges separate the n_dom-th from the next, the sets are equal
    for g in range(counts.shape[0]):
        rest = np.setdiff1d(np.arange(counts.shape[1]), ref_dom[g])
        if rest.size == 0 or lo[g, ref_dom[g]].min() > hi[g, rest].max():
            assert np.array_equal(dom[g], ref_dom[g]), g
    say(f"  counts inside the fp32 bounds; {n_amb} ambiguous (query, pair) overlaps, "
        f"{int(exact.sum())}/{exact.size} counts fixed exactly")
    if name == "small-planted":
        assert np.array_equal(dom, planted)
    if name == "all-keys-all-pairs":
        # k_cal = L: every selection holds the whole window
        assert np.all(counts == cfg.group * cfg.M * cfg.L)
        assert np.array_equal(dom, np.tile(np.arange(32), (cfg.Hkv, 1)))


def test_calibrated_set_drives_token_scoring(sa):
    """The calibrated set is a dom_pairs argument of sa_token_score as it is."""
    cfg = W.CAL_SMALL
    q, k, planted = W.calibration_inputs_host(cfg)
    dom, _ = _run(sa, q, k, cfg.k_cal, cfg.n_dom)
    qt = torch.from_numpy(np.ascontiguousarray(q[:, 0], np.float32)).to(DEV).to(torch.bfloat16)
    kt = torch.from_numpy(np.ascontiguousarray(k, np.float32)).to(DEV).to(torch.bfloat16)
    scores = torch.empty((1, cfg.Hq, cfg.L), dtype=torch.float32, device=DEV)
    lens = torch.full((1,), cfg.L, dtype=torch.int32, device=DEV)
    sa.sa_token_score(qt[None], kt[None], scores, lens, torch.from_numpy(dom).to(DEV),
                      sm_scale=1.0)
    torch.cuda.synchronize()
    assert torch.isfinite(scores).all()
