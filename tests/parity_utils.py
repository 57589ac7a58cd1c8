"""Comparison rules used by the GPU parity tests.

* Scores (fp32 on the GPU, fp64 in the oracle): |gpu - ref| <= 1e-4 *
  max(|ref|, rms of the row's finite refs); -inf entries must match exactly.
* Selected index sets: where the oracle's k-th and (k+1)-th candidate scores
  differ by more than 1e-3 relative (same floor), the sets must be equal;
  everywhere the GPU's set must be threshold-consistent with the oracle's
  scores: the worst kept candidate is not clearly worse than the best dropped
  one (each side widened by the score tolerance), and the count is right.
* Attention outputs: within 2e-2 absolute for bf16 storage, 1e-5 for fp32.
* Rotated cache rows (:func:`rotated_bounds`): the GPU rotates in fp32 with
  an fp64-reduced angle, so each value lies within 2^-20 (|x_i| + |x_{i+P}|)
  of the oracle's fp64 rotation; stored as bf16 it must be one of the
  roundings of that interval (one value except next to a rounding midpoint).
"""
from __future__ import annotations

import sys

import numpy as np

SCORE_RTOL = 1e-4
# log-sum-exp of the bf16 attention paths: the probabilities are rounded to
# bf16 for the P V product and the denominator sums those same rounded values.
# bf16 keeps 8 significant bits, so round-to-nearest moves each value by at
# most 2^-8 of itself; log l then moves by at most log(1 + 2^-8) < 2^-8.  The
# fp32 score accumulation of ordinary logits adds far less than 1e-4.
LSE_ATOL_BF16 = 2.0 ** -8 + 1e-4
GAP_RTOL = 1e-3
OUT_ATOL = {"bf16": 2e-2, "f32": 1e-5}


ROT_ERR = 2.0 ** -20


def rotated_bounds(ref: np.ndarray, x_raw: np.ndarray, dtype: str):
    """Admissible [lo, hi] for the stored GPU rotation of ``x_raw`` given the
    oracle's fp64 rotation ``ref`` (same shape, last axis d)."""
    from synth import round_to_bf16
    P = x_raw.shape[-1] // 2
    pair = np.abs(x_raw[..., :P]).astype(np.float64) + np.abs(x_raw[..., P:])
    e = ROT_ERR * np.concatenate([pair, pair], axis=-1) + 2.0 ** -23 * np.abs(ref)
    lo, hi = ref - e, ref + e
    if dtype == "bf16":
        return (round_to_bf16(lo).astype(np.float64), round_to_bf16(hi).astype(np.float64))
    return lo, hi


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def row_floor(ref_row: np.ndarray) -> float:
    fin = ref_row[np.isfinite(ref_row)]
    return float(np.sqrt(np.mean(fin ** 2))) if fin.size else 0.0


def assert_scores_close(gpu: np.ndarray, ref: np.ndarray, rtol: float = SCORE_RTOL):
    g = np.asarray(gpu, np.float64).reshape(-1, gpu.shape[-1])
    r = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    assert g.shape == r.shape
    inf_r = ~np.isfinite(r)
    assert np.array_equal(~np.isfinite(g), inf_r), "infinite entries differ"
    assert np.array_equal(g[inf_r], r[inf_r])
    worst = 0.0
    for i in range(r.shape[0]):
        fin = np.isfinite(r[i])
        if not fin.any():
            continue
        tol = rtol * np.maximum(np.abs(r[i][fin]), row_floor(r[i]))
        err = np.abs(g[i][fin] - r[i][fin])
        worst = max(worst, float((err / tol).max()))
        assert np.all(err <= tol), f"row {i}: max err {err.max():.3e} > tol"
    return worst


def candidates(valid_len: int, n_sink: int, n_local: int) -> np.ndarray:
    forced = set(range(min(n_sink, valid_len))) | set(range(max(0, valid_len - n_local), valid_len))
    return np.array([j for j in range(valid_len) if j not in forced], dtype=np.int64), forced


def check_selection(gpu_sel, ref_scores, valid_len, k, n_sink, n_local, rtol=SCORE_RTOL,
                    tol=None):
    """Validate one row's GPU selection against the oracle's scores.

    ``tol`` (optional, per column) replaces the relative score tolerance
    when the GPU scores carry a larger derived error bound.  Returns True if
    the gap rule applied (and so the sets were compared for equality), False
    if only threshold consistency could be checked.
    """
    gsel = np.asarray(gpu_sel, dtype=np.int64)
    assert np.all(np.diff(gsel) > 0), "selection not strictly ascending"
    cand, forced = candidates(int(valid_len), n_sink, n_local)
    assert forced <= set(gsel.tolist()), "forced column missing"
    kk = min(int(k), cand.size)
    chosen = np.array(sorted(set(gsel.tolist()) - forced), dtype=np.int64)
    assert chosen.size == kk, f"kept {chosen.size} candidates, expected {kk}"
    assert np.all(np.isin(chosen, cand))
    if kk == 0 or kk == cand.size:
        return True
    s = np.asarray(ref_scores, np.float64)[cand]
    s = np.where(np.isnan(s), -np.inf, s)
    floor = row_floor(s)
    if tol is None:
        t = np.where(np.isfinite(s), rtol * np.maximum(np.abs(s), floor), 0.0)
    else:
        t = np.where(np.isfinite(s), np.asarray(tol, np.float64)[cand], 0.0)
    order = np.lexsort((cand, -s))
    kth, nxt = s[order[kk - 1]], s[order[kk]]
    gap_need = max(GAP_RTOL * max(abs(kth), floor), 2.0 * (t[order[kk - 1]] + t[order[kk]]))
    gap_applies = np.isfinite(kth) and (kth - nxt) > gap_need
    if gap_applies:
        assert np.array_equal(np.sort(cand[order[:kk]]), chosen), "selection differs despite a clear gap"
        return True
    is_kept = np.isin(cand, chosen)
    worst_kept = np.min((s + t)[is_kept])
    best_dropped = np.max((s - t)[~is_kept])
    assert worst_kept >= best_dropped, "selection not threshold-consistent"
    return False


# ----------------------------------------------------------------------------- top-k under rounding
def count_greater(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """For each t: the number of u with (a_u, -u) > (b_t, -t), i.e. entries
    that rank above position t's value b_t in a top-k by (value descending,
    index ascending).  u = t is counted when a_t > b_t."""
    n = a.shape[0]
    idx = np.arange(n)
    val = np.concatenate([a, b]).astype(np.float64)
    neg = np.concatenate([-idx, -idx])
    typ = np.concatenate([np.zeros(n, np.int64), np.ones(n, np.int64)])
    # ascending by (value, -index, type): an a-entry equal to a b-entry sorts
    # before it, so every a-entry after a b-entry is strictly greater
    order = np.lexsort((typ, neg, val))
    is_a = (typ[order] == 0).astype(np.int64)
    a_after = is_a.sum() - np.cumsum(is_a)
    out = np.empty(n, np.int64)
    bpos = np.nonzero(typ[order] == 1)[0]
    out[order[bpos] - n] = a_after[bpos]
    return out


def topk_status(s: np.ndarray, tol: np.ndarray, k: int):
    """Top-k (value descending, index ascending) of scores known only to lie
    in [s - tol, s + tol].  Returns (sure_in, ambiguous) masks: a sure_in
    entry is in every top-k the rounded scores can give, an entry in neither
    mask is in none, and exactly k - sure_in.sum() of the ambiguous ones are
    chosen."""
    s = np.asarray(s, np.float64)
    tol = np.asarray(tol, np.float64)
    n = s.shape[0]
    if k >= n:
        return np.ones(n, bool), np.zeros(n, bool)
    lo, hi = s - tol, s + tol
    could = count_greater(hi, lo) - (hi > lo)   # others that may rank above
    sure = count_greater(lo, hi)                # others that rank above for certain (lo_t < hi_t)
    sure_in = could < k
    sure_out = sure >= k
    assert not np.any(sure_in & sure_out)
    return sure_in, ~(sure_in | sure_out)


def overlap_range(f_in, f_amb, kf: int, p_in, p_amb, kp: int):
    """Smallest and largest |F & P| over the selections F (all of f_in plus
    kf - |f_in| of f_amb) and P (all of p_in plus kp - |p_in| of p_amb)."""
    f_out = ~(f_in | f_amb)
    p_out = ~(p_in | p_amb)
    rf = kf - int(f_in.sum())
    rp = kp - int(p_in.sum())
    assert 0 <= rf <= int(f_amb.sum()) and 0 <= rp <= int(p_amb.sum())
    SS = int((f_in & p_in).sum())
    SA = int((f_in & p_amb).sum())
    AS = int((f_amb & p_in).sum())
    AA = int((f_amb & p_amb).sum())
    AO = int((f_amb & p_out).sum())
    OA = int((f_out & p_amb).sum())
    lo_best, hi_best = None, None
    for xa in range(min(AA, rf) + 1):
        xs_lo, xs_hi = max(0, rf - xa - AO), min(AS, rf - xa)
        if xs_lo > xs_hi:
            continue
        for ya in range(min(AA, rp) + 1):
            ys_lo, ys_hi = max(0, rp - ya - OA), min(SA, rp - ya)
            if ys_lo > ys_hi:
                continue
            z_lo, z_hi = max(0, xa + ya - AA), min(xa, ya)
            lo = SS + xs_lo + ys_lo + z_lo
            hi = SS + xs_hi + ys_hi + z_hi
            lo_best = lo if lo_best is None else min(lo_best, lo)
            hi_best = hi if hi_best is None else max(hi_best, hi)
    assert lo_best is not None
    return lo_best, hi_best


# fp32 rounding of the calibration scores: the full score is a running fp32
# sum of d exact products (bf16 x bf16), a pair score one rounding of the sum
# of two exact products.  Recursive summation of n terms is within
# gamma_n * sum |terms| of the exact sum, gamma_n = n u / (1 - n u), u = 2^-24.
def gamma(n: int, u: float = 2.0 ** -24) -> float:
    return n * u / (1.0 - n * u)


def calibration_count_bounds(q: np.ndarray, k: np.ndarray, k_cal: int):
    """Admissible per-pair counts [lo, hi] ([Hkv, P] each) of an fp32
    calibration against the oracle's fp64 scores, plus the number of
    (query, pair) overlaps that were ambiguous."""
    from oracle import calibration as C
    Hq, M, d = q.shape
    Hkv, L = k.shape[:2]
    P = d // 2
    grp = Hq // Hkv
    lo = np.zeros((Hkv, P), np.int64)
    hi = np.zeros((Hkv, P), np.int64)
    n_amb = 0
    for h in range(Hq):
        g = h // grp
        ak = np.abs(k[g].astype(np.float64))
        for m in range(M):
            full, pairs = C.calibration_scores(q[h, m], k[g])
            aq = np.abs(q[h, m].astype(np.float64))
            # fp32 bound plus the fp64 oracle's own (far smaller) rounding
            t_full = (gamma(d) + gamma(d, 2.0 ** -53)) * (ak @ aq)
            t_pair = (gamma(2) + gamma(2, 2.0 ** -53)) * (ak[:, :P] * aq[:P] + ak[:, P:] * aq[P:]).T
            f_in, f_amb = topk_status(full, t_full, k_cal)
            for i in range(P):
                p_in, p_amb = topk_status(pairs[i], t_pair[i], k_cal)
                a, b = overlap_range(f_in, f_amb, k_cal, p_in, p_amb, k_cal)
                lo[g, i] += a
                hi[g, i] += b
                n_amb += a != b
    return lo, hi, n_amb
