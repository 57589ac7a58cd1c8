"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each check below ties one oracle function to something fixed independently:
a textbook or library routine in a special case, a closed form, an
invariant, brute force on a tiny input, or planted structure.  The
``test_planted_*`` tests at the end put a plausible mistake into the oracle
(on the CPU) and require that at least one pin catches it.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import sparse_attention as sa
from synth import workloads as W
import synth

def _gauss(shape, seed):
    return synth.gaussian_tensor(seed, 9, shape, "f32").astype(np.float64)


# ----------------------------------------------------------------------------- V5 RoPE
def check_rope_complex_form(d=64, theta=1e4, S=300):
    """RoPE written as complex multiplication z_i * exp(1j * p * omega_i) with
    z_i = x_i + 1j x_{i+P} (RoFormer's complex form), omega_i from the
    geometric progression theta^(-2i/d) built by repeated multiplication."""
    x = _gauss((S, d), 1)
    pos = np.arange(S) * 7 + 3
    P = d // 2
    ratio = theta ** (-2.0 / d)
    omega = np.array([ratio ** i for i in range(P)])
    z = x[:, :P] + 1j * x[:, P:]
    zr = z * np.exp(1j * pos[:, None] * omega[None, :])
    ref = np.concatenate([zr.real, zr.imag], axis=1)
    got = sa.rope(x, pos, theta)
    assert np.allclose(got, ref, rtol=0, atol=1e-11), np.abs(got - ref).max()


def check_rope_invariants(d=128, theta=5e5):
    x = _gauss((64, d), 2)
    y = _gauss((64, d), 3)
    P = d // 2
    pos = np.arange(64) * 2047 + 5
    xr = sa.rope(x, pos, theta)
    # per-pair norm is preserved
    n0 = x[:, :P] ** 2 + x[:, P:] ** 2
    n1 = xr[:, :P] ** 2 + xr[:, P:] ** 2
    assert np.allclose(n0, n1, rtol=1e-12, atol=1e-12)
    # position 0 is the identity
    assert np.array_equal(sa.rope(x, np.zeros(64), theta), x)
    # shift invariance: <R(t) q, R(s) k> = <R(t - s) q, k>
    t, s = 131071, 70001
    lhs = np.sum(sa.rope(x, np.full(64, t), theta) * sa.rope(y, np.full(64, s), theta), axis=1)
    rhs = np.sum(sa.rope(x, np.full(64, t - s), theta) * y, axis=1)
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-9), np.abs(lhs - rhs).max()


def test_v5_rope_complex_form():
    check_rope_complex_form()
    check_rope_complex_form(d=128, theta=5e5, S=64)


def test_v5_rope_invariants():
    check_rope_invariants()


# ----------------------------------------------------------------------------- V2a pooling
def _brute_block_score(q_rot_block, k_rot_block, split, calibrate, scale):
    """Score of one (query block, key block) pair from token-level sums only."""
    Bs, d = q_rot_block.shape
    P = d // 2
    bands = []
    if split > 0:
        bands.append(list(range(0, split)) + list(range(P, P + split)))
    if split < P:
        bands.append(list(range(split, P)) + list(range(P + split, 2 * P)))
    total = 0.0
    for ch in bands:
        # <mean q, mean k> = average over the Bs^2 token pairs
        cross = 0.0
        for t in range(Bs):
            for s in range(Bs):
                cross += float(np.dot(q_rot_block[t, ch], k_rot_block[s, ch]))
        cross /= Bs * Bs
        if calibrate:
            def energies(xb):
                tok = sum(float(np.dot(xb[t, ch], xb[t, ch])) for t in range(Bs)) / (Bs * len(ch))
                gram = 0.0
                for t in range(Bs):
                    for u in range(Bs):
                        gram += float(np.dot(xb[t, ch], xb[u, ch]))
                pool = gram / (Bs * Bs) / len(ch)
                return math.sqrt(tok), math.sqrt(pool)
            tq, pq = energies(q_rot_block)
            tk, pk = energies(k_rot_block)
            cross *= (tq * tk) / (pq * pk)
        total += cross
    return scale * total


@pytest.mark.parametrize("split,calibrate", [(0, 0), (8, 0), (8, 1), (32, 1), (0, 1)])
def test_v2a_pooled_score_brute_force(split, calibrate):
    d, Bs, N = 64, 16, 4
    S = Bs * N
    q = _gauss((1, 4, S, d), 4)
    k = _gauss((1, 2, S, d), 5)
    pos = np.arange(S)
    qr, kr = sa.rope(q, pos, 1e4), sa.rope(k, pos, 1e4)
    pq = sa.pool_blocks(qr, Bs, split, calibrate)
    pk = sa.pool_blocks(kr, Bs, split, calibrate)
    s = sa.block_scores(pq, pk, 0.125, causal=True)
    for h in range(4):
        for I in range(N):
            for J in range(N):
                if J > I:
                    assert s[0, h, I, J] == -np.inf
                    continue
                ref = _brute_block_score(qr[0, h, I * Bs:(I + 1) * Bs],
                                         kr[0, h // 2, J * Bs:(J + 1) * Bs], split, calibrate, 0.125)
                assert abs(s[0, h, I, J] - ref) <= 1e-12 * max(1.0, abs(ref)), (h, I, J)


# ----------------------------------------------------------------------------- V3 band collapse
def dirichlet_pooled(c, t0, Bs, omega):
    """Closed form of the block mean of a constant pair c rotated at t0..t0+Bs-1.

    Geometric series: (1/Bs) sum_t exp(i t w) = exp(i (t0 + (Bs-1)/2) w)
    * sin(Bs w / 2) / (Bs sin(w / 2)).
    """
    amp = np.sin(Bs * omega / 2) / (Bs * np.sin(omega / 2))
    return c * np.exp(1j * (t0 + (Bs - 1) / 2.0) * omega) * amp


@pytest.mark.parametrize("cfg", [W.C1, W.C2])
def test_v3_band_collapse_closed_form(cfg):
    d, Bs, split = cfg.d, cfg.block, cfg.band_split_pair
    P = d // 2
    c = _gauss((d,), 6)
    t0 = 5 * Bs
    S = 6 * Bs
    x = np.broadcast_to(c, (S, d)).copy()
    pooled = sa.pool_blocks(sa.rope(x, np.arange(S), cfg.theta), Bs, split, calibrate=False)[5]
    ratio = cfg.theta ** (-2.0 / d)
    omega = np.array([ratio ** i for i in range(P)])
    ref = dirichlet_pooled(c[:P] + 1j * c[P:], t0, Bs, omega)
    got = pooled[:P] + 1j * pooled[P:]
    assert np.allclose(got, ref, rtol=0, atol=1e-12)
    # the pages' claim: high-frequency pairs collapse, low-frequency pairs survive
    amp2 = (np.sin(Bs * omega / 2) / (Bs * np.sin(omega / 2))) ** 2
    high, low = amp2[:split].mean(), amp2[split:].mean()
    expect = {W.C1.name: (0.271, 0.995), W.C2.name: (0.0068, 0.921)}[cfg.name]
    assert abs(high - expect[0]) < 5e-3 * max(1, expect[0] * 10) and abs(low - expect[1]) < 5e-3
    e = np.abs(got) ** 2 / np.abs(c[:P] + 1j * c[P:]) ** 2
    assert np.allclose(e, amp2, rtol=1e-9)
    assert e[:split].mean() < 0.3 and e[split:].mean() > 0.9


def test_v3_calibration_restores_band_energy():
    """With calibration the pooled band RMS equals the token band RMS."""
    d, Bs, split = 128, 128, 16
    x = _gauss((2 * Bs, d), 7)
    xr = sa.rope(x, np.arange(2 * Bs), 5e5)
    m = sa.pool_blocks(xr, Bs, split, calibrate=True)
    for ch in sa.band_channels(d, split):
        for blk in range(2):
            tok = np.sqrt((xr[blk * Bs:(blk + 1) * Bs][:, ch] ** 2).mean())
            pool = np.sqrt((m[blk, ch] ** 2).mean())
            assert abs(tok - pool) < 1e-12


# ----------------------------------------------------------------------------- V7 band extremes
def test_v7_band_extremes_single_band():
    d, Bs = 64, 32
    x = _gauss((1, 1, 4 * Bs, d), 8)
    xr = sa.rope(x, np.arange(4 * Bs), 1e4)
    a = sa.pool_blocks(xr, Bs, 0, True)
    b = sa.pool_blocks(xr, Bs, d // 2, True)
    assert np.array_equal(a, b)
    # single band: m * e_tok / e_pool over all channels, computed per block with plain loops
    for blk in range(4):
        rows = xr[0, 0, blk * Bs:(blk + 1) * Bs]
        m = [sum(rows[t, c] for t in range(Bs)) / Bs for c in range(d)]
        e_tok = math.sqrt(sum(rows[t, c] ** 2 for t in range(Bs) for c in range(d)) / (Bs * d))
        e_pool = math.sqrt(sum(v * v for v in m) / d)
        ref = np.array(m) * e_tok / e_pool
        assert np.allclose(a[0, 0, blk], ref, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------- V2b top-k
def _sort_reference(scores, valid_len, k, n_sink, n_local):
    """Full sort with Python's stable ``sorted`` on (-score, index)."""
    forced = {j for j in range(valid_len) if j < n_sink or j >= valid_len - n_local}

    def canon(v):
        v = float(v)
        if v != v:
            return -math.inf
        return 0.0 if v == 0.0 else v
    cand = [j for j in range(valid_len) if j not in forced]
    ranked = sorted(cand, key=lambda j: (-canon(scores[j]), j))
    return sorted(forced | set(ranked[:min(k, len(ranked))]))


def _tricky_rows(rows, cols, seed):
    g = np.random.default_rng(seed)
    s = g.standard_normal((rows, cols)).astype(np.float32).astype(np.float64)
    s[:, ::7] = np.round(s[:, ::7])              # many exact ties
    s[0, :] = 1.0                                  # all equal
    s[1, ::3] = np.nan
    s[2, ::2] = -0.0
    s[2, 1::2] = 0.0
    s[3, ::5] = -np.inf
    s[4, :] = -np.inf
    return s


@pytest.mark.parametrize("cols,k,n_sink,n_local", [(37, 5, 1, 2), (64, 0, 0, 0), (100, 100, 2, 3),
                                                   (257, 31, 1, 1), (1000, 64, 0, 0)])
def test_v2b_selection_vs_full_sort(cols, k, n_sink, n_local):
    s = _tricky_rows(12, cols, cols)
    g = np.random.default_rng(cols + 1)
    for r in range(12):
        vl = int(g.integers(0, cols + 1)) if r > 5 else cols
        got = sa.select_row(s[r], vl, k, n_sink, n_local)
        ref = _sort_reference(s[r], vl, k, n_sink, n_local)
        assert got.tolist() == ref, (r, vl)
        assert np.all(np.diff(got) > 0)


def test_keep_budget_exact_ceiling():
    b = sa.keep_budget(256, keep_percent=10)
    assert b[0] == 1 and b[9] == 1 and b[10] == 2 and b[29] == 3 and b[255] == 26
    b = sa.keep_budget(1024, keep_percent=5)
    assert b[19] == 1 and b[20] == 2 and b[1023] == 52
    assert sa.keep_budget(8, keep_const=4) == [4] * 8


# ----------------------------------------------------------------------------- V1 / V2c attention
def _sdpa(q, k, v, mask=None, causal=False):
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=None if mask is None else torch.from_numpy(mask), is_causal=causal)
    return out.numpy()


def test_v1_selected_all_equals_dense_causal():
    B, Hq, Hkv, S, d, Bs = 1, 4, 2, 256, 64, 32
    N = S // Bs
    q = _gauss((B, Hq, S, d), 10)
    k = _gauss((B, Hkv, S, d), 11)
    v = _gauss((B, Hkv, S, d), 12)
    sel = [[[list(range(I + 1)) for I in range(N)] for _ in range(Hq)]]
    out, lse = sa.prefill_attention(q, k, v, sel, Bs, d ** -0.5, causal=True)
    kk = np.repeat(k, Hq // Hkv, axis=1)
    vv = np.repeat(v, Hq // Hkv, axis=1)
    ref = _sdpa(q, kk, vv, causal=True)
    assert np.allclose(out, ref, rtol=0, atol=1e-12)
    logits = np.einsum("bhtd,bhsd->bhts", q, kk) * d ** -0.5
    logits = np.where(np.tril(np.ones((S, S), bool)), logits, -np.inf)
    assert np.allclose(lse, scipy.special.logsumexp(logits, axis=-1), atol=1e-12)


def test_v2c_sparse_attention_vs_masked_dense():
    B, Hq, Hkv, S, d, Bs = 2, 2, 1, 192, 32, 16
    N = S // Bs
    q = _gauss((B, Hq, S, d), 13)
    k = _gauss((B, Hkv, S, d), 14)
    v = _gauss((B, Hkv, S, d), 15)
    g = np.random.default_rng(0)
    sel = [[[sorted(set(g.choice(I + 1, size=min(I + 1, 3), replace=False).tolist()) | {I})
             for I in range(N)] for _ in range(Hq)] for _ in range(B)]
    out, _ = sa.prefill_attention(q, k, v, sel, Bs, d ** -0.5, causal=True)
    for b in range(B):
        for h in range(Hq):
            mask = np.zeros((S, S), bool)
            for I in range(N):
                for J in sel[b][h][I]:
                    mask[I * Bs:(I + 1) * Bs, J * Bs:(J + 1) * Bs] = True
            mask &= np.tril(np.ones((S, S), bool))
            ref = _sdpa(q[b, h][None], k[b, 0][None], v[b, 0][None], mask=mask[None])[0]
            assert np.allclose(out[b, h], ref, atol=1e-12)


def test_prefill_non_causal_and_empty_selection():
    S, d, Bs = 64, 16, 16
    q, k, v = _gauss((1, 1, S, d), 16), _gauss((1, 1, S, d), 17), _gauss((1, 1, S, d), 18)
    sel = [[[[0, 3], [], [1, 2, 3], [3]]]]
    out, lse = sa.prefill_attention(q, k, v, sel, Bs, 0.25, causal=False)
    assert np.all(out[0, 0, Bs:2 * Bs] == 0) and np.all(lse[0, 0, Bs:2 * Bs] == -np.inf)
    mask = np.zeros((S, S), bool)
    for I, blocks in enumerate(sel[0][0]):
        for J in blocks:
            mask[I * Bs:(I + 1) * Bs, J * Bs:(J + 1) * Bs] = True
    rows = np.r_[0:Bs, 2 * Bs:S]
    ref = _sdpa(q[0, 0, rows][None], k[0, 0][None], v[0, 0][None], mask=mask[rows][None])[0]
    # sdpa scales by 1/sqrt(d) = 0.25 for d = 16
    assert np.allclose(out[0, 0, rows], ref, atol=1e-12)


# ----------------------------------------------------------------------------- V6 FASA reduction
def test_v6_all_pairs_dominant_gives_full_logits_and_dense_decode():
    B, Hq, Hkv, L, d = 2, 4, 2, 300, 64
    q = _gauss((B, Hq, d), 20)
    kc = _gauss((B, Hkv, L, d), 21)
    vc = _gauss((B, Hkv, L, d), 22)
    lens = np.array([300, 171])
    dom = np.tile(np.arange(d // 2), (Hkv, 1))
    qr = sa.decode_query(q, lens, 5e5)
    s = sa.token_scores(qr, kc, dom, lens, d ** -0.5)
    for b in range(B):
        for h in range(Hq):
            ref = [float(np.dot(qr[b, h], kc[b, h // 2, t])) * d ** -0.5 for t in range(lens[b])]
            assert np.allclose(s[b, h, :lens[b]], ref, atol=1e-12)
            assert np.all(s[b, h, lens[b]:] == -np.inf)
    r = sa.decode_pipeline(q, kc, vc, lens, dom, theta=5e5, k=L, sm_scale=d ** -0.5)
    for b in range(B):
        for h in range(Hq):
            n = lens[b]
            ref = _sdpa(qr[b, h][None, None], kc[b, h // 2, :n][None], vc[b, h // 2, :n][None])[0, 0]
            assert np.allclose(r["out"][b, h], ref, atol=1e-12)


def test_decode_query_position():
    q = _gauss((2, 3, 64), 23)
    lens = np.array([10, 4097])
    got = sa.decode_query(q, lens, 1e4)
    for b in range(2):
        assert np.allclose(got[b], sa.rope(q[b], np.full(3, lens[b] - 1), 1e4))


# ----------------------------------------------------------------------------- V8 slab layout
def test_v8_slab_layout_round_trip_and_scores():
    cfg = W.C5.with_(B=2, L=64)
    dom = W.dominant_pairs(cfg)
    k = _gauss((2, cfg.Hkv, 64, cfg.d), 24)
    kd, kr = sa.standard_to_slab(k, dom)
    assert kd.shape[-1] == 2 * cfg.n_dom and kr.shape[-1] == cfg.d - 2 * cfg.n_dom
    assert np.array_equal(sa.slab_to_standard(kd, kr, dom), k)
    P = cfg.d // 2
    for g in range(cfg.Hkv):
        assert np.array_equal(kd[:, g, :, :cfg.n_dom], k[:, g][..., dom[g]])
        assert np.array_equal(kd[:, g, :, cfg.n_dom:], k[:, g][..., dom[g] + P])
    # scores from the slab alone equal the oracle's scores from the full cache
    q = _gauss((2, cfg.Hq, cfg.d), 25)
    lens = np.array([64, 50])
    s = sa.token_scores(q, k, dom, lens, 0.1)
    for b in range(2):
        for h in range(cfg.Hq):
            g = h // cfg.group
            qd = np.concatenate([q[b, h, dom[g]], q[b, h, dom[g] + P]])
            assert np.allclose(s[b, h, :lens[b]], 0.1 * kd[b, g, :lens[b]] @ qd, atol=1e-12)


# ----------------------------------------------------------------------------- V9 recentering
def test_v9_key_recentering_invariance():
    B, Hq, S, d, Bs = 1, 2, 128, 32, 16
    N = S // Bs
    q, k, v = _gauss((B, Hq, S, d), 26), _gauss((B, 1, S, d), 27), _gauss((B, 1, S, d), 28)
    g = np.random.default_rng(3)
    sel = [[[sorted(set(g.choice(I + 1, size=min(I + 1, 2), replace=False).tolist()) | {I})
             for I in range(N)] for _ in range(Hq)]]
    kbar = k.mean(axis=2, keepdims=True)
    o1, l1 = sa.prefill_attention(q, k, v, sel, Bs, d ** -0.5, True)
    o2, l2 = sa.prefill_attention(q, k - kbar, v, sel, Bs, d ** -0.5, True)
    assert np.allclose(o1, o2, atol=1e-12)
    shift = d ** -0.5 * np.einsum("bhsd,bd->bhs", q, kbar[:, 0, 0])
    assert np.allclose(l1 - l2, shift, atol=1e-10)
    # decode
    qd, kc, vc = _gauss((1, 2, d), 29), _gauss((1, 1, 90, d), 30), _gauss((1, 1, 90, d), 31)
    selt = [[list(range(0, 90, 3)), list(range(5, 60))]]
    a, _ = sa.decode_attention(qd, kc, vc, selt, 0.2)
    b_, _ = sa.decode_attention(qd, kc - kc.mean(axis=2, keepdims=True), vc, selt, 0.2)
    assert np.allclose(a, b_, atol=1e-12)


# ----------------------------------------------------------------------------- V4 needle recall
def test_v4_prefill_needle_recall():
    """Every planted needle pair (J, I) is selected in row I by all query heads
    of its group (one KV group of the 32K layer, shortened to 8192 tokens)."""
    cfg = W.C2.with_(S=8192, Hq=4, Hkv=1, needle_pairs=16)
    q, k, v, _ = W.prefill_inputs_host(cfg)
    pos = np.arange(cfg.S)
    pq = sa.pool_blocks(sa.rope(q, pos, cfg.theta), cfg.block, cfg.band_split_pair, True)
    pk = sa.pool_blocks(sa.rope(k, pos, cfg.theta), cfg.block, cfg.band_split_pair, True)
    s = sa.block_scores(pq, pk, cfg.d ** -0.5, True)
    budget = sa.keep_budget(cfg.N, keep_percent=cfg.keep_percent)
    found = total = 0
    for g, J, I, _u in W.prefill_needle_pairs(cfg):
        for h in range(cfg.Hq):
            sel = sa.select_row(s[0, h, I], I + 1, budget[I], cfg.n_sink, cfg.n_local)
            total += 1
            found += int(J in sel)
    assert found == total, (found, total)


def test_v4_decode_needle_recall():
    cfg = W.C4.with_(B=2, L=8192, k=256)
    x = W.decode_inputs_host(cfg)
    r = sa.decode_pipeline(x["q_raw"].astype(np.float64), x["k"].astype(np.float64),
                           x["v"].astype(np.float64), x["lens"], x["dom"], theta=cfg.theta,
                           k=cfg.k, sm_scale=cfg.d ** -0.5)
    for b, h, p in W.decode_needles(cfg, x["lens"]):
        assert p in set(r["sel"][b][h].tolist()), (b, h, p)


def test_c1_needle_report():
    """Tiny fp32 case: single-token needles under mean pooling are reported,
    not asserted (pooling dilutes one token by 1/64)."""
    cfg = W.C1
    q, k, v, _ = W.prefill_inputs_host(cfg)
    r = sa.prefill_pipeline(q, k, v, theta=cfg.theta, block=cfg.block, split_pair=cfg.band_split_pair,
                            calibrate=True, sm_scale=cfg.d ** -0.5, causal=True,
                            budget=sa.keep_budget(cfg.N, keep_const=cfg.keep_const),
                            n_sink=cfg.n_sink, n_local=cfg.n_local)
    last = set(r["sel"][0][0][cfg.N - 1].tolist())
    blocks = [b for b, _ in W.tiny_needle_keys(cfg)]
    print("C1 needle blocks", blocks, "selected in last row:", sorted(last))
    assert len(r["sel"][0][0][cfg.N - 1]) == cfg.keep_const + 2


# ----------------------------------------------------------------------------- planted mistakes
def _fails(fn, *a, **kw):
    try:
        fn(*a, **kw)
    except AssertionError:
        return True
    return False


def test_planted_rope_mistakes_are_caught(monkeypatch):
    good = sa.rope

    def wrong_sign(x, positions, theta):
        y = good(x, -np.asarray(positions), theta)
        return y

    def interleaved(x, positions, theta):
        x = np.asarray(x, dtype=np.float64)
        d = x.shape[-1]
        perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
        inv = np.argsort(perm)
        return good(x[..., perm], positions, theta)[..., inv]

    def wrong_freq(x, positions, theta):
        return good(x, positions, theta ** 0.5)

    for mutant in (wrong_sign, interleaved, wrong_freq):
        monkeypatch.setattr(sa, "rope", mutant)
        assert _fails(check_rope_complex_form) or _fails(check_rope_invariants), mutant.__name__
    monkeypatch.setattr(sa, "rope", good)


def test_planted_pooling_mistakes_are_caught(monkeypatch):
    good = sa.pool_blocks

    def no_calibration(x, block, split, calibrate):
        return good(x, block, split, False)

    def swapped_bands(x, block, split, calibrate):
        d = np.asarray(x).shape[-1]
        return good(x, block, d // 2 - split, calibrate)

    def sum_not_mean(x, block, split, calibrate):
        return good(x, block, split, calibrate) * (block if not calibrate else 1.0) * 1.5

    for mutant in (no_calibration, swapped_bands, sum_not_mean):
        monkeypatch.setattr(sa, "pool_blocks", mutant)
        caught = (_fails(test_v2a_pooled_score_brute_force, 8, 1)
                  or _fails(test_v2a_pooled_score_brute_force, 8, 0)
                  or _fails(test_v3_calibration_restores_band_energy))
        assert caught, mutant.__name__
    monkeypatch.setattr(sa, "pool_blocks", good)


def test_planted_score_and_selection_mistakes_are_caught(monkeypatch):
    good_scores, good_sel = sa.block_scores, sa.select_row

    def no_causal(pq, pk, scale, causal):
        return good_scores(pq, pk, scale, False)

    def wrong_group(pq, pk, scale, causal):
        return good_scores(pq, pk[:, ::-1].copy(), scale, causal)

    for mutant in (no_causal, wrong_group):
        monkeypatch.setattr(sa, "block_scores", mutant)
        assert _fails(test_v2a_pooled_score_brute_force, 8, 1), mutant.__name__
    monkeypatch.setattr(sa, "block_scores", good_scores)

    def ties_high_index(scores, valid_len, k, n_sink, n_local):
        rev = np.asarray(scores)[:valid_len][::-1]
        got = good_sel(rev, valid_len, k, n_local, n_sink)
        return np.sort(valid_len - 1 - got)

    def nan_high(scores, valid_len, k, n_sink, n_local):
        s = np.where(np.isnan(scores), np.inf, scores)
        return good_sel(s, valid_len, k, n_sink, n_local)

    for mutant in (ties_high_index, nan_high):
        monkeypatch.setattr(sa, "select_row", mutant)
        assert _fails(test_v2b_selection_vs_full_sort, 37, 5, 1, 2), mutant.__name__
    monkeypatch.setattr(sa, "select_row", good_sel)


def test_planted_attention_mistakes_are_caught(monkeypatch):
    good = sa.prefill_attention

    def no_token_mask(q, k, v, sel, block, scale, causal):
        return good(q, k, v, sel, block, scale, False)

    def wrong_scale(q, k, v, sel, block, scale, causal):
        return good(q, k, v, sel, block, scale * 1.01, causal)

    for mutant in (no_token_mask, wrong_scale):
        monkeypatch.setattr(sa, "prefill_attention", mutant)
        assert _fails(test_v1_selected_all_equals_dense_causal), mutant.__name__
    monkeypatch.setattr(sa, "prefill_attention", good)

    good_ts = sa.token_scores

    def one_channel_per_pair(q, k, dom, lens, scale):
        q2 = np.array(q, dtype=np.float64)
        q2[..., q2.shape[-1] // 2:] = 0
        return good_ts(q2, k, dom, lens, scale)

    monkeypatch.setattr(sa, "token_scores", one_channel_per_pair)
    assert _fails(test_v6_all_pairs_dominant_gives_full_logits_and_dense_decode)
    monkeypatch.setattr(sa, "token_scores", good_ts)
