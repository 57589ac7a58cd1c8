"""fp64 reference definitions of every step of the sparse-attention path.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Everything is
computed in float64 from the stored input values (fp32 and bf16 inputs
convert to fp64 exactly).  Loops run in the order the definitions are
stated; numpy's matmul, sort and exp serve as single steps.

Notation: B batch, Hq / Hkv query / KV heads, query head h reads KV head
h // (Hq/Hkv), S sequence, d head dim, P = d/2 rotary pairs, Bs block size,
N = S/Bs blocks.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

NEG_INF = -np.inf


# ----------------------------------------------------------------------------- RoPE
def rope_frequencies(d: int, theta: float) -> np.ndarray:
    """omega_i = theta ** (-2 i / d) for rotary pair i = 0 .. d/2 - 1.

    FASA sec. 2.A treats RoPE as a set of frequency chunks; Prism sec. 2
    calls the fast-rotating dimensions "high frequency".  Pair 0 is the
    fastest (omega_0 = 1).
    """
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / d)


def rope(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate every pair (i, i + d/2) of ``x[..., S, d]`` by angle p * omega_i.

    Reading: half-split pairing (channels i and i + d/2 form pair i), the
    Llama convention; positions are absolute token positions (FASA sec. 2.B,
    FAC keeps the original absolute positions).
        x'_i       = x_i cos(p w_i) - x_{i+P} sin(p w_i)
        x'_{i+P}   = x_{i+P} cos(p w_i) + x_i sin(p w_i)
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    P = d // 2
    w = rope_frequencies(d, theta)
    ang = np.asarray(positions, dtype=np.float64)[..., :, None] * w  # [S, P]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :P], x[..., P:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# ----------------------------------------------------------------------------- pooling
def band_channels(d: int, split_pair: int) -> list[np.ndarray]:
    """Channel lists of the two bands (Prism sec. 3, item 1).

    High band = rotary pairs [0, split_pair), low band = [split_pair, d/2);
    both channels of every pair belong to its band.  An empty band is dropped,
    so split_pair = 0 or d/2 gives single-band pooling.
    """
    P = d // 2
    out = []
    for lo, hi in ((0, split_pair), (split_pair, P)):
        if hi > lo:
            pairs = np.arange(lo, hi)
            out.append(np.concatenate([pairs, pairs + P]))
    return out


def pool_blocks(x_rot: np.ndarray, block: int, split_pair: int, calibrate: bool) -> np.ndarray:
    """Calibrated dual-band block means of rotated vectors ``x_rot[..., S, d]``.

    Prism sec. 1: block importance is estimated from the mean of each block's
    vectors.  Sec. 3, item 1: the mean is taken separately on a high- and a
    low-frequency band.  Sec. 3, item 2: a temperature from the RMS energy
    density of the vectors restores the logit amplitude that pooling loses.

    Reading (the pages give no formula): per (block, band b)
        m      = (1/Bs) sum_t x'_t[b]
        e_tok  = sqrt( sum_t |x'_t[b]|^2 / (Bs |b|) )     token RMS energy
        e_pool = sqrt( |m|^2 / |b| )                      pooled RMS energy
        m~[b]  = m * e_tok / e_pool     (0 if e_pool == 0)
    so a band logit <m~_q, m~_k> equals <m_q, m_k> divided by the temperature
    tau_q * tau_k with tau = e_pool / e_tok.  With ``calibrate`` false,
    m~ = m.
    """
    x = np.asarray(x_rot, dtype=np.float64)
    S, d = x.shape[-2], x.shape[-1]
    N = S // block
    xb = x.reshape(x.shape[:-2] + (N, block, d))
    m = xb.mean(axis=-2)
    out = np.zeros_like(m)
    for ch in band_channels(d, split_pair):
        mb = m[..., ch]
        if calibrate:
            e_tok = np.sqrt((xb[..., ch] ** 2).sum(axis=(-2, -1)) / (block * ch.size))
            e_pool = np.sqrt((mb ** 2).sum(axis=-1) / ch.size)
            with np.errstate(divide="ignore", invalid="ignore"):
                f = np.where(e_pool > 0, e_tok / e_pool, 0.0)
            out[..., ch] = mb * f[..., None]
        else:
            out[..., ch] = mb
    return out


def block_scores(pq: np.ndarray, pk: np.ndarray, sm_scale: float, causal: bool) -> np.ndarray:
    """s(h, I, J) = sm_scale * <m~_q(h, I), m~_k(g(h), J)>; -inf for J > I if causal.

    Prism sec. 3, item 2 and sec. 5: estimation is a block-level matrix
    product only.  Reading: the calibrated band logits are summed, which is
    the single dot product over all channels of the calibrated vectors.
    pq: [B, Hq, N, d], pk: [B, Hkv, N, d] -> [B, Hq, N, N].
    """
    B, Hq, N, d = pq.shape
    Hkv = pk.shape[1]
    grp = Hq // Hkv
    s = np.empty((B, Hq, N, N))
    for b in range(B):
        for h in range(Hq):
            s[b, h] = sm_scale * (pq[b, h] @ pk[b, h // grp].T)
    if causal:
        I, J = np.meshgrid(np.arange(N), np.arange(N), indexing="ij")
        s[..., J > I] = NEG_INF
    return s


# ----------------------------------------------------------------------------- selection
def keep_budget(N: int, keep_const: int = 0, keep_percent: int = 0) -> list[int]:
    """Top-k size per query block I: a constant, or ceil(percent/100 * (I + 1)).

    Reading: a keep budget of "p% of blocks" counts the causally visible
    blocks of query block I; forced blocks come on top of it.  Exact
    rational arithmetic.
    """
    if keep_const:
        return [keep_const] * N
    out = []
    for I in range(N):
        q = Fraction(keep_percent, 100) * (I + 1)
        out.append(int(-((-q.numerator) // q.denominator)))
    return out


def _canonical(v: np.ndarray) -> np.ndarray:
    """NaN ranks as -inf and -0 as +0 (deterministic selection)."""
    v = np.asarray(v, dtype=np.float64)
    v = np.where(np.isnan(v), NEG_INF, v)
    return np.where(v == 0, 0.0, v)


def select_row(scores: np.ndarray, valid_len: int, k: int, n_sink: int, n_local: int) -> np.ndarray:
    """Indices kept for one row, ascending.

    Prism sec. 1 keeps a subset of relevant blocks; FASA sec. 2.B selects a
    critical token subset T_t from the predicted importance.  Reading:
    forced = sink columns [0, n_sink) and the last n_local valid columns;
    from the other valid columns take the min(k, count) best by
    (score descending, index ascending); return forced plus those, sorted.
    """
    valid_len = int(valid_len)
    forced = set(range(min(n_sink, valid_len))) | set(range(max(0, valid_len - n_local), valid_len))
    is_cand = np.ones(valid_len, dtype=bool)
    is_cand[sorted(forced)] = False
    cand = np.nonzero(is_cand)[0].astype(np.int64)
    keys = _canonical(np.asarray(scores)[cand])
    order = np.lexsort((cand, -keys))  # primary: score desc; secondary: index asc
    take = cand[order[: max(0, min(k, cand.size))]]
    return np.array(sorted(forced | set(int(t) for t in take)), dtype=np.int64)


def select_rows(scores: np.ndarray, valid_len, k, n_sink: int, n_local: int) -> list[np.ndarray]:
    """select_row over the rows of a 2-D score array; valid_len / k per row or scalar."""
    rows = scores.shape[0]
    vl = np.broadcast_to(np.asarray(valid_len), (rows,))
    kk = np.broadcast_to(np.asarray(k), (rows,))
    return [select_row(scores[r], int(vl[r]), int(kk[r]), n_sink, n_local) for r in range(rows)]


# ----------------------------------------------------------------------------- prefill attention
def prefill_attention(q_rot, k_rot, v, sel, block: int, sm_scale: float, causal: bool):
    """Block-sparse softmax attention (Prism sec. 1: attention only over the
    selected key blocks).

    For a query at position t in block I of head h, the key set is the union
    of the selected blocks J in sel[b][h][I]; with ``causal`` only keys s <= t
    count (inside the diagonal block this is a token-level mask).  Keys and
    values come from KV head h // (Hq/Hkv).
        l_s = sm_scale <q'_t, k'_s>,   o_t = sum_s softmax(l)_s v_s,
        lse_t = log sum_s exp(l_s)
    A query with no key gets o = 0 and lse = -inf.
    Returns (out [B, Hq, S, d], lse [B, Hq, S]).
    """
    B, Hq, S, d = q_rot.shape
    Hkv = k_rot.shape[1]
    grp = Hq // Hkv
    N = S // block
    out = np.zeros((B, Hq, S, d))
    lse = np.full((B, Hq, S), NEG_INF)
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            for I in range(N):
                blocks = np.asarray(sel[b][h][I], dtype=np.int64)
                if blocks.size == 0:
                    continue
                keys = np.concatenate([np.arange(J * block, (J + 1) * block) for J in blocks])
                qs = np.arange(I * block, (I + 1) * block)
                logits = sm_scale * (q_rot[b, h, qs] @ k_rot[b, g, keys].T)
                if causal:
                    logits = np.where(keys[None, :] <= qs[:, None], logits, NEG_INF)
                mx = logits.max(axis=1)
                has = np.isfinite(mx)
                safe = np.where(has, mx, 0.0)
                p = np.exp(logits - safe[:, None])
                den = p.sum(axis=1)
                o = (p @ v[b, g, keys]) / np.where(has, den, 1.0)[:, None]
                out[b, h, qs] = np.where(has[:, None], o, 0.0)
                lse[b, h, qs] = np.where(has, safe + np.log(np.where(has, den, 1.0)), NEG_INF)
    return out, lse


# ----------------------------------------------------------------------------- decode
def decode_query(q: np.ndarray, cache_len: np.ndarray, theta: float) -> np.ndarray:
    """Rotate the decode query q[B, Hq, d] at position cache_len[b] - 1.

    Reading: the cache holds the keys of positions 0 .. L_b - 1, the newest
    token (the one decoding) at L_b - 1 (FASA sec. 2.B, original positions).
    """
    out = np.empty(q.shape, dtype=np.float64)
    for b in range(q.shape[0]):
        pos = np.array([int(cache_len[b]) - 1])
        out[b] = rope(q[b][:, None, :], pos, theta)[:, 0, :]
    return out


def token_scores(q_rot, k_cache, dom_pairs, cache_len, sm_scale: float) -> np.ndarray:
    """Token Importance Predictor (FASA sec. 2.B, item 1).

    Scores use only the dominant frequency chunks of the query head's KV
    head: s(b, h, t) = sm_scale * sum_{i in D_g} (q_i k_{t,i} + q_{i+P} k_{t,i+P})
    for t < L_b, -inf for L_b <= t < Lmax.  ``k_cache`` [B, Hkv, Lmax, d] holds
    rotated keys; ``dom_pairs`` [Hkv, n_dom].
    """
    B, Hq, d = q_rot.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    grp = Hq // Hkv
    P = d // 2
    s = np.full((B, Hq, Lmax), NEG_INF)
    for b in range(B):
        L = int(cache_len[b])
        for h in range(Hq):
            g = h // grp
            D = np.asarray(dom_pairs[g], dtype=np.int64)
            ch = np.concatenate([D, D + P])
            s[b, h, :L] = sm_scale * (k_cache[b, g, :L][:, ch] @ q_rot[b, h, ch])
    return s


def decode_attention(q_rot, k_cache, v_cache, sel, sm_scale: float):
    """Focused Attention Computation (FASA sec. 2.B, item 2): full-dimension
    softmax attention over the selected tokens only, at their original
    positions (the cache already holds rotated keys).

    sel[b][h] = selected token indices.  Returns (out [B, Hq, d], lse [B, Hq]).
    """
    B, Hq, d = q_rot.shape
    Hkv = k_cache.shape[1]
    grp = Hq // Hkv
    out = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), NEG_INF)
    for b in range(B):
        for h in range(Hq):
            t = np.asarray(sel[b][h], dtype=np.int64)
            if t.size == 0:
                continue
            g = h // grp
            logits = sm_scale * (k_cache[b, g, t] @ q_rot[b, h])
            mx = logits.max()
            p = np.exp(logits - mx)
            out[b, h] = (p @ v_cache[b, g, t]) / p.sum()
            lse[b, h] = mx + np.log(p.sum())
    return out, lse


def standard_to_slab(k_cache: np.ndarray, dom_pairs: np.ndarray):
    """Split a standard K cache into the dominant slab and the rest.

    FASA sec. 2.C (computation-optimised variant): only a sparse subset of
    the key states is read when scoring.  Layout reading: slab channel j <
    n_dom holds channel D[j], channel n_dom + j holds D[j] + P; the rest slab
    holds every other channel in ascending order.
    """
    B, Hkv, L, d = k_cache.shape
    P = d // 2
    n = dom_pairs.shape[1]
    k_dom = np.empty((B, Hkv, L, 2 * n), k_cache.dtype)
    k_rest = np.empty((B, Hkv, L, d - 2 * n), k_cache.dtype)
    for g in range(Hkv):
        D = np.asarray(dom_pairs[g], dtype=np.int64)
        dom_ch = np.concatenate([D, D + P])
        rest = np.array([c for c in range(d) if c not in set(dom_ch.tolist())], dtype=np.int64)
        k_dom[:, g] = k_cache[:, g][..., dom_ch]
        k_rest[:, g] = k_cache[:, g][..., rest]
    return k_dom, k_rest


def slab_to_standard(k_dom: np.ndarray, k_rest: np.ndarray, dom_pairs: np.ndarray) -> np.ndarray:
    """Inverse of :func:`standard_to_slab`."""
    B, Hkv, L, nd = k_dom.shape
    d = nd + k_rest.shape[-1]
    P = d // 2
    out = np.empty((B, Hkv, L, d), k_dom.dtype)
    for g in range(Hkv):
        D = np.asarray(dom_pairs[g], dtype=np.int64)
        dom_ch = np.concatenate([D, D + P])
        rest = np.array([c for c in range(d) if c not in set(dom_ch.tolist())], dtype=np.int64)
        out[:, g][..., dom_ch] = k_dom[:, g]
        out[:, g][..., rest] = k_rest[:, g]
    return out


# ----------------------------------------------------------------------------- pipelines
def prefill_pipeline(q, k, v, *, theta, block, split_pair, calibrate, sm_scale, causal,
                     budget, n_sink, n_local, q_heads=None, group=None):
    """Whole prefill path from stored (pre-rotation) Q, K, V.

    Rotation at positions 0 .. S-1, calibrated dual-band pooling, block
    scores, per-row selection (row I sees I + 1 causal blocks, or all N when
    not causal) and block-sparse attention.  ``q_heads`` names the global
    query-head index of each row of ``q`` (for sampled runs with a subset of
    heads) and ``group`` the query heads per KV head (default: nh / Hkv of
    the arrays given); ``budget`` is the top-k per query block.
    Returns dict(q_rot, k_rot, pq, pk, scores, sel, out, lse).
    """
    B, nh, S, d = q.shape
    Hkv = k.shape[1]
    if q_heads is None:
        q_heads = list(range(nh))
    pos = np.arange(S)
    q_rot = rope(q, pos, theta)
    k_rot = rope(k, pos, theta)
    pq = pool_blocks(q_rot, block, split_pair, calibrate)
    pk = pool_blocks(k_rot, block, split_pair, calibrate)
    N = S // block
    grp = group if group is not None else max(1, nh // Hkv)
    scores = np.empty((B, nh, N, N))
    for i, h in enumerate(q_heads):
        scores[:, i] = block_scores(pq[:, i:i + 1], pk[:, h // grp:h // grp + 1], sm_scale, causal)[:, 0]
    sel = []
    for b in range(B):
        per_h = []
        for i in range(nh):
            vl = np.arange(1, N + 1) if causal else np.full(N, N)
            per_h.append(select_rows(scores[b, i], vl, np.asarray(budget), n_sink, n_local))
        sel.append(per_h)
    # attention per head, with the right KV head
    out = np.zeros((B, nh, S, d))
    lse = np.full((B, nh, S), NEG_INF)
    for i, h in enumerate(q_heads):
        g = h // grp
        o, l = prefill_attention(q_rot[:, i:i + 1], k_rot[:, g:g + 1], v[:, g:g + 1],
                                 [[sel[b][i]] for b in range(B)], block, sm_scale, causal)
        out[:, i], lse[:, i] = o[:, 0], l[:, 0]
    return dict(q_rot=q_rot, k_rot=k_rot, pq=pq, pk=pk, scores=scores, sel=sel, out=out, lse=lse)


def decode_pipeline(q_raw, k_cache, v_cache, cache_len, dom_pairs, *, theta, k, sm_scale):
    """Whole decode step: rotate q at L_b - 1, TIP scores, top-k, FAC attention.

    Returns dict(q_rot, scores, sel, out, lse).
    """
    q_rot = decode_query(q_raw, cache_len, theta)
    s = token_scores(q_rot, k_cache, dom_pairs, cache_len, sm_scale)
    B, Hq = q_rot.shape[:2]
    sel = [[select_row(s[b, h], int(cache_len[b]), k, 0, 0) for h in range(Hq)] for b in range(B)]
    out, lse = decode_attention(q_rot, k_cache, v_cache, sel, sm_scale)
    return dict(q_rot=q_rot, scores=s, sel=sel, out=out, lse=lse)
