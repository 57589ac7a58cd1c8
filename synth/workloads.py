"""The five synthetic workloads and their needle structure.

Shapes follow a Llama-3.1-8B attention layer (32 query heads, 8 KV heads,
head_dim 128).  All values are seeded; every tensor element is an
Irwin-Hall(12) normal variate from :mod:`synth`, except the rows that carry a
planted needle.

Needles are planted in the rotated (post-position-encoding) frame, the frame
the method's scores are computed in:

* prefill needle *pairs*: a vector ``a*u`` (``u`` a random unit vector,
  ``a = sqrt(3*sqrt(d))``) is added to every key of a key block J and to every
  query of a later query block I, so each of the block's token logits gains
  +3 after the 1/sqrt(d) scale;
* the tiny fp32 case plants 4 single needle *keys* equal to
  ``3*sqrt(d)`` times the unit mean direction of the last block's rotated
  queries;
* decode needles are cached keys equal to ``3*sqrt(d)`` times the unit
  direction of one query head's rotated decode query.

Prefill tensors are stored before the position rotation, so a needle is
written into them through the inverse rotation at the token's own position.
That rotation lives here as part of *input construction*; the oracle and the
GPU path each apply their own rotation to whatever is stored.
"""
from __future__ import annotations

import dataclasses
import functools
from dataclasses import dataclass

import numpy as np

from . import (TID_K, TID_NEEDLE, TID_DOM, TID_Q, TID_V, gaussian_f32, gaussian_tensor,
               round_to_bf16, uniform01, uniform_int)


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    dtype: str          # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    S: int
    d: int
    theta: float
    block: int
    band_split_pair: int
    n_sink: int
    n_local: int
    keep_const: int = 0       # constant top-k per query block (if > 0)
    keep_percent: int = 0     # else ceil(keep_percent/100 * (I+1))
    needle_pairs: int = 0     # needle pairs per KV group
    needle_keys: int = 0      # single needle keys (tiny case)
    seed: int = 1
    calibrate: int = 1
    causal: int = 1

    @property
    def N(self) -> int:
        return self.S // self.block

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def with_(self, **kw) -> "PrefillConfig":
        return dataclasses.replace(self, **kw)


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    L: int
    d: int
    theta: float
    n_dom: int
    k: int
    slab: int
    needles_per_head: int = 4
    seed: int = 4
    ragged: int = 0           # if > 0, cache lengths vary in [L - ragged, L]
    full_rows: int = 0        # slab layout: full rotated rows for the attention, not a rest slab

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def with_(self, **kw) -> "DecodeConfig":
        return dataclasses.replace(self, **kw)


C1 = PrefillConfig("tiny causal prefill fp32 (1 head, d=64, seq 512)", "f32", 1, 1, 1, 512, 64,
                   1e4, 64, 16, n_sink=1, n_local=1, keep_const=4, needle_keys=4, seed=1)
C2 = PrefillConfig("Llama-3.1-8B-shaped prefill layer, seq 32768, bf16", "bf16", 1, 32, 8, 32768,
                   128, 5e5, 128, 16, n_sink=1, n_local=2, keep_percent=10, needle_pairs=16, seed=2)
C3 = PrefillConfig("Llama-3.1-8B-shaped prefill layer, seq 131072, bf16", "bf16", 1, 32, 8,
                   131072, 128, 5e5, 128, 16, n_sink=1, n_local=2, keep_percent=5,
                   needle_pairs=64, seed=3)
C4 = DecodeConfig("token-sparse decode, batch 16, KV length 65536, bf16", "bf16", 16, 32, 8,
                  65536, 128, 5e5, n_dom=16, k=2048, slab=0, seed=4)
C5 = DecodeConfig("token-sparse decode, batch 64, KV length 131072, dominant slab + full rows, bf16",
                  "bf16", 64, 32, 8, 131072, 128, 5e5, n_dom=16, k=4096, slab=1, seed=5,
                  full_rows=1)

# the 64K decode workload with the 128K workload's cache layout: the same logical
# K cache (same seed and channels) as C4, stored as the dominant slab plus full rows
C4_SLAB = C4.with_(name="token-sparse decode, batch 16, KV length 65536, dominant slab + full rows, "
                        "bf16", slab=1, full_rows=1)

CONFIGS = {"C1": C1, "C2": C2, "C3": C3, "C4": C4, "C5": C5, "C4_SLAB": C4_SLAB}


# ---------------------------------------------------------------- rotation used to plant
def _inverse_rotate_rows(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rows ``y`` such that rotating ``y`` at ``positions`` gives ``x`` (fp64).

    Half-split pairing: pair i is channels (i, i + d/2), angle pos * theta**(-2i/d).
    """
    d = x.shape[-1]
    half = d // 2
    freq = np.power(float(theta), -2.0 * np.arange(half, dtype=np.float64) / d)
    ang = -np.asarray(positions, dtype=np.float64)[:, None] * freq[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def _forward_rotate_rows(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    return _inverse_rotate_rows(x, -np.asarray(positions, dtype=np.float64), theta)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_to_bf16(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def _unit_gauss(seed: int, base: int, d: int) -> np.ndarray:
    u = gaussian_f32(seed, TID_NEEDLE, np.arange(base, base + d, dtype=np.uint64)).astype(np.float64)
    return u / np.linalg.norm(u)


# ---------------------------------------------------------------- prefill
def prefill_needle_pairs(cfg: PrefillConfig) -> list[tuple[int, int, int, np.ndarray]]:
    """List of (kv_group, key_block J, query_block I, unit vector u)."""
    out = []
    N = cfg.N
    for g in range(cfg.Hkv):
        for p in range(cfg.needle_pairs):
            base = ((g * max(cfg.needle_pairs, 1) + p) << 10)
            J = int(uniform_int(cfg.seed, TID_NEEDLE, np.array([base]), 1, N - 4)[0])
            I = int(uniform_int(cfg.seed, TID_NEEDLE, np.array([base + 1]), J + 3, N - 1)[0])
            u = _unit_gauss(cfg.seed, base + 512, cfg.d)
            out.append((g, J, I, u))
    return out


def tiny_needle_keys(cfg: PrefillConfig) -> list[tuple[int, int]]:
    """(block, offset) of the single needle keys: distinct blocks in 1..N-2."""
    blocks = np.arange(1, cfg.N - 1)
    order = np.argsort(uniform01(cfg.seed, TID_NEEDLE, np.arange(blocks.size, dtype=np.uint64)),
                       kind="stable")
    chosen = np.sort(blocks[order[: cfg.needle_keys]])
    offs = uniform_int(cfg.seed, TID_NEEDLE, 100 + np.arange(cfg.needle_keys, dtype=np.uint64), 0,
                       cfg.block - 1)
    return [(int(b), int(o)) for b, o in zip(chosen, offs)]


def base_rows(cfg, tid: int, n_heads: int, b: int, h: int, rows: np.ndarray, length: int) -> np.ndarray:
    """fp32 generator values of rows ``rows`` of head (b, h) of a [B,H,length,d] tensor."""
    d = cfg.d
    flat = ((b * n_heads + h) * length + np.asarray(rows, dtype=np.int64))[:, None] * d + np.arange(d)
    return gaussian_f32(cfg.seed, tid, flat.astype(np.uint64)).astype(np.float64)


def prefill_patches(cfg: PrefillConfig):
    """Needle rows to write over the generator's prefill tensors.

    Returns a list of (tensor_id, b, head, row_index_array, stored_rows[n, d] fp32).
    Overlapping needles on one row are summed before rounding.
    """
    adds: dict[tuple[int, int, int], np.ndarray] = {}
    d, Bs = cfg.d, cfg.block

    def add(tid, h, blk, vec):
        key = (tid, h, blk)
        adds[key] = adds.get(key, 0.0) + vec

    if cfg.needle_pairs:
        a = np.sqrt(3.0 * np.sqrt(d))
        for g, J, I, u in prefill_needle_pairs(cfg):
            add(TID_K, g, J, a * u)
            for hq in range(g * cfg.group, (g + 1) * cfg.group):
                add(TID_Q, hq, I, a * u)
    patches = []
    for b in range(cfg.B):
        for (tid, h, blk), vec in sorted(adds.items(), key=lambda kv: kv[0]):
            rows = np.arange(blk * Bs, (blk + 1) * Bs)
            n_heads = cfg.Hq if tid == TID_Q else cfg.Hkv
            base = base_rows(cfg, tid, n_heads, b, h, rows, cfg.S)
            planted = base + _inverse_rotate_rows(np.broadcast_to(vec, (Bs, d)), rows, cfg.theta)
            patches.append((tid, b, h, rows, _store(planted, cfg.dtype)))
    if cfg.needle_keys:
        # needle direction: unit mean of the last block's rotated queries (head 0 of each group)
        for b in range(cfg.B):
            for g in range(cfg.Hkv):
                hq = g * cfg.group
                last = np.arange((cfg.N - 1) * Bs, cfg.N * Bs)
                qrows = _store(base_rows(cfg, TID_Q, cfg.Hq, b, hq, last, cfg.S), cfg.dtype)
                qrot = _forward_rotate_rows(qrows.astype(np.float64), last, cfg.theta)
                mean = qrot.mean(axis=0)
                target = 3.0 * np.sqrt(d) * mean / np.linalg.norm(mean)
                for blk, off in tiny_needle_keys(cfg):
                    row = np.array([blk * Bs + off])
                    planted = _inverse_rotate_rows(target[None, :], row, cfg.theta)
                    patches.append((TID_K, b, g, row, _store(planted, cfg.dtype)))
    return patches


def prefill_inputs_host(cfg: PrefillConfig, q_heads=None):
    """Stored Q, K, V (fp32 arrays holding the stored values) on the host.

    ``q_heads``: optional list of query heads to generate (the KV heads they
    read are generated in full); returns (q[B, len(q_heads), S, d], k, v, q_heads).
    """
    if q_heads is None:
        q_heads = list(range(cfg.Hq))
    kv_heads = sorted({h // cfg.group for h in q_heads})
    shape_q = (cfg.B, len(q_heads), cfg.S, cfg.d)
    q = np.empty(shape_q, np.float32)
    for i, h in enumerate(q_heads):
        for b in range(cfg.B):
            base = ((b * cfg.Hq + h) * cfg.S) * cfg.d
            q[b, i] = gaussian_tensor(cfg.seed, TID_Q, (cfg.S, cfg.d), cfg.dtype, base)
    k = np.zeros((cfg.B, cfg.Hkv, cfg.S, cfg.d), np.float32)
    v = np.zeros_like(k)
    for g in kv_heads:
        for b in range(cfg.B):
            base = ((b * cfg.Hkv + g) * cfg.S) * cfg.d
            k[b, g] = gaussian_tensor(cfg.seed, TID_K, (cfg.S, cfg.d), cfg.dtype, base)
            v[b, g] = gaussian_tensor(cfg.seed, TID_V, (cfg.S, cfg.d), cfg.dtype, base)
    pos_of = {h: i for i, h in enumerate(q_heads)}
    for tid, b, h, rows, vals in prefill_patches(cfg):
        if tid == TID_Q and h in pos_of:
            q[b, pos_of[h], rows] = vals
        elif tid == TID_K and h in kv_heads:
            k[b, h, rows] = vals
    return q, k, v, q_heads


def keep_budget(cfg: PrefillConfig) -> np.ndarray:
    """Top-k size per query block I, as exact integers."""
    I = np.arange(cfg.N, dtype=np.int64)
    if cfg.keep_const:
        return np.full(cfg.N, cfg.keep_const, np.int64)
    return (cfg.keep_percent * (I + 1) + 99) // 100


# ---------------------------------------------------------------- decode
def dominant_pairs(cfg: DecodeConfig) -> np.ndarray:
    """[Hkv, n_dom] ascending distinct rotary-pair indices per KV head."""
    P = cfg.d // 2
    out = np.empty((cfg.Hkv, cfg.n_dom), np.int32)
    for g in range(cfg.Hkv):
        u = uniform01(cfg.seed, TID_DOM, np.arange(g * P, (g + 1) * P, dtype=np.uint64))
        out[g] = np.sort(np.argsort(u, kind="stable")[: cfg.n_dom])
    return out


def slab_channels(dom: np.ndarray, d: int) -> tuple[np.ndarray, np.ndarray]:
    """Channel maps of the dominant-slab layout for one KV head.

    slab channel j < n_dom holds channel dom[j]; j >= n_dom holds
    dom[j - n_dom] + d/2.  The rest slab holds all other channels ascending.
    """
    P = d // 2
    dom_ch = np.concatenate([dom, dom + P]).astype(np.int64)
    rest = np.setdiff1d(np.arange(d), dom_ch)
    return dom_ch, rest


def cache_lengths(cfg: DecodeConfig) -> np.ndarray:
    if not cfg.ragged:
        return np.full(cfg.B, cfg.L, np.int32)
    r = uniform_int(cfg.seed, TID_NEEDLE, (1 << 30) + np.arange(cfg.B, dtype=np.uint64),
                    cfg.L - cfg.ragged, cfg.L)
    r[0] = cfg.L
    return r.astype(np.int32)


def decode_needles(cfg: DecodeConfig, lens: np.ndarray) -> list[tuple[int, int, int]]:
    """(b, q_head, position) of every needle token; positions distinct per (b, group)."""
    out = []
    for b in range(cfg.B):
        for g in range(cfg.Hkv):
            n = cfg.needles_per_head * cfg.group
            if n == 0:
                continue
            base = (1 << 32) + ((b * cfg.Hkv + g) << 12)
            hi = int(lens[b]) - 2
            pos = []
            j = 0
            while len(pos) < n:
                p = int(uniform_int(cfg.seed, TID_NEEDLE, np.array([base + j]), 0, hi)[0])
                j += 1
                if p not in pos:
                    pos.append(p)
            for i, p in enumerate(pos):
                out.append((b, g * cfg.group + i // cfg.needles_per_head, p))
    return out


def decode_inputs_host(cfg: DecodeConfig, batches=None, kv_heads=None):
    """Stored decode inputs on the host for batch rows ``batches``.

    Returns dict with q_raw[nb, Hq, d], k[nb, Hkv, L, d] (standard layout,
    already rotated), v[nb, Hkv, L, d], lens[nb], dom[Hkv, n_dom], batches.
    With ``kv_heads`` only those KV heads' caches are generated (the others
    stay zero), for sampled checks of large workloads.
    """
    if batches is None:
        batches = list(range(cfg.B))
    if kv_heads is None:
        kv_heads = list(range(cfg.Hkv))
    lens_all = cache_lengths(cfg)
    nb = len(batches)
    q = np.empty((nb, cfg.Hq, cfg.d), np.float32)
    k = np.zeros((nb, cfg.Hkv, cfg.L, cfg.d), np.float32)
    v = np.zeros_like(k)
    for i, b in enumerate(batches):
        q[i] = gaussian_tensor(cfg.seed, TID_Q, (cfg.Hq, cfg.d), cfg.dtype, b * cfg.Hq * cfg.d)
        for g in kv_heads:
            base = (b * cfg.Hkv + g) * cfg.L * cfg.d
            k[i, g] = gaussian_tensor(cfg.seed, TID_K, (cfg.L, cfg.d), cfg.dtype, base)
            v[i, g] = gaussian_tensor(cfg.seed, TID_V, (cfg.L, cfg.d), cfg.dtype, base)
    for b, h, p, row in decode_patches(cfg, lens_all):
        if b in batches and h // cfg.group in kv_heads:
            k[batches.index(b), h // cfg.group, p] = row
    return dict(q_raw=q, k=k, v=v, lens=lens_all[batches], dom=dominant_pairs(cfg),
                batches=batches)


def decode_cache_values(cfg: DecodeConfig, tid: int, b: int, g: int, rows, channels=None):
    """Stored values of cache tensor ``tid`` (TID_K or TID_V, standard layout)
    at rows ``rows`` and channels ``channels`` (default: all) of batch row b,
    KV head g, as fp32 [len(rows), len(channels)], needle keys included.

    The generator is counter-based, so a sampled check of a large cache can
    regenerate just the elements it reads."""
    rows = np.asarray(rows, dtype=np.int64)
    ch = np.arange(cfg.d, dtype=np.int64) if channels is None else np.asarray(channels, np.int64)
    base = (b * cfg.Hkv + g) * cfg.L * cfg.d
    n = (base + rows[:, None] * cfg.d + ch[None, :]).astype(np.uint64)
    z = gaussian_f32(cfg.seed, tid, n)
    out = round_to_bf16(z) if cfg.dtype == "bf16" else z.astype(np.float32)
    if tid == TID_K:
        where = {int(t): j for j, t in enumerate(rows.tolist())}
        for bb, h, p, row in _decode_patches_cached(cfg):
            if bb == b and h // cfg.group == g and p in where:
                out[where[p]] = row[ch]
    return out


@functools.lru_cache(maxsize=4)
def _decode_patches_cached(cfg: DecodeConfig):
    return decode_patches(cfg, cache_lengths(cfg))


def decode_patches(cfg: DecodeConfig, lens: np.ndarray):
    """Needle key rows: list of (b, q_head, position, stored row[d])."""
    out = []
    needles = decode_needles(cfg, lens)
    by_bh: dict[tuple[int, int], list[int]] = {}
    for b, h, p in needles:
        by_bh.setdefault((b, h), []).append(p)
    for (b, h), ps in sorted(by_bh.items()):
        qrow = gaussian_tensor(cfg.seed, TID_Q, (cfg.d,), cfg.dtype, (b * cfg.Hq + h) * cfg.d)
        qrot = _forward_rotate_rows(qrow[None, :].astype(np.float64),
                                    np.array([int(lens[b]) - 1]), cfg.theta)[0]
        target = 3.0 * np.sqrt(cfg.d) * qrot / np.linalg.norm(qrot)
        stored = _store(target, cfg.dtype)
        for p in ps:
            out.append((b, h, p, stored))
    return out


# ---------------------------------------------------------------- calibration
@dataclass(frozen=True)
class CalibConfig:
    """Offline calibration of the dominant rotary pairs (FASA sec. 2.B item 1:
    a one-time calibration identifies the dominant frequency chunks).

    Inputs are rotated calibration queries q [Hq, M, d] and keys k [Hkv, L, d]
    (stored bf16).  Each KV head gets a planted dominant set of n_dom pairs:
    for every calibration query, k_cal / 2 keys of the window (disjoint
    between the group's queries) receive amp times the unit direction of that
    query's components on the planted pairs, on those pairs only.  The rest
    is Irwin-Hall(12) noise.
    """
    name: str
    Hq: int
    Hkv: int
    M: int
    L: int
    d: int
    n_dom: int
    k_cal: int
    amp: float = 12.0
    seed: int = 9
    dtype: str = "bf16"

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def with_(self, **kw) -> "CalibConfig":
        return dataclasses.replace(self, **kw)


CAL_SMALL = CalibConfig("calibration, 8 query / 2 KV heads, 8 queries, window 2048, d=128", 8, 2,
                        8, 2048, 128, n_dom=16, k_cal=64)
CAL_LLAMA = CalibConfig("calibration, Llama-3.1-8B-shaped heads, 16 queries, window 8192, d=128",
                        32, 8, 16, 8192, 128, n_dom=16, k_cal=256)


def planted_pairs(cfg: CalibConfig) -> np.ndarray:
    """[Hkv, n_dom] ascending distinct rotary pairs planted as dominant."""
    P = cfg.d // 2
    out = np.empty((cfg.Hkv, cfg.n_dom), np.int32)
    for g in range(cfg.Hkv):
        u = uniform01(cfg.seed, TID_DOM, np.arange(g * P, (g + 1) * P, dtype=np.uint64))
        out[g] = np.sort(np.argsort(u, kind="stable")[: cfg.n_dom])
    return out


def calibration_inputs_host(cfg: CalibConfig):
    """(q [Hq, M, d], k [Hkv, L, d], planted [Hkv, n_dom]) as stored values."""
    P = cfg.d // 2
    r = cfg.k_cal // 2
    if cfg.group * cfg.M * r > cfg.L:
        raise ValueError("window too short for disjoint relevant key sets")
    q = gaussian_tensor(cfg.seed, TID_Q, (cfg.Hq, cfg.M, cfg.d), cfg.dtype).astype(np.float64)
    k = gaussian_tensor(cfg.seed, TID_K, (cfg.Hkv, cfg.L, cfg.d), cfg.dtype).astype(np.float64)
    dom = planted_pairs(cfg)
    for g in range(cfg.Hkv):
        ch = np.concatenate([dom[g], dom[g] + P]).astype(np.int64)
        u = uniform01(cfg.seed, TID_NEEDLE, (g << 24) + np.arange(cfg.L, dtype=np.uint64))
        perm = np.argsort(u, kind="stable")
        for hh in range(cfg.group):
            h = g * cfg.group + hh
            for m in range(cfg.M):
                keys = perm[(hh * cfg.M + m) * r:(hh * cfg.M + m + 1) * r]
                dirn = q[h, m, ch] / np.linalg.norm(q[h, m, ch])
                k[g, keys[:, None], ch[None, :]] += cfg.amp * dirn[None, :]
    return _store(q, cfg.dtype), _store(k, cfg.dtype), dom
