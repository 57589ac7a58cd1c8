"""GPU parity of the decode KV-cache append and of the prefill -> decode handoff.

"FASA: Frequency-aware Sparse Attention", sec. 2.B item 2: the cached keys
keep their original absolute positions, so a new token's key is rotated at
its own position when it enters the cache; sec. 2.C: the computation-
optimised variant keeps the dominant channels of every key together (the
dominant slab).  The oracle rotates in fp64 (``rope``) and splits a standard
cache with ``standard_to_slab``; each stored GPU value must lie in the
admissible interval of ``tests.parity_utils.rotated_bounds``, untouched rows
must keep their old contents bit for bit, and values are copied exactly.

The handoff test runs two prompts of different lengths through the prefill
layer, appends each prompt's keys and values to a shared cache, then decodes
several tokens, each appended at its batch row's own position first; every
step is compared with the oracle's decode path on the oracle's own cache.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import sparse_attention as O
from synth import workloads as W
from tests.parity_utils import rotated_bounds, say
from tests.test_gpu_end_to_end import _HostCache, _all_samples, _compare_decode, _compare_prefill, _layer

pytestmark = pytest.mark.gpu
DEV = "cuda"
SENTINEL = 100.0  # outside the range of any rotated Irwin-Hall(12) pair (|x| <= 6 sqrt 2)


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import long_context_sparse_apply_amd as m
    return m


def _dev(a, dtype):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(dt)


def _host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _dom(Hkv, d, n_dom, seed):
    return W.dominant_pairs(W.C5.with_(Hkv=Hkv, d=d, n_dom=n_dom, seed=seed))


class HostCache:
    """The oracle's view of a cache: fp64 rotated keys, raw key pairs (for the
    admissible interval), stored values, and which rows were written."""

    def __init__(self, B, Hkv, Lmax, d):
        self.k = np.zeros((B, Hkv, Lmax, d))
        self.raw = np.zeros((B, Hkv, Lmax, d))
        self.v = np.zeros((B, Hkv, Lmax, d))
        self.written = np.zeros((B, Lmax), bool)
        self.Lmax = Lmax

    def append(self, b, k_new, v_new, start, theta):
        """k_new, v_new [Hkv, S, d] stored raw values for batch row b."""
        S = k_new.shape[1]
        rows = np.arange(S)
        pos = start + rows
        keep = pos < self.Lmax
        pos, rows = pos[keep], rows[keep]
        self.k[b][:, pos] = O.rope(k_new[:, rows].astype(np.float64), pos, theta)
        self.raw[b][:, pos] = k_new[:, rows]
        self.v[b][:, pos] = v_new[:, rows]
        self.written[b, pos] = True

    def bounds(self, dtype):
        return rotated_bounds(self.k, self.raw, dtype)


def _check_cache(cache_k, cache_rest, cache_v, hc, dtype, dom, slab):
    """Stored GPU cache vs the oracle's: admissible intervals on written rows,
    the sentinel on every other row, values bit for bit."""
    lo, hi = hc.bounds(dtype)
    g_v = _host(cache_v)
    w = hc.written
    for b in range(w.shape[0]):
        rows = np.nonzero(w[b])[0]
        other = np.nonzero(~w[b])[0]
        assert np.array_equal(g_v[b][:, rows], hc.v[b][:, rows]), ("v", b)
        assert np.all(g_v[b][:, other] == SENTINEL), ("v untouched", b)
    if slab == 2:  # slab + full rows: the slab, then every channel in the standard order
        lo_s, hi_s = O.standard_to_slab(lo, dom), O.standard_to_slab(hi, dom)
        for t, l_, h_ in ((cache_k, lo_s[0], hi_s[0]), (cache_rest, lo, hi)):
            g = _host(t)
            for b in range(w.shape[0]):
                rows = np.nonzero(w[b])[0]
                other = np.nonzero(~w[b])[0]
                gv = g[b][:, rows]
                bad = (gv < l_[b][:, rows]) | (gv > h_[b][:, rows])
                assert not bad.any(), ("slab + full rows", b, int(bad.sum()))
                assert np.all(g[b][:, other] == SENTINEL), ("k untouched", b)
    elif slab:
        parts = [(cache_k, 0)] + ([(cache_rest, 1)] if cache_rest is not None else [])
        lo_s, hi_s = O.standard_to_slab(lo, dom), O.standard_to_slab(hi, dom)
        for t, which in parts:
            g = _host(t)
            for b in range(w.shape[0]):
                rows = np.nonzero(w[b])[0]
                other = np.nonzero(~w[b])[0]
                gl, gh = lo_s[which][b][:, rows], hi_s[which][b][:, rows]
                gv = g[b][:, rows]
                bad = (gv < gl) | (gv > gh)
                assert not bad.any(), ("slab part", which, b, int(bad.sum()))
                assert np.all(g[b][:, other] == SENTINEL), ("k untouched", which, b)
    else:
        g = _host(cache_k)
        for b in range(w.shape[0]):
            rows = np.nonzero(w[b])[0]
            other = np.nonzero(~w[b])[0]
            gv = g[b][:, rows]
            bad = (gv < lo[b][:, rows]) | (gv > hi[b][:, rows])
            assert not bad.any(), ("k", b, int(bad.sum()))
            assert np.all(g[b][:, other] == SENTINEL), ("k untouched", b)


APPEND_CASES = [
    # dtype, d, slab, n_dom
    ("bf16", 128, False, 16),
    ("bf16", 128, True, 16),
    ("f32", 64, True, 8),
    ("f32", 64, False, 8),
    ("bf16", 128, True, 64),   # every pair dominant: no rest slab
    ("bf16", 64, True, 1),
    ("bf16", 128, 2, 16),      # slab + full rows
    ("f32", 64, 2, 4),
]


@pytest.mark.parametrize("dtype,d,slab,n_dom", APPEND_CASES,
                         ids=[f"{c[0]}-d{c[1]}-{['std', 'slab', 'slab-full'][int(c[2])]}-n{c[3]}"
                              for c in APPEND_CASES])
def test_kv_cache_append(sa, dtype, d, slab, n_dom):
    say(f"case: kv append {dtype} d={d} slab={slab} n_dom={n_dom}")
    B, Hkv, Lmax, theta = 3, 2, 200, 5e5
    dom = _dom(Hkv, d, n_dom, 31)
    domt = torch.from_numpy(dom).to(DEV)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kd = 2 * n_dom if slab else d
    k_cache = torch.full((B, Hkv, Lmax, kd), SENTINEL, dtype=tdt, device=DEV)
    rest_w = d if slab == 2 else d - kd
    k_rest = (torch.full((B, Hkv, Lmax, rest_w), SENTINEL, dtype=tdt, device=DEV)
              if slab and rest_w > 0 else None)
    v_cache = torch.full((B, Hkv, Lmax, d), SENTINEL, dtype=tdt, device=DEV)
    hc = HostCache(B, Hkv, Lmax, d)
    # first call: 37 tokens per row at ragged starts, the last row running past Lmax;
    # second call: one token each, including the cache's last row
    for call, (S, starts) in enumerate([(37, [0, 91, 180]), (1, [37, 128, 199])]):
        shape = (B, Hkv, S, d)
        k_new = synth.gaussian_tensor(40 + call, synth.TID_K, shape, dtype)
        v_new = synth.gaussian_tensor(40 + call, synth.TID_V, shape, dtype)
        start = torch.tensor(starts, dtype=torch.int32, device=DEV)
        sa.sa_kv_cache_append(_dev(k_new, dtype), _dev(v_new, dtype), start, k_cache, v_cache,
                              theta=theta, k_rest=k_rest, dom_pairs=domt if slab else None,
                              slab=bool(slab), full_rows=slab == 2)
        for b in range(B):
            hc.append(b, k_new[b], v_new[b], starts[b], theta)
    torch.cuda.synchronize()
    _check_cache(k_cache, k_rest, v_cache, hc, dtype, dom, slab)


def test_kv_cache_append_standard_matches_rope_apply(sa):
    """The standard layout's rows equal sa_rope_apply's rotation at the same
    positions (both use one rotation rule), for positions near 2^17."""
    B, Hkv, S, d, Lmax, theta = 2, 2, 64, 128, 131072, 5e5
    k_new = synth.gaussian_tensor(44, synth.TID_K, (B, Hkv, S, d), "bf16")
    v_new = synth.gaussian_tensor(44, synth.TID_V, (B, Hkv, S, d), "bf16")
    starts = [Lmax - S, 70000]
    kc = torch.zeros((B, Hkv, Lmax, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    sa.sa_kv_cache_append(_dev(k_new, "bf16"), _dev(v_new, "bf16"),
                          torch.tensor(starts, dtype=torch.int32, device=DEV), kc, vc, theta=theta)
    pos = np.stack([s + np.arange(S) for s in starts]).astype(np.int32)
    rot = torch.empty((B, Hkv, S, d), dtype=torch.bfloat16, device=DEV)
    sa.sa_rope_apply(_dev(k_new, "bf16"), rot, theta, pos=torch.from_numpy(pos.ravel()).to(DEV))
    torch.cuda.synchronize()
    for b in range(B):
        assert torch.equal(kc[b, :, starts[b]:starts[b] + S], rot[b])
    hc = HostCache(B, Hkv, Lmax, d)
    for b in range(B):
        hc.append(b, k_new[b], v_new[b], starts[b], theta)
    for b in range(B):
        sl = slice(starts[b], starts[b] + S)
        lo, hi = rotated_bounds(hc.k[b][:, sl], hc.raw[b][:, sl], "bf16")
        g = _host(kc[b, :, sl])
        assert np.all((g >= lo) & (g <= hi))


@pytest.mark.parametrize("slab,host_rest,full_rows",
                         [(False, False, False), (True, False, False), (True, True, False),
                          (True, False, True)],
                         ids=["std", "slab", "slab-host-rest", "slab-full-rows"])
def test_prefill_decode_handoff(sa, slab, host_rest, full_rows):
    """Two prompts (2048 and 1536 tokens) through the prefill layer into one
    cache, then 3 decode steps with per-row positions, each against the oracle.
    With host_rest the non-dominant keys and the values live in pinned host
    memory (FASA-M) and are written and read over the host link."""
    from long_context_sparse_apply_amd.pipeline import DecodeCache
    say(f"case: prefill -> decode handoff slab={slab} host_rest={host_rest} full_rows={full_rows}")
    lens0 = [2048, 1536]
    T, top_k, n_dom = 3, 256, 16
    base = W.C2.with_(Hq=8, Hkv=2, needle_pairs=4)
    B, Hq, Hkv, d, theta = 2, base.Hq, base.Hkv, base.d, base.theta
    Lmax = max(lens0) + T
    dom = _dom(Hkv, d, n_dom, 32)
    cache = DecodeCache(B, Hkv, Lmax, d, dtype=torch.bfloat16, device=DEV, theta=theta,
                        dom_pairs=torch.from_numpy(dom).to(DEV), slab=slab, host_rest=host_rest,
                        full_rows=full_rows)
    if host_rest:
        assert not cache.v.is_cuda and cache.v.is_pinned() and cache.k_rest.is_pinned()
    second = cache.k_full if full_rows else cache.k_rest
    cache.k.fill_(SENTINEL)
    cache.v.fill_(SENTINEL)
    if second is not None:
        second.fill_(SENTINEL)
    layout = 2 if full_rows else int(slab)
    hc = HostCache(B, Hkv, Lmax, d)
    for b, S in enumerate(lens0):
        cfg = base.with_(S=S, seed=50 + b)
        q, k, v, heads = W.prefill_inputs_host(cfg)
        kt, vt = _dev(k, cfg.dtype), _dev(v, cfg.dtype)
        layer = _layer(sa, cfg, _dev(q, cfg.dtype), kt, vt)
        layer.run()
        cache.append(kt, vt, batch=b)
        torch.cuda.synchronize()
        _compare_prefill(cfg, layer, q[:, [0, Hq - 1]], k, v, [0, Hq - 1])
        hc.append(b, k[0], v[0], 0, theta)
        del layer
    assert cache.lens.cpu().tolist() == lens0
    _check_cache(cache.k, second, cache.v, hc, "bf16", dom, layout)
    dcfg = W.C5.with_(B=B, Hq=Hq, Hkv=Hkv, L=Lmax, d=d, theta=theta, n_dom=n_dom, k=top_k,
                      slab=int(slab))
    lens = np.array(lens0, np.int32)
    for t in range(T):
        q_new = synth.gaussian_tensor(60 + t, synth.TID_Q, (B, Hq, d), "bf16")
        k_new = synth.gaussian_tensor(60 + t, synth.TID_K, (B, Hkv, 1, d), "bf16")
        v_new = synth.gaussian_tensor(60 + t, synth.TID_V, (B, Hkv, 1, d), "bf16")
        cache.append(_dev(k_new, "bf16"), _dev(v_new, "bf16"))
        for b in range(B):
            hc.append(b, k_new[b], v_new[b], int(lens[b]), theta)
        lens = lens + 1
        step = cache.step(_dev(q_new, "bf16"), top_k=top_k)
        step.run()
        torch.cuda.synchronize()
        assert cache.lens.cpu().numpy().tolist() == lens.tolist()
        # the oracle's cache: its own rotation, stored in bf16
        k_or = synth.round_to_bf16(hc.k).astype(np.float64)
        lo, hi = hc.bounds("bf16")
        x = dict(q_raw=q_new, k=k_or, v=hc.v, lens=lens, dom=dom, batches=list(range(B)))
        say(f"  step {t}: lens {lens.tolist()}")
        _compare_decode(dcfg, step, _HostCache(dcfg, x), _all_samples(dcfg, range(B)), k_amb=hi - lo)
    _check_cache(cache.k, second, cache.v, hc, "bf16", dom, layout)


def test_decode_host_placement(sa):
    """FASA-M placement on the decode step: the dominant slab in device memory,
    the rest of each key and the values in pinned host memory.  The step must
    equal the all-device step bit for bit (same kernels, same data) and match
    the oracle."""
    import synth.device as SD
    from long_context_sparse_apply_amd.pipeline import DecodeStep
    from tests.test_gpu_end_to_end import _decode_step
    cfg = W.C5.with_(B=2, L=8192, k=256, ragged=1000, full_rows=0)
    say("case: decode with host-placed k_rest / v (slab-8k)")
    x = W.decode_inputs_host(cfg)
    dt = SD.decode_tensors(cfg)
    dev_step = _decode_step(sa, cfg, x, dt)
    dev_step.run()
    k_rest_h = torch.empty(dt["k_rest"].shape, dtype=dt["k_rest"].dtype, pin_memory=True)
    v_h = torch.empty(dt["v"].shape, dtype=dt["v"].dtype, pin_memory=True)
    k_rest_h.copy_(dt["k_rest"])
    v_h.copy_(dt["v"])
    torch.cuda.synchronize()
    host_step = DecodeStep(dt["q_raw"], dt["k"], v_h, dt["lens"], dt["dom"], theta=cfg.theta,
                           top_k=cfg.k, slab=True, k_rest=k_rest_h)
    host_step.run()
    torch.cuda.synchronize()
    assert torch.equal(host_step.tok_idx, dev_step.tok_idx)
    assert torch.equal(host_step.out, dev_step.out)
    assert torch.equal(host_step.lse, dev_step.lse)
    _compare_decode(cfg, host_step, _HostCache(cfg, x), _all_samples(cfg, range(cfg.B)))
