"""GPU parity of the fused token top-k (sa_token_topk) against the two calls it
replaces, sa_token_score then sa_topk_select: the selections must be equal
bit for bit (indices and counts), on the same device inputs, for the
dominant-slab and the standard cache layouts.

The two-step path is itself checked against the fp64 oracle elsewhere (staged
and end-to-end decode tests), so equality here carries that parity over.
Cases cover the sampled-threshold path, rows too short to sample (every token
a candidate), k at or above a row's length, empty rows, several slab widths,
group sizes and both dtypes, and the exact fallback: a cache whose scores all
tie sends every token past the threshold, so the candidate list overflows and
the row is selected again from recomputed scores.
"""
import numpy as np
import pytest
import torch

import synth
from synth import workloads as W
from tests.guards import check_all, guarded
from tests.parity_utils import say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import long_context_sparse_apply_amd as m
    import synth.device  # noqa: F401
    return m


def _two_step(sa, q_rope, k_dom, lens, dom, scale, k_top, slab=True):
    B, Hq, _ = q_rope.shape
    Lmax = k_dom.shape[2]
    scores = torch.empty((B, Hq, Lmax), dtype=torch.float32, device=DEV)
    sa.sa_token_score(q_rope, k_dom, scores, lens, dom, sm_scale=scale, slab=slab)
    idx = torch.empty((B, Hq, k_top), dtype=torch.int32, device=DEV)
    cnt = torch.empty((B, Hq), dtype=torch.int32, device=DEV)
    sa.sa_topk_select(scores, idx, cnt, k_const=k_top,
                      valid_len=lens.repeat_interleave(Hq).to(torch.int32).contiguous())
    return idx, cnt


def _fused(sa, q_rope, k_dom, lens, dom, scale, k_top, max_out=None, slab=True):
    B, Hq, _ = q_rope.shape
    Lmax = k_dom.shape[2]
    max_out = k_top if max_out is None else max_out
    ws, g_ws = guarded((sa.workspace_bytes(sa.SA_OP_TOKEN_TOPK, rows=B * Hq, cols=Lmax,
                                           max_k=k_top),), torch.uint8)
    idx, g_i = guarded((B, Hq, max_out), torch.int32)
    cnt, g_c = guarded((B, Hq), torch.int32)
    sa.sa_token_topk(q_rope, k_dom, lens, dom, idx, cnt, ws, sm_scale=scale, k_top=k_top, slab=slab)
    torch.cuda.synchronize()
    check_all(("workspace", g_ws), ("idx", g_i), ("count", g_c))
    return idx, cnt


def _inputs(dtype, B, Hq, Hkv, Lmax, n_dom, lens, seed, tie=False, slab=True, d=128):
    q = synth.gaussian_tensor(seed, synth.TID_Q, (B, Hq, d), dtype)
    kd = synth.gaussian_tensor(seed, synth.TID_K, (B, Hkv, Lmax, 2 * n_dom if slab else d), dtype)
    if tie:
        kd[:] = kd[:, :, :1, :]  # every token the same key: every score ties
    g = np.random.default_rng(seed)
    dom = np.sort(np.stack([g.choice(d // 2, n_dom, replace=False) for _ in range(Hkv)]), axis=1)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return (torch.from_numpy(q).to(DEV).to(tdt), torch.from_numpy(kd).to(DEV).to(tdt),
            torch.tensor(lens, dtype=torch.int32, device=DEV),
            torch.from_numpy(dom.astype(np.int32)).to(DEV).contiguous())


CASES = [  # name, dtype, B, Hq, Hkv, Lmax, n_dom, lens, k_top, tie
    ("bf16-32k-sampled", "bf16", 2, 8, 2, 32768, 16, [32768, 20000], 1024, False),
    ("bf16-64k-grp8", "bf16", 1, 8, 1, 65536, 16, [65536], 2048, False),
    ("bf16-ragged-short", "bf16", 4, 4, 4, 9000, 16, [9000, 700, 1, 0], 512, False),
    ("bf16-k-above-len", "bf16", 2, 4, 2, 3000, 16, [3000, 2500], 2800, False),
    ("bf16-narrow-slab", "bf16", 1, 4, 1, 20000, 4, [19999], 300, False),
    ("bf16-wide-slab", "bf16", 1, 2, 1, 20000, 32, [20000], 640, False),
    ("f32-sampled", "f32", 2, 4, 2, 20000, 8, [20000, 15000], 700, False),
    ("f32-narrow", "f32", 1, 2, 2, 6000, 4, [6000], 100, False),
    ("bf16-all-tied-fallback", "bf16", 1, 4, 1, 16384, 16, [16384], 512, True),
    # 256 (batch, KV head) groups: one work-group samples and searches a group
    # (fewer groups: four work-groups share the samples, a pick kernel searches)
    ("bf16-256-groups", "bf16", 64, 8, 4, 8192, 16, [8192 - 37 * i for i in range(64)], 512, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_token_topk_equals_score_then_select(sa, case):
    name, dtype, B, Hq, Hkv, Lmax, n_dom, lens, k_top, tie = case
    say(f"case: token top-k {name}")
    q, kd, lens_t, dom = _inputs(dtype, B, Hq, Hkv, Lmax, n_dom, lens, 40 + len(name), tie)
    scale = 128 ** -0.5
    ri, rc = _two_step(sa, q, kd, lens_t, dom, scale, k_top)
    fi, fc = _fused(sa, q, kd, lens_t, dom, scale, k_top)
    torch.cuda.synchronize()
    assert torch.equal(fc, rc), (fc.cpu(), rc.cpu())
    assert torch.equal(fi, ri)
    # a second call repeats the first bit for bit
    fi2, fc2 = _fused(sa, q, kd, lens_t, dom, scale, k_top)
    assert torch.equal(fi2, fi) and torch.equal(fc2, fc)
    # counts are min(k, length): a row never loses a selected token
    exp = np.minimum(k_top, np.repeat(np.asarray(lens), Hq)).reshape(B, Hq)
    assert np.array_equal(fc.cpu().numpy(), exp)


STD_CASES = [  # name, dtype, d, B, Hq, Hkv, Lmax, n_dom, lens, k_top, tie
    ("std-bf16-64k-c4-shape", "bf16", 128, 2, 8, 2, 65536, 16, [65536, 40000], 2048, False),
    ("std-bf16-ragged", "bf16", 128, 4, 4, 4, 9000, 16, [9000, 700, 1, 0], 512, False),
    ("std-bf16-grp1-n5", "bf16", 128, 1, 2, 2, 20000, 5, [19999], 300, False),
    ("std-bf16-grp8-n40", "bf16", 128, 1, 8, 1, 30000, 40, [30000], 1000, False),
    ("std-bf16-d64", "bf16", 64, 2, 4, 1, 16384, 8, [16384, 9000], 600, False),
    ("std-f32", "f32", 128, 2, 4, 2, 20000, 16, [20000, 15000], 700, False),
    ("std-bf16-k-above-len", "bf16", 128, 2, 4, 2, 3000, 16, [3000, 2500], 2800, False),
    ("std-bf16-all-tied-fallback", "bf16", 128, 1, 4, 1, 16384, 16, [16384], 512, True),
    ("std-bf16-256-groups", "bf16", 128, 64, 8, 4, 8192, 16, [8192 - 37 * i for i in range(64)], 512,
     False),
]


@pytest.mark.parametrize("case", STD_CASES, ids=[c[0] for c in STD_CASES])
def test_token_topk_standard_layout(sa, case):
    """The standard cache layout (full rows, the dominant channels read from
    each): the fused selection equals score-then-select bit for bit."""
    name, dtype, d, B, Hq, Hkv, Lmax, n_dom, lens, k_top, tie = case
    say(f"case: token top-k {name}")
    q, kd, lens_t, dom = _inputs(dtype, B, Hq, Hkv, Lmax, n_dom, lens, 90 + len(name), tie,
                                 slab=False, d=d)
    scale = d ** -0.5
    ri, rc = _two_step(sa, q, kd, lens_t, dom, scale, k_top, slab=False)
    fi, fc = _fused(sa, q, kd, lens_t, dom, scale, k_top, slab=False)
    torch.cuda.synchronize()
    assert torch.equal(fc, rc), (fc.cpu(), rc.cpu())
    assert torch.equal(fi, ri)
    exp = np.minimum(k_top, np.repeat(np.asarray(lens), Hq)).reshape(B, Hq)
    assert np.array_equal(fc.cpu().numpy(), exp)


def test_token_topk_slab_d64(sa):
    """Head dim 64 (32 rotary pairs), 8 dominant pairs: 32-byte slab rows."""
    say("case: token top-k slab d=64")
    q, kd, lens_t, dom = _inputs("bf16", 2, 4, 2, 24000, 8, [24000, 17000], 61, d=64)
    scale = 64 ** -0.5
    ri, rc = _two_step(sa, q, kd, lens_t, dom, scale, 900)
    fi, fc = _fused(sa, q, kd, lens_t, dom, scale, 900)
    torch.cuda.synchronize()
    assert torch.equal(fc, rc)
    assert torch.equal(fi, ri)


def test_token_topk_pads_wider_output(sa):
    """max_out above k_top: the selection is the same and the rest is -1."""
    q, kd, lens_t, dom = _inputs("bf16", 1, 4, 1, 12000, 16, [11000], 77)
    scale = 128 ** -0.5
    ri, rc = _two_step(sa, q, kd, lens_t, dom, scale, 256)
    fi, fc = _fused(sa, q, kd, lens_t, dom, scale, 256, max_out=300)
    torch.cuda.synchronize()
    assert torch.equal(fc, rc)
    assert torch.equal(fi[..., :256], ri)
    assert bool((fi[..., 256:] == -1).all())


def test_token_topk_decode_c5_shape(sa):
    """The 128K slab decode workload (batch 64, top-4096), as the bench runs
    it: the fused step's selection equals the two-step selection."""
    from long_context_sparse_apply_amd.pipeline import DecodeStep
    import synth.device as SD
    cfg = W.C5
    dt = SD.decode_tensors(cfg)
    fused = DecodeStep(dt["q_raw"], dt["k"], dt["v"], dt["lens"], dt["dom"], theta=cfg.theta,
                       top_k=cfg.k, slab=True, k_rest=dt["k_rest"], fused=True)
    fused.rope()
    fused.score_select()
    ri, rc = _two_step(sa, fused.q_rope, fused.k, fused.cache_len, fused.dom, fused.scale, cfg.k)
    torch.cuda.synchronize()
    assert torch.equal(fused.tok_cnt, rc)
    assert torch.equal(fused.tok_idx, ri)


def test_token_topk_decode_c4_shape(sa):
    """The 64K standard-layout decode workload (batch 16, top-2048), as the
    bench runs it: the fused step's selection equals the two-step one."""
    from long_context_sparse_apply_amd.pipeline import DecodeStep
    import synth.device as SD
    cfg = W.C4
    dt = SD.decode_tensors(cfg)
    fused = DecodeStep(dt["q_raw"], dt["k"], dt["v"], dt["lens"], dt["dom"], theta=cfg.theta,
                       top_k=cfg.k, slab=bool(cfg.slab), k_rest=dt["k_rest"], fused=True)
    fused.rope()
    fused.score_select()
    ri, rc = _two_step(sa, fused.q_rope, fused.k, fused.cache_len, fused.dom, fused.scale, cfg.k,
                       slab=bool(cfg.slab))
    torch.cuda.synchronize()
    assert torch.equal(fused.tok_cnt, rc)
    assert torch.equal(fused.tok_idx, ri)


def test_decode_c4_slab_layout_matches_standard(sa):
    """The 64K decode workload (batch 16, top-2048) on the dominant slab +
    full-row cache: the slab holds the dominant channels in the order the
    standard layout scores them, and the full rows equal the standard cache,
    so the step selects the same tokens and attends to the same output, bit
    for bit, as on the standard cache."""
    from long_context_sparse_apply_amd.pipeline import DecodeStep
    import synth.device as SD
    res = []
    for cfg in (W.C4, W.C4_SLAB):
        dt = SD.decode_tensors(cfg)
        step = DecodeStep(dt["q_raw"], dt["k"], dt["v"], dt["lens"], dt["dom"], theta=cfg.theta,
                          top_k=cfg.k, slab=bool(cfg.slab), k_rest=dt["k_rest"],
                          k_full=dt["k_full"])
        assert step.fused
        step.run()
        torch.cuda.synchronize()
        res.append((step.tok_idx.clone(), step.tok_cnt.clone(), step.out.clone()))
        del step, dt
        torch.cuda.empty_cache()
    (i0, c0, o0), (i1, c1, o1) = res
    assert torch.equal(c0, c1)
    assert torch.equal(i0, i1)
    assert torch.equal(o0, o1)
