"""The allocation-free decode entry point (sa_sparse_attn_decode_static: the
split-K partials in the library's fixed per-GPU array) against the entry
point it mirrors (sa_sparse_attn_decode with a caller's workspace), through
the C ABI: two calls in a row, the second with a smaller input, each equal
to the workspace variant bit for bit and within 2e-2 of the fp64 oracle over
the same selection.  A size whose partials exceed the array is refused."""
import numpy as np
import pytest
import torch

import synth
from oracle import sparse_attention as O
from synth import workloads as W
from tests.guards import check_all, guarded
from tests.parity_utils import OUT_ATOL, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import long_context_sparse_apply_amd as m
    return m


def _case(sa, B, Hq, Hkv, L, max_k, slab, seed):
    cfg = W.C4.with_(B=B, Hq=Hq, Hkv=Hkv, L=L, n_dom=16, ragged=L // 4, seed=seed,
                     needles_per_head=2)
    x = W.decode_inputs_host(cfg)
    q = synth.gaussian_tensor(seed, 8, (B, Hq, 128), "bf16")
    g = np.random.default_rng(seed)
    tok = np.full((B, Hq, max_k), -1, np.int32)
    cnt = np.zeros((B, Hq), np.int32)
    sel = [[None] * Hq for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            n = int(g.integers(0, min(max_k, int(x["lens"][b])) + 1))
            t = np.sort(g.choice(int(x["lens"][b]), size=n, replace=False)).astype(np.int32)
            tok[b, h, :n], cnt[b, h], sel[b][h] = t, n, t
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV).to(torch.bfloat16)
    kw = {}
    if slab:
        kd, kr = O.standard_to_slab(x["k"], x["dom"])
        kt, kw["k_rest"] = dev(kd), dev(kr)
        kw["dom_pairs"] = torch.from_numpy(x["dom"]).to(DEV)
    else:
        kt = dev(x["k"])
    args = (dev(q), kt, dev(x["v"]), torch.from_numpy(tok).to(DEV), torch.from_numpy(cnt).to(DEV))
    ref, _ = O.decode_attention(q.astype(np.float64), x["k"].astype(np.float64),
                                x["v"].astype(np.float64), sel, 128 ** -0.5)
    return args, kw, ref


@pytest.mark.parametrize("first,second", [
    ((4, 32, 8, 5000, 2048, 0, 61), (2, 8, 2, 3000, 700, 1, 62)),
], ids=["std-then-smaller-slab"])
def test_static_decode_matches_workspace_decode(sa, first, second):
    for B, Hq, Hkv, L, max_k, slab, seed in (first, second):
        say(f"case: static decode B={B} Hq={Hq} L={L} max_k={max_k} slab={slab}")
        args, kw, ref = _case(sa, B, Hq, Hkv, L, max_k, slab, seed)
        ws, g_ws = guarded((sa.workspace_bytes(sa.SA_OP_DECODE, B=B, Hq=Hq, max_k=max_k),),
                           torch.uint8)
        out_w, g_ow = guarded((B, Hq, 128), torch.bfloat16)
        lse_w, g_lw = guarded((B, Hq), torch.float32)
        sa.sa_sparse_attn_decode(*args, out_w, ws, sm_scale=128 ** -0.5, slab=bool(slab),
                                 lse=lse_w, **kw)
        out_s, g_os = guarded((B, Hq, 128), torch.bfloat16)
        lse_s, g_ls = guarded((B, Hq), torch.float32)
        sa.sa_sparse_attn_decode_static(*args, out_s, sm_scale=128 ** -0.5, slab=bool(slab),
                                        lse=lse_s, **kw)
        torch.cuda.synchronize()
        check_all(("ws", g_ws), ("out ws", g_ow), ("lse ws", g_lw), ("out static", g_os),
                  ("lse static", g_ls))
        assert torch.equal(out_s, out_w)
        assert torch.equal(lse_s, lse_w)
        err = np.abs(out_s.float().cpu().numpy() - ref).max()
        assert err <= OUT_ATOL["bf16"], err


def test_static_decode_refuses_oversize(sa):
    """511 lists with 64 splits each need more partials than the array holds."""
    B, Hq, Hkv, L, max_k = 1, 511, 511, 64, 16384
    q = torch.zeros((B, Hq, 128), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((B, Hkv, L, 128), dtype=torch.bfloat16, device=DEV)
    tok = torch.zeros((B, Hq, max_k), dtype=torch.int32, device=DEV)
    cnt = torch.zeros((B, Hq), dtype=torch.int32, device=DEV)
    out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(sa.SAError) as e:
        sa.sa_sparse_attn_decode_static(q, k, k, tok, cnt, out, sm_scale=1.0)
    assert e.value.status == sa.SA_ERR_WORKSPACE
