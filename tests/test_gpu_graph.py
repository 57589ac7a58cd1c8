"""A decode step captured once in a HIP graph and replayed: the fused token
top-k (sa_token_topk) then the decode attention (sa_sparse_attn_decode with
its workspace, or the allocation-free sa_sparse_attn_decode_static), on the
standard and the dominant-slab cache layouts; and the prefill layer
(sa_block_score, sa_topk_select, sa_sparse_attn_prefill) likewise.  The library issues only
kernel launches on the caller's stream (no memory set, copy, allocation or
synchronisation), so a serving loop can capture the step and replay it
with new queries written into the captured query buffer.

Each replay follows eager work of the program's own (the same step run
eagerly into separate buffers, with synchronisation in between) and must
equal that eager step bit for bit: selected indices, counts, output and
log-sum-exp.  The eager step is itself checked against the fp64 oracle by
the parity tests.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import sparse_attention as O
from synth import workloads as W
from tests.parity_utils import say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import long_context_sparse_apply_amd as m
    return m


CASES = [  # name, slab, static decode, B, Hq, Hkv, L, d, n_dom, k_top
    ("std-ws", False, False, 2, 8, 2, 4096, 128, 16, 256),
    ("slab-ws", True, False, 2, 8, 2, 4096, 128, 16, 256),
    ("std-static", False, True, 2, 8, 2, 4096, 128, 16, 256),
    ("slab-static-onepass", True, True, 16, 32, 8, 2048, 128, 16, 128),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_step_graph_replay(sa, case):
    name, slab, static, B, Hq, Hkv, L, d, n_dom, k_top = case
    say(f"case: decode step in a graph {name}")
    cfg = W.C4.with_(dtype="bf16", B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, n_dom=n_dom, ragged=300,
                     seed=61, needles_per_head=2)
    x = W.decode_inputs_host(cfg)
    bf = torch.bfloat16
    if slab:
        k_dom, k_rest = O.standard_to_slab(x["k"], x["dom"])
        k_score = torch.from_numpy(np.ascontiguousarray(k_dom, np.float32)).to(DEV).to(bf)
        k_rest_t = torch.from_numpy(np.ascontiguousarray(k_rest, np.float32)).to(DEV).to(bf)
    else:
        k_score = torch.from_numpy(np.ascontiguousarray(x["k"], np.float32)).to(DEV).to(bf)
        k_rest_t = None
    v = torch.from_numpy(np.ascontiguousarray(x["v"], np.float32)).to(DEV).to(bf)
    lens = torch.from_numpy(x["lens"]).to(DEV)
    dom = torch.from_numpy(x["dom"]).to(DEV)
    scale = d ** -0.5

    def buffers():
        return dict(
            idx=torch.empty((B, Hq, k_top), dtype=torch.int32, device=DEV),
            cnt=torch.empty((B, Hq), dtype=torch.int32, device=DEV),
            out=torch.empty((B, Hq, d), dtype=bf, device=DEV),
            lse=torch.empty((B, Hq), dtype=torch.float32, device=DEV),
            ws_t=torch.empty(sa.workspace_bytes(sa.SA_OP_TOKEN_TOPK, rows=B * Hq, cols=L, max_k=k_top),
                             dtype=torch.uint8, device=DEV),
            ws_d=torch.empty(sa.workspace_bytes(sa.SA_OP_DECODE, B=B, Hq=Hq, max_k=k_top),
                             dtype=torch.uint8, device=DEV))

    def step(qb, o):
        sa.sa_token_topk(qb, k_score, lens, dom, o["idx"], o["cnt"], o["ws_t"], sm_scale=scale,
                         k_top=k_top, slab=slab)
        kw = dict(sm_scale=scale, cache_len=lens, dom_pairs=dom if slab else None, slab=slab,
                  k_rest=k_rest_t, lse=o["lse"])
        if static:
            sa.sa_sparse_attn_decode_static(qb, k_score, v, o["idx"], o["cnt"], o["out"], **kw)
        else:
            sa.sa_sparse_attn_decode(qb, k_score, v, o["idx"], o["cnt"], o["out"], o["ws_d"], **kw)

    def query(seed):
        return synth.gaussian_tensor(seed, 8, (B, Hq, d), "bf16")

    q_static = torch.from_numpy(query(70)).to(DEV).to(bf)
    g_buf, e_buf = buffers(), buffers()
    # warm-up outside the capture (first calls set up the library's state)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(q_static, g_buf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(q_static, g_buf)
    torch.cuda.synchronize()

    for r in range(4):
        q_static.copy_(torch.from_numpy(query(71 + r)).to(DEV).to(bf))
        step(q_static, e_buf)  # the eager step into its own buffers
        torch.cuda.synchronize()
        for key in ("idx", "cnt", "out", "lse"):
            g_buf[key].fill_(-3)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        cnt = g_buf["cnt"]
        assert torch.equal(cnt, e_buf["cnt"]), f"replay {r}: counts differ"
        assert bool((cnt > 0).all()), f"replay {r}: an empty selection"
        assert torch.equal(g_buf["idx"], e_buf["idx"]), f"replay {r}: indices differ"
        assert torch.equal(g_buf["out"], e_buf["out"]), f"replay {r}: outputs differ"
        assert torch.equal(g_buf["lse"], e_buf["lse"]), f"replay {r}: lse differs"
        say(f"  replay {r}: equal to the eager step")
    del graph


def test_prefill_layer_graph_replay(sa):
    """The prefill layer (block scores with the fused rotation and pooling,
    block top-k, block-sparse attention) captured once and replayed with new
    queries: every replay equals the same layer run eagerly into its own
    buffers, bit for bit (scores, lists, counts, output, lse)."""
    from long_context_sparse_apply_amd.pipeline import PrefillLayer
    say("case: prefill layer in a graph")
    B, Hq, Hkv, S, d = 1, 8, 2, 4096, 128
    bf = torch.bfloat16

    def tensor(seed, H):
        return torch.from_numpy(synth.gaussian_tensor(seed, 8, (B, H, S, d), "bf16")).to(DEV).to(bf)

    q, k, v = tensor(80, Hq), tensor(81, Hkv), tensor(82, Hkv)
    kw = dict(theta=5e5, block=128, band_split_pair=16, n_sink=1, n_local=2, keep_percent=10)
    lg, le = PrefillLayer(q, k, v, **kw), PrefillLayer(q, k, v, **kw)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lg.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lg.run()
    torch.cuda.synchronize()
    names = ("scores", "blk_idx", "blk_cnt", "out", "lse")
    for r in range(3):
        q.copy_(tensor(83 + r, Hq))
        le.run()
        torch.cuda.synchronize()
        for n in names:
            getattr(lg, n).fill_(-3)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(getattr(lg, n), getattr(le, n)), f"replay {r}: {n} differs"
        say(f"  replay {r}: equal to the eager layer")
    del graph
