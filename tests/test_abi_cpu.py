"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any launch (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "sa.h")) as f:
        src = f.read()
    return sorted(set(re.findall(r"^\s*(?:sa_status|size_t|const char\*|int)\s+(sa_\w+)\(", src, re.M)))


def test_header_declares_the_six_entry_points():
    names = _declared()
    for n in ("sa_rope_apply", "sa_block_score", "sa_token_score", "sa_topk_select",
              "sa_sparse_attn_prefill", "sa_sparse_attn_decode"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import long_context_sparse_apply_amd as sa
    lib = ctypes.CDLL(sa.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n
    assert set(_declared()) <= set(sa.EXPORTED)


def test_status_strings_and_version():
    import long_context_sparse_apply_amd as sa
    assert sa.status_string(0) == "ok"
    assert "workspace" in sa.status_string(sa.SA_ERR_WORKSPACE)
    assert sa.lib.sa_version() >= 100


def _fake(n=1):
    # non-NULL host addresses: only reached if validation wrongly passed, never dereferenced
    return ctypes.c_void_p(0x1000 * n)


def test_validation_errors_before_launch():
    import long_context_sparse_apply_amd as sa
    L = sa.lib
    P = _fake
    # rope: null, bad d, bad theta, bad dtype
    assert L.sa_rope_apply(None, P(), 1, 1, 1, 8, 128, None, 0, 1e4, None) == sa.SA_ERR_NULL
    assert L.sa_rope_apply(P(), P(), 1, 1, 1, 8, 96, None, 0, 1e4, None) == sa.SA_ERR_SHAPE
    assert L.sa_rope_apply(P(), P(), 1, 1, 1, 8, 128, None, 0, 1.0, None) == sa.SA_ERR_RANGE
    assert L.sa_rope_apply(P(), P(), 7, 1, 1, 8, 128, None, 0, 1e4, None) == sa.SA_ERR_DTYPE
    # kv cache append: null pointers, shapes, theta, slab rules
    def kva(kn=True, start=True, B=2, Hkv=2, S=4, d=128, Lmax=64, theta=1e4, slab=0, dom=None,
            n_dom=16, rest=None, dtype=1):
        return L.sa_kv_cache_append(P() if kn else None, P(), dtype, B, Hkv, S, d, Lmax,
                                    P() if start else None, theta, slab, dom, n_dom, P(), rest, P(),
                                    None)
    assert kva(kn=False) == sa.SA_ERR_NULL
    assert kva(start=False) == sa.SA_ERR_NULL
    assert kva(S=0) == sa.SA_ERR_SHAPE
    assert kva(Lmax=0) == sa.SA_ERR_SHAPE
    assert kva(d=96) == sa.SA_ERR_SHAPE
    assert kva(theta=0.5) == sa.SA_ERR_RANGE
    assert kva(dtype=5) == sa.SA_ERR_DTYPE
    assert kva(slab=1) == sa.SA_ERR_NULL                      # no dominant pairs
    assert kva(slab=1, dom=P(), n_dom=65) == sa.SA_ERR_RANGE
    assert kva(slab=1, dom=P(), n_dom=16) == sa.SA_ERR_NULL   # no k_rest while 2*n_dom < d
    # block score: S % block, Hq % Hkv, split range, workspace
    args = dict(theta=1e4, block=64, split=16)
    def bs(B=1, Hq=4, Hkv=2, S=512, d=64, block=64, split=16, ws=None, wsb=0, pq=None, pk=None,
           qsc=1.0):
        return L.sa_block_score(P(), P(), 0, B, Hq, Hkv, S, d, 1e4, block, split, 1, 0.1, 1,
                                None, qsc, None, pq, pk, P(), ws, wsb, None)
    assert bs(S=500) == sa.SA_ERR_SHAPE
    assert bs(Hq=3) == sa.SA_ERR_SHAPE
    assert bs(block=48) == sa.SA_ERR_SHAPE
    assert bs(split=33) == sa.SA_ERR_RANGE
    assert bs(qsc=float("inf")) == sa.SA_ERR_RANGE
    assert bs(qsc=float("nan")) == sa.SA_ERR_RANGE
    assert bs() == sa.SA_ERR_WORKSPACE
    assert bs(ws=P(), wsb=100) == sa.SA_ERR_WORKSPACE
    # topk: shapes, ranges, max_out
    assert L.sa_topk_select(P(), 4, 0, None, None, 2, 0, 0, P(), 4, P(), None, 0, None) == sa.SA_ERR_SHAPE
    assert L.sa_topk_select(P(), 4, 300000, None, None, 2, 0, 0, P(), 4, P(), None, 0, None) == sa.SA_ERR_SHAPE
    assert L.sa_topk_select(P(), 4, 10, None, None, -1, 0, 0, P(), 4, P(), None, 0, None) == sa.SA_ERR_RANGE
    assert L.sa_topk_select(P(), 4, 10, None, None, 4, 1, 1, P(), 5, P(), None, 0, None) == sa.SA_ERR_RANGE
    assert L.sa_topk_select(None, 4, 10, None, None, 2, 0, 0, P(), 4, P(), None, 0, None) == sa.SA_ERR_NULL
    assert L.sa_topk_select(None, 0, 10, None, None, 2, 0, 0, None, 4, None, None, 0, None) == sa.SA_OK
    # token score: group size, slab width
    assert L.sa_token_score(P(), P(), None, 1, 1, 6, 2, 64, 128, P(), P(), 16, 0, 0.1, P(), None) == sa.SA_ERR_UNSUPPORTED
    assert L.sa_token_score(P(), P(), None, 1, 1, 8, 2, 64, 128, P(), P(), 6, 1, 0.1, P(), None) == sa.SA_ERR_UNSUPPORTED
    assert L.sa_token_score(P(), P(), None, 1, 1, 8, 2, 64, 128, P(), P(), 65, 0, 0.1, P(), None) == sa.SA_ERR_RANGE
    # prefill attention
    assert L.sa_sparse_attn_prefill(P(), P(), P(), 1, 1, 4, 2, 1000, 128, 128, P(), P(), 4, 1, 0.1, P(), None, None) == sa.SA_ERR_SHAPE
    assert L.sa_sparse_attn_prefill(P(), P(), P(), 1, 1, 4, 2, 1024, 128, 128, P(), P(), 0, 1, 0.1, P(), None, None) == sa.SA_ERR_RANGE
    assert L.sa_sparse_attn_prefill(None, P(), P(), 1, 1, 4, 2, 1024, 128, 128, P(), P(), 4, 1, 0.1, P(), None, None) == sa.SA_ERR_NULL
    # decode attention: workspace and slab rules
    need = sa.workspace_bytes(sa.SA_OP_DECODE, B=2, Hq=8, max_k=512)
    assert need > 2 * 8 * 2 * 128 * 4
    assert L.sa_sparse_attn_decode(P(), P(), None, P(), 1, 2, 8, 2, 1024, 128, P(), None, 0, 0,
                                   P(), P(), 512, 0.1, P(), None, P(), need - 1, None) == sa.SA_ERR_WORKSPACE
    assert L.sa_sparse_attn_decode(P(), P(), None, P(), 1, 2, 8, 2, 1024, 128, P(), P(), 6, 1,
                                   P(), P(), 512, 0.1, P(), None, P(), need, None) == sa.SA_ERR_UNSUPPORTED
    assert L.sa_sparse_attn_decode(P(), P(), None, P(), 1, 2, 8, 2, 1024, 128, P(), P(), 16, 1,
                                   P(), P(), 512, 0.1, P(), None, P(), need, None) == sa.SA_ERR_NULL
    # host placement: k_rest / v may be pinned host memory, never pageable memory (refused
    # before any launch; without a GPU no host memory is reachable either)
    pageable = ctypes.create_string_buffer(1 << 16)
    hp = ctypes.cast(pageable, ctypes.c_void_p)
    assert L.sa_sparse_attn_decode(P(), P(), None, hp, 1, 2, 8, 2, 1024, 128, P(), None, 0, 0,
                                   P(), P(), 512, 0.1, P(), None, P(), need, None) == sa.SA_ERR_ACCESS
    assert L.sa_kv_cache_append(P(), P(), 1, 2, 2, 4, 128, 64, P(), 1e4, 0, None, 0, P(), None,
                                hp, None) == sa.SA_ERR_ACCESS
    assert "accessible" in sa.status_string(sa.SA_ERR_ACCESS)
    # calibration of the dominant pairs: sizes, ranges, bf16 only, workspace
    need = sa.calibrate_workspace_bytes(8, 2, 4, 2048, 128, 64)
    assert need > 8 * 4 * 64 * 2048 * 4
    assert sa.calibrate_workspace_bytes(8, 3, 4, 2048, 128, 64) == 0
    assert sa.calibrate_workspace_bytes(8, 2, 4, 2048, 128, 4096) == 0
    def cal(q=True, Hq=8, Hkv=2, M=4, L=2048, d=128, kc=64, nd=16, dtype=1, ws=True, wsb=None):
        return L_.sa_calibrate_dominant(P() if q else None, P(), dtype, Hq, Hkv, M, L, d, kc, nd,
                                        P(), P(), P() if ws else None,
                                        need if wsb is None else wsb, None)
    L_ = L
    assert cal(q=False) == sa.SA_ERR_NULL
    assert cal(Hkv=3) == sa.SA_ERR_SHAPE
    assert cal(d=96) == sa.SA_ERR_SHAPE
    assert cal(L=300000) == sa.SA_ERR_SHAPE
    assert cal(kc=0) == sa.SA_ERR_RANGE
    assert cal(kc=2049) == sa.SA_ERR_RANGE
    assert cal(nd=65) == sa.SA_ERR_RANGE
    assert cal(dtype=0) == sa.SA_ERR_UNSUPPORTED
    assert cal(dtype=9) == sa.SA_ERR_DTYPE
    assert cal(ws=False) == sa.SA_ERR_WORKSPACE
    assert cal(wsb=need - 1) == sa.SA_ERR_WORKSPACE
    # k-sparse feature codes
    assert L.sa_sfa_sparsify(P(), P(), 1, -1, 128, 16, None) == sa.SA_ERR_SHAPE
    assert L.sa_sfa_sparsify(P(), P(), 1, 10, 96, 16, None) == sa.SA_ERR_SHAPE
    assert L.sa_sfa_sparsify(P(), P(), 1, 10, 128, -1, None) == sa.SA_ERR_RANGE
    assert L.sa_sfa_sparsify(P(), P(), 9, 10, 128, 16, None) == sa.SA_ERR_DTYPE
    assert L.sa_sfa_sparsify(None, P(), 1, 10, 128, 16, None) == sa.SA_ERR_NULL
    assert L.sa_sfa_sparsify(None, None, 1, 0, 128, 16, None) == sa.SA_OK


def test_token_topk_validation():
    """sa_token_topk: argument checks on the host, no launch."""
    import long_context_sparse_apply_amd as sa
    L = sa.lib
    P = lambda: ctypes.c_void_p(16)  # noqa: E731 (never dereferenced: every call fails a check)
    ws_ok = sa.workspace_bytes(sa.SA_OP_TOKEN_TOPK, rows=16, cols=4096, max_k=256)

    def tt(q=True, dtype=1, B=2, Hq=8, Hkv=2, Lmax=4096, d=128, n_dom=16, slab=1, k=256,
           max_out=256, ws=True, wsb=None):
        return L.sa_token_topk(P() if q else None, P(), dtype, B, Hq, Hkv, Lmax, d, P(), P(),
                               n_dom, slab, 0.1, k, P(), max_out, P(), P() if ws else None,
                               ws_ok if wsb is None else wsb, None)
    assert tt(q=False) == sa.SA_ERR_NULL
    assert tt(dtype=7) == sa.SA_ERR_DTYPE
    assert tt(Lmax=0) == sa.SA_ERR_SHAPE
    assert tt(Lmax=300000) == sa.SA_ERR_SHAPE
    assert tt(Hq=7) == sa.SA_ERR_SHAPE
    assert tt(Hq=6, Hkv=2) == sa.SA_ERR_UNSUPPORTED
    assert tt(n_dom=0) == sa.SA_ERR_RANGE
    assert tt(k=-1) == sa.SA_ERR_RANGE
    assert tt(max_out=255) == sa.SA_ERR_RANGE
    assert tt(n_dom=48) == sa.SA_ERR_UNSUPPORTED          # 192-byte slab rows
    assert tt(n_dom=2) == sa.SA_ERR_UNSUPPORTED           # 8-byte slab rows
    assert tt(dtype=0, n_dom=32) == sa.SA_ERR_UNSUPPORTED  # fp32: 256-byte slab rows
    # the standard layout reads any n_dom of the full rows: no slab-width rule
    assert tt(slab=0, n_dom=48, ws=False) == sa.SA_ERR_WORKSPACE
    assert tt(slab=0, n_dom=2, ws=False) == sa.SA_ERR_WORKSPACE
    assert tt(slab=0, d=96) == sa.SA_ERR_SHAPE
    assert tt(slab=0, n_dom=65) == sa.SA_ERR_RANGE
    assert tt(ws=False) == sa.SA_ERR_WORKSPACE
    assert tt(wsb=ws_ok - 1) == sa.SA_ERR_WORKSPACE


def test_workspace_sizes():
    import long_context_sparse_apply_amd as sa
    assert sa.workspace_bytes(sa.SA_OP_TOPK, 100, 1000) == 0
    # thresholds and counts, then per row up to k + k/4 + 1024 (64-aligned) composites
    assert sa.workspace_bytes(sa.SA_OP_TOKEN_TOPK, rows=2048, cols=131072, max_k=4096) >= 2048 * 6144 * 8
    assert sa.workspace_bytes(sa.SA_OP_TOKEN_TOPK, rows=0, cols=10, max_k=4) == 0
    n = 1 * (32 + 8) * 256
    assert sa.workspace_bytes(sa.SA_OP_BLOCK_SCORE, n, 128) >= n * 128 * 4
    assert sa.workspace_bytes(99) == 0


def test_prefill_row_params_budget():
    import long_context_sparse_apply_amd as sa
    vl, kr, kmax = sa.prefill_row_params(1, 2, 256, keep_percent=10, device="cpu")
    assert vl.shape[0] == 512 and int(vl[0]) == 1 and int(vl[255]) == 256 and int(vl[256]) == 1
    assert int(kr[9]) == 1 and int(kr[10]) == 2 and int(kr[255]) == 26 and kmax == 26


def test_prefill_row_params_match_the_oracle_budget():
    """The library's keep budget (host helper of the C ABI) equals the
    oracle's exact-rational ceil(p (I + 1) / 100) on every row, for the
    32K and 128K layers and a constant budget; errors come back negative."""
    import numpy as np
    import long_context_sparse_apply_amd as sa
    from oracle import sparse_attention as O
    for N, kc, kp in ((256, 0, 10), (1024, 0, 5), (8, 4, 0), (77, 0, 33), (5, 0, 100)):
        vl, kr, kmax = sa.prefill_row_params(2, 3, N, keep_const=kc, keep_percent=kp, device="cpu")
        want = np.array(O.keep_budget(N, keep_const=kc, keep_percent=kp))
        assert np.array_equal(kr.numpy(), np.tile(want, 6)) and kmax == want.max()
        assert np.array_equal(vl.numpy(), np.tile(np.arange(1, N + 1), 6))
    vl, kr, _ = sa.prefill_row_params(1, 1, 10, keep_percent=10, causal=False, device="cpu")
    assert bool((vl == 10).all()) and bool((kr == 1).all())
    L = sa.lib
    assert L.sa_prefill_row_params(0, 4, 1, 0, 10, None, None) == -sa.SA_ERR_SHAPE
    assert L.sa_prefill_row_params(1 << 20, 1 << 12, 1, 0, 10, None, None) == -sa.SA_ERR_SHAPE
    assert L.sa_prefill_row_params(8, 4, 1, 0, 0, None, None) == -sa.SA_ERR_RANGE
    assert L.sa_prefill_row_params(8, 4, 1, 0, 101, None, None) == -sa.SA_ERR_RANGE
    assert L.sa_prefill_row_params(8, 4, 1, -1, 0, None, None) == -sa.SA_ERR_RANGE
    assert L.sa_prefill_row_params(8, 4, 1, 3, 0, None, None) == 3
