"""GPU parity of Sparse Feature Attention ("Scaling Attention via Feature
Sparsity", sec. 2): the k-sparse codes bit for bit, and attention over the
codes against the oracle (2e-2 absolute for bf16, 1e-5 for fp32)."""
import numpy as np
import pytest
import torch

import synth
from oracle import feature_sparse as F
from tests.parity_utils import LSE_ATOL_BF16, OUT_ATOL, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import long_context_sparse_apply_amd as m
    return m


def _dev(a, dtype):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(dt)


def _inputs(shape, dtype, seed, tid=synth.TID_Q, ties=False):
    x = synth.gaussian_tensor(seed, tid, shape, dtype).astype(np.float64)
    if ties:  # coarse values: many equal magnitudes inside a row
        x = np.round(x * 2.0) / 2.0
    return x


@pytest.mark.parametrize("dtype,d,rows,kf,ties", [
    ("bf16", 128, 1001, 16, False), ("bf16", 128, 1001, 16, True), ("bf16", 128, 64, 1, True),
    ("bf16", 128, 64, 128, False), ("bf16", 128, 64, 200, False), ("bf16", 128, 64, 0, False),
    ("f32", 64, 333, 8, True), ("f32", 64, 333, 37, False)])
def test_sparsify_bit_exact(sa, dtype, d, rows, kf, ties):
    say(f"case: sfa sparsify {dtype} d={d} rows={rows} k={kf} ties={ties}")
    x = _inputs((rows, d), dtype, 21, ties=ties)
    xt = _dev(x, dtype)
    out = torch.full_like(xt, 7.0)
    sa.sa_sfa_sparsify(xt, out, k_feat=kf)
    torch.cuda.synchronize()
    ref = F.sparsify(x, kf)
    assert np.array_equal(out.float().cpu().numpy().astype(np.float64), ref)
    # in place gives the same codes
    sa.sa_sfa_sparsify(xt, xt, k_feat=kf)
    torch.cuda.synchronize()
    assert torch.equal(xt, out)


@pytest.mark.parametrize("dtype,Hq,Hkv,S,d,kf", [
    ("bf16", 4, 2, 1024, 128, 16), ("bf16", 2, 2, 512, 64, 8), ("f32", 2, 1, 256, 128, 16)])
def test_sfa_attention(sa, dtype, Hq, Hkv, S, d, kf):
    from long_context_sparse_apply_amd.pipeline import SFALayer
    say(f"case: sfa attention {dtype} Hq={Hq} Hkv={Hkv} S={S} d={d} k={kf}")
    q = _inputs((1, Hq, S, d), dtype, 22, synth.TID_Q)
    k = _inputs((1, Hkv, S, d), dtype, 22, synth.TID_K)
    v = _inputs((1, Hkv, S, d), dtype, 22, synth.TID_V)
    layer = SFALayer(_dev(q, dtype), _dev(k, dtype), _dev(v, dtype), k_feat=kf, block=64 if S <= 512 else 128)
    layer.run()
    torch.cuda.synchronize()
    assert np.array_equal(layer.q_code.float().cpu().numpy().astype(np.float64), F.sparsify(q, kf))
    ref, ref_lse = F.sfa_attention(q, k, v, kf, d ** -0.5)
    err = np.abs(layer.out.float().cpu().numpy() - ref).max()
    assert err <= OUT_ATOL[dtype], err
    assert np.abs(layer.lse.cpu().numpy() - ref_lse).max() <= (LSE_ATOL_BF16 if dtype == "bf16" else 1e-5)


def test_sfa_attention_llama_shaped_sampled(sa):
    """The bench's launch shape (32 query / 8 KV heads, 8192 tokens, k = 16)
    with sampled heads and query rows checked against the oracle."""
    from long_context_sparse_apply_amd.pipeline import SFALayer
    Hq, Hkv, S, d, kf = 32, 8, 8192, 128, 16
    say("case: sfa attention 32/8 heads, 8192 tokens, sampled")
    q = _inputs((1, Hq, S, d), "bf16", 23, synth.TID_Q)
    k = _inputs((1, Hkv, S, d), "bf16", 23, synth.TID_K)
    v = _inputs((1, Hkv, S, d), "bf16", 23, synth.TID_V)
    layer = SFALayer(_dev(q, "bf16"), _dev(k, "bf16"), _dev(v, "bf16"), k_feat=kf)
    layer.run()
    torch.cuda.synchronize()
    out = layer.out.float().cpu().numpy()
    rows = np.array([0, 1, 127, 128, 4095, 8191])
    for h in (0, 13, 31):
        g = h // (Hq // Hkv)
        qs = F.sparsify(q[0, h, rows], kf)
        ks = F.sparsify(k[0, g], kf)
        s = d ** -0.5 * (qs @ ks.T)
        s = np.where(np.arange(S)[None, :] <= rows[:, None], s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        ref = (p @ v[0, g]) / p.sum(axis=1, keepdims=True)
        err = np.abs(out[0, h, rows] - ref).max()
        assert err <= OUT_ATOL["bf16"], (h, err)
