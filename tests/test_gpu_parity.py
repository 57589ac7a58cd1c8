"""GPU parity: every C-ABI entry point against the fp64 oracle on identical
seeded inputs.  Needs an MI355X; every call goes through the C ABI.

Staged tests feed both sides the same stored inputs (the same index lists for
the attention stages, drawn from a seeded numpy generator); the end-to-end
tests run the whole path on each side and compare scores, selections and the
attention over the GPU's own selection.  Every output is carved from a
guarded allocation (tests/guards.py) whose bands are checked after each call,
and the selection and attention stages are run twice and must repeat bit for
bit.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import sparse_attention as O
from synth import workloads as W
from tests.guards import check_all, guarded
from tests.parity_utils import LSE_ATOL_BF16, OUT_ATOL, assert_scores_close, check_selection, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import long_context_sparse_apply_amd as m
    import synth.device  # noqa: F401
    return m


def _dt(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def _host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _stored(shape, dtype, seed):
    """Seeded stored values (fp32 array holding exactly representable values)."""
    return synth.gaussian_tensor(seed, 8, shape, dtype)


def _dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(_dt(dtype))


# ----------------------------------------------------------------------------- generator
def test_device_generator_matches_host(sa):
    import synth.device as SD
    say("case: generator fp32 / bf16 / channel map")
    t = torch.empty((3, 5, 64), dtype=torch.float32, device=DEV)
    SD.fill(t, 7, synth.TID_K, base=11)
    ref = synth.gaussian_f32(7, synth.TID_K, np.arange(11, 11 + t.numel(), dtype=np.uint64))
    assert np.array_equal(t.cpu().numpy().ravel().view(np.uint32), ref.view(np.uint32))
    tb = torch.empty((4, 128), dtype=torch.bfloat16, device=DEV)
    SD.fill(tb, 3, synth.TID_Q)
    refb = synth.f32_to_bf16_bits(synth.gaussian_f32(3, synth.TID_Q, np.arange(512, dtype=np.uint64)))
    assert np.array_equal(tb.view(torch.int16).cpu().numpy().view(np.uint16).ravel(), refb)
    chmap = torch.tensor([[5, 1, 64], [0, 2, 127]], dtype=torch.int32, device=DEV)
    tm = torch.empty((2, 3, 3), dtype=torch.float32, device=DEV)  # 2 heads x 3 rows
    SD.fill(tm, 5, synth.TID_K, logical_d=128, chmap=chmap, rows_per_head=3, n_heads=2)
    full = synth.gaussian_f32(5, synth.TID_K, np.arange(6 * 128, dtype=np.uint64)).reshape(6, 128)
    want = np.stack([full[r, chmap.cpu().numpy()[r // 3]] for r in range(6)])
    assert np.array_equal(tm.cpu().numpy().reshape(6, 3), want)


# ----------------------------------------------------------------------------- RoPE
@pytest.mark.parametrize("dtype,d,pos0,use_pos", [("f32", 64, 0, False), ("bf16", 128, 131000, False),
                                                  ("bf16", 128, 0, True), ("f32", 128, 65530, True)])
def test_rope_apply(sa, dtype, d, pos0, use_pos):
    say(f"case: rope {dtype} d={d} pos0={pos0} pos_array={use_pos}")
    B, H, S, theta = 2, 3, 40, 5e5
    x = _stored((B, H, S, d), dtype, 1)
    pos = np.stack([np.arange(S) * 3277 + b for b in range(B)]).astype(np.int32) if use_pos else None
    xt = _dev(x, dtype)
    out, g_out = guarded(xt.shape, xt.dtype)
    sa.sa_rope_apply(xt, out, theta, pos=None if pos is None else torch.from_numpy(pos.ravel()).to(DEV),
                     pos0=pos0)
    torch.cuda.synchronize()
    g_out.check("rope out")
    ref = np.empty((B, H, S, d))
    for b in range(B):
        p = pos[b] if use_pos else pos0 + np.arange(S)
        ref[b] = O.rope(x[b].astype(np.float64), p, theta)
    got = _host(out)
    if dtype == "f32":
        assert np.abs(got - ref).max() < 1e-5
    else:  # one bf16 rounding of an fp32 value within 1e-6 of the reference
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5)
    # in place
    sa.sa_rope_apply(xt, xt, theta, pos=None if pos is None else torch.from_numpy(pos.ravel()).to(DEV),
                     pos0=pos0)
    assert torch.equal(xt, out)


# ----------------------------------------------------------------------------- block scores
BLOCK_CASES = [
    ("C1", W.C1, None),
    ("gqa-bf16-ragged", W.C2.with_(S=128 * 100, Hq=8, Hkv=2, needle_pairs=4), None),
    ("d64-bf16-block32-nocal", W.C1.with_(dtype="bf16", S=32 * 70, Hq=4, Hkv=4, block=32,
                                          needle_keys=0, calibrate=0), None),
    ("single-band-block256", W.C2.with_(S=256 * 12, Hq=4, Hkv=1, block=256, band_split_pair=0,
                                        needle_pairs=0), None),
    # the pooling pass's other thread shapes: 512 threads with one row a
    # thread (d 64, block 128), two rows (fp32 d 64, block 256) and four rows
    # (fp32 d 128, block 256); 256 threads over a block of 16 rows (half of
    # them idle)
    ("d64-bf16-block128", W.C1.with_(dtype="bf16", S=128 * 20, Hq=4, Hkv=2, block=128,
                                     needle_keys=0), None),
    ("d64-f32-block256", W.C1.with_(S=256 * 6, Hq=2, Hkv=1, block=256, needle_keys=0), None),
    ("d128-f32-block256", W.C2.with_(dtype="f32", S=256 * 5, Hq=4, Hkv=2, block=256,
                                     needle_pairs=0), None),
    ("d128-bf16-block16", W.C2.with_(S=16 * 90, Hq=4, Hkv=1, block=16, needle_pairs=0), None),
]


@pytest.mark.parametrize("name,cfg,_", BLOCK_CASES, ids=[c[0] for c in BLOCK_CASES])
def test_block_score(sa, name, cfg, _):
    say(f"case: block_score {name}")
    q, k, v, _h = W.prefill_inputs_host(cfg)
    qt, kt = _dev(q, cfg.dtype), _dev(k, cfg.dtype)
    N = cfg.N
    scores, g_s = guarded((cfg.B, cfg.Hq, N, N), torch.float32)
    pq, g_pq = guarded((cfg.B, cfg.Hq, N, cfg.d), torch.float32)
    pk, g_pk = guarded((cfg.B, cfg.Hkv, N, cfg.d), torch.float32)
    qr, g_qr = guarded(qt.shape, qt.dtype)
    kr, g_kr = guarded(kt.shape, kt.dtype)
    scale = cfg.d ** -0.5
    sa.sa_block_score(qt, kt, scores, theta=cfg.theta, block=cfg.block,
                      band_split_pair=cfg.band_split_pair, calibrate=bool(cfg.calibrate),
                      sm_scale=scale, causal=True, q_rope_out=qr, k_rope_out=kr,
                      pooled_q_out=pq, pooled_k_out=pk)
    torch.cuda.synchronize()
    check_all(("scores", g_s), ("pooled q", g_pq), ("pooled k", g_pk), ("rotated q", g_qr),
              ("rotated k", g_kr))
    pos = np.arange(cfg.S)
    q_rot = O.rope(q.astype(np.float64), pos, cfg.theta)
    k_rot = O.rope(k.astype(np.float64), pos, cfg.theta)
    rpq = O.pool_blocks(q_rot, cfg.block, cfg.band_split_pair, cfg.calibrate)
    rpk = O.pool_blocks(k_rot, cfg.block, cfg.band_split_pair, cfg.calibrate)
    rs = O.block_scores(rpq, rpk, scale, True)
    # pooled vectors: within 1e-4 of the vector's RMS
    for got, ref in ((_host(pq), rpq), (_host(pk), rpk)):
        rms = np.sqrt((ref ** 2).mean(axis=-1, keepdims=True))
        assert np.all(np.abs(got - ref) <= 1e-4 * rms + 1e-7)
    assert_scores_close(_host(scores), rs)
    # rotated outputs: one dtype rounding away from the fp64 rotation
    for got, ref in ((_host(qr), q_rot), (_host(kr), k_rot)):
        if cfg.dtype == "f32":
            assert np.abs(got - ref).max() < 1e-5
        else:
            assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5)
    # workspace variant (pooled outputs not requested) gives identical scores
    ws, g_ws = guarded((sa.workspace_bytes(sa.SA_OP_BLOCK_SCORE, cfg.B * (cfg.Hq + cfg.Hkv) * N,
                                           cfg.d),), torch.uint8)
    s2, g_s2 = guarded(scores.shape, scores.dtype)
    sa.sa_block_score(qt, kt, s2, theta=cfg.theta, block=cfg.block,
                      band_split_pair=cfg.band_split_pair, calibrate=bool(cfg.calibrate),
                      sm_scale=scale, causal=True, ws=ws)
    torch.cuda.synchronize()
    check_all(("workspace", g_ws), ("scores (workspace variant)", g_s2))
    assert torch.equal(s2, scores)


def test_block_score_q_rope_scale(sa):
    """q_rope_scale multiplies the stored rotated Q (one bf16 rounding of the
    fp32 product) and leaves the pooled vectors and the scores unchanged."""
    cfg = W.C2.with_(S=128 * 6, Hq=4, Hkv=2, needle_pairs=0)
    say("case: block_score q_rope_scale")
    q, k, v, _h = W.prefill_inputs_host(cfg)
    qt, kt = _dev(q, cfg.dtype), _dev(k, cfg.dtype)
    N, scale = cfg.N, cfg.d ** -0.5
    c = scale * np.log2(np.e)
    outs = []
    for qsc in (1.0, c):
        scores = torch.empty((cfg.B, cfg.Hq, N, N), dtype=torch.float32, device=DEV)
        pq = torch.empty((cfg.B, cfg.Hq, N, cfg.d), dtype=torch.float32, device=DEV)
        pk = torch.empty((cfg.B, cfg.Hkv, N, cfg.d), dtype=torch.float32, device=DEV)
        qr, kr = torch.empty_like(qt), torch.empty_like(kt)
        sa.sa_block_score(qt, kt, scores, theta=cfg.theta, block=cfg.block,
                          band_split_pair=cfg.band_split_pair, calibrate=True, sm_scale=scale,
                          causal=True, q_rope_out=qr, q_rope_scale=qsc, k_rope_out=kr,
                          pooled_q_out=pq, pooled_k_out=pk)
        outs.append((scores, pq, qr, kr))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[0][3], outs[1][3])
    q_rot = O.rope(q.astype(np.float64), np.arange(cfg.S), cfg.theta) * c
    got = _host(outs[1][2])
    assert np.all(np.abs(got - q_rot) <= 2.0 ** -8 * np.abs(q_rot) + 1e-5)


# ----------------------------------------------------------------------------- top-k
def _tricky_scores(rows, cols, seed):
    g = np.random.default_rng(seed)
    s = g.standard_normal((rows, cols)).astype(np.float32)
    s[:, ::7] = np.round(s[:, ::7])
    if rows > 5:
        s[0, :] = 1.0
        s[1, ::3] = np.nan
        s[2, ::2] = -0.0
        s[2, 1::2] = 0.0
        s[3, ::5] = -np.inf
        s[4, :] = -np.inf
    if rows > 8:
        s[6, :] = np.arange(cols, dtype=np.float32)            # best at the end
        s[7, :] = -np.arange(cols, dtype=np.float32)           # best at the start
        s[8, ::97] += 50.0                                     # sparse strong entries
    return s


TOPK_CASES = [  # rows, cols, k_const, n_sink, n_local, per-row valid_len, per-row k
    (40, 37, 5, 1, 2, True, True),
    (64, 128, 16, 0, 0, False, False),
    (33, 256, 26, 1, 2, True, True),
    (70, 1024, 52, 1, 2, True, True),
    (9, 1000, 0, 2, 0, True, False),
    (12, 5000, 300, 0, 0, True, False),
    (10, 65536, 2048, 0, 0, False, False),
    (7, 131072, 4096, 0, 0, True, False),
    (5, 20000, 4500, 3, 3, True, True),
]


@pytest.mark.parametrize("case", TOPK_CASES, ids=[f"r{c[0]}c{c[1]}k{c[2]}" for c in TOPK_CASES])
def test_topk_bit_exact(sa, case):
    rows, cols, kc, ns, nl, per_vl, per_k = case
    say(f"case: topk rows={rows} cols={cols} k={kc}")
    s = _tricky_scores(rows, cols, cols + kc)
    g = np.random.default_rng(rows * 7 + cols)
    vl = g.integers(0, cols + 1, rows).astype(np.int32) if per_vl else np.full(rows, cols, np.int32)
    if per_vl:
        vl[0] = cols
    kr = g.integers(0, kc + 1, rows).astype(np.int32) if per_k else np.full(rows, kc, np.int32)
    max_out = ns + nl + kc
    st = torch.from_numpy(s).to(DEV)
    runs = []
    for rep in range(2):  # a second call must repeat the first bit for bit
        idx, g_i = guarded((rows, max_out), torch.int32)
        cnt, g_c = guarded((rows,), torch.int32)
        sa.sa_topk_select(st, idx, cnt, k_const=kc,
                          valid_len=torch.from_numpy(vl).to(DEV) if per_vl else None,
                          k_per_row=torch.from_numpy(kr).to(DEV) if per_k else None,
                          n_sink=ns, n_local=nl)
        torch.cuda.synchronize()
        check_all(("idx", g_i), ("count", g_c))
        runs.append((idx, cnt))
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    for r in range(rows):
        ref = O.select_row(s[r].astype(np.float64), int(vl[r]), int(kr[r]), ns, nl)
        assert gc[r] == ref.size, (r, gc[r], ref.size)
        assert np.array_equal(gi[r, :gc[r]], ref), r
        assert np.all(gi[r, gc[r]:] == -1)


# ----------------------------------------------------------------------------- prefill attention
def _random_selection(B, Hq, N, max_sel, seed, causal=True, empty_rows=0):
    g = np.random.default_rng(seed)
    idx = np.full((B, Hq, N, max_sel), -1, np.int32)
    cnt = np.zeros((B, Hq, N), np.int32)
    sel = [[[None] * N for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            for I in range(N):
                hi = I + 1 if causal else N
                n = int(g.integers(1, min(max_sel, hi) + 1))
                ch = set(g.choice(hi, size=n, replace=False).tolist())
                if causal:
                    ch.add(I)
                    ch = set(sorted(ch)[-max_sel:]) if len(ch) > max_sel else ch
                if empty_rows and g.random() < 0.1:
                    ch = set()
                lst = sorted(ch)
                sel[b][h][I] = lst
                cnt[b, h, I] = len(lst)
                idx[b, h, I, :len(lst)] = lst
    return idx, cnt, sel


PREFILL_CASES = [  # name, dtype, B, Hq, Hkv, S, d, block, max_sel, causal, empty
    ("f32-d64-b64", "f32", 1, 1, 1, 512, 64, 64, 6, True, False),
    ("bf16-d128-b128-gqa", "bf16", 1, 8, 2, 2048, 128, 128, 6, True, False),
    ("bf16-d64-b64-batch2", "bf16", 2, 4, 1, 1024, 64, 64, 5, True, True),
    ("bf16-d128-b64-noncausal", "bf16", 1, 2, 2, 768, 128, 64, 4, False, False),
    ("bf16-d128-b32-plain", "bf16", 1, 2, 1, 256, 128, 32, 4, True, False),
    ("f32-d128-b128-dense", "f32", 1, 2, 1, 512, 128, 128, 4, True, False),
    ("bf16-d128-b128-grp8-batch2", "bf16", 2, 8, 1, 2048, 128, 128, 5, True, True),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_sparse_attn_prefill(sa, case):
    name, dtype, B, Hq, Hkv, S, d, block, max_sel, causal, empty = case
    say(f"case: prefill {name}")
    N = S // block
    q = _stored((B, Hq, S, d), dtype, 11)
    k = _stored((B, Hkv, S, d), dtype, 12)
    v = _stored((B, Hkv, S, d), dtype, 13)
    if name.endswith("dense"):
        max_sel = N
        idx = np.full((B, Hq, N, N), -1, np.int32)
        cnt = np.zeros((B, Hq, N), np.int32)
        sel = [[[list(range(I + 1)) for I in range(N)] for _ in range(Hq)] for _ in range(B)]
        for b in range(B):
            for h in range(Hq):
                for I in range(N):
                    idx[b, h, I, :I + 1] = np.arange(I + 1)
                    cnt[b, h, I] = I + 1
    else:
        idx, cnt, sel = _random_selection(B, Hq, N, max_sel, S + Hq, causal, empty)
    scale = d ** -0.5
    qd, kd, vd = _dev(q, dtype), _dev(k, dtype), _dev(v, dtype)
    idx_d, cnt_d = torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV)
    runs = []
    for rep in range(2):  # a second call must repeat the first bit for bit
        out, g_o = guarded((B, Hq, S, d), _dt(dtype))
        lse, g_l = guarded((B, Hq, S), torch.float32)
        sa.sa_sparse_attn_prefill(qd, kd, vd, idx_d, cnt_d, out, block=block, sm_scale=scale,
                                  causal=causal, lse=lse)
        torch.cuda.synchronize()
        check_all(("out", g_o), ("lse", g_l))
        runs.append((out, lse))
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])
    ref, rlse = O.prefill_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                    sel, block, scale, causal)
    got = _host(out)
    err = np.abs(got - ref).max()
    say(f"  max |out - ref| = {err:.3e}")
    assert err <= OUT_ATOL[dtype]
    gl = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(gl), fin)
    assert np.abs(gl[fin] - rlse[fin]).max() <= (1e-4 if dtype == "f32" else LSE_ATOL_BF16)


UNIT_CASES = [  # name, B, Hq, Hkv, S, d, block, max_sel, causal, empty, logit_gain
    ("d128-b128-gqa", 1, 8, 2, 2048, 128, 128, 6, True, False, 1.0),
    ("d128-b128-wide-logits", 1, 4, 1, 2048, 128, 128, 8, True, True, 40.0),
    ("d128-b64-wide-logits-noncausal", 1, 2, 2, 1024, 128, 64, 6, False, False, 40.0),
    ("d64-b64-wide-logits", 2, 2, 1, 1024, 64, 64, 5, True, False, 25.0),
    ("d64-b128-tiny-logits", 1, 2, 2, 1024, 64, 128, 4, True, False, 1e-3),
]


@pytest.mark.parametrize("case", UNIT_CASES, ids=[c[0] for c in UNIT_CASES])
def test_sparse_attn_prefill_base2(sa, case):
    """sm_scale = ln 2 (the float nearest): the bf16 kernel takes the logits as
    base-2 exponents as they stand.  Q holds the folded factor (here
    logit_gain * d^-1/2 * log2 e, rounded to bf16) and keys grow in size along
    the sequence, so with a large gain later chunks exceed the running
    reference by far more than 64 (base 2) and the reference moves several
    times per row."""
    name, B, Hq, Hkv, S, d, block, max_sel, causal, empty, gain = case
    say(f"case: prefill base-2 {name}")
    N = S // block
    c = gain * d ** -0.5 * np.log2(np.e)
    q = synth.round_to_bf16(_stored((B, Hq, S, d), "bf16", 21) * c)
    ramp = (1.0 + 3.0 * np.arange(S) / S)[None, None, :, None]
    k = synth.round_to_bf16(_stored((B, Hkv, S, d), "bf16", 22) * ramp)
    v = _stored((B, Hkv, S, d), "bf16", 23)
    idx, cnt, sel = _random_selection(B, Hq, N, max_sel, S + Hq + 7, causal, empty)
    out, g_o = guarded((B, Hq, S, d), torch.bfloat16)
    lse, g_l = guarded((B, Hq, S), torch.float32)
    ln2 = float(np.float32(np.log(2.0)))
    sa.sa_sparse_attn_prefill(_dev(q, "bf16"), _dev(k, "bf16"), _dev(v, "bf16"),
                              torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV), out,
                              block=block, sm_scale=ln2, causal=causal, lse=lse)
    torch.cuda.synchronize()
    check_all(("out", g_o), ("lse", g_l))
    ref, rlse = O.prefill_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                    sel, block, ln2, causal)
    err = np.abs(_host(out) - ref).max()
    say(f"  max |out - ref| = {err:.3e}")
    assert err <= OUT_ATOL["bf16"]
    gl = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(gl), fin)
    # Each base-2 logit is an fp32 sum of d exact bf16 products started from
    # -m_ref, a multiple of 64 with |m_ref| <= A + 32, A = max over keys of
    # sum_i |q_i k_i|: its error is at most (d + 1) 2^-24 (2 A + 32).  lse
    # (natural) moves by at most ln 2 times that, on top of the bf16 bound.
    grp = Hq // Hkv
    A = np.stack([np.abs(q[:, h]) @ np.abs(k[:, h // grp]).transpose(0, 2, 1) for h in range(Hq)],
                 axis=1).max(axis=-1)
    tol = LSE_ATOL_BF16 + np.log(2.0) * (d + 1) * 2.0 ** -24 * (2 * A + 32)
    assert np.all(np.abs(gl[fin] - rlse[fin]) <= tol[fin])


# ----------------------------------------------------------------------------- token scores
TOKEN_CASES = [  # name, dtype, B, Hq, Hkv, L, d, n_dom, slab, ragged
    ("bf16-std", "bf16", 2, 8, 2, 3000, 128, 16, 0, 500),
    ("bf16-slab", "bf16", 3, 32, 8, 1024, 128, 16, 1, 300),
    ("f32-std-d64", "f32", 1, 4, 4, 777, 64, 5, 0, 0),
    ("f32-slab-grp8", "f32", 2, 8, 1, 600, 128, 32, 1, 100),
]


def _decode_case_inputs(dtype, B, Hq, Hkv, L, d, n_dom, ragged, seed):
    cfg = W.C4.with_(dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, n_dom=n_dom, ragged=ragged,
                     seed=seed, needles_per_head=2)
    x = W.decode_inputs_host(cfg)
    return cfg, x


@pytest.mark.parametrize("case", TOKEN_CASES, ids=[c[0] for c in TOKEN_CASES])
def test_token_score(sa, case):
    name, dtype, B, Hq, Hkv, L, d, n_dom, slab, ragged = case
    say(f"case: token_score {name}")
    cfg, x = _decode_case_inputs(dtype, B, Hq, Hkv, L, d, n_dom, ragged, 21)
    q_rot = O.decode_query(x["q_raw"].astype(np.float64), x["lens"], cfg.theta)
    q_store = synth.round_to_bf16(q_rot) if dtype == "bf16" else q_rot.astype(np.float32)
    kf = x["k"].astype(np.float64)
    ref = O.token_scores(q_store.astype(np.float64), kf, x["dom"], x["lens"], d ** -0.5)
    scores, g_s = guarded((B, Hq, L), torch.float32)
    dom_t = torch.from_numpy(x["dom"]).to(DEV)
    if slab:
        kd, _kr = O.standard_to_slab(x["k"], x["dom"])
        ktensor = _dev(kd, dtype)
    else:
        ktensor = _dev(x["k"], dtype)
    sa.sa_token_score(_dev(q_store, dtype), ktensor, scores, torch.from_numpy(x["lens"]).to(DEV),
                      dom_t, sm_scale=d ** -0.5, slab=bool(slab))
    torch.cuda.synchronize()
    g_s.check("scores")
    assert_scores_close(_host(scores), ref)


# ----------------------------------------------------------------------------- decode attention
DECODE_CASES = [  # name, dtype, B, Hq, Hkv, L, d, n_dom, slab, max_k
    ("bf16-std", "bf16", 2, 8, 2, 3000, 128, 16, 0, 700),
    ("bf16-slab", "bf16", 2, 8, 2, 2048, 128, 16, 1, 512),
    ("bf16-std-grp8", "bf16", 2, 16, 2, 2000, 128, 16, 0, 500),
    ("bf16-slab-grp8", "bf16", 1, 8, 1, 2500, 128, 8, 1, 800),
    ("f32-std-d64", "f32", 2, 4, 1, 999, 64, 8, 0, 300),
    ("f32-slab", "f32", 1, 4, 4, 1500, 128, 8, 1, 1100),
    ("bf16-std-d64", "bf16", 2, 4, 2, 2500, 64, 8, 0, 600),
    ("bf16-slab-d64", "bf16", 2, 4, 1, 1800, 64, 8, 1, 500),
    # B*Hq >= 512: one work-group per selection list (online softmax across its chunks)
    ("bf16-std-onepass", "bf16", 16, 32, 8, 1200, 128, 16, 0, 700),
    ("bf16-slab-onepass", "bf16", 16, 32, 8, 1100, 128, 16, 1, 900),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_sparse_attn_decode(sa, case):
    name, dtype, B, Hq, Hkv, L, d, n_dom, slab, max_k = case
    say(f"case: decode {name}")
    cfg, x = _decode_case_inputs(dtype, B, Hq, Hkv, L, d, n_dom, 200, 31)
    q = _stored((B, Hq, d), dtype, 32)  # used directly as the rotated query
    g = np.random.default_rng(L)
    tok = np.full((B, Hq, max_k), -1, np.int32)
    cnt = np.zeros((B, Hq), np.int32)
    sel = [[None] * Hq for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            n = 0 if (b == 0 and h == 1) else int(g.integers(1, min(max_k, x["lens"][b]) + 1))
            t = np.sort(g.choice(int(x["lens"][b]), size=n, replace=False)).astype(np.int32)
            tok[b, h, :n] = t
            cnt[b, h] = n
            sel[b][h] = t
    ref, rlse = O.decode_attention(q.astype(np.float64), x["k"].astype(np.float64),
                                   x["v"].astype(np.float64), sel, d ** -0.5)
    ws, g_ws = guarded((sa.workspace_bytes(sa.SA_OP_DECODE, B=B, Hq=Hq, max_k=max_k),), torch.uint8)
    kw = {}
    if slab:
        kd, kr = O.standard_to_slab(x["k"], x["dom"])
        ktensor, kw["k_rest"] = _dev(kd, dtype), _dev(kr, dtype)
        kw["dom_pairs"] = torch.from_numpy(x["dom"]).to(DEV)
    else:
        ktensor = _dev(x["k"], dtype)
    qd, vd = _dev(q, dtype), _dev(x["v"], dtype)
    tok_d, cnt_d = torch.from_numpy(tok).to(DEV), torch.from_numpy(cnt).to(DEV)
    runs = []
    for rep in range(2):  # a second call must repeat the first bit for bit
        out, g_o = guarded((B, Hq, d), _dt(dtype))
        lse, g_l = guarded((B, Hq), torch.float32)
        sa.sa_sparse_attn_decode(qd, ktensor, vd, tok_d, cnt_d, out, ws, sm_scale=d ** -0.5,
                                 cache_len=torch.from_numpy(x["lens"]).to(DEV), slab=bool(slab),
                                 lse=lse, **kw)
        torch.cuda.synchronize()
        check_all(("out", g_o), ("lse", g_l), ("workspace", g_ws))
        runs.append((out, lse))
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])
    err = np.abs(_host(out) - ref).max()
    say(f"  max |out - ref| = {err:.3e}")
    assert err <= OUT_ATOL[dtype]
    gl = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(gl), fin)
    assert np.abs(gl[fin] - rlse[fin]).max() <= (1e-4 if dtype == "f32" else 1e-2)


# ----------------------------------------------------------------------------- count clamping
@pytest.mark.parametrize("dtype,block", [("bf16", 128), ("f32", 64)], ids=["bf16-mfma", "f32-plain"])
def test_prefill_count_above_width_is_clamped(sa, dtype, block):
    """blk_cnt above max_sel (a caller's stale buffer) is clamped on the
    device to max_sel, and a negative count to 0: the output equals the one
    with the count at the width, bit for bit, and a clamped-empty row gives
    out = 0, lse = -inf.  The lists sit in a guarded allocation, so even an
    unclamped read would stay inside it."""
    say(f"case: prefill count clamping {dtype} block {block}")
    B, Hq, Hkv, S, d, max_sel = 1, 2, 1, 1024, 128, 4
    N = S // block
    q = _stored((B, Hq, S, d), dtype, 41)
    k = _stored((B, Hkv, S, d), dtype, 42)
    v = _stored((B, Hkv, S, d), dtype, 43)
    idx, _cnt, _sel = _random_selection(B, Hq, N, max_sel, 5, True, False)
    qd, kd, vd = _dev(q, dtype), _dev(k, dtype), _dev(v, dtype)
    idx_d, g_idx = guarded(idx.shape, torch.int32)
    idx_d.copy_(torch.from_numpy(idx))
    full = np.array([[[min(max_sel, int((idx[0, h, I] >= 0).sum())) for I in range(N)]
                      for h in range(Hq)]], np.int32)
    outs = []
    for cnt in (full, np.where(full == max_sel, max_sel + 1000, full).astype(np.int32),
                np.full_like(full, -3)):
        out, g_o = guarded((B, Hq, S, d), _dt(dtype))
        lse, g_l = guarded((B, Hq, S), torch.float32)
        sa.sa_sparse_attn_prefill(qd, kd, vd, idx_d, torch.from_numpy(cnt).to(DEV), out,
                                  block=block, sm_scale=d ** -0.5, causal=True, lse=lse)
        torch.cuda.synchronize()
        check_all(("out", g_o), ("lse", g_l), ("idx", g_idx))
        outs.append((out, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert bool((outs[2][0] == 0).all()) and bool(torch.isneginf(outs[2][1]).all())


@pytest.mark.parametrize("dtype,block", [("bf16", 128), ("bf16", 64), ("f32", 64)],
                         ids=["bf16-b128", "bf16-b64", "f32-plain"])
def test_prefill_unusable_entries_are_skipped(sa, dtype, block):
    """List entries outside [0, N) and, with the causal mask, above the
    diagonal are skipped wherever they sit in the list (first entry
    included): the output matches the oracle over the usable entries only,
    and a list of unusable entries alone gives out = 0, lse = -inf."""
    say(f"case: prefill unusable list entries {dtype} block {block}")
    B, Hq, Hkv, S, d, max_sel = 1, 4, 1, 1024, 128, 9
    N = S // block
    q = _stored((B, Hq, S, d), dtype, 51)
    k = _stored((B, Hkv, S, d), dtype, 52)
    v = _stored((B, Hkv, S, d), dtype, 53)
    g = np.random.default_rng(54)
    idx = np.full((B, Hq, N, max_sel), -1, np.int32)
    cnt = np.zeros((B, Hq, N), np.int32)
    sel = [[[None] * N for _ in range(Hq)]]
    for h in range(Hq):
        for I in range(N):
            good = sorted(set(g.choice(I + 1, size=min(I + 1, 3), replace=False).tolist()) | {I})
            if h == Hq - 1 and I % 3 == 0:
                good = []  # only unusable entries
            bad = [-1, N + 5, -7] + ([I + 1] if I + 1 < N else [N])
            lst = list(good)
            for j, x in enumerate(bad):  # the first bad one goes first, the rest in between
                lst.insert(0 if j == 0 else int(g.integers(0, len(lst) + 1)), x)
            lst = lst[:max_sel]
            idx[0, h, I, :len(lst)] = lst
            cnt[0, h, I] = len(lst)
            sel[0][h][I] = sorted(x for x in lst if 0 <= x <= I)
    qd, kd, vd = _dev(q, dtype), _dev(k, dtype), _dev(v, dtype)
    idx_d, g_idx = guarded(idx.shape, torch.int32)
    idx_d.copy_(torch.from_numpy(idx))
    out, g_o = guarded((B, Hq, S, d), _dt(dtype))
    lse, g_l = guarded((B, Hq, S), torch.float32)
    scale = d ** -0.5
    sa.sa_sparse_attn_prefill(qd, kd, vd, idx_d, torch.from_numpy(cnt).to(DEV), out, block=block,
                              sm_scale=scale, causal=True, lse=lse)
    torch.cuda.synchronize()
    check_all(("out", g_o), ("lse", g_l), ("idx", g_idx))
    ref, rlse = O.prefill_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                    sel, block, scale, True)
    got = _host(out)
    err = np.abs(got - ref).max()
    say(f"  max |out - ref| = {err:.3e}")
    assert err <= OUT_ATOL[dtype]
    gl = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(gl), fin)
    assert np.abs(gl[fin] - rlse[fin]).max() <= (1e-4 if dtype == "f32" else LSE_ATOL_BF16)
    for I in range(0, N, 3):  # the lists of unusable entries alone
        rows = slice(I * block, (I + 1) * block)
        assert bool((out[0, Hq - 1, rows] == 0).all()) and bool(torch.isneginf(lse[0, Hq - 1, rows]).all())


@pytest.mark.parametrize("B,Hq", [(2, 8), (16, 32)], ids=["split-k", "one-pass"])
def test_decode_count_above_width_is_clamped(sa, B, Hq):
    """tok_cnt above max_k is clamped on the device to max_k (negative to 0)."""
    say(f"case: decode count clamping B={B} Hq={Hq}")
    dtype, Hkv, L, d, max_k = "bf16", 8 if Hq == 32 else 2, 1500, 128, 600
    cfg, x = _decode_case_inputs(dtype, B, Hq, Hkv, L, d, 16, 0, 44)
    q = _stored((B, Hq, d), dtype, 45)
    g = np.random.default_rng(46)
    tok = np.stack([[np.sort(g.choice(L, size=max_k, replace=False)) for _ in range(Hq)]
                    for _ in range(B)]).astype(np.int32)
    tok_d, g_tok = guarded(tok.shape, torch.int32)
    tok_d.copy_(torch.from_numpy(tok))
    ws, g_ws = guarded((sa.workspace_bytes(sa.SA_OP_DECODE, B=B, Hq=Hq, max_k=max_k),), torch.uint8)
    qd, kd, vd = _dev(q, dtype), _dev(x["k"], dtype), _dev(x["v"], dtype)
    outs = []
    for c in (max_k, max_k + 77, -1):
        cnt = torch.full((B, Hq), c, dtype=torch.int32, device=DEV)
        out, g_o = guarded((B, Hq, d), torch.bfloat16)
        lse, g_l = guarded((B, Hq), torch.float32)
        sa.sa_sparse_attn_decode(qd, kd, vd, tok_d, cnt, out, ws, sm_scale=d ** -0.5, lse=lse)
        torch.cuda.synchronize()
        check_all(("out", g_o), ("lse", g_l), ("workspace", g_ws), ("tok_idx", g_tok))
        outs.append((out, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert bool((outs[2][0] == 0).all()) and bool(torch.isneginf(outs[2][1]).all())
