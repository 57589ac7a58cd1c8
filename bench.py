"""Benchmark of the sparse-attention hot path on one MI355X.

A step is one prefill layer of the 32K-token Llama-3.1-8B-shaped workload
(32 query / 8 KV heads, d=128, bf16, block 128, keep 10% + sink + 2 local):
fused RoPE + dual-band pooling + block scores, block top-k, and block-sparse
attention.  Inputs are generated in HBM before timing.  The JSON line also
carries the 128K prefill layer and the 64K / 128K decode steps measured in
the same run ("secondary"), the roofline of the dominant kernel, and the
fp64 CPU oracle timed on the same 32K layer.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-secondary] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse prefill tok/s @32K/128K; decode µs/step @64K; % MFMA/HBM peak"
PEAK_BF16_FLOPS = 2.5e15
PEAK_HBM_BPS = 8.0e12
# counter summary of the prefill attention kernel and the source it measured
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "prefill_attn_mfma_32k_traffic.md")
PREFILL_SOURCE = os.path.join(ROOT, "long_context_sparse_apply_amd", "csrc", "attn_prefill.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def prefill_flops(blk_idx, blk_cnt, block, d, causal=True):
    """Algorithmic FLOPs of the sparse attention: 4*d per unmasked selected
    (query, key) pair; also the tile FLOPs (diagonal tiles counted whole)."""
    B, Hq, N, _ = blk_idx.shape
    pairs = 0
    tiles = 0
    for I in range(N):
        c = blk_cnt[:, :, I]
        sel = blk_idx[:, :, I, :]
        valid = (np.arange(sel.shape[-1])[None, None, :] < c[..., None]) & (sel >= 0)
        below = valid & (sel < I)
        diag = valid & (sel == I)
        pairs += int(below.sum()) * block * block + int(diag.sum()) * block * (block + 1) // 2
        tiles += int((below | diag).sum()) * block * block
    return 4.0 * d * pairs, 4.0 * d * tiles


def decode_bytes(tok_cnt, d, elem=2):
    """Gathered K and V bytes per call: every selected token of every (b, h)."""
    return float(tok_cnt.sum()) * 2 * d * elem


def decode_dedup_bytes(tok_idx, tok_cnt, hkv, d, elem=2):
    """K and V bytes if each KV head's rows were gathered once for its query heads:
    the union of the selections of the query heads that share a KV head."""
    B, Hq, _ = tok_idx.shape
    grp = Hq // hkv
    rows = 0
    for b in range(B):
        for g in range(hkv):
            sel = [tok_idx[b, h, :tok_cnt[b, h]] for h in range(g * grp, (g + 1) * grp)]
            rows += np.unique(np.concatenate(sel)).size
    return float(rows) * 2 * d * elem


class CacheFlush:
    """Reads a 1 GiB buffer before each timed step, so L2 and the MALL hold
    nothing from the previous iteration.  A read sweep, not a fill: the
    previous step's dirty lines are written back during the sweep, and the
    sweep leaves no dirty lines of its own to be written back inside the
    timed step.  Not timed."""

    def __init__(self, torch, enabled=True):
        self.buf = None
        self.torch = torch
        if enabled:
            self.buf = torch.zeros(1 << 27, dtype=torch.int64, device="cuda")  # 1 GiB
            self.out = torch.empty((), dtype=torch.int64, device="cuda")

    def __call__(self):
        if self.buf is not None:
            self.torch.amax(self.buf, dim=0, out=self.out)


def _stats(x):
    x = np.asarray(x, dtype=np.float64)
    return float(np.median(x)), float(np.percentile(x, 10)), float(np.percentile(x, 90))


def time_prefill(layer, steps, warmup, torch, flush):
    for _ in range(warmup):
        layer.run()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        flush()
        e = ev[i]
        e[0].record()
        layer.score()
        e[1].record()
        layer.select()
        e[2].record()
        layer.attend()
        e[3].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    parts = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in ev])  # ms
    step = np.array([e[0].elapsed_time(e[3]) for e in ev])
    r = dict(wall_ms=wall * 1e3, attend_ms_mean=float(parts[:, 2].mean()))
    for name, col in (("step_ms", step), ("score_ms", parts[:, 0]), ("select_ms", parts[:, 1]),
                      ("attend_ms", parts[:, 2])):
        r[name], r[name + "_p10"], r[name + "_p90"] = _stats(col)
    return r


def time_decode(step, steps, warmup, torch, flush):
    """Per-stage HIP-event times of the decode step.  A fused step (slab
    layout: one sa_token_topk call scores and selects) has no score / select
    split: score_us and select_us are None and score_select_us covers both."""
    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for i in range(steps):
        flush()
        e = ev[i]
        e[0].record()
        step.rope()
        e[1].record()
        if step.fused:
            step.score_select()
            e[2].record()
        else:
            step.score()
            e[2].record()
            step.select()
        e[3].record()
        step.attend()
        e[4].record()
    torch.cuda.synchronize()
    parts = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in ev]) * 1e3
    total = np.array([e[0].elapsed_time(e[4]) for e in ev]) * 1e3
    r = dict(attend_us_mean=float(parts[:, 3].mean()), fused=bool(step.fused))
    cols = [("step_us", total), ("rope_us", parts[:, 0]), ("attend_us", parts[:, 3]),
            ("score_select_us", parts[:, 1] + parts[:, 2])]
    if not step.fused:
        cols += [("score_us", parts[:, 1]), ("select_us", parts[:, 2])]
    else:
        r["score_us"] = r["select_us"] = None
    for name, col in cols:
        r[name], r[name + "_p10"], r[name + "_p90"] = _stats(col)
    return r


def time_call(fn, steps, warmup, torch, flush):
    """Median / p10 / p90 (us) of one enqueued call, HIP events around it."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for e0, e1 in ev:
        flush()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return _stats(np.array([e0.elapsed_time(e1) for e0, e1 in ev]) * 1e3)


def run_decode_host_rest(cfg, steps, warmup, torch, flush):
    """FASA-M placement (memory-optimised variant): the dominant slab and the
    scores in device memory; the non-dominant key channels and the values in
    pinned host memory.  Scoring reads the slab only; the attention reads the
    selected rows of k_rest and v over the host link.  Host-link bytes per
    step = selected (b, h, token) x (rest-of-key + value row bytes)."""
    import synth.device as SD
    from long_context_sparse_apply_amd.pipeline import DecodeStep
    dt = SD.decode_tensors(cfg)
    k_rest = torch.empty(dt["k_rest"].shape, dtype=dt["k_rest"].dtype, pin_memory=True)
    v = torch.empty(dt["v"].shape, dtype=dt["v"].dtype, pin_memory=True)
    k_rest.copy_(dt["k_rest"])
    v.copy_(dt["v"])
    torch.cuda.synchronize()
    del dt["k_rest"], dt["v"]
    torch.cuda.empty_cache()
    step = DecodeStep(dt["q_raw"], dt["k"], v, dt["lens"], dt["dom"], theta=cfg.theta,
                      top_k=cfg.k, slab=True, k_rest=k_rest)
    t = time_decode(step, steps, warmup, torch, flush)
    cnt = step.tok_cnt.cpu().numpy()
    row_host = (cfg.d - 2 * cfg.n_dom) * 2 + cfg.d * 2
    host_bytes = float(cnt.sum()) * row_host
    t["host_link_bytes"] = host_bytes
    t["host_link_GBps"] = host_bytes / (t["attend_us"] * 1e-6) / 1e9
    t["device_resident_bytes"] = float(dt["k"].numel() * 2)
    t["host_resident_bytes"] = float((k_rest.numel() + v.numel()) * 2)
    del step, dt, k_rest, v
    torch.cuda.empty_cache()
    return t


def run_calibration(cfg, steps, warmup, torch, flush):
    """The one-time calibration of the dominant pairs (FASA sec. 2.B item 1)
    on a Llama-shaped window.  Algorithmic bytes: the keys and queries read
    once, the full and pair scores written once and read once by the top-k,
    their selections written once and read once by the overlap count."""
    from long_context_sparse_apply_amd import calibrate_workspace_bytes, sa_calibrate_dominant
    from synth import workloads as W
    q, k, planted = W.calibration_inputs_host(cfg)
    qt = torch.from_numpy(q).to("cuda").to(torch.bfloat16)
    kt = torch.from_numpy(k).to("cuda").to(torch.bfloat16)
    ws = torch.empty(calibrate_workspace_bytes(cfg.Hq, cfg.Hkv, cfg.M, cfg.L, cfg.d, cfg.k_cal),
                     dtype=torch.uint8, device="cuda")
    dom = torch.empty((cfg.Hkv, cfg.n_dom), dtype=torch.int32, device="cuda")
    counts = torch.empty((cfg.Hkv, cfg.d // 2), dtype=torch.int32, device="cuda")

    def fn():
        sa_calibrate_dominant(qt, kt, dom, counts, ws, k_cal=cfg.k_cal)
    med, p10, p90 = time_call(fn, steps, warmup, torch, flush)
    rows = cfg.Hq * cfg.M * (cfg.d // 2 + 1)
    nbytes = (qt.numel() + kt.numel()) * 2 + 2.0 * rows * cfg.L * 4 + 2.0 * rows * cfg.k_cal * 4
    recovered = bool((dom.cpu().numpy() == planted).all())
    del qt, kt, ws
    torch.cuda.empty_cache()
    return {"workload": cfg.name, "us": med, "us_p10_p90": [p10, p90], "bytes": nbytes,
            "hbm_frac": nbytes / (med * 1e-6) / PEAK_HBM_BPS, "planted_set_recovered": recovered}


def run_sfa(steps, warmup, torch, flush, S=8192, Hq=32, Hkv=8, d=128, kf=16):
    """Sparse Feature Attention over one causal prefill layer: k-sparse codes
    of Q and K, then exact attention over every causal block of the codes on
    the matrix unit.  FLOPs counted as the kernel performs them: 4 d per
    visible (query, key) pair."""
    import synth
    import synth.device as SD
    from long_context_sparse_apply_amd.pipeline import SFALayer
    q = torch.empty((1, Hq, S, d), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((1, Hkv, S, d), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    SD.fill(q, 23, synth.TID_Q)
    SD.fill(k, 23, synth.TID_K)
    SD.fill(v, 23, synth.TID_V)
    layer = SFALayer(q, k, v, k_feat=kf)
    codes = time_call(layer.codes, steps, warmup, torch, flush)
    attend = time_call(layer.attend, steps, warmup, torch, flush)
    flops = 4.0 * d * Hq * S * (S + 1) / 2
    res = {"workload": f"SFA causal prefill, {Hq} query / {Hkv} KV heads, {S} tokens, d={d}, "
                       f"k={kf} active channels per token, bf16",
           "codes_us": codes[0], "attend_ms": attend[0] / 1e3,
           "tok_per_s": S / ((codes[0] + attend[0]) * 1e-6),
           # the dense matrix-unit work the kernel performs over the zero-filled
           # codes (4 d per visible pair), not the method's intersection work
           # (about (k/d)^2 of it), so a rate of the kernel, not of SFA
           "attend_dense_equiv_tflops": flops / (attend[0] * 1e-6) / 1e12,
           "attend_dense_equiv_mfma_frac": flops / (attend[0] * 1e-6) / PEAK_BF16_FLOPS,
           "intersection_flops_share": (kf / d) ** 2}
    del layer, q, k, v
    torch.cuda.empty_cache()
    return res


def run_cache_append(cfg_p, cfg_d, steps, warmup, torch, flush):
    """sa_kv_cache_append at its two uses: the prefill -> decode handoff (the
    whole prompt's keys rotated and values copied into a decode cache) and one
    decode token per batch row.  Algorithmic bytes: raw K and V read once,
    rotated K and V written once."""
    import synth
    import synth.device as SD
    from long_context_sparse_apply_amd import sa_kv_cache_append
    from synth import workloads as W
    dev = "cuda"
    q, k, v = SD.prefill_tensors(cfg_p)
    del q
    dom = torch.from_numpy(W.dominant_pairs(cfg_d)).to(dev)
    n = dom.shape[1]
    out = {}

    def one(name, k_new, v_new, Lmax, start_row):
        B, Hkv, S, d = k_new.shape
        start = torch.full((B,), start_row, dtype=torch.int32, device=dev)
        for slab in (False, True):
            kc = torch.zeros((B, Hkv, Lmax, 2 * n if slab else d), dtype=k_new.dtype, device=dev)
            kr = (torch.zeros((B, Hkv, Lmax, d - 2 * n), dtype=k_new.dtype, device=dev)
                  if slab else None)
            vc = torch.zeros((B, Hkv, Lmax, d), dtype=k_new.dtype, device=dev)

            def fn():
                sa_kv_cache_append(k_new, v_new, start, kc, vc, theta=cfg_p.theta, k_rest=kr,
                                   dom_pairs=dom if slab else None, slab=slab)
            med, p10, p90 = time_call(fn, steps, warmup, torch, flush)
            nbytes = 4.0 * k_new.numel() * k_new.element_size()
            key = f"{name}_{'slab' if slab else 'std'}"
            out[key] = {"us": med, "us_p10_p90": [p10, p90], "bytes": nbytes,
                        "hbm_frac": nbytes / (med * 1e-6) / PEAK_HBM_BPS}
            del kc, kr, vc
    one("prompt_32k", k, v, cfg_p.S, 0)
    del k, v
    kt = torch.empty((cfg_d.B, cfg_d.Hkv, 1, cfg_d.d), dtype=torch.bfloat16, device=dev)
    vt = torch.empty_like(kt)
    SD.fill(kt, cfg_d.seed, synth.TID_K)
    SD.fill(vt, cfg_d.seed, synth.TID_V)
    one("token_b64", kt, vt, 4096, 4000)
    torch.cuda.empty_cache()
    return out


def copy_reference(torch, reps=5):
    """Achieved GB/s of a 1 GiB device-to-device copy (1 GiB read + 1 GiB
    written), timed in the same run as a practical HBM reference."""
    src = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * (1 << 30) / (float(np.median(ts)) * 1e-3) / 1e9


def gemm_reference(torch, n=8192, per_group=25, groups=3):
    """Achieved TFLOP/s of a plain bf16 matrix product (n x n times n x n,
    contiguous operands, torch.matmul on the vendor GEMM library), timed in
    the same run as a practical matrix-unit reference: `per_group` products
    back to back between two events, so the chip settles at the clock it
    sustains under matrix load; the median over `groups` groups."""
    a = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    c = torch.matmul(a, b)
    torch.cuda.synchronize()
    ts = []
    for _ in range(groups):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(per_group):
            torch.matmul(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / per_group)
    del a, b, c
    torch.cuda.empty_cache()
    return 2.0 * n ** 3 / (float(np.median(ts)) * 1e-3) / 1e12


def run_prefill(cfg, steps, warmup, torch, flush):
    import synth.device as SD
    from long_context_sparse_apply_amd.pipeline import PrefillLayer
    q, k, v = SD.prefill_tensors(cfg)
    layer = PrefillLayer(q, k, v, theta=cfg.theta, block=cfg.block,
                         band_split_pair=cfg.band_split_pair, n_sink=cfg.n_sink,
                         n_local=cfg.n_local, keep_const=cfg.keep_const,
                         keep_percent=cfg.keep_percent)
    t = time_prefill(layer, steps, warmup, torch, flush)
    fl, tile_fl = prefill_flops(layer.blk_idx.cpu().numpy(), layer.blk_cnt.cpu().numpy(),
                                cfg.block, cfg.d)
    t["attend_tflops"] = fl / (t["attend_ms"] * 1e-3) / 1e12
    t["attend_mfma_frac"] = fl / (t["attend_ms"] * 1e-3) / PEAK_BF16_FLOPS
    t["attend_flops"] = fl
    t["attend_tile_flops"] = tile_fl
    t["tok_per_s"] = cfg.B * cfg.S / (t["step_ms"] * 1e-3)
    # fused RoPE + pooling reads Q and K and writes rotated Q and K once
    rp_bytes = 2.0 * (q.numel() + k.numel()) * q.element_size()
    t["score_hbm_bytes"] = rp_bytes
    del layer, q, k, v
    torch.cuda.empty_cache()
    return t


def run_decode(cfg, steps, warmup, torch, flush):
    import synth.device as SD
    from long_context_sparse_apply_amd.pipeline import DecodeStep
    dt = SD.decode_tensors(cfg)
    step = DecodeStep(dt["q_raw"], dt["k"], dt["v"], dt["lens"], dt["dom"], theta=cfg.theta,
                      top_k=cfg.k, slab=bool(cfg.slab), k_rest=dt["k_rest"], k_full=dt["k_full"])
    t = time_decode(step, steps, warmup, torch, flush)
    t["cache_layout"] = ("standard" if not cfg.slab else
                         "dominant slab + full rows" if cfg.full_rows else "dominant slab + rest")
    t["cache_device_bytes"] = float(sum(x.numel() * x.element_size()
                                        for x in (dt["k"], dt["k_rest"], dt["k_full"], dt["v"])
                                        if x is not None))
    cnt = step.tok_cnt.cpu().numpy()
    gb = decode_bytes(cnt, cfg.d)
    t["attend_gather_bytes"] = gb
    t["attend_hbm_frac"] = gb / (t["attend_us"] * 1e-6) / PEAK_HBM_BPS
    t["attend_gather_bytes_dedup_per_kv_head"] = decode_dedup_bytes(step.tok_idx.cpu().numpy(), cnt,
                                                                    cfg.Hkv, cfg.d)
    row = 2 * cfg.n_dom if cfg.slab else cfg.d
    key_bytes = float(cfg.B) * cfg.Hkv * cfg.L * row * 2
    if step.fused:
        # the fused top-k reads the key rows once and writes no scores; its
        # fraction is over the whole score + select time
        t["score_bytes"] = key_bytes
        t["score_hbm_frac"] = key_bytes / (t["score_select_us"] * 1e-6) / PEAK_HBM_BPS
        # the two calls it replaces, on the same inputs, for comparison
        two = DecodeStep(dt["q_raw"], dt["k"], dt["v"], dt["lens"], dt["dom"], theta=cfg.theta,
                         top_k=cfg.k, slab=bool(cfg.slab), k_rest=dt["k_rest"], k_full=dt["k_full"],
                         fused=False)
        two.rope()

        def score_then_select():
            two.score()
            two.select()
        t["two_step_score_select_us"] = time_call(score_then_select, max(3, steps // 2), 1, torch,
                                                  flush)[0]
        torch.cuda.synchronize()
        t["two_step_equal"] = bool(torch.equal(two.tok_idx, step.tok_idx)
                                   and torch.equal(two.tok_cnt, step.tok_cnt))
        del two
    else:
        scan = key_bytes + float(cfg.B) * cfg.Hq * cfg.L * 4  # key rows read, scores written
        t["score_bytes"] = scan
        t["score_hbm_frac"] = scan / (t["score_us"] * 1e-6) / PEAK_HBM_BPS
    del step, dt
    torch.cuda.empty_cache()
    return t


def host_info():
    """Cores in this process's affinity mask, BLAS threads, CPU model."""
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        blas = 1
    cpu_model = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    return affinity, blas, cpu_model


def _spot_check(host, seed, tid, base, rng, n=4096):
    """The copied inputs are the seeded generator's values: a random sample of
    elements regenerated on the host must match bit for bit."""
    import synth
    flat = host.reshape(-1)
    idx = rng.integers(0, flat.size, n)
    want = synth.round_to_bf16(synth.gaussian_f32(seed, tid, (base + idx).astype(np.uint64)))
    assert np.array_equal(flat[idx].astype(np.float32), want), "inputs differ from the generator"


def _baseline(value, unit, seconds, sample):
    affinity, blas, cpu_model = host_info()
    return {"value": value, "unit": unit, "cores": int(blas), "kind": "oracle",
            "sample": f"{sample}: {seconds:.1f} s on {cpu_model}",
            "affinity_cores": int(affinity), "blas_threads": int(blas),
            "python_threads": 1, "cpu_model": cpu_model}


def cpu_baseline_prefill(cfg, torch, kv_groups=None):
    """The fp64 oracle on a prefill layer: block scoring, selection and
    block-sparse attention, timed on the host cores.  ``kv_groups`` limits it
    to those KV groups (their query heads), extrapolated linearly in heads.
    Inputs come from the device-side seeded generator (copied to the host and
    spot-checked against the host generator); only the oracle is timed."""
    import synth
    import synth.device as SD
    from oracle import sparse_attention as O
    groups = list(range(cfg.Hkv)) if kv_groups is None else list(kv_groups)
    heads = [g * cfg.group + i for g in groups for i in range(cfg.group)]
    qd, kd, vd = SD.prefill_tensors(cfg)
    q = qd[:, heads].float().cpu().numpy()
    k = kd.float().cpu().numpy()
    v = vd.float().cpu().numpy()
    del qd, kd, vd
    torch.cuda.empty_cache()
    rng = np.random.default_rng(0)
    _spot_check(v, cfg.seed, synth.TID_V, 0, rng)
    t0 = time.perf_counter()
    O.prefill_pipeline(q, k, v, theta=cfg.theta, block=cfg.block,
                       split_pair=cfg.band_split_pair, calibrate=True, sm_scale=cfg.d ** -0.5,
                       causal=True, budget=O.keep_budget(cfg.N, keep_percent=cfg.keep_percent),
                       n_sink=cfg.n_sink, n_local=cfg.n_local, q_heads=heads, group=cfg.group)
    dt = time.perf_counter() - t0
    scale = cfg.Hq / len(heads)
    what = (f"the whole {cfg.S // 1024}K prefill layer ({cfg.Hq} query heads), one pass"
            if scale == 1 else
            f"{len(groups)} KV group(s) ({len(heads)} of {cfg.Hq} query heads) of the "
            f"{cfg.S // 1024}K prefill layer, extrapolated x{scale:g} (work is linear in heads)")
    return _baseline(cfg.B * cfg.S / (dt * scale), "tok/s", dt, what)


def cpu_baseline_decode(cfg, torch, batches):
    """The fp64 oracle on a decode step (rotate q, token scores over the
    dominant pairs, top-k, attention) for the sampled batch rows, extrapolated
    linearly to the whole batch (work is linear in batch rows)."""
    import synth
    import synth.device as SD
    from oracle import sparse_attention as O
    dt_ = SD.decode_tensors(cfg)
    bs = list(batches)
    kfull = dt_["k_full"] if dt_.get("k_full") is not None else dt_["k"]
    if cfg.slab and dt_.get("k_full") is None:
        raise ValueError("the decode baseline reads full key rows")
    q = dt_["q_raw"][bs].float().cpu().numpy()
    k = kfull[bs].float().cpu().numpy()
    v = dt_["v"][bs].float().cpu().numpy()
    lens, dom = dt_["lens_host"][bs], dt_["dom_host"]
    del dt_, kfull
    torch.cuda.empty_cache()
    rng = np.random.default_rng(1)
    _spot_check(v[0], cfg.seed, synth.TID_V, bs[0] * cfg.Hkv * cfg.L * cfg.d, rng)
    t0 = time.perf_counter()
    O.decode_pipeline(q, k, v, lens, dom, theta=cfg.theta, k=cfg.k, sm_scale=cfg.d ** -0.5)
    dt = time.perf_counter() - t0
    scale = cfg.B / len(bs)
    what = (f"batch rows {bs[0]}-{bs[-1]} of {cfg.B} ({len(bs) * cfg.Hq} of {cfg.B * cfg.Hq} "
            f"query rows), KV length {cfg.L}, top-{cfg.k}, extrapolated x{scale:g}")
    return _baseline(dt * scale * 1e6, "us/step", dt, what)


def measured_traffic(summary_path, kernel_source):
    """HBM bytes per launch from a committed counter summary, or None when the
    kernel source has changed since the counters were taken (the summary
    records the sha256 of the source it measured)."""
    try:
        text = open(summary_path).read()
        src = open(kernel_source, "rb").read()
    except OSError:
        return None
    h = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not h or not b or hashlib.sha256(src).hexdigest() != h.group(1):
        return None
    return float(b.group(1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default=None, help="C2|C3|C4|C4_SLAB|C5: run one workload (profiling)")
    ap.add_argument("--no-flush", action="store_true",
                    help="do not clear L2 / MALL with a 1 GiB read sweep before each timed step")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first copy 1 GiB device-to-device 3 times (a kernel of known bytes "
                         "that scales the HBM traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(how it would shard is a design note, not code).", file=sys.stderr)
        sys.exit(2)
    import torch
    import long_context_sparse_apply_amd  # noqa: F401  (fails loudly if not built)
    from synth import workloads as W
    torch.cuda.set_device(0)

    if args.calib_copy:
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied 1 GiB x3")
        del src, dst
        torch.cuda.empty_cache()
    flush = CacheFlush(torch, enabled=not args.no_flush)
    if args.only:
        cfg = W.CONFIGS[args.only]
        log(f"running {args.only} only")
        r = run_prefill(cfg, args.steps, args.warmup, torch, flush) if args.only in ("C2", "C3") \
            else run_decode(cfg, args.steps, args.warmup, torch, flush)
        log(json.dumps(r))
        return

    copy_gbps = copy_reference(torch)
    log(f"1 GiB device copy: {copy_gbps:.0f} GB/s")
    gemm_tflops = gemm_reference(torch)
    log(f"bf16 8192^3 library matrix product: {gemm_tflops:.0f} TFLOP/s")
    cfg = W.C2
    log("C2: prefill 32K")
    main_r = run_prefill(cfg, args.steps, args.warmup, torch, flush)
    log(json.dumps(main_r))
    secondary = {}
    if not args.no_secondary:
        log("C3: prefill 128K")
        r3 = run_prefill(W.C3, max(3, args.steps // 4), 2, torch, flush)
        log(json.dumps(r3))
        secondary["prefill_128k"] = {"tok_per_s": r3["tok_per_s"], "ms_per_step": r3["step_ms"],
                                     "ms_per_step_p10_p90": [r3["step_ms_p10"], r3["step_ms_p90"]],
                                     "attend_ms": r3["attend_ms"],
                                     "attend_mfma_frac": r3["attend_mfma_frac"],
                                     "score_ms": r3["score_ms"], "select_ms": r3["select_ms"]}
        for name, c in (("decode_64k", W.C4), ("decode_64k_slab", W.C4_SLAB),
                        ("decode_128k_slab", W.C5),
                        ("decode_128k_slab_rest", W.C5.with_(full_rows=0))):
            log(f"{name}")
            rd = run_decode(c, args.steps, args.warmup, torch, flush)
            log(json.dumps(rd))
            secondary[name] = {"us_per_step": rd["step_us"],
                               "us_per_step_p10_p90": [rd["step_us_p10"], rd["step_us_p90"]],
                               "rope_us": rd["rope_us"], "fused_score_select": rd["fused"],
                               "score_select_us": rd["score_select_us"],
                               "score_us": rd["score_us"],
                               "select_us": rd["select_us"], "attend_us": rd["attend_us"],
                               "attend_hbm_frac": rd["attend_hbm_frac"],
                               "attend_gather_bytes": rd["attend_gather_bytes"],
                               "attend_gather_bytes_dedup_per_kv_head":
                                   rd["attend_gather_bytes_dedup_per_kv_head"],
                               "score_hbm_frac": rd["score_hbm_frac"],
                               "cache_layout": rd["cache_layout"],
                               "cache_device_bytes": rd["cache_device_bytes"]}
            if rd["fused"]:
                secondary[name]["two_step_score_select_us"] = rd["two_step_score_select_us"]
                secondary[name]["two_step_equal"] = rd["two_step_equal"]
        log("decode_64k_slab_host_rest (FASA-M placement)")
        cfg_m = W.C5.with_(B=16, L=65536, k=2048, full_rows=0)
        rm = run_decode_host_rest(cfg_m, max(2, args.steps // 5), 1, torch, flush)
        log(json.dumps(rm))
        secondary["decode_64k_slab_host_rest"] = {
            "workload": "batch 16, KV length 65536, dominant slab (16 pairs) in HBM, "
                        "rest of K and V in pinned host memory, top-2048, bf16",
            "us_per_step": rm["step_us"], "score_select_us": rm["score_select_us"],
            "attend_us": rm["attend_us"],
            "host_link_bytes": rm["host_link_bytes"], "host_link_GBps": rm["host_link_GBps"],
            "device_resident_bytes": rm["device_resident_bytes"],
            "host_resident_bytes": rm["host_resident_bytes"]}
        log("sfa_prefill_8k (Sparse Feature Attention)")
        rs = run_sfa(max(3, args.steps // 4), 1, torch, flush)
        log(json.dumps(rs))
        secondary["sfa_prefill_8k"] = rs
        log("calibration of the dominant pairs")
        rc = run_calibration(W.CAL_LLAMA, max(3, args.steps // 4), 1, torch, flush)
        log(json.dumps(rc))
        secondary["calibration"] = rc
        log("cache append (prefill -> decode handoff, decode token)")
        ra = run_cache_append(cfg, W.C5, args.steps, args.warmup, torch, flush)
        log(json.dumps(ra))
        secondary["cache_append"] = ra
    cpu = None
    cpu_more = None
    if not args.no_cpu:
        log("cpu baseline (oracle): 32K prefill layer")
        cpu = cpu_baseline_prefill(cfg, torch)
        log(json.dumps(cpu))
        if not args.no_secondary:
            cpu_more = {}
            log("cpu baseline (oracle): 128K prefill, one KV group")
            cpu_more["prefill_128k"] = cpu_baseline_prefill(W.C3, torch, kv_groups=[0])
            log("cpu baseline (oracle): 64K decode, batch rows 0-1")
            cpu_more["decode_64k"] = cpu_baseline_decode(W.C4, torch, [0, 1])
            log("cpu baseline (oracle): 128K slab decode, batch rows 0-3")
            cpu_more["decode_128k_slab"] = cpu_baseline_decode(W.C5, torch, [0, 1, 2, 3])
            log(json.dumps(cpu_more))
    # the roofline uses the attention kernel's mean launch duration (as a
    # kernel trace reports it); the step figures are medians
    achieved = main_r["attend_flops"] / (main_r["attend_ms_mean"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": main_r["tok_per_s"],
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_r["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B-shaped sparse prefill layer, seq 32768, 32 Q / 8 KV "
                               "heads, d=128, block 128, keep 10% + sink + 2 local, bf16",
                   "seq_len": cfg.S, "batch": cfg.B, "q_heads": cfg.Hq, "kv_heads": cfg.Hkv,
                   "head_dim": cfg.d, "block": cfg.block, "keep_percent": cfg.keep_percent},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_FLOPS / 1e12,
                     "unit": "TFLOP/s", "frac": achieved * 1e12 / PEAK_BF16_FLOPS,
                     "traffic": measured_traffic(TRAFFIC_SUMMARY, PREFILL_SOURCE),
                     "kernel": "prefill_mfma_kernel",
                     "avg_launch_ms": main_r["attend_ms_mean"],
                     "flops_per_launch": main_r["attend_flops"],
                     "tile_flops_per_launch": main_r["attend_tile_flops"]},
        "ms_per_step_p10_p90": [main_r["step_ms_p10"], main_r["step_ms_p90"]],
        "stages_ms": {"score": main_r["score_ms"], "select": main_r["select_ms"],
                      "attend": main_r["attend_ms"]},
        "timing": ("HIP events on the kernels' stream; medians of the timed steps; L2 and MALL "
                   "cleared by a 1 GiB read sweep before each step" if not args.no_flush else
                   "HIP events on the kernels' stream; medians of the timed steps; no cache flush"),
        "hbm_reference": {"copy_GBps": copy_gbps, "peak_GBps": PEAK_HBM_BPS / 1e9},
        "mfma_reference": {"gemm_TFLOPs": gemm_tflops, "peak_TFLOPs": PEAK_BF16_FLOPS / 1e12,
                           "gemm": "bf16 8192 x 8192 x 8192, torch.matmul (vendor library)",
                           "attend_vs_gemm": main_r["attend_tflops"] / gemm_tflops},
        "cpu_baseline": cpu,
        "cpu_baseline_secondary": cpu_more,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
