"""Build the synthetic workloads directly in GPU memory.

Bulk values come from the device generator (``libsynth_gen.so``, built from
``synth/gen.hip``), which reproduces the host generator bit for bit; the few
rows that carry a planted needle are computed on the host (fp64, then
rounded) and copied over.  Input construction only.
"""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import numpy as np

from . import IH_SCALE, TID_K, TID_Q, TID_V
from . import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsynth_gen.so")
_lib = None


def build(verbose: bool = True) -> str:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(HERE, "gen.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"synth generator build failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}", flush=True)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built")
        _lib = ctypes.CDLL(LIB_PATH)
        _lib.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_float, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                    ctypes.c_void_p]
        _lib.synth_fill.restype = ctypes.c_int
    return _lib


def fill(t, seed: int, tid: int, *, logical_d: int | None = None, base: int = 0, chmap=None,
         rows_per_head: int = 1, n_heads: int = 1):
    """Fill GPU tensor ``t`` (rows x last dim) with generator values."""
    import torch
    cols = t.shape[-1]
    rows = t.numel() // cols
    ld = logical_d if logical_d is not None else cols
    st = torch.cuda.current_stream().cuda_stream
    r = lib().synth_fill(ctypes.c_void_p(t.data_ptr()), 1 if t.dtype == torch.bfloat16 else 0,
                         rows, cols, ld, base, seed, tid, float(IH_SCALE),
                         None if chmap is None else ctypes.c_void_p(chmap.data_ptr()),
                         rows_per_head, n_heads, ctypes.c_void_p(st))
    if r != 0:
        raise RuntimeError(f"synth_fill failed ({r})")
    return t


def torch_dtype(name: str):
    import torch
    return torch.bfloat16 if name == "bf16" else torch.float32


def prefill_tensors(cfg: W.PrefillConfig, device="cuda"):
    """Stored (pre-rotation) Q, K, V of a prefill workload on the GPU."""
    import torch
    dt = torch_dtype(cfg.dtype)
    q = torch.empty((cfg.B, cfg.Hq, cfg.S, cfg.d), dtype=dt, device=device)
    k = torch.empty((cfg.B, cfg.Hkv, cfg.S, cfg.d), dtype=dt, device=device)
    v = torch.empty_like(k)
    fill(q, cfg.seed, TID_Q)
    fill(k, cfg.seed, TID_K)
    fill(v, cfg.seed, TID_V)
    for tid, b, h, rows, vals in W.prefill_patches(cfg):
        dst = q if tid == TID_Q else k
        dst[b, h, int(rows[0]):int(rows[-1]) + 1] = torch.from_numpy(
            np.ascontiguousarray(vals, dtype=np.float32)).to(device=device, dtype=dt)
    torch.cuda.synchronize()
    return q, k, v


def decode_tensors(cfg: W.DecodeConfig, device="cuda"):
    """Decode workload on the GPU: q_raw, rotated K cache (standard or slab), V."""
    import torch
    dt = torch_dtype(cfg.dtype)
    lens = W.cache_lengths(cfg)
    dom = W.dominant_pairs(cfg)
    q = torch.empty((cfg.B, cfg.Hq, cfg.d), dtype=dt, device=device)
    fill(q, cfg.seed, TID_Q)
    v = torch.empty((cfg.B, cfg.Hkv, cfg.L, cfg.d), dtype=dt, device=device)
    fill(v, cfg.seed, TID_V)
    patches = W.decode_patches(cfg, lens)
    out = dict(q_raw=q, v=v, lens=torch.from_numpy(lens).to(device),
               dom=torch.from_numpy(dom).to(device), lens_host=lens, dom_host=dom)
    if not cfg.slab:
        k = torch.empty_like(v)
        fill(k, cfg.seed, TID_K)
        for b, h, p, row in patches:
            k[b, h // cfg.group, p] = torch.from_numpy(row).to(device=device, dtype=dt)
        out["k"] = k
        out["k_rest"] = None
        out["k_full"] = None
    else:
        maps = [W.slab_channels(dom[g], cfg.d) for g in range(cfg.Hkv)]
        dom_map = torch.from_numpy(np.stack([m[0] for m in maps]).astype(np.int32)).to(device)
        rest_map = torch.from_numpy(np.stack([m[1] for m in maps]).astype(np.int32)).to(device)
        nd = 2 * cfg.n_dom
        k_dom = torch.empty((cfg.B, cfg.Hkv, cfg.L, nd), dtype=dt, device=device)
        fill(k_dom, cfg.seed, TID_K, logical_d=cfg.d, chmap=dom_map, rows_per_head=cfg.L,
             n_heads=cfg.Hkv)
        if cfg.full_rows:
            # the full rows the attention gathers, in the standard channel order
            k_second = torch.empty((cfg.B, cfg.Hkv, cfg.L, cfg.d), dtype=dt, device=device)
            fill(k_second, cfg.seed, TID_K)
        else:
            k_second = torch.empty((cfg.B, cfg.Hkv, cfg.L, cfg.d - nd), dtype=dt, device=device)
            fill(k_second, cfg.seed, TID_K, logical_d=cfg.d, chmap=rest_map, rows_per_head=cfg.L,
                 n_heads=cfg.Hkv)
        for b, h, p, row in patches:
            g = h // cfg.group
            dm, rm = maps[g]
            k_dom[b, g, p] = torch.from_numpy(row[dm]).to(device=device, dtype=dt)
            k_second[b, g, p] = torch.from_numpy(row if cfg.full_rows else row[rm]).to(
                device=device, dtype=dt)
        out["k"] = k_dom
        out["k_rest"] = None if cfg.full_rows else k_second
        out["k_full"] = k_second if cfg.full_rows else None
    torch.cuda.synchronize()
    return out
