"""One prefill layer and one decode step as chains of C-ABI calls.

Buffers are allocated once per shape (torch is the allocator); ``run()``
only enqueues the library's kernels on the current stream.

Prefill ("Prism: Spectral-Aware Block-Sparse Attention"):
    sa_block_score  -> rotated Q/K, calibrated dual-band pooled vectors, block scores
    sa_topk_select  -> per query block: sink + local + top-k blocks
    sa_sparse_attn_prefill -> attention over the selected blocks
Decode ("FASA: Frequency-aware Sparse Attention"):
    sa_kv_cache_append -> the new token's key rotated at its position, written
                      with its value into the cache (standard or dominant slab)
    sa_rope_apply   -> the decode query rotated at position L_b - 1
    sa_token_score  -> dominant-chunk token scores
    sa_topk_select  -> top-k tokens
      (dominant-slab layout: sa_token_topk does both without a score array)
    sa_sparse_attn_decode -> split-K attention over the selected tokens
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import (SA_OP_BLOCK_SCORE, SA_OP_DECODE, SA_OP_TOKEN_TOPK, prefill_row_params,
               sa_block_score, sa_kv_cache_append, sa_rope_apply, sa_sfa_sparsify,
               sa_sparse_attn_decode, sa_sparse_attn_prefill, sa_token_score, sa_token_topk,
               sa_topk_select, workspace_bytes)


class PrefillLayer:
    def __init__(self, q, k, v, *, theta, block, band_split_pair, n_sink, n_local, keep_const=0,
                 keep_percent=0, calibrate=True, causal=True, sm_scale=None, keep_pooled=False):
        self.q, self.k, self.v = q, k, v
        B, Hq, S, d = q.shape
        Hkv = k.shape[1]
        self.B, self.Hq, self.Hkv, self.S, self.d = B, Hq, Hkv, S, d
        self.block, self.N = block, S // block
        self.theta, self.split = theta, band_split_pair
        self.calibrate, self.causal = calibrate, causal
        self.n_sink, self.n_local = n_sink, n_local
        self.scale = sm_scale if sm_scale is not None else d ** -0.5
        # bf16: the stored Q carries sm_scale * log2(e) and the attention runs
        # with sm_scale = ln 2, so its logits are base-2 exponents as they
        # stand (the same softmax, one multiply-add less per score)
        if q.dtype == torch.bfloat16:
            self.q_rope_scale = self.scale * math.log2(math.e)
            self.attn_scale = float(np.float32(math.log(2.0)))
        else:
            self.q_rope_scale, self.attn_scale = 1.0, self.scale
        dev = q.device
        N = self.N
        self.q_rope = torch.empty_like(q)
        self.k_rope = torch.empty_like(k)
        self.scores = torch.empty((B, Hq, N, N), dtype=torch.float32, device=dev)
        if keep_pooled:
            self.pq = torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev)
            self.pk = torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev)
            self.ws = None
        else:
            self.pq = self.pk = None
            self.ws = torch.empty(workspace_bytes(SA_OP_BLOCK_SCORE, B * (Hq + Hkv) * N, d),
                                  dtype=torch.uint8, device=dev)
        self.valid_len, self.k_rows, kmax = prefill_row_params(
            B, Hq, N, keep_const=keep_const, keep_percent=keep_percent, causal=causal, device=dev)
        self.k_max = kmax
        self.max_sel = min(N, n_sink + n_local + kmax)
        self.max_out = n_sink + n_local + kmax
        self.blk_idx = torch.empty((B, Hq, N, self.max_out), dtype=torch.int32, device=dev)
        self.blk_cnt = torch.empty((B, Hq, N), dtype=torch.int32, device=dev)
        self.out = torch.empty_like(q)
        self.lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)

    def score(self):
        sa_block_score(self.q, self.k, self.scores, theta=self.theta, block=self.block,
                       band_split_pair=self.split, calibrate=self.calibrate, sm_scale=self.scale,
                       causal=self.causal, q_rope_out=self.q_rope,
                       q_rope_scale=self.q_rope_scale, k_rope_out=self.k_rope,
                       pooled_q_out=self.pq, pooled_k_out=self.pk, ws=self.ws)

    def select(self):
        sa_topk_select(self.scores, self.blk_idx, self.blk_cnt, k_const=self.k_max,
                       valid_len=self.valid_len, k_per_row=self.k_rows, n_sink=self.n_sink,
                       n_local=self.n_local)

    def attend(self):
        sa_sparse_attn_prefill(self.q_rope, self.k_rope, self.v, self.blk_idx, self.blk_cnt,
                               self.out, block=self.block, sm_scale=self.attn_scale,
                               causal=self.causal, lse=self.lse)

    def run(self):
        self.score()
        self.select()
        self.attend()
        return self.out


class SFALayer:
    """Sparse Feature Attention ("Scaling Attention via Feature Sparsity",
    sec. 2) over one causal prefill layer: k-sparse codes of Q and K
    (sa_sfa_sparsify), then exact attention over every causal block of the
    codes (sa_sparse_attn_prefill with the full causal block list, built once
    per shape)."""

    def __init__(self, q, k, v, *, k_feat, block=128, sm_scale=None):
        self.q, self.k, self.v = q, k, v
        B, Hq, S, d = q.shape
        self.block, self.N, self.k_feat = block, S // block, k_feat
        self.scale = sm_scale if sm_scale is not None else d ** -0.5
        dev = q.device
        N = self.N
        self.q_code = torch.empty_like(q)
        self.k_code = torch.empty_like(k)
        # every block J <= I of query block I (the kernel skips J > I when causal)
        self.blk_idx = torch.arange(N, dtype=torch.int32, device=dev).repeat(B * Hq * N).view(
            B, Hq, N, N).contiguous()
        self.blk_cnt = torch.arange(1, N + 1, dtype=torch.int32, device=dev).repeat(B * Hq).view(
            B, Hq, N).contiguous()
        self.out = torch.empty_like(q)
        self.lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)

    def codes(self):
        sa_sfa_sparsify(self.q, self.q_code, k_feat=self.k_feat)
        sa_sfa_sparsify(self.k, self.k_code, k_feat=self.k_feat)

    def attend(self):
        sa_sparse_attn_prefill(self.q_code, self.k_code, self.v, self.blk_idx, self.blk_cnt,
                               self.out, block=self.block, sm_scale=self.scale, causal=True,
                               lse=self.lse)

    def run(self):
        self.codes()
        self.attend()
        return self.out


class DecodeCache:
    """A decode KV cache of ``Lmax`` rows per (batch, KV head) plus its lengths.

    Keys are stored rotated at their absolute positions (the row index), in
    the standard layout ``k [B, Hkv, Lmax, d]`` or, with ``slab``, as the
    dominant slab ``k [B, Hkv, Lmax, 2*n_dom]`` plus either ``k_rest [B, Hkv,
    Lmax, d - 2*n_dom]`` or, with ``full_rows``, ``k_full [B, Hkv, Lmax, d]``
    (every channel in the standard order: the attention then gathers whole
    256-byte rows, for 2*n_dom channels of extra memory per token).  ``lens``
    (int32 [B], on the device) counts the rows written so far; appends go to
    row ``lens[b]`` onward.

    ``host_rest`` (slab layout only): FASA's memory-optimised variant
    (FASA-M, sec. 2.C).  Only the dominant slab stays in device memory;
    ``k_rest`` and ``v`` live in pinned host memory, and the decode step
    reads the selected rows of them over the host link when it attends.
    """

    def __init__(self, B, Hkv, Lmax, d, *, dtype, device, theta, dom_pairs, slab=False,
                 full_rows=False, host_rest=False):
        if host_rest and not slab:
            raise ValueError("host placement keeps the dominant slab on the device: needs slab")
        if full_rows and (not slab or host_rest):
            raise ValueError("full rows go with the device-resident slab layout")
        self.B, self.Hkv, self.Lmax, self.d = B, Hkv, Lmax, d
        self.theta, self.slab, self.full_rows, self.dom = theta, slab, full_rows, dom_pairs
        n_dom = dom_pairs.shape[1]
        kd = 2 * n_dom if slab else d
        rest_kw = dict(device="cpu", pin_memory=True) if host_rest else dict(device=device)
        self.k = torch.zeros((B, Hkv, Lmax, kd), dtype=dtype, device=device)
        self.k_rest = (torch.zeros((B, Hkv, Lmax, d - kd), dtype=dtype, **rest_kw)
                       if slab and not full_rows and kd < d else None)
        self.k_full = (torch.zeros((B, Hkv, Lmax, d), dtype=dtype, device=device)
                       if full_rows else None)
        self.v = torch.zeros((B, Hkv, Lmax, d), dtype=dtype, **rest_kw)
        self.lens = torch.zeros(B, dtype=torch.int32, device=device)

    def append(self, k_new, v_new, batch=None):
        """Append ``S`` raw tokens ``[B, Hkv, S, d]`` to every batch row, or
        ``[1, Hkv, S, d]`` to batch row ``batch`` alone.  Rows past ``Lmax``
        are dropped and not counted."""
        S = k_new.shape[2]
        sl = slice(None) if batch is None else slice(batch, batch + 1)
        second = self.k_full if self.full_rows else self.k_rest
        lens = self.lens[sl]
        sa_kv_cache_append(k_new, v_new, lens, self.k[sl], self.v[sl], theta=self.theta,
                           k_rest=None if second is None else second[sl], dom_pairs=self.dom,
                           slab=self.slab, full_rows=self.full_rows)
        lens.add_(S).clamp_(max=self.Lmax)

    def step(self, q_raw, *, top_k, sm_scale=None):
        """A decode step for the query ``q_raw [B, Hq, d]`` of the newest token."""
        return DecodeStep(q_raw, self.k, self.v, self.lens, self.dom, theta=self.theta,
                          top_k=top_k, slab=self.slab, k_rest=self.k_rest, k_full=self.k_full,
                          sm_scale=sm_scale)


class DecodeStep:
    """One decode step.  ``fused`` (the default for the slab layout, and for
    the standard layout in bf16 with at most 16 dominant pairs) scores and
    selects the tokens with sa_token_topk, which writes no score array;
    otherwise sa_token_score then sa_topk_select (the same selection).
    ``k_full`` (slab layout): the full rotated rows the attention gathers,
    in place of the slab and ``k_rest``."""

    def __init__(self, q_raw, k, v, cache_len, dom_pairs, *, theta, top_k, slab=False, k_rest=None,
                 k_full=None, sm_scale=None, cache_len_host=None, fused=None):
        self.q_raw, self.k, self.v, self.k_rest, self.k_full = q_raw, k, v, k_rest, k_full
        B, Hq, d = q_raw.shape
        Hkv, L = v.shape[1], v.shape[2]
        self.B, self.Hq, self.Hkv, self.L, self.d = B, Hq, Hkv, L, d
        self.theta, self.top_k, self.slab = theta, top_k, slab
        self.cache_len, self.dom = cache_len, dom_pairs
        self.scale = sm_scale if sm_scale is not None else d ** -0.5
        dev = q_raw.device
        # position of the decoding token per batch row: cache_len - 1 (int32, [B])
        self.pos = (cache_len - 1).to(torch.int32).contiguous()
        self.q_rope = torch.empty_like(q_raw)
        # fused by default with the slab, and with the standard layout where
        # its threshold reads the rows coalesced (bf16, at most 16 dominant
        # pairs); elsewhere that threshold's scattered reads cost more than
        # the score array saves
        fast_std = q_raw.dtype == torch.bfloat16 and 2 * dom_pairs.shape[1] <= 32
        self.fused = (slab or fast_std) if fused is None else bool(fused)
        if self.fused:
            self.scores = None
            self.ws_sel = torch.empty(workspace_bytes(SA_OP_TOKEN_TOPK, rows=B * Hq, cols=L,
                                                      max_k=top_k), dtype=torch.uint8, device=dev)
        else:
            self.scores = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
        self.valid_len = cache_len.repeat_interleave(Hq).to(torch.int32).contiguous()
        self.tok_idx = torch.empty((B, Hq, top_k), dtype=torch.int32, device=dev)
        self.tok_cnt = torch.empty((B, Hq), dtype=torch.int32, device=dev)
        self.ws = torch.empty(workspace_bytes(SA_OP_DECODE, B=B, Hq=Hq, max_k=top_k),
                              dtype=torch.uint8, device=dev)
        self.out = torch.empty_like(q_raw)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)

    def rope(self):
        # q_raw viewed as [B, Hq, 1, d]: one token per (b, h) at position pos[b]
        sa_rope_apply(self.q_raw.view(self.B, self.Hq, 1, self.d),
                      self.q_rope.view(self.B, self.Hq, 1, self.d), self.theta, pos=self.pos)

    def score(self):
        sa_token_score(self.q_rope, self.k, self.scores, self.cache_len, self.dom,
                       sm_scale=self.scale, slab=self.slab, k_rest=self.k_rest)

    def select(self):
        sa_topk_select(self.scores, self.tok_idx, self.tok_cnt, k_const=self.top_k,
                       valid_len=self.valid_len)

    def score_select(self):
        sa_token_topk(self.q_rope, self.k, self.cache_len, self.dom, self.tok_idx, self.tok_cnt,
                      self.ws_sel, sm_scale=self.scale, k_top=self.top_k, slab=self.slab)

    def attend(self):
        if self.k_full is not None:
            # slab + full rows: the attention gathers whole rows of the full cache
            sa_sparse_attn_decode(self.q_rope, self.k_full, self.v, self.tok_idx, self.tok_cnt,
                                  self.out, self.ws, sm_scale=self.scale,
                                  cache_len=self.cache_len, lse=self.lse)
            return
        sa_sparse_attn_decode(self.q_rope, self.k, self.v, self.tok_idx, self.tok_cnt, self.out,
                              self.ws, sm_scale=self.scale, cache_len=self.cache_len,
                              dom_pairs=self.dom, slab=self.slab, k_rest=self.k_rest,
                              lse=self.lse)

    def run(self):
        self.rope()
        if self.fused:
            self.score_select()
        else:
            self.score()
            self.select()
        self.attend()
        return self.out
