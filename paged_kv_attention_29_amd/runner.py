"""Caller-side driver of the library for a seeded workload: allocates the
paged cache on the GPU (unwritten slots NaN), writes the cached context and
each step's new tokens through ``reshape_and_cache``, and runs the step's
decode / prefill calls (plus ``merge_attn_states`` for split decode).

It does what a serving engine's attention backend does around the four
entry points; all attention arithmetic happens in the library's kernels.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from . import (merge_attn_states, paged_attn_decode, paged_attn_decode_merged, paged_attn_prefill,
               reshape_and_cache, scaled_fp8_quant)


@dataclass
class CallBuffers:
    """Device-resident inputs and outputs of one attention call."""
    kind: str
    q: torch.Tensor
    cu_seqlens_q: torch.Tensor
    seq_lens: torch.Tensor
    block_table: torch.Tensor
    max_seqlen_q: int
    max_seqlen_k: int
    num_splits: int
    out: torch.Tensor
    lse: torch.Tensor
    part_out: Optional[torch.Tensor] = None
    part_lse: Optional[torch.Tensor] = None
    causal: bool = True
    # split decode merged in the decode launch (paged_attn_decode_merged):
    # its zeroed counters; None runs decode then merge_attn_states
    split_counters: Optional[torch.Tensor] = None


class PagedCache:
    """One layer's K/V cache for a workload.  With ``kv_scales = (k_scale,
    v_scale)`` the cache holds fp8 (e4m3) codes written by the quantising
    reshape_and_cache with those per-tensor scales (unwritten slots hold the
    NaN code 0x7F); otherwise it holds the workload's 16-bit dtype."""

    def __init__(self, w, device: str = "cuda", kv_scales=None):
        self.w = w
        self.device = device
        shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_size)
        if kv_scales is None:
            self.key_cache = torch.full(shape, float("nan"), dtype=w.dtype, device=device)
            self.k_scale = self.v_scale = None
        else:
            self.key_cache = torch.full(shape, 0x7F, dtype=torch.uint8, device=device)
            self.k_scale = torch.tensor([float(kv_scales[0])], device=device)
            self.v_scale = torch.tensor([float(kv_scales[1])], device=device)
        self.value_cache = self.key_cache.clone()
        self.block_table = torch.from_numpy(w.block_table).to(device)
        self.alibi = None if w.alibi_slopes is None else w.alibi_slopes.to(device)
        self.sinks = None  # optional fp32 [num_heads] attention-sink logits on the device
        # fp8 cache only: a device fp32 scalar; the calls then quantise q with
        # it (scaled_fp8_quant) and attend the codes with this descale
        self.q_scale = None

    def write(self, key: torch.Tensor, value: torch.Tensor, slots: torch.Tensor) -> None:
        reshape_and_cache(key.to(self.device), value.to(self.device), self.key_cache,
                          self.value_cache, slots.to(self.device), k_scale=self.k_scale,
                          v_scale=self.v_scale)

    def fill_context(self) -> None:
        for _, k, v, s in self.w.context_tokens():
            self.write(k, v, s)
        torch.cuda.synchronize()

    def step_inputs(self, step):
        """(key, value, slots) of a step, resident on the device."""
        k, v, s = self.w.step_tokens(step)
        return k.to(self.device), v.to(self.device), s.to(self.device)

    def call_buffers(self, call, num_splits: Optional[int] = None,
                     merged: bool = False) -> CallBuffers:
        w, dev = self.w, self.device
        S = call.num_splits if num_splits is None else num_splits
        T = call.q.shape[0]
        out = torch.empty(T, w.num_heads, w.head_size, dtype=w.dtype, device=dev)
        lse = torch.empty(w.num_heads, T, dtype=torch.float32, device=dev)
        po = pl = None
        if call.kind == "decode" and S > 1:
            po = torch.empty(S, T, w.num_heads, w.head_size, dtype=torch.float32, device=dev)
            pl = torch.empty(S, w.num_heads, T, dtype=torch.float32, device=dev)
        cnt = None
        if call.kind == "decode" and S > 1 and merged:
            cnt = torch.zeros(T * w.num_heads, dtype=torch.int32, device=dev)
        ids = torch.from_numpy(np.asarray(call.seq_ids, dtype=np.int64)).to(dev)
        q = call.q.to(dev)
        if self.q_scale is not None:
            q = scaled_fp8_quant(torch.empty(q.shape, dtype=torch.uint8, device=dev), q,
                                 self.q_scale)
        return CallBuffers(
            kind=call.kind, q=q,
            cu_seqlens_q=torch.from_numpy(call.cu_seqlens_q).to(dev),
            seq_lens=torch.from_numpy(call.seq_lens.astype(np.int32)).to(dev),
            block_table=self.block_table.index_select(0, ids).contiguous(),
            max_seqlen_q=int(call.query_lens.max()), max_seqlen_k=int(call.seq_lens.max()),
            num_splits=S, out=out, lse=lse, part_out=po, part_lse=pl, causal=bool(call.causal),
            split_counters=cnt)

    def run(self, cb: CallBuffers, stream=None) -> None:
        w = self.w
        if cb.kind == "prefill":
            paged_attn_prefill(cb.out, cb.q, self.key_cache, self.value_cache, cb.cu_seqlens_q,
                               cb.seq_lens, cb.block_table, cb.max_seqlen_q, cb.max_seqlen_k,
                               w.scale, cb.causal, w.window_left, w.softcap, self.alibi, lse=cb.lse,
                               stream=stream, sinks=self.sinks, k_scale=self.k_scale,
                               v_scale=self.v_scale, q_scale=self.q_scale)
        elif cb.num_splits == 1:
            paged_attn_decode(cb.out, cb.q, self.key_cache, self.value_cache, cb.seq_lens,
                              cb.block_table, cb.max_seqlen_k, w.scale, w.window_left, w.softcap,
                              self.alibi, 1, lse=cb.lse, stream=stream, sinks=self.sinks,
                              k_scale=self.k_scale, v_scale=self.v_scale, q_scale=self.q_scale)
        elif cb.split_counters is not None:
            paged_attn_decode_merged(cb.out, cb.q, self.key_cache, self.value_cache, cb.seq_lens,
                                     cb.block_table, cb.max_seqlen_k, w.scale, cb.num_splits,
                                     cb.part_out, cb.part_lse, cb.split_counters, w.window_left,
                                     w.softcap, self.alibi, lse=cb.lse, stream=stream,
                                     sinks=self.sinks, k_scale=self.k_scale, v_scale=self.v_scale,
                                     q_scale=self.q_scale)
        else:
            paged_attn_decode(None, cb.q, self.key_cache, self.value_cache, cb.seq_lens,
                              cb.block_table, cb.max_seqlen_k, w.scale, w.window_left, w.softcap,
                              self.alibi, cb.num_splits, part_out=cb.part_out,
                              part_lse=cb.part_lse, stream=stream, sinks=self.sinks,
                              k_scale=self.k_scale, v_scale=self.v_scale, q_scale=self.q_scale,
                              out_dtype=w.dtype)
            merge_attn_states(cb.out, cb.part_out, cb.part_lse, out_lse=cb.lse, stream=stream)


def run_workload(w, num_splits: Optional[int] = None, device: str = "cuda"):
    """Fill the cache, run every step in order; returns (cache, [[CallBuffers]])."""
    cache = PagedCache(w, device)
    cache.fill_context()
    results: List[List[CallBuffers]] = []
    for step in w.steps:
        k, v, s = cache.step_inputs(step)
        cache.write(k, v, s)
        bufs = [cache.call_buffers(c, num_splits) for c in step.calls]
        for cb in bufs:
            cache.run(cb)
        results.append(bufs)
    torch.cuda.synchronize()
    return cache, results
