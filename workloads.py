"""Seeded synthetic inputs for the paged-KV attention workloads.

This module only draws inputs: sequence lengths, block tables, slot mappings
and Q/K/V values.  It holds none of the attention arithmetic and imports
neither the oracle nor the HIP library; both sides receive the same bytes
from here.

Recipe (all draws are deterministic functions of the workload seed):
  * integers (lengths, block permutation): numpy PCG64(seed), lengths first,
    then one permutation of the block pool; sequence b takes the next
    ceil(L_b / block_size) entries of that permutation, rows are padded
    with 0;
  * values: one torch CPU generator per (tensor, sequence, kv-head) — or per
    (step, sequence) for queries — seeded from a hash of those indices;
    standard normal in float32, multiplied by the workload's value scale in
    float32, then rounded to fp16/bf16 (round-to-nearest-even);
  * a token at logical position j of sequence b is stored in slot
    block_table[b, j // block_size] * block_size + j % block_size;
  * the pool holds ceil(1.1 * sum_b ceil(L_b / block_size)) blocks unless a
    workload fixes it; slots never written stay NaN ("poison") so a kernel
    that reads past a sequence's end shows up as NaN.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

# positions drawn per generator call for K/V, and the tensor tags
KV_CHUNK = 4096
_TAG_K, _TAG_V, _TAG_Q = 1, 2, 3


def _seed_of(*words: int) -> int:
    h = hashlib.blake2b(repr(tuple(int(w) for w in words)).encode(), digest_size=8)
    return int.from_bytes(h.digest(), "little") & ((1 << 63) - 1)


def normal(shape, seed_words: Sequence[int], mult: float, dtype: torch.dtype) -> torch.Tensor:
    g = torch.Generator().manual_seed(_seed_of(*seed_words))
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if mult != 1.0:
        x = x * mult
    return x.to(dtype)


def cu_seqlens(lengths: Sequence[int]) -> np.ndarray:
    """Running start offsets, e.g. lengths [4, 6] -> [0, 4, 10]."""
    out = np.zeros(len(lengths) + 1, dtype=np.int32)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return out


@dataclass
class AttnCall:
    """One attention call of a step over a subset of the workload's sequences."""
    kind: str                      # "decode" or "prefill"
    seq_ids: np.ndarray            # rows of the workload block table, in call order
    query_lens: np.ndarray         # int32 [B]
    seq_lens: np.ndarray           # int32 [B], keys visible after the step's writes
    q: torch.Tensor                # [sum(query_lens), num_heads, head_size]
    causal: bool = True
    num_splits: int = 1            # decode only

    @property
    def cu_seqlens_q(self) -> np.ndarray:
        return cu_seqlens(self.query_lens)

    @property
    def num_seqs(self) -> int:
        return len(self.seq_ids)


@dataclass
class Step:
    """New tokens written through reshape_and_cache, then attention calls."""
    new_positions: List[np.ndarray]   # per workload sequence: logical positions written
    calls: List[AttnCall]


@dataclass
class Workload:
    name: str
    seed: int
    dtype: torch.dtype
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    num_blocks: int
    final_lens: np.ndarray            # int32 [B]: length of each sequence after all steps
    context_lens: np.ndarray          # int32 [B]: tokens cached before the first step
    block_table: np.ndarray           # int32 [B, max_blocks]
    value_mult: float = 1.0
    scale: float = 1.0
    window_left: int = -1
    softcap: float = 0.0
    alibi_slopes: Optional[torch.Tensor] = None   # fp32 [num_heads]
    steps: List[Step] = field(default_factory=list)

    @property
    def num_seqs(self) -> int:
        return len(self.final_lens)

    def slots(self, b: int, positions: np.ndarray) -> np.ndarray:
        """Cache slots (int64) of logical positions of sequence b."""
        positions = np.asarray(positions, dtype=np.int64)
        blk = self.block_table[b][positions // self.block_size].astype(np.int64)
        return blk * self.block_size + positions % self.block_size

    def sequence_kv(self, b: int, lo: int = 0, hi: Optional[int] = None,
                    kv_heads: Optional[Sequence[int]] = None):
        """Logical K and V rows [lo, hi) of sequence b: [hi-lo, n_heads, D].

        Values are drawn in chunks of KV_CHUNK positions per (sequence,
        kv-head), so any slice can be regenerated without drawing the rest."""
        L = int(self.final_lens[b])
        hi = L if hi is None else hi
        heads = range(self.num_kv_heads) if kv_heads is None else kv_heads
        c0, c1 = lo // KV_CHUNK, (hi - 1) // KV_CHUNK
        ks, vs = [], []
        for g in heads:
            kc, vc = [], []
            for c in range(c0, c1 + 1):
                n = min(KV_CHUNK, L - c * KV_CHUNK)
                kc.append(normal((n, self.head_size), (self.seed, _TAG_K, b, g, c),
                                 self.value_mult, self.dtype))
                vc.append(normal((n, self.head_size), (self.seed, _TAG_V, b, g, c),
                                 self.value_mult, self.dtype))
            base = c0 * KV_CHUNK
            ks.append(torch.cat(kc)[lo - base:hi - base])
            vs.append(torch.cat(vc)[lo - base:hi - base])
        return torch.stack(ks, dim=1), torch.stack(vs, dim=1)

    def step_tokens(self, step: Step):
        """(key, value, slot_mapping) written by one step, concatenated over
        sequences in workload order."""
        ks, vs, ss = [], [], []
        for b, pos in enumerate(step.new_positions):
            if len(pos) == 0:
                continue
            k, v = self.sequence_kv(b, int(pos[0]), int(pos[-1]) + 1)
            ks.append(k)
            vs.append(v)
            ss.append(self.slots(b, pos))
        return torch.cat(ks), torch.cat(vs), torch.from_numpy(np.concatenate(ss))

    def context_tokens(self, seq_ids: Optional[Sequence[int]] = None):
        """(key, value, slot_mapping) of the cached context, sequence by
        sequence; yields one triple per sequence to bound memory."""
        ids = range(self.num_seqs) if seq_ids is None else seq_ids
        for b in ids:
            C = int(self.context_lens[b])
            if C == 0:
                continue
            k, v = self.sequence_kv(b, 0, C)
            yield b, k, v, torch.from_numpy(self.slots(b, np.arange(C)))


def _block_table(rng: np.random.Generator, lens: np.ndarray, block_size: int,
                 num_blocks: Optional[int] = None):
    need = [-(-int(L) // block_size) for L in lens]
    if num_blocks is None:
        num_blocks = math.ceil(1.1 * sum(need))
    perm = rng.permutation(num_blocks)
    table = np.zeros((len(lens), max(need)), dtype=np.int32)
    at = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[at:at + n]
        at += n
    return num_blocks, table


def _query(seed: int, step: int, b: int, n: int, heads: int, D: int, mult: float, dtype) -> torch.Tensor:
    return normal((n, heads, D), (seed, _TAG_Q, step, b), mult, dtype)


def tiny(seed: int = 1) -> Workload:
    """fp16, 2 sequences with cached context 17 and 40, block 16, 4 query /
    2 KV heads of size 64, scale 1/8, block table a permutation of 8 blocks.
    Step 0: one new token per sequence, then decode.  Step 1: a causal
    prefill chunk of 5 new tokens on sequence 0."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = np.array([17, 40], dtype=np.int32)
    final = np.array([17 + 1 + 5, 40 + 1], dtype=np.int32)
    perm = rng.permutation(8)
    table = np.stack([perm[:4], perm[4:]]).astype(np.int32)
    w = Workload("tiny_fp16", seed, torch.float16, 4, 2, 64, 16, 8, final, ctx, table,
                 scale=1.0 / math.sqrt(64))
    q0 = torch.cat([_query(seed, 0, b, 1, 4, 64, 1.0, torch.float16) for b in range(2)])
    w.steps.append(Step([np.array([17]), np.array([40])], [
        AttnCall("decode", np.array([0, 1]), np.array([1, 1], np.int32),
                 np.array([18, 41], np.int32), q0)]))
    q1 = _query(seed, 1, 0, 5, 4, 64, 1.0, torch.float16)
    w.steps.append(Step([np.arange(18, 23), np.array([], np.int64)], [
        AttnCall("prefill", np.array([0]), np.array([5], np.int32),
                 np.array([23], np.int32), q1)]))
    return w


def _decode_workload(name, seed, lens, Hq, Hkv, D, bs, num_splits, dtype=torch.bfloat16,
                     window_left=-1, softcap=0.0, alibi=None, rng=None) -> Workload:
    rng = rng or np.random.Generator(np.random.PCG64(seed))
    nb, table = _block_table(rng, lens, bs)
    w = Workload(name, seed, dtype, Hq, Hkv, D, bs, nb, lens.astype(np.int32),
                 (lens - 1).astype(np.int32), table, scale=1.0 / math.sqrt(D),
                 window_left=window_left, softcap=softcap, alibi_slopes=alibi)
    B = len(lens)
    q = torch.cat([_query(seed, 0, b, 1, Hq, D, 1.0, dtype) for b in range(B)])
    w.steps.append(Step([np.array([L - 1]) for L in lens], [
        AttnCall("decode", np.arange(B), np.ones(B, np.int32), lens.astype(np.int32), q,
                 num_splits=num_splits)]))
    return w


def decode_batch(seed: int = 2, num_splits: int = 8) -> Workload:
    """bf16 decode: 64 sequences, context uniform in [512, 4096], 32 query /
    8 KV heads of size 128, block 16, shuffled pool sized for the context
    plus 10%, no masks."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(512, 4096, size=64, endpoint=True)
    return _decode_workload("decode_b64_l512-4096_h32-8-128_bs16", seed, lens, 32, 8, 128, 16,
                            num_splits, rng=rng)


def prefill_batch(seed: int = 3) -> Workload:
    """bf16 varlen causal prefill: 16 sequences of length uniform in
    [256, 2048], no prior context, 32 query / 8 KV heads of size 128,
    block 16, Q/K/V scaled by 0.5; K/V reach the cache through
    reshape_and_cache before attention."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(256, 2048, size=16, endpoint=True)
    nb, table = _block_table(rng, lens, 16)
    w = Workload("prefill_b16_l256-2048_h32-8-128_bs16", seed, torch.bfloat16, 32, 8, 128, 16,
                 nb, lens.astype(np.int32), np.zeros(16, np.int32), table, value_mult=0.5,
                 scale=1.0 / math.sqrt(128))
    q = torch.cat([_query(seed, 0, b, int(L), 32, 128, 0.5, torch.bfloat16)
                   for b, L in enumerate(lens)])
    w.steps.append(Step([np.arange(L) for L in lens], [
        AttnCall("prefill", np.arange(16), lens.astype(np.int32), lens.astype(np.int32), q)]))
    return w


def mixed_batch(seed: int = 4, num_splits: int = 16) -> Workload:
    """bf16 mixed chunked-prefill: 48 decode sequences (context uniform in
    [1024, 8192]) and 4 prefill chunks of 512 new tokens on contexts uniform
    in [2048, 8192]; 32 query / 8 KV heads of size 128, block 32, sliding
    window 4096, logits softcap 50.  Decodes come first in the token order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dec = rng.integers(1024, 8192, size=48, endpoint=True)
    pctx = rng.integers(2048, 8192, size=4, endpoint=True)
    final = np.concatenate([dec, pctx + 512]).astype(np.int32)
    ctx = np.concatenate([dec - 1, pctx]).astype(np.int32)
    nb, table = _block_table(rng, final, 32)
    w = Workload("mixed_d48_p4x512_h32-8-128_bs32_w4096_cap50", seed, torch.bfloat16, 32, 8,
                 128, 32, nb, final, ctx, table, scale=1.0 / math.sqrt(128),
                 window_left=4095, softcap=50.0)
    qd = torch.cat([_query(seed, 0, b, 1, 32, 128, 1.0, torch.bfloat16) for b in range(48)])
    qp = torch.cat([_query(seed, 0, 48 + i, 512, 32, 128, 1.0, torch.bfloat16) for i in range(4)])
    positions = [np.array([L - 1]) for L in dec] + [np.arange(c, c + 512) for c in pctx]
    w.steps.append(Step(positions, [
        AttnCall("decode", np.arange(48), np.ones(48, np.int32), dec.astype(np.int32), qd,
                 num_splits=num_splits),
        AttnCall("prefill", np.arange(48, 52), np.full(4, 512, np.int32),
                 (pctx + 512).astype(np.int32), qp)]))
    return w


def alibi_slopes(num_heads: int) -> torch.Tensor:
    """Slope of head h (0-based) is 2^(-8 (h + 1) / num_heads)."""
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / num_heads) for h in range(num_heads)],
                        dtype=torch.float32)


def long_decode(seed: int = 5, context: int = 131072, num_seqs: int = 8) -> Workload:
    """bf16 long-context split-KV decode: 8 sequences of 131072 tokens,
    64 query / 8 KV heads of size 256, block 16, ALiBi slopes 2^(-8h/64),
    32 key partitions merged by log-sum-exp."""
    lens = np.full(num_seqs, context, dtype=np.int64)
    return _decode_workload(f"long_decode_b{num_seqs}_l{context}_h64-8-256_bs16_alibi_s32",
                            seed, lens, 64, 8, 256, 16, 32, alibi=alibi_slopes(64))


WORKLOADS = {
    "tiny": tiny,
    "decode": decode_batch,
    "prefill": prefill_batch,
    "mixed": mixed_batch,
    "long": long_decode,
}


def custom(name: str, seed: int, ctx_lens, q_lens, num_heads: int, num_kv_heads: int,
           head_size: int, block_size: int, dtype=torch.bfloat16, kind: str = "prefill",
           window_left: int = -1, softcap: float = 0.0, alibi: bool = False,
           num_splits: int = 1, value_mult: float = 1.0) -> Workload:
    """A one-step workload of arbitrary shape (edge cases in tests): sequence b
    has ctx_lens[b] cached tokens and q_lens[b] new tokens, written by
    reshape_and_cache, then one decode (all q_lens 1) or prefill call."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    ql = np.asarray(q_lens, dtype=np.int64)
    final = ctx + ql
    nb, table = _block_table(rng, np.maximum(final, 1), block_size)
    w = Workload(name, seed, dtype, num_heads, num_kv_heads, head_size, block_size, nb,
                 final.astype(np.int32), ctx.astype(np.int32), table, value_mult=value_mult,
                 scale=1.0 / math.sqrt(head_size), window_left=window_left, softcap=softcap,
                 alibi_slopes=alibi_slopes(num_heads) if alibi else None)
    B = len(final)
    q = torch.cat([_query(seed, 0, b, int(ql[b]), num_heads, head_size, value_mult, dtype)
                   for b in range(B)])
    if kind == "decode":
        assert (ql == 1).all()
    w.steps.append(Step([np.arange(c, c + n) for c, n in zip(ctx, ql)], [
        AttnCall(kind, np.arange(B), ql.astype(np.int32), final.astype(np.int32), q,
                 num_splits=num_splits)]))
    return w
