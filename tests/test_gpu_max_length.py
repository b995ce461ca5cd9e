"""Prefill and split decode at the longest sequence the library accepts:
2^24 - 1 keys (the block division is a multiply-high reciprocal exact below
2^24; longer sequences are rejected on the host).  One KV head of 64, block
256, bf16; the cache holds the sequence through a shuffled block table.
The last three positions are the queries of a causal prefill; the last one
is also decoded alone with 64 splits and merged.  Both are compared with
the oracle, element by element.

The sequence's K/V rows are drawn once (about 2 x 2 GB) and used twice: the
GPU cache is filled with reshape_and_cache through the shuffled table, and
the oracle's cache is the same rows in position order (block b of the
sequence in cache block b), read through the identity table — the slot
rule that maps one to the other is pinned on its own in the CPU tests."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle_side import assert_attn_close, assert_lse_close

pytestmark = pytest.mark.gpu

L = (1 << 24) - 1
BS = 256
NQ = 3
SPLITS = 64


def _announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_attention_29_amd as pa
    return pa


@pytest.mark.timeout(900)
def test_prefill_and_decode_at_the_longest_sequence(pa):
    _announce(f"max-length sequence: L={L}, block {BS}, prefill {NQ} queries, decode {SPLITS} splits")
    w = W.custom("max_len", 41, [L - NQ], [NQ], 1, 1, 64, BS, torch.bfloat16, "prefill")
    call = w.steps[0].calls[0]
    k, v = w.sequence_kv(0, 0, L)  # [L, 1, 64], positions in order
    dev = torch.device("cuda")

    # ---- GPU: the cache through the workload's shuffled block table
    nb = w.num_blocks
    kc = torch.full((nb, BS, 1, 64), float("nan"), dtype=torch.bfloat16, device=dev)
    vc = torch.full_like(kc, float("nan"))
    table = torch.from_numpy(np.ascontiguousarray(w.block_table)).to(dev)
    pos = torch.arange(L, dtype=torch.int64, device=dev)
    slots = table[0].to(torch.int64)[pos // BS] * BS + pos % BS
    pa.reshape_and_cache(k.to(dev), v.to(dev), kc, vc, slots)
    del pos, slots
    q = call.q.to(dev)
    lens = torch.tensor([L], dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((1, NQ), dtype=torch.float32, device=dev)
    pa.paged_attn_prefill(out, q, kc, vc, torch.tensor([0, NQ], dtype=torch.int32, device=dev),
                          lens, table, NQ, L, w.scale, True, lse=lse)
    qd = q[NQ - 1:].contiguous()
    part_out = torch.empty((SPLITS, 1, 1, 64), dtype=torch.float32, device=dev)
    part_lse = torch.empty((SPLITS, 1, 1), dtype=torch.float32, device=dev)
    pa.paged_attn_decode(None, qd, kc, vc, lens, table, L, w.scale, num_splits=SPLITS,
                         part_out=part_out, part_lse=part_lse)
    dout = torch.empty_like(qd)
    dlse = torch.empty((1, 1), dtype=torch.float32, device=dev)
    pa.merge_attn_states(dout, part_out, part_lse, out_lse=dlse)
    torch.cuda.synchronize()
    res = [t.cpu() for t in (out, lse, dout, dlse)]
    del kc, vc, table, q, out, lse, qd, part_out, part_lse, dout, dlse
    torch.cuda.empty_cache()

    # ---- oracle: the same rows in position order, identity block table
    _announce("oracle over 2^24 - 1 keys")
    nblk = -(-L // BS)
    pad = nblk * BS - L
    nan_row = torch.full((pad, 1, 64), float("nan"), dtype=torch.bfloat16)
    kco = torch.cat([k, nan_row]).view(nblk, BS, 1, 64)
    vco = torch.cat([v, nan_row]).view(nblk, BS, 1, 64)
    del k, v
    ident = torch.arange(nblk, dtype=torch.int32)[None]
    ref_out, ref_lse = oracle.attend(call.q, kco, vco, [0, NQ], [L], ident, w.scale, True)

    assert_attn_close(res[0], ref_out, "prefill at 2^24 - 1 keys")
    assert_lse_close(res[1], ref_lse, "prefill lse at 2^24 - 1 keys")
    assert_attn_close(res[2], ref_out[NQ - 1:], "split decode at 2^24 - 1 keys")
    assert_lse_close(res[3], ref_lse[:, NQ - 1:], "split decode lse at 2^24 - 1 keys")
