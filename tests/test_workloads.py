"""Input generators: determinism, shapes and the page-printed metadata
examples (no GPU)."""
import hashlib
import json
import os

import numpy as np
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        if isinstance(a, torch.Tensor):
            a = a.contiguous().view(torch.uint8).numpy() if a.dtype in (torch.float16, torch.bfloat16) \
                else a.numpy()
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_cu_seqlens_matches_page_example():
    ex = json.load(open(os.path.join(GOLDEN, "metadata_examples.json")))["cu_seqlens"]
    assert W.cu_seqlens(ex["lengths"]).tolist() == ex["cumulative"]


def test_slot_formula_matches_page_block_table_example():
    ex = json.load(open(os.path.join(GOLDEN, "metadata_examples.json")))["block_table"]
    w = W.tiny()
    w.block_table = np.array([ex["row"]], dtype=np.int32)
    w.block_size = ex["block_size"]
    for tok, blk, off in ex["token_to_block_offset"]:
        assert w.slots(0, np.array([tok]))[0] == blk * ex["block_size"] + off


def test_same_seed_same_bytes():
    for make in (W.tiny, W.prefill_batch):
        a, b = make(), make()
        assert _digest(a.block_table, a.final_lens) == _digest(b.block_table, b.final_lens)
        ka, va, sa = a.step_tokens(a.steps[0])
        kb, vb, sb = b.step_tokens(b.steps[0])
        assert _digest(ka, va, sa, a.steps[0].calls[0].q) == _digest(kb, vb, sb, b.steps[0].calls[0].q)


def test_chunked_generation_is_slice_consistent():
    w = W.mixed_batch()
    b = 50                                 # a prefill sequence longer than one chunk
    L = int(w.final_lens[b])
    k_all, v_all = w.sequence_kv(b)
    k_mid, v_mid = w.sequence_kv(b, 4000, 4200, kv_heads=[3])
    assert torch.equal(k_all[4000:4200, 3:4], k_mid) and torch.equal(v_all[4000:4200, 3:4], v_mid)
    assert k_all.shape == (L, 8, 128) and k_all.dtype == torch.bfloat16


def test_block_tables_are_valid_and_disjoint():
    for make in (W.tiny, W.decode_batch, W.prefill_batch, W.mixed_batch):
        w = make()
        used = []
        for b in range(w.num_seqs):
            n = -(-int(w.final_lens[b]) // w.block_size)
            row = w.block_table[b, :n]
            assert ((row >= 0) & (row < w.num_blocks)).all()
            used.extend(row.tolist())
        assert len(used) == len(set(used))


def test_config_shapes():
    t = W.tiny()
    assert t.context_lens.tolist() == [17, 40] and t.num_blocks == 8
    assert [c.seq_lens.tolist() for s in t.steps for c in s.calls] == [[18, 41], [23]]
    d = W.decode_batch()
    assert d.num_seqs == 64 and d.final_lens.min() >= 512 and d.final_lens.max() <= 4096
    assert d.num_blocks == int(np.ceil(1.1 * sum(-(-int(L) // 16) for L in d.final_lens)))
    p = W.prefill_batch()
    assert (p.context_lens == 0).all() and p.steps[0].calls[0].q.shape[0] == p.final_lens.sum()
    m = W.mixed_batch()
    dec, pre = m.steps[0].calls
    assert dec.num_seqs == 48 and pre.query_lens.tolist() == [512] * 4 and m.block_size == 32
    assert m.window_left == 4095 and m.softcap == 50.0
    l = W.long_decode()
    assert (l.final_lens == 131072).all() and l.steps[0].calls[0].num_splits == 32
    assert abs(float(l.alibi_slopes[0]) - 2 ** -0.125) < 1e-7 and float(l.alibi_slopes[-1]) == 2 ** -8
