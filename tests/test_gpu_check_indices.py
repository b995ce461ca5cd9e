"""GPU test of pa_check_indices, the debug validation of the index arrays
the attention calls trust: its three counts equal the counts computed here
with numpy (integers: exact), for crafted arrays with known bad entries and
for the configured workloads' own tables (all valid)."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_attention_29_amd as pa
    return pa


def _expected(slots, table, lens, num_blocks, bs):
    bad_slot = int((slots >= num_blocks * bs).sum()) if slots is not None else 0
    bad_id = bad_len = 0
    if lens is not None:
        for b, L in enumerate(lens.tolist()):
            used = -(-L // bs) if L > 0 else 0
            if L < 0 or used > table.shape[1]:
                bad_len += 1
                continue
            row = table[b, :used]
            bad_id += int(((row < 0) | (row >= num_blocks)).sum())
    return [bad_slot, bad_id, bad_len]


def test_counts_match_crafted_errors(pa):
    print("\n[gpu-case] pa_check_indices crafted", flush=True)
    rng = np.random.default_rng(3)
    num_blocks, bs = 50, 16
    slots = rng.integers(-3, num_blocks * bs, size=3000).astype(np.int64)
    slots[::97] = num_blocks * bs + rng.integers(0, 1000, size=slots[::97].shape)
    B, cols = 300, 12
    table = rng.integers(0, num_blocks, size=(B, cols)).astype(np.int32)
    lens = rng.integers(0, cols * bs + 1, size=B).astype(np.int32)
    table[:, -2:] = 2 ** 30                      # padding past most rows: bad but unread
    for b in range(0, B, 17):                    # bad ids inside used ranges
        used = -(-int(lens[b]) // bs)
        if used:
            table[b, used - 1] = -5 if b % 2 else num_blocks
    lens[5] = -1
    lens[6] = cols * bs + 1                      # more blocks than a row holds
    counts = torch.full((3,), 12345, dtype=torch.int32, device="cuda")
    pa.check_indices(num_blocks, bs, torch.from_numpy(slots).cuda(),
                     torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda(), counts=counts)
    torch.cuda.synchronize()
    exp = _expected(slots, table, lens, num_blocks, bs)
    assert exp[0] > 0 and exp[1] > 0 and exp[2] == 2
    assert counts.cpu().tolist() == exp
    # slots only, and a table only
    c1 = pa.check_indices(num_blocks, bs, slot_mapping=torch.from_numpy(slots).cuda())
    c2 = pa.check_indices(num_blocks, bs, block_table=torch.from_numpy(table).cuda(),
                          seq_lens=torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    assert c1.cpu().tolist() == [exp[0], 0, 0] and c2.cpu().tolist() == [0, exp[1], exp[2]]


@pytest.mark.parametrize("make", [W.tiny, W.decode_batch, W.prefill_batch, W.mixed_batch])
def test_workload_tables_are_clean(pa, make):
    w = make()
    print(f"\n[gpu-case] pa_check_indices {w.name}", flush=True)
    table = torch.from_numpy(np.ascontiguousarray(w.block_table)).cuda()
    lens = torch.from_numpy(w.final_lens.astype(np.int32)).cuda()
    # the slot of every position of every sequence
    slots = torch.from_numpy(np.concatenate(
        [w.slots(b, np.arange(int(L))) for b, L in enumerate(w.final_lens)]).astype(np.int64)).cuda()
    c = pa.check_indices(w.num_blocks, w.block_size, slot_mapping=slots, block_table=table,
                         seq_lens=lens)
    torch.cuda.synchronize()
    assert c.cpu().tolist() == [0, 0, 0]
