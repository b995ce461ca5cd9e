"""Pins of the CPU oracle against things other than itself (no GPU).

Each test ties an oracle function to a page-printed example, a closed form,
an invariant, a library routine on a special case, or pure-Python brute force
on tiny inputs.  Together they are chosen so that a dropped term, a wrong
sign or index, or a transposed operand anywhere in the oracle fails one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NAN = float("nan")


# ----------------------------------------------------------------------------
# helpers: a small paged problem built from logical K/V the test keeps
# ----------------------------------------------------------------------------
class Paged:
    """Logical per-sequence K/V plus a shuffled paged cache holding them."""

    def __init__(self, lens, Hkv, D, bs, dtype=torch.float32, seed=0, pool_extra=3,
                 kmult=1.0):
        g = torch.Generator().manual_seed(seed)
        self.lens = list(lens)
        self.bs, self.Hkv, self.D = bs, Hkv, D
        need = [-(-L // bs) for L in lens]
        self.nb = sum(need) + pool_extra
        perm = torch.randperm(self.nb, generator=g)
        self.table = torch.zeros(len(lens), max(need), dtype=torch.int32)
        at = 0
        for b, n in enumerate(need):
            self.table[b, :n] = perm[at:at + n]
            at += n
        self.K = [(torch.randn(L, Hkv, D, generator=g) * kmult).to(dtype) for L in lens]
        self.V = [torch.randn(L, Hkv, D, generator=g).to(dtype) for L in lens]
        self.kc = torch.full((self.nb, bs, Hkv, D), NAN, dtype=dtype)
        self.vc = torch.full((self.nb, bs, Hkv, D), NAN, dtype=dtype)
        for b, L in enumerate(lens):
            for j in range(L):
                blk = int(self.table[b, j // bs])
                self.kc[blk, j % bs] = self.K[b][j]
                self.vc[blk, j % bs] = self.V[b][j]


def brute_force(q, kc, vc, cu, lens, table, scale, causal, wl, cap, slopes, key_ranges=None):
    """Pure-Python float64 attention, addressing the cache slot by slot."""
    q = q.double().tolist()
    kcl = kc.double().tolist()
    vcl = vc.double().tolist()
    T, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv, bs = len(kcl[0][0]), len(kcl[0])
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(T)]
    lse = [[-math.inf] * T for _ in range(Hq)]
    for b in range(len(lens)):
        nq, L = cu[b + 1] - cu[b], lens[b]
        for t in range(nq):
            row, p = cu[b] + t, L - nq + t
            for h in range(Hq):
                g = (h * Hkv) // Hq
                scores, vrows = [], []
                for j in range(L):
                    if causal and j > p:
                        continue
                    if wl >= 0 and j < p - wl:
                        continue
                    if key_ranges is not None and not (key_ranges[b][0] <= j < key_ranges[b][1]):
                        continue
                    blk, off = int(table[b][j // bs]), j % bs
                    k = kcl[blk][off][g]
                    s = scale * sum(q[row][h][d] * k[d] for d in range(D))
                    if cap > 0:
                        s = cap * math.tanh(s / cap)
                    if slopes is not None:
                        s -= float(slopes[h]) * abs(p - j)
                    scores.append(s)
                    vrows.append(vcl[blk][off][g])
                if not scores:
                    continue
                m = max(scores)
                ws = [math.exp(s - m) for s in scores]
                tot = sum(ws)
                for d in range(D):
                    out[row][h][d] = sum(w * v[d] for w, v in zip(ws, vrows)) / tot
                lse[h][row] = m + math.log(tot)
    return torch.tensor(out, dtype=torch.float64), torch.tensor(lse, dtype=torch.float64)


# ----------------------------------------------------------------------------
# a1: scatter
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_scatter_bitexact_vs_numpy_fancy_index(dtype):
    g = torch.Generator().manual_seed(7)
    nb, bs, Hkv, D, T = 6, 16, 2, 64, 40
    key = torch.randn(T + 3, Hkv, D, generator=g).to(dtype)      # padded rows
    val = torch.randn(T + 3, Hkv, D, generator=g).to(dtype)
    slots = torch.randperm(nb * bs, generator=g)[:T].to(torch.int64)
    slots[[3, 11, 30]] = -1                                        # padding slots
    sentinel = 0x7E01 if dtype == torch.float16 else 0x7FC1
    kc = torch.full((nb, bs, Hkv, D), 0, dtype=torch.int16).fill_(sentinel).view(dtype)
    vc = kc.clone()
    oracle.scatter(key, val, slots, kc, vc)

    kn = np.full((nb * bs, Hkv, D), sentinel, dtype=np.uint16)
    vn = kn.copy()
    s = slots.numpy()
    ok = s >= 0
    kn[s[ok]] = key[:T].view(torch.int16).numpy().view(np.uint16)[ok]
    vn[s[ok]] = val[:T].view(torch.int16).numpy().view(np.uint16)[ok]
    assert np.array_equal(kc.view(torch.int16).numpy().view(np.uint16).reshape(nb * bs, Hkv, D), kn)
    assert np.array_equal(vc.view(torch.int16).numpy().view(np.uint16).reshape(nb * bs, Hkv, D), vn)


def test_gather_matches_page_block_table_example():
    ex = json.load(open(os.path.join(GOLDEN, "metadata_examples.json")))["block_table"]
    bs = ex["block_size"]
    row = torch.tensor(ex["row"], dtype=torch.int32)
    cache = torch.zeros(3, bs, 1, 2)
    for blk in range(3):
        for off in range(bs):
            cache[blk, off, 0, 0] = blk
            cache[blk, off, 0, 1] = off
    rows = oracle.gather_sequence(cache, row, 3 * bs)
    for tok, blk, off in ex["token_to_block_offset"]:
        assert rows[tok, 0, 0] == blk and rows[tok, 0, 1] == off


# ----------------------------------------------------------------------------
# a2-a7: attention against brute force, SDPA and closed forms
# ----------------------------------------------------------------------------
BF_CASES = [
    # lens, query_lens, Hq, Hkv, D, bs, causal, wl, cap, alibi
    ([18, 41], [1, 1], 4, 2, 8, 16, True, -1, 0.0, False),        # decode, config-1 shape
    ([23], [5], 4, 2, 8, 16, True, -1, 0.0, False),               # prefill chunk
    ([23, 9], [5, 9], 4, 2, 8, 16, True, 6, 0.0, False),          # window
    ([23, 9], [5, 3], 4, 1, 8, 16, True, -1, 1.0, False),         # strong softcap
    ([23, 9], [5, 3], 6, 2, 8, 16, True, -1, 5.0, True),          # softcap + alibi, G=3
    ([20, 7], [4, 7], 2, 2, 8, 32, False, -1, 0.0, True),         # non-causal alibi
    ([33], [33], 8, 2, 4, 16, True, 3, 0.0, True),                # window + alibi
]


@pytest.mark.parametrize("case", BF_CASES)
def test_attend_vs_brute_force(case):
    lens, qlens, Hq, Hkv, D, bs, causal, wl, cap, alibi = case
    P = Paged(lens, Hkv, D, bs, seed=len(lens) + D, kmult=2.0)
    g = torch.Generator().manual_seed(11)
    cu = W.cu_seqlens(qlens).tolist()
    q = torch.randn(cu[-1], Hq, D, generator=g)
    slopes = W.alibi_slopes(Hq) if alibi else None
    scale = 1.0 / math.sqrt(D)
    o, l = oracle.attend(q, P.kc, P.vc, cu, lens, P.table, scale, causal, wl, cap, slopes)
    ob, lb = brute_force(q, P.kc, P.vc, cu, lens, P.table.tolist(), scale, causal, wl, cap, slopes)
    assert torch.allclose(o, ob, atol=1e-12, rtol=1e-12)
    assert torch.allclose(l, lb, atol=1e-12, rtol=1e-12)


def _dense_mask(qlen, L, causal, wl):
    p = torch.arange(L - qlen, L)[:, None]
    j = torch.arange(L)[None, :]
    m = torch.ones(qlen, L, dtype=torch.bool)
    if causal:
        m &= j <= p
    if wl >= 0:
        m &= p - j <= wl
    return m


@pytest.mark.parametrize("alibi", [False, True])
@pytest.mark.parametrize("wl", [-1, 37])
def test_attend_vs_torch_sdpa(alibi, wl):
    lens, qlens, Hq, Hkv, D, bs = [150, 97, 64], [150, 20, 1], 8, 2, 32, 16
    P = Paged(lens, Hkv, D, bs, seed=3)
    g = torch.Generator().manual_seed(5)
    cu = W.cu_seqlens(qlens).tolist()
    q = torch.randn(cu[-1], Hq, D, generator=g)
    slopes = W.alibi_slopes(Hq) if alibi else None
    scale = 0.3
    o, l = oracle.attend(q, P.kc, P.vc, cu, lens, P.table, scale, True, wl, 0.0, slopes)
    for b, (L, nq) in enumerate(zip(lens, qlens)):
        K = P.K[b].double().repeat_interleave(Hq // Hkv, dim=1).permute(1, 0, 2)[None]
        V = P.V[b].double().repeat_interleave(Hq // Hkv, dim=1).permute(1, 0, 2)[None]
        Q = q[cu[b]:cu[b + 1]].double().permute(1, 0, 2)[None]
        vis = _dense_mask(nq, L, True, wl)
        bias = torch.zeros(Hq, nq, L, dtype=torch.float64)
        if alibi:
            dist = (torch.arange(L - nq, L)[:, None] - torch.arange(L)[None, :]).double()
            bias = -slopes.double()[:, None, None] * dist[None]
        bias = bias.masked_fill(~vis[None], float("-inf"))
        ref = F.scaled_dot_product_attention(Q, K, V, attn_mask=bias[None], scale=scale)[0]
        assert torch.allclose(o[cu[b]:cu[b + 1]].permute(1, 0, 2), ref, atol=1e-10)
        # LSE from the library's own logsumexp over the biased scores
        s = scale * (Q[0] @ K[0].transpose(-1, -2)) + bias
        assert torch.allclose(l[:, cu[b]:cu[b + 1]], torch.logsumexp(s, dim=-1), atol=1e-10)


def test_zero_query_gives_mean_and_log_count():
    lens, qlens = [40, 23], [6, 1]
    P = Paged(lens, 2, 16, 16, seed=9)
    cu = W.cu_seqlens(qlens).tolist()
    q = torch.zeros(cu[-1], 4, 16)
    o, l = oracle.attend(q, P.kc, P.vc, cu, lens, P.table, 0.7, True, 9, 0.0, None)
    for b, (L, nq) in enumerate(zip(lens, qlens)):
        for t in range(nq):
            p = L - nq + t
            lo = max(0, p - 9)
            n = p - lo + 1
            for h in range(4):
                mean = P.V[b][lo:p + 1, h // 2].double().mean(dim=0)
                assert torch.allclose(o[cu[b] + t, h], mean, atol=1e-12)
                assert abs(float(l[h, cu[b] + t]) - math.log(n)) < 1e-12


def test_zero_query_alibi_geometric_closed_form():
    L = 50
    P = Paged([L], 1, 8, 16, seed=2)
    q = torch.zeros(L, 2, 8)
    slopes = torch.tensor([0.5, 0.125])
    o, l = oracle.attend(q, P.kc, P.vc, [0, L], [L], P.table, 1.0, True, -1, 0.0, slopes)
    for h, sig in enumerate([0.5, 0.125]):
        for p in range(L):
            n = p + 1
            closed = math.log((1 - math.exp(-sig * n)) / (1 - math.exp(-sig)))
            assert abs(float(l[h, p]) - closed) < 1e-12


def test_window_zero_returns_own_value_row():
    lens = [37]
    P = Paged(lens, 2, 16, 16, seed=4)
    q = torch.randn(37, 2, 16)
    o, _ = oracle.attend(q, P.kc, P.vc, [0, 37], lens, P.table, 1.0, True, 0, 0.0, None)
    assert torch.equal(o, P.V[0].double())


def test_single_key_returns_that_value():
    P = Paged([1, 1], 1, 8, 16, seed=6)
    q = torch.randn(2, 3, 8)
    o, l = oracle.decode(q, P.kc, P.vc, [1, 1], P.table, 0.5)
    for b in range(2):
        assert torch.equal(o[b], P.V[b][0, 0].double().expand(3, 8))
        sc = 0.5 * (q[b].double() @ P.K[b][0, 0].double())
        assert torch.allclose(l[:, b], sc, atol=1e-14)


def test_sequence_without_keys_gives_zero_and_neg_inf():
    """A decode row of a zero-length sequence sees no key: out 0, lse -inf,
    and the other rows are those of the batch without it."""
    P = Paged([0, 1, 21], 2, 8, 16, seed=7)
    q = torch.randn(3, 4, 8)
    o, l = oracle.decode(q, P.kc, P.vc, [0, 1, 21], P.table, 0.5)
    assert torch.equal(o[0], torch.zeros(4, 8, dtype=torch.float64))
    assert torch.isneginf(l[:, 0]).all()
    o2, l2 = oracle.decode(q[1:], P.kc, P.vc, [1, 21], P.table[1:], 0.5)
    assert torch.equal(o[1:], o2) and torch.equal(l[:, 1:], l2)
    assert torch.equal(o[1], P.V[1][0].double().repeat_interleave(2, dim=0))
    po, pl = oracle.decode_splits(q, P.kc, P.vc, [0, 1, 21], P.table, 0.5, 3)
    assert torch.equal(po[:, 0], torch.zeros(3, 4, 8, dtype=torch.float64))
    assert torch.isneginf(pl[:, :, 0]).all()


def test_huge_softcap_equals_no_softcap():
    P = Paged([30, 12], 2, 16, 16, seed=8)
    q = torch.randn(2, 4, 16)
    a = oracle.decode(q, P.kc, P.vc, [30, 12], P.table, 0.25, softcap=1e30)
    b = oracle.decode(q, P.kc, P.vc, [30, 12], P.table, 0.25)
    assert torch.allclose(a[0], b[0], atol=1e-12) and torch.allclose(a[1], b[1], atol=1e-12)


def test_softmax_rows_sum_to_one_via_constant_values():
    P = Paged([64, 17], 2, 8, 16, seed=10)
    P.vc[~torch.isnan(P.vc)] = 1.0
    cu = [0, 64, 65]
    q = torch.randn(65, 4, 8) * 3
    o, _ = oracle.attend(q, P.kc, P.vc, cu, [64, 17], P.table, 1.0, True, 20, 7.0,
                         W.alibi_slopes(4))
    assert (o - 1.0).abs().max() < 1e-6


# ----------------------------------------------------------------------------
# paging, causality and decode/prefill invariants
# ----------------------------------------------------------------------------
def test_permuting_physical_blocks_is_bit_identical():
    P = Paged([70, 33], 2, 16, 16, seed=12)
    cu = [0, 70, 73]
    q = torch.randn(73, 4, 16)
    o1, l1 = oracle.attend(q, P.kc, P.vc, cu, [70, 33], P.table, 0.2, True, 25, 3.0, None)
    perm = torch.randperm(P.nb)
    kc2, vc2 = torch.empty_like(P.kc), torch.empty_like(P.vc)
    kc2[perm] = P.kc
    vc2[perm] = P.vc
    table2 = perm[P.table.long()].to(torch.int32)
    o2, l2 = oracle.attend(q, kc2, vc2, cu, [70, 33], table2, 0.2, True, 25, 3.0, None)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_identity_table_equals_dense_attention():
    L, Hkv, D = 40, 1, 8
    P = Paged([L], Hkv, D, 64, seed=13, pool_extra=0)
    assert P.nb == 1
    q = torch.randn(L, 1, D)
    o, _ = oracle.attend(q, P.kc, P.vc, [0, L], [L], torch.zeros(1, 1, dtype=torch.int32),
                         0.5, True)
    K, V = P.K[0][:, 0].double(), P.V[0][:, 0].double()
    s = 0.5 * q[:, 0].double() @ K.T
    s = s.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
    assert torch.allclose(o[:, 0], torch.softmax(s, dim=-1) @ V, atol=1e-12)


def test_causal_output_ignores_future_keys():
    P = Paged([48], 2, 16, 16, seed=14)
    q = torch.randn(48, 4, 16)
    o1, l1 = oracle.attend(q, P.kc, P.vc, [0, 48], [48], P.table, 0.3, True)
    kc, vc = P.kc.clone(), P.vc.clone()
    for j in range(30, 48):
        blk = int(P.table[0, j // 16])
        kc[blk, j % 16] += 5.0
        vc[blk, j % 16] -= 3.0
    o2, l2 = oracle.attend(q, kc, vc, [0, 48], [48], P.table, 0.3, True)
    assert torch.equal(o1[:30], o2[:30]) and torch.equal(l1[:, :30], l2[:, :30])
    assert not torch.equal(o1[30:], o2[30:])


def test_decode_equals_last_row_of_prefill():
    lens = [57, 16]
    P = Paged(lens, 2, 16, 16, seed=15)
    q = torch.randn(sum(lens), 4, 16)
    cu = W.cu_seqlens(lens).tolist()
    op, lp = oracle.attend(q, P.kc, P.vc, cu, lens, P.table, 0.25, True, 20, 4.0,
                           W.alibi_slopes(4))
    last = [cu[b + 1] - 1 for b in range(2)]
    od, ld = oracle.decode(q[last], P.kc, P.vc, lens, P.table, 0.25, 20, 4.0, W.alibi_slopes(4))
    assert torch.allclose(od, op[last], atol=1e-13) and torch.allclose(ld, lp[:, last], atol=1e-13)


# ----------------------------------------------------------------------------
# a8-a9: split boundaries and merge
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("L,S,bs,mx", [(131072, 32, 16, None), (1000, 3, 16, None),
                                       (17, 4, 16, None), (5, 8, 32, None), (4096, 7, 32, None),
                                       (1000, 3, 16, 4096), (700, 8, 16, 4096), (5000, 4, 16, 4096)])
def test_split_bounds_partition_block_aligned(L, S, bs, mx):
    b = oracle.split_bounds(L, S, bs, mx)
    assert len(b) == S and b[0][0] == 0 and b[-1][1] == L
    for (lo, hi), (lo2, _) in zip(b, b[1:]):
        assert hi == lo2 and lo <= hi and (lo % bs == 0 or lo == hi == L)
    if (L, S) == (131072, 32):
        assert all(hi - lo == 4096 for lo, hi in b)


def test_split_bounds_fixed_chunks_from_the_batch_bound():
    # chunk = 16 * ceil(ceil(4096 / 3) / 16) = 1376 keys: a short sequence sits
    # in the first split; the others are empty
    assert oracle.split_bounds(1000, 3, 16, 4096) == [(0, 1000), (1000, 1000), (1000, 1000)]
    # chunk = 1024; the bound is loose (5000 > 4096): the last split takes the rest
    assert oracle.split_bounds(5000, 4, 16, 4096) == [(0, 1024), (1024, 2048), (2048, 3072),
                                                      (3072, 5000)]
    # every split but the last of a long sequence holds exactly one chunk
    assert oracle.split_bounds(4000, 8, 32, 4096) == [(512 * p, min(512 * (p + 1), 4000))
                                                      for p in range(8)]


@pytest.mark.parametrize("S,mx", [(2, None), (3, None), (32, None), (4, 640), (3, 100)])
def test_split_then_merge_equals_unsplit(S, mx):
    lens = [200, 45, 16, 1]
    P = Paged(lens, 2, 16, 16, seed=16)
    q = torch.randn(4, 8, 16)
    slopes = W.alibi_slopes(8)
    po, pl = oracle.decode_splits(q, P.kc, P.vc, lens, P.table, 0.25, S, 60, 6.0, slopes,
                                  max_seq_len=mx)
    mo, ml = oracle.merge(po, pl)
    o, l = oracle.decode(q, P.kc, P.vc, lens, P.table, 0.25, 60, 6.0, slopes)
    assert torch.allclose(mo, o, atol=1e-12) and torch.allclose(ml, l, atol=1e-12)


def test_merge_identical_states_adds_log2():
    o = torch.randn(1, 5, 3, 8, dtype=torch.float64)
    l = torch.randn(1, 3, 5, dtype=torch.float64)
    mo, ml = oracle.merge(torch.cat([o, o]), torch.cat([l, l]))
    assert torch.allclose(mo, o[0], atol=1e-14)
    assert torch.allclose(ml, l[0] + math.log(2.0), atol=1e-14)


def test_merge_with_empty_part_is_identity_and_all_empty_is_zero():
    o = torch.randn(1, 4, 2, 8, dtype=torch.float64)
    l = torch.randn(1, 2, 4, dtype=torch.float64)
    empty_o = torch.zeros_like(o)
    empty_l = torch.full_like(l, float("-inf"))
    mo, ml = oracle.merge(torch.cat([empty_o, o, empty_o]), torch.cat([empty_l, l, empty_l]))
    assert torch.equal(mo, o[0]) and torch.equal(ml, l[0])
    zo, zl = oracle.merge(torch.cat([empty_o, empty_o]), torch.cat([empty_l, empty_l]))
    assert torch.equal(zo, torch.zeros_like(o[0])) and torch.isneginf(zl).all()


def test_merge_two_parts_matches_softmax_over_union():
    # two disjoint key sets; the merge of their states is attention over both
    g = torch.Generator().manual_seed(17)
    s1, s2 = torch.randn(7, generator=g, dtype=torch.float64), torch.randn(4, generator=g, dtype=torch.float64)
    v1, v2 = torch.randn(7, 3, generator=g, dtype=torch.float64), torch.randn(4, 3, generator=g, dtype=torch.float64)
    o1 = torch.softmax(s1, 0) @ v1
    o2 = torch.softmax(s2, 0) @ v2
    parts_o = torch.stack([o1, o2])[:, None, None, :]
    parts_l = torch.stack([torch.logsumexp(s1, 0), torch.logsumexp(s2, 0)])[:, None, None]
    mo, ml = oracle.merge(parts_o, parts_l)
    s = torch.cat([s1, s2])
    assert torch.allclose(mo[0, 0], torch.softmax(s, 0) @ torch.cat([v1, v2]), atol=1e-14)
    assert abs(float(ml[0, 0]) - float(torch.logsumexp(s, 0))) < 1e-14


def _shared_prefix_case(seed, B, P, q_lens, extra, Hq, Hkv, D, bs):
    """A cache whose sequences share their first P keys (same physical
    blocks), random K/V in every block, and queries after the prefix."""
    g = torch.Generator().manual_seed(seed)
    n = P // bs
    lens = [P + e + ql for e, ql in zip(extra, q_lens)]
    own = [-(-(L - P) // bs) for L in lens]
    nb = n + sum(own) + 2
    perm = torch.randperm(nb, generator=g)
    table = torch.zeros(B, n + max(own), dtype=torch.int32)
    table[:, :n] = perm[:n]
    at = n
    for b in range(B):
        table[b, n:n + own[b]] = perm[at:at + own[b]]
        at += own[b]
    kc = torch.randn(nb, bs, Hkv, D, generator=g)
    vc = torch.randn(nb, bs, Hkv, D, generator=g)
    cu = [0]
    for ql in q_lens:
        cu.append(cu[-1] + ql)
    q = torch.randn(cu[-1], Hq, D, generator=g)
    return q, kc, vc, cu, lens, table


@pytest.mark.parametrize("cap", [0.0, 3.0])
def test_cascade_equals_plain_causal(cap):
    """The cascade decomposition (shared prefix non-causal, suffix causal,
    LSE merge) reproduces plain causal attention."""
    q, kc, vc, cu, lens, table = _shared_prefix_case(9, 5, 48, [1, 7, 3, 16, 2], [0, 5, 17, 40, 1],
                                                     8, 2, 16, 16)
    o, l = oracle.cascade(q, kc, vc, cu, lens, table, 0.3, 48, softcap=cap)
    ro, rl = oracle.attend(q, kc, vc, cu, lens, table, 0.3, True, -1, cap, None)
    assert torch.allclose(o, ro, atol=1e-12, rtol=0) and torch.allclose(l, rl, atol=1e-12, rtol=0)


def test_cascade_matches_brute_force_tiny():
    q, kc, vc, cu, lens, table = _shared_prefix_case(10, 3, 16, [2, 1, 3], [1, 0, 2], 4, 2, 8, 16)
    o, l = oracle.cascade(q, kc, vc, cu, lens, table, 0.5, 16)
    bo, bl = brute_force(q, kc, vc, cu, lens, table, 0.5, True, -1, 0.0, None)
    assert torch.allclose(o, bo, atol=1e-12, rtol=0) and torch.allclose(l, bl, atol=1e-12, rtol=0)


def test_cascade_rejects_unshared_prefix():
    q, kc, vc, cu, lens, table = _shared_prefix_case(11, 2, 32, [1, 1], [0, 0], 4, 2, 8, 16)
    table[1, 0] = table[1, 0] + 100
    with pytest.raises(AssertionError):
        oracle.cascade(q, kc, vc, cu, lens, table, 0.5, 32)


# ----------------------------------------------------------------------------
# chunked local attention (next row): keys of the query's own chunk only
# ----------------------------------------------------------------------------
def test_chunked_attention_with_one_chunk_is_plain_causal():
    P = Paged([30, 7], 2, 16, 16, seed=21)
    q = torch.randn(12, 4, 16)
    cu = [0, 9, 12]
    a = oracle.attend(q, P.kc, P.vc, cu, [30, 7], P.table, 0.3, True, attn_chunk_size=32)
    b = oracle.attend(q, P.kc, P.vc, cu, [30, 7], P.table, 0.3, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_chunked_attention_query_at_chunk_start_sees_itself():
    P = Paged([40], 1, 8, 16, seed=22)
    q = torch.randn(9, 2, 8)                    # positions 31..39
    o, l = oracle.attend(q, P.kc, P.vc, [0, 9], [40], P.table, 0.7, True, attn_chunk_size=8)
    t = 32 - 31                                 # row of position 32, a chunk start
    assert torch.equal(o[t], P.V[0][32, 0].double().expand(2, 8))
    assert torch.allclose(l[:, t], 0.7 * (q[t].double() @ P.K[0][32, 0].double()), atol=1e-14)


def test_chunked_attention_equals_causal_attention_per_chunk():
    """Each chunk of a sequence, taken as its own sequence (its keys from the
    chunk start), gives the same rows as chunked attention over the whole."""
    chunk, L, nq = 16, 53, 30                   # queries at positions 23..52
    P = Paged([L], 2, 8, 16, seed=23)
    q = torch.randn(nq, 4, 8)
    o, l = oracle.attend(q, P.kc, P.vc, [0, nq], [L], P.table, 0.4, True, attn_chunk_size=chunk)
    p0 = L - nq
    for c0 in range(0, L, chunk):
        rows = [t for t in range(nq) if c0 <= p0 + t < c0 + chunk]
        if not rows:
            continue
        Lc = p0 + rows[-1] + 1 - c0             # keys c0 .. the chunk's last query
        table = P.table[:, c0 // 16:]
        oc, lc = oracle.attend(q[rows[0]:rows[-1] + 1], P.kc, P.vc, [0, len(rows)], [Lc], table,
                               0.4, True)
        assert torch.allclose(o[rows[0]:rows[-1] + 1], oc, atol=1e-12, rtol=0)
        assert torch.allclose(l[:, rows[0]:rows[-1] + 1], lc, atol=1e-12, rtol=0)


# ----------------------------------------------------------------------------
# attention sinks (next row): one more logit per head in the denominator
# ----------------------------------------------------------------------------
def test_sinks_of_minus_inf_change_nothing():
    P = Paged([30, 9], 2, 16, 16, seed=31)
    q = torch.randn(12, 4, 16)
    cu, lens = [0, 8, 12], [30, 9]
    a = oracle.attend(q, P.kc, P.vc, cu, lens, P.table, 0.3, True,
                      sinks=torch.full((4,), float("-inf")))
    b = oracle.attend(q, P.kc, P.vc, cu, lens, P.table, 0.3, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_sink_with_one_key_is_a_sigmoid_gate():
    """One visible key with score s and value v: out = v * sigmoid(s - sink),
    lse = ln(e^s + e^sink)."""
    P = Paged([1], 1, 8, 16, seed=32)
    q = torch.randn(1, 2, 8)
    sinks = torch.tensor([0.7, -1.3])
    o, l = oracle.decode(q, P.kc, P.vc, [1], P.table, 0.5, sinks=sinks)
    for h in range(2):
        s = 0.5 * float(q[0, h].double() @ P.K[0][0, 0].double())
        gate = 1.0 / (1.0 + math.exp(float(sinks[h]) - s))
        assert torch.allclose(o[0, h], P.V[0][0, 0].double() * gate, atol=1e-14, rtol=0)
        assert abs(float(l[h, 0]) - math.log(math.exp(s) + math.exp(float(sinks[h])))) < 1e-13


def test_sink_is_an_extra_state_with_zero_output():
    """Merging the sinkless result with a state (out 0, lse = sink) gives the
    result with the sink (the LSE merge the pages use for partial states)."""
    P = Paged([40, 3, 17], 2, 16, 16, seed=33)
    q = torch.randn(3, 4, 16)
    sinks = torch.tensor([0.5, -2.0, 3.0, 0.0])
    o, l = oracle.decode(q, P.kc, P.vc, [40, 3, 17], P.table, 0.25, softcap=2.0, sinks=sinks)
    o0, l0 = oracle.decode(q, P.kc, P.vc, [40, 3, 17], P.table, 0.25, softcap=2.0)
    ls = sinks.double()[:, None].expand(4, 3)
    mo, ml = oracle.merge(torch.stack([o0, torch.zeros_like(o0)]), torch.stack([l0, ls]))
    assert torch.allclose(o, mo, atol=1e-13, rtol=0) and torch.allclose(l, ml, atol=1e-13, rtol=0)


def test_sinks_split_then_merge_and_empty_sequence():
    P = Paged([0, 60, 33], 2, 8, 16, seed=34)
    q = torch.randn(3, 4, 8)
    sinks = torch.tensor([1.0, -0.5, 0.25, 2.0])
    o, l = oracle.decode(q, P.kc, P.vc, [0, 60, 33], P.table, 0.4, sinks=sinks)
    po, pl = oracle.decode_splits(q, P.kc, P.vc, [0, 60, 33], P.table, 0.4, 4, sinks=sinks)
    mo, ml = oracle.merge(po, pl)
    assert torch.allclose(o, mo, atol=1e-13, rtol=0) and torch.allclose(l, ml, atol=1e-13, rtol=0)
    assert torch.equal(o[0], torch.zeros(4, 8, dtype=torch.float64))
    assert torch.equal(l[:, 0], sinks.double())          # no key: the sink alone


def test_cascade_with_sinks_equals_plain_causal_with_sinks():
    """Sinks folded into the prefix part only give the same result as plain
    causal attention with the sinks."""
    q, kc, vc, cu, lens, table = _shared_prefix_case(11, 4, 32, [1, 5, 2, 9], [3, 0, 20, 7],
                                                     8, 2, 16, 16)
    sinks = torch.tensor([0.3, -1.0, 2.5, 0.0, -0.7, 1.1, 4.0, -3.0])
    o, l = oracle.cascade(q, kc, vc, cu, lens, table, 0.3, 32, sinks=sinks)
    ro, rl = oracle.attend(q, kc, vc, cu, lens, table, 0.3, True, sinks=sinks)
    assert torch.allclose(o, ro, atol=1e-12, rtol=0) and torch.allclose(l, rl, atol=1e-12, rtol=0)
