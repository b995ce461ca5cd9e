"""GPU parity of attention sinks (one fp32 logit per query head that joins
the softmax denominator without a value) in paged_attn_prefill,
paged_attn_decode (unsplit, and split then merged: the sink joins split 0
only) and paged_attn_cascade (the prefix part only), against the oracle in
float64: outputs to max-abs 2e-2 / mean-abs 2e-3, LSE to 1e-2.  The sinks
mix small, dominant (+8) and absent (-inf) values; sequences of length 0
must give out = 0 and lse = the sink."""
import pytest
import torch

import oracle
from oracle_side import assert_attn_close, assert_lse_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_attention_29_amd as pa
    return pa


def _sinks(Hq, seed):
    g = torch.Generator().manual_seed(1000 + seed)
    s = torch.randn(Hq, generator=g) * 2.0
    s[0] = float("-inf")
    if Hq > 2:
        s[Hq // 2] = 8.0
    return s


def _cache(seed, lens, Hkv, D, bs, dtype, spare_cols=2):
    """Random K/V, a random block table (spare columns and blocks hold NaN,
    never read)."""
    g = torch.Generator().manual_seed(seed)
    need = [-(-L // bs) for L in lens]
    nb = sum(need) + 3
    perm = torch.randperm(nb, generator=g)
    table = torch.zeros(len(lens), max(need + [1]) + spare_cols, dtype=torch.int32)
    table[:] = int(perm[-1])
    at = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[at:at + n]
        at += n
    kc = torch.randn(nb, bs, Hkv, D, generator=g).to(dtype)
    vc = torch.randn(nb, bs, Hkv, D, generator=g).to(dtype)
    for spare in perm[at:].tolist():
        kc[spare] = float("nan")
        vc[spare] = float("nan")
    return kc, vc, table


PREFILL = [
    # name, ctx, q, Hq, Hkv, D, bs, dtype, window_left, softcap, alibi
    ("g4_d128", [0, 300, 7], [200, 65, 1], 8, 2, 128, 16, torch.bfloat16, -1, 0.0, False),
    ("g2_d64_cap_window", [40, 0], [100, 33], 4, 2, 64, 32, torch.float16, 31, 4.0, False),
    ("g1_d256_alibi", [10], [90], 2, 2, 256, 16, torch.bfloat16, -1, 0.0, True),
]


@pytest.mark.parametrize("case", PREFILL, ids=[c[0] for c in PREFILL])
def test_prefill_sinks(pa, case):
    name, ctx, ql, Hq, Hkv, D, bs, dtype, wl, cap, alibi = case
    print(f"\n[gpu-case] prefill sinks {name}", flush=True)
    seed = len(name)
    lens = [c + q for c, q in zip(ctx, ql)]
    kc, vc, table = _cache(seed, lens, Hkv, D, bs, dtype)
    cu = [0]
    for q in ql:
        cu.append(cu[-1] + q)
    g = torch.Generator().manual_seed(seed + 1)
    q = (torch.randn(cu[-1], Hq, D, generator=g) * 0.5).to(dtype)
    slopes = torch.rand(Hq, generator=g) * 0.1 if alibi else None
    sinks = _sinks(Hq, seed)
    scale = D ** -0.5
    out = torch.full((cu[-1], Hq, D), float("nan"), dtype=dtype, device="cuda")
    lse = torch.full((Hq, cu[-1]), float("nan"), device="cuda")
    pa.paged_attn_prefill(out, q.cuda(), kc.cuda(), vc.cuda(),
                          torch.tensor(cu, dtype=torch.int32, device="cuda"),
                          torch.tensor(lens, dtype=torch.int32, device="cuda"), table.cuda(),
                          max(ql), max(lens), scale, True, wl, cap,
                          None if slopes is None else slopes.cuda(), lse=lse,
                          sinks=sinks.cuda())
    torch.cuda.synchronize()
    ro, rl = oracle.attend(q, kc, vc, cu, lens, table, scale, True, wl, cap, slopes, sinks=sinks)
    assert_attn_close(out, ro, name)
    assert_lse_close(lse, rl, f"{name} lse")


DECODE = [
    # name, lens, Hq, Hkv, D, bs, dtype, window_left, softcap, splits
    ("g4_d128_s1", [0, 1, 17, 300, 1024], 32, 8, 128, 16, torch.bfloat16, -1, 0.0, 1),
    ("g4_d128_s4", [0, 1, 17, 300, 1024], 32, 8, 128, 16, torch.bfloat16, -1, 0.0, 4),
    ("g8_d64_window_s3", [5, 700, 64], 16, 2, 64, 32, torch.float16, 40, 3.0, 3),
    ("g1_d256_s2", [0, 33, 260], 4, 4, 256, 16, torch.bfloat16, -1, 0.0, 2),
    ("g24_d128_s3", [0, 40, 900], 48, 2, 128, 16, torch.bfloat16, -1, 0.0, 3),
]


@pytest.mark.parametrize("case", DECODE, ids=[c[0] for c in DECODE])
def test_decode_sinks(pa, case):
    name, lens, Hq, Hkv, D, bs, dtype, wl, cap, S = case
    print(f"\n[gpu-case] decode sinks {name}", flush=True)
    seed = len(name) + 50
    kc, vc, table = _cache(seed, lens, Hkv, D, bs, dtype)
    g = torch.Generator().manual_seed(seed + 1)
    B = len(lens)
    q = (torch.randn(B, Hq, D, generator=g) * 0.5).to(dtype)
    sinks = _sinks(Hq, seed)
    scale = D ** -0.5
    qd, kcd, vcd, td = q.cuda(), kc.cuda(), vc.cuda(), table.cuda()
    lensd = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = torch.full((B, Hq, D), float("nan"), dtype=dtype, device="cuda")
    lse = torch.full((Hq, B), float("nan"), device="cuda")
    if S == 1:
        pa.paged_attn_decode(out, qd, kcd, vcd, lensd, td, max(lens), scale, wl, cap,
                             lse=lse, sinks=sinks.cuda())
    else:
        po = torch.full((S, B, Hq, D), float("nan"), device="cuda")
        pl = torch.full((S, Hq, B), float("nan"), device="cuda")
        pa.paged_attn_decode(None, qd, kcd, vcd, lensd, td, max(lens), scale, wl, cap,
                             num_splits=S, part_out=po, part_lse=pl, sinks=sinks.cuda())
        pa.merge_attn_states(out, po, pl, out_lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(q, kc, vc, lens, table, scale, wl, cap, sinks=sinks)
    if S > 1:
        rpo, rpl = oracle.decode_splits(q, kc, vc, lens, table, scale, S, wl, cap, sinks=sinks)
        assert_attn_close(po, rpo, f"{name} parts")
        assert_lse_close(pl, rpl, f"{name} part lse")
    assert_attn_close(out, ro, name)
    assert_lse_close(lse, rl, f"{name} lse")
    for b, L in enumerate(lens):
        if L == 0:   # no key: the sink alone
            assert torch.equal(out[b].float().cpu(), torch.zeros(Hq, D))
            assert_lse_close(lse[:, b], sinks.double(), f"{name} empty sequence lse")


def _shared_prefix(seed, prefix, q_lens, extra, Hq, Hkv, D, bs, dtype):
    g = torch.Generator().manual_seed(seed)
    B, n = len(q_lens), prefix // bs
    lens = [prefix + e + ql for e, ql in zip(extra, q_lens)]
    own = [-(-(L - prefix) // bs) for L in lens]
    nb = n + sum(own) + 1
    perm = torch.randperm(nb, generator=g)
    table = torch.zeros(B, n + max(own), dtype=torch.int32)
    table[:, :n] = perm[:n]
    at = n
    for b in range(B):
        table[b, n:n + own[b]] = perm[at:at + own[b]]
        at += own[b]
    kc = torch.randn(nb, bs, Hkv, D, generator=g).to(dtype)
    vc = torch.randn(nb, bs, Hkv, D, generator=g).to(dtype)
    cu = [0]
    for ql in q_lens:
        cu.append(cu[-1] + ql)
    q = (torch.randn(cu[-1], Hq, D, generator=g) * 0.5).to(dtype)
    return q, kc, vc, cu, lens, table


CASCADE = [
    # name, prefix, q_lens, extra, Hq, Hkv, D, bs, dtype
    ("prefill_g4", 128, [1, 37, 70], [0, 20, 100], 16, 4, 128, 16, torch.bfloat16),
    ("decode_q1_splits", 1024, [1] * 24, list(range(3, 24 * 9, 9)), 32, 8, 128, 16,
     torch.bfloat16),
]


@pytest.mark.parametrize("case", CASCADE, ids=[c[0] for c in CASCADE])
def test_cascade_sinks(pa, case):
    name, prefix, ql, extra, Hq, Hkv, D, bs, dtype = case
    print(f"\n[gpu-case] cascade sinks {name}", flush=True)
    q, kc, vc, cu, lens, table = _shared_prefix(len(name) + 7, prefix, ql, extra, Hq, Hkv, D, bs,
                                                dtype)
    sinks = _sinks(Hq, len(name))
    scale = D ** -0.5
    T = cu[-1]
    out = torch.full((T, Hq, D), float("nan"), dtype=dtype, device="cuda")
    lse = torch.full((Hq, T), float("nan"), device="cuda")
    pa.paged_attn_cascade(out, q.cuda(), kc.cuda(), vc.cuda(),
                          torch.tensor(cu, dtype=torch.int32, device="cuda"),
                          torch.tensor(lens, dtype=torch.int32, device="cuda"), table.cuda(),
                          max(ql), max(lens), scale, prefix, lse=lse, sinks=sinks.cuda())
    torch.cuda.synchronize()
    ro, rl = oracle.cascade(q, kc, vc, cu, lens, table, scale, prefix, sinks=sinks)
    assert_attn_close(out, ro, name)
    assert_lse_close(lse, rl, f"{name} lse")
