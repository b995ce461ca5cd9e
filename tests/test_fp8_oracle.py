"""Pins of the oracle's fp8 (e4m3) cache arithmetic against torch's own
float8_e4m3fn type (a library routine written independently of the code
table here), closed-form code values and the rounding error bound."""
import math

import torch

from oracle.fp8 import E4M3_MAX, e4m3_dequantize, e4m3_quantize, e4m3_values, scatter_fp8


def test_code_table_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64)
    mine = e4m3_values()
    nan = torch.isnan(ref)
    assert torch.equal(nan, torch.isnan(mine)) and nan.sum() == 2
    assert torch.equal(mine[~nan], ref[~nan])


def test_closed_form_codes():
    v = e4m3_values()
    assert v[0x01] == 2.0 ** -9          # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert v[0x08] == 2.0 ** -6          # smallest normal
    assert v[0x38] == 1.0 and v[0xB8] == -1.0
    assert v[0x7E] == E4M3_MAX == 448.0
    assert v[0x80] == 0.0 and math.copysign(1.0, float(v[0x80])) < 0
    assert all(v[c] < v[c + 1] for c in range(126))   # codes 0..126 increase


def _torch_quantize(x, scale):
    t = x.to(torch.float32) / torch.tensor(scale, dtype=torch.float32)
    return t.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)


def test_quantize_matches_torch_on_random_ties_and_saturation():
    g = torch.Generator().manual_seed(5)
    mag = torch.exp2(torch.rand(20000, generator=g, dtype=torch.float64) * 24 - 14)
    sgn = torch.where(torch.rand(20000, generator=g) < 0.5, -1.0, 1.0).double()
    x = (mag * sgn).float()
    v = e4m3_values()[:127]
    mids = ((v[1:] + v[:-1]) / 2).float()              # every tie (exact in fp32)
    edge = torch.tensor([0.0, -0.0, 448.0, 449.0, 464.0, 465.0, 1e6, -1e6, 2.0 ** -10,
                         -2.0 ** -10, 2.0 ** -11, float("inf"), float("-inf")])
    for xs in (x, mids, -mids, v.float(), edge):
        assert torch.equal(e4m3_quantize(xs, 1.0), _torch_quantize(xs, 1.0))
    for s in (0.0173, 3.5, 2.0 ** -5):
        assert torch.equal(e4m3_quantize(x, s), _torch_quantize(x, s))


def test_ties_go_to_the_even_code_and_nan_keeps_its_sign():
    v = e4m3_values()
    for c in range(0, 126):
        mid = torch.tensor([(float(v[c]) + float(v[c + 1])) / 2])
        got = int(e4m3_quantize(mid, 1.0)[0])
        assert got == (c if c % 2 == 0 else c + 1)
    q = e4m3_quantize(torch.tensor([float("nan"), -float("nan")]), 1.0)
    assert int(q[0]) & 0x7F == 0x7F


def test_round_trip_and_error_bound():
    v = e4m3_values()
    finite = torch.tensor([c for c in range(256) if not math.isnan(float(v[c]))])
    assert torch.equal(e4m3_quantize(v[finite].float(), 1.0).long(), finite)
    g = torch.Generator().manual_seed(6)
    x = torch.randn(50000, generator=g, dtype=torch.float64).float() * 100
    s = 0.37
    back = e4m3_dequantize(e4m3_quantize(x, s), s)
    t = x.double() / s
    inside = t.abs() <= E4M3_MAX
    # half a unit in the last place: 2^(e-4) for normals, 2^-10 for subnormals
    e = torch.floor(torch.log2(t.abs().clamp(min=2.0 ** -6)))
    bound = torch.exp2(e - 4) * s
    assert ((back - x.double()).abs()[inside] <= bound[inside] * (1 + 1e-6)).all()
    assert torch.equal(back[~inside].abs(), torch.full_like(back[~inside], 448.0 * s))


def test_scatter_fp8_writes_codes_and_skips_padding():
    g = torch.Generator().manual_seed(7)
    key = torch.randn(5, 2, 8, generator=g).bfloat16()
    val = torch.randn(5, 2, 8, generator=g).bfloat16()
    kc = torch.zeros(3, 4, 2, 8, dtype=torch.uint8)
    vc = torch.zeros_like(kc)
    slots = torch.tensor([5, -1, 0, 11, 6])
    scatter_fp8(key, val, slots, kc, vc, 0.25, 0.5)
    assert torch.equal(kc[1, 1], e4m3_quantize(key[0], 0.25))
    assert torch.equal(vc[2, 3], e4m3_quantize(val[3], 0.5))
    assert torch.equal(kc[0, 1], torch.zeros(2, 8, dtype=torch.uint8))   # slot of the padding row untouched


# ----------------------------------------------------------------------------
# the quantised query (an fp8 query with q_descale)
# ----------------------------------------------------------------------------
def test_query_quantiser_matches_torch_float8():
    from oracle.fp8 import scaled_fp8_quant
    g = torch.Generator().manual_seed(11)
    q = (torch.randn(7, 4, 64, generator=g) * 3).to(torch.bfloat16)
    for scale in (0.0125, 0.02, 1.0 / 64):
        assert torch.equal(scaled_fp8_quant(q, scale), _torch_quantize(q, scale))


def test_lossless_query_codes_give_the_16bit_attention():
    """A query whose elements are e4m3 values times a power-of-two scale
    quantises without loss, so attention through the fp8-query path equals
    attention with the 16-bit query exactly."""
    import oracle
    from oracle.fp8 import dequantize_query, scaled_fp8_quant
    g = torch.Generator().manual_seed(12)
    q_scale = 2.0 ** -5
    codes = torch.randint(0, 126, (3, 4, 64), generator=g, dtype=torch.uint8)
    codes |= (torch.rand(3, 4, 64, generator=g) < 0.5).to(torch.uint8) << 7
    q16 = (e4m3_values()[codes.long()] * q_scale).to(torch.bfloat16)
    assert torch.equal(q16.double(), e4m3_values()[codes.long()] * q_scale)   # exact in bf16
    assert torch.equal(scaled_fp8_quant(q16, q_scale) & 0x7F, codes & 0x7F)
    kc = torch.randn(4, 16, 2, 64, generator=g).to(torch.bfloat16)
    vc = torch.randn(4, 16, 2, 64, generator=g).to(torch.bfloat16)
    bt = torch.tensor([[0, 1], [2, 3]], dtype=torch.int32)
    args = (kc, vc, [0, 1, 3], [20, 31], bt, 0.125)
    qd = dequantize_query(scaled_fp8_quant(q16, q_scale), q_scale)
    o8, l8 = oracle.attend(qd, *args)
    o16, l16 = oracle.attend(q16, *args)
    assert torch.equal(o8, o16) and torch.equal(l8, l16)


def test_fp8_query_attention_by_brute_force():
    """Tiny fp8 case (fp8 query, fp8 cache) against a pure-Python loop that
    quantises through torch's float8_e4m3fn type and multiplies the
    descales in, one score at a time."""
    import oracle
    from oracle.fp8 import dequantize_query, scaled_fp8_quant
    g = torch.Generator().manual_seed(13)
    Hq, Hkv, D, bs, L = 4, 2, 8, 16, 21
    q_scale, k_scale, v_scale, scale = 0.011, 0.023, 0.017, D ** -0.5
    q = torch.randn(1, Hq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(L, Hkv, D, generator=g).to(torch.bfloat16)
    v = torch.randn(L, Hkv, D, generator=g).to(torch.bfloat16)
    kc = torch.zeros(2, bs, Hkv, D, dtype=torch.uint8)
    vc = torch.zeros(2, bs, Hkv, D, dtype=torch.uint8)
    scatter_fp8(k, v, torch.arange(L), kc, vc, k_scale, v_scale)
    bt = torch.tensor([[0, 1]], dtype=torch.int32)
    qd = dequantize_query(scaled_fp8_quant(q, q_scale), q_scale)
    out, lse = oracle.decode(qd, e4m3_dequantize(kc, k_scale), e4m3_dequantize(vc, v_scale),
                             [L], bt, scale)
    f8 = lambda x, s: float(_torch_quantize(x, s).view(torch.float8_e4m3fn).double())
    for h in range(Hq):
        gk = h // (Hq // Hkv)
        s = []
        for j in range(L):
            acc = 0.0
            for d in range(D):
                acc += f8(q[0, h, d], q_scale) * f8(k[j, gk, d], k_scale)
            s.append(scale * q_scale * k_scale * acc)
        m = max(s)
        w = [math.exp(x - m) for x in s]
        den = sum(w)
        for d in range(D):
            ref = v_scale * sum(w[j] * f8(v[j, gk, d], v_scale) for j in range(L)) / den
            assert abs(out[0, h, d].item() - ref) < 1e-12
        assert abs(lse[h, 0].item() - (m + math.log(den))) < 1e-12
