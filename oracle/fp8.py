"""FP8 (e4m3) KV cache: the code table, quantisation and dequantisation.

TEST INFRASTRUCTURE ONLY (part of the oracle package).

The pages store the cache as float8_e4m3fn when kv_cache_dtype is "fp8" or
"fp8_e4m3" and pass one fp32 scale per tensor: reshape_and_cache_flash gets
``layer._k_scale`` / ``layer._v_scale`` with the kv_cache_dtype, and the
attention call gets the same scales as k_descale / v_descale  [vLLM
flash_attn.py (e2f56c3), FlashAttentionBackend.get_fp8_dtype_for_flashattn;
FlashAttentionImpl.forward, the reshape_and_cache_flash call and the
descale arguments].  The arithmetic is not printed.  Readings used here:

* the format is OCP e4m3 "fn": sign, 4 exponent bits (bias 7), 3 mantissa
  bits, subnormals, no infinities, S.1111.111 is NaN; the largest finite
  magnitude is 448;
* a stored code is the element x divided by the scale in fp32 (correctly
  rounded), then rounded to the nearest code, ties to the even code (the
  one whose mantissa ends in 0), saturating at +-448 (so +-inf gives
  +-448); the sign of the element is kept (so -0 and small negatives that
  round to zero give the code 0x80); NaN gives 0x7F with the element's sign;
* the dequantised element is value(code) * scale (a descale multiplies).

The query: with an fp8 cache the page quantises the query too, per tensor
with the static scale ``layer._q_scale`` (``ops.scaled_fp8_quant(query,
layer._q_scale)``), and passes that scale to the attention call as
``q_descale`` beside k_descale / v_descale  [vLLM flash_attn.py (v0.9.0.1
docs), FlashAttentionImpl.forward, the fp8 branch; vLLM flash_attn.py
(e2f56c3), "queries are quantized in the attention layer" and the
q_descale argument].  Reading used here: the query codes are made exactly
as the cache codes are (``e4m3_quantize(q, q_scale)``), and the attention
reads value(code) * q_scale, so attention with an fp8 query is attention
over the dequantised query (``scaled_fp8_quant`` / ``dequantize_query``).
Keeping the query in 16 bits (another backend's option) is plain attention
with the unquantised query.
"""
from __future__ import annotations

import torch

_F64 = torch.float64
E4M3_MAX = 448.0


def e4m3_values() -> torch.Tensor:
    """Value of every code 0..255 (float64; NaN for 0x7F and 0xFF), from the
    bit fields: exponent field 0 is subnormal, m/8 * 2^-6; otherwise
    (1 + m/8) * 2^(e - 7)."""
    vals = torch.empty(256, dtype=_F64)
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            v = float("nan")
        elif e == 0:
            v = (m / 8.0) * 2.0 ** -6
        else:
            v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        vals[code] = -v if s else v
    return vals


def e4m3_quantize(x: torch.Tensor, scale: float) -> torch.Tensor:
    """uint8 codes of x / scale (see the module readings).  x is any float
    tensor; the division is done in fp32."""
    t = x.to(torch.float32) / torch.tensor(scale, dtype=torch.float32)
    pos = e4m3_values()[:127]                     # codes 0x00..0x7E, increasing values
    a = t.abs().to(_F64).clamp(max=E4M3_MAX)       # saturate (inf -> 448)
    hi = torch.searchsorted(pos, a.flatten()).clamp(max=126).reshape(a.shape)
    lo = (hi - 1).clamp(min=0)
    d_hi = (pos[hi] - a).abs()
    d_lo = (a - pos[lo]).abs()
    # nearest; on a tie the even code
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = torch.where(pick_lo, lo, hi)
    code = torch.where(torch.isnan(t), torch.full_like(code, 0x7F), code)
    sign = torch.signbit(t).to(torch.long) << 7
    return (code | sign).to(torch.uint8)


def e4m3_dequantize(codes: torch.Tensor, scale: float) -> torch.Tensor:
    """value(code) * scale in float64."""
    return e4m3_values()[codes.to(torch.long)] * float(scale)


def scatter_fp8(key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor,
                key_cache: torch.Tensor, value_cache: torch.Tensor, k_scale: float,
                v_scale: float) -> None:
    """reshape_and_cache into an fp8 cache (uint8 codes): each token row is
    quantised with its tensor's scale, then written to its slot as in
    ``scatter`` (negative slots skipped)."""
    bs = key_cache.shape[1]
    for i, s in enumerate(slot_mapping.tolist()):
        if s < 0:
            continue
        blk, off = divmod(int(s), bs)
        key_cache[blk, off] = e4m3_quantize(key[i], k_scale)
        value_cache[blk, off] = e4m3_quantize(value[i], v_scale)


def scaled_fp8_quant(x: torch.Tensor, scale: float) -> torch.Tensor:
    """The query quantiser with a static per-tensor scale: uint8 e4m3 codes
    of x / scale, the same arithmetic as the cache codes (see the module
    readings)  [vLLM flash_attn.py (v0.9.0.1 docs), FlashAttentionImpl
    .forward, ops.scaled_fp8_quant(query, layer._q_scale)]."""
    return e4m3_quantize(x, scale)


def dequantize_query(codes: torch.Tensor, q_scale: float) -> torch.Tensor:
    """What the attention reads from an fp8 query: value(code) * q_scale
    (q_descale), float64, for ``attend`` / ``decode``."""
    return e4m3_dequantize(codes, q_scale)
