"""K/V caches at device addresses whose low 32 bits have bit 31 set.

The prefill kernel's K/V DMA takes the cache base as a scalar 64-bit
address; a base rebuilt from 32-bit halves must not sign-extend the low half
into the high one (such an address faults).  Ordinary allocations may or may
not land on such addresses, so these cases place both caches there on
purpose: the caches are views into one 4 GiB + buffer at offsets where the
low word of the address is 0x80000000 (K) and 0xC0000000 (V).  Results are
compared with the oracle as in the other parity tests."""
import pytest
import torch

import workloads as W
from oracle_side import assert_attn_close, assert_lse_close, oracle_cache, oracle_call

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def runner():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_attention_29_amd import runner
    return runner


def _place_high(cache):
    """Move the cache's K and V into views at addresses with low word
    0x80000000 and 0xC0000000 (contents copied)."""
    kc, vc = cache.key_cache, cache.value_cache
    nbytes = kc.numel() * kc.element_size()
    assert nbytes <= 1 << 30
    buf = torch.empty((1 << 32) + 2 * nbytes + 4096, dtype=torch.uint8, device=kc.device)
    lo = buf.data_ptr() & 0xFFFFFFFF
    views = []
    for want, src in ((0x80000000, kc), (0xC0000000, vc)):
        off = (want - lo) % (1 << 32)
        view = buf[off:off + nbytes].view(src.dtype).view(src.shape)
        assert view.data_ptr() & 0xFFFFFFFF == want
        view.copy_(src)
        views.append(view)
    cache.key_cache, cache.value_cache = views
    cache._high_buffer = buf  # keeps the views' storage alive with the cache
    return cache


def _run(runner, w):
    cache = _place_high(runner.PagedCache(w))
    cache.fill_context()
    step = w.steps[0]
    k, v, s = cache.step_inputs(step)
    cache.write(k, v, s)
    bufs = [cache.call_buffers(c) for c in step.calls]
    for cb in bufs:
        cache.run(cb)
    torch.cuda.synchronize()
    assert cache.key_cache.data_ptr() & 0xFFFFFFFF == 0x80000000
    return bufs


@pytest.mark.parametrize("D", [64, 128, 256])
def test_prefill_high_address_cache(runner, D):
    _announce(f"prefill, caches at high-bit addresses, D={D}")
    w = W.custom(f"high_addr_prefill_d{D}", 31, [40, 0, 300], [70, 130, 1], 8, 2, D, 16,
                 torch.bfloat16, "prefill", window_left=100)
    (cb,) = _run(runner, w)
    kc, vc = oracle_cache(w, 0)
    ref = oracle_call(w, kc, vc, w.steps[0].calls[0])
    assert_attn_close(cb.out, ref[0], f"high-address prefill D={D}")
    assert_lse_close(cb.lse, ref[1], f"high-address prefill D={D} lse")


def test_decode_high_address_cache(runner):
    _announce("decode, caches at high-bit addresses")
    w = W.custom("high_addr_decode", 32, [500, 37, 2000], [1, 1, 1], 16, 2, 128, 16,
                 torch.bfloat16, "decode", num_splits=4)
    (cb,) = _run(runner, w)
    kc, vc = oracle_cache(w, 0)
    ref = oracle_call(w, kc, vc, w.steps[0].calls[0])
    assert_attn_close(cb.out, ref[0], "high-address decode")
    assert_lse_close(cb.lse, ref[1], "high-address decode lse")
