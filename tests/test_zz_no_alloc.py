"""paged_attn_decode_noalloc (the entry point for callers that cannot
allocate: its split partials live in the library's fixed device scratch)
against the existing path, paged_attn_decode with caller workspace followed
by merge_attn_states, through the C ABI: two calls in a row on the same
GPU, the second with a smaller batch, each compared element by element
(the two paths run the same kernels, so the results must be identical) and
against the oracle at the attention tolerance."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle_side import assert_attn_close, assert_lse_close, oracle_cache, oracle_call

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_attention_29_amd as pa
    return pa


def _existing_and_noalloc(pa, runner, w, S):
    cache, res = runner.run_workload(w, num_splits=S)
    call, cb = w.steps[0].calls[0], res[0][0]
    out = torch.full_like(cb.out, float("nan"))
    lse = torch.full_like(cb.lse, float("nan"))
    rc = pa.lib.paged_attn_decode_noalloc(
        out.data_ptr(), lse.data_ptr(), cb.q.data_ptr(), cache.key_cache.data_ptr(),
        cache.value_cache.data_ptr(), cb.seq_lens.data_ptr(), cb.block_table.data_ptr(),
        cb.block_table.stride(0), call.num_seqs, cb.max_seqlen_k, w.num_heads, w.num_kv_heads,
        w.head_size, w.block_size, w.num_blocks, w.scale, w.window_left, w.softcap,
        None if cache.alibi is None else cache.alibi.data_ptr(), None, S,
        pa.PA_BF16 if w.dtype == torch.bfloat16 else pa.PA_F16,
        pa.PA_BF16 if w.dtype == torch.bfloat16 else pa.PA_F16, None, None, None,
        torch.cuda.current_stream().cuda_stream)
    assert rc == 0, pa.pa_last_error()
    torch.cuda.synchronize()
    return cb, out, lse


def test_noalloc_decode_two_calls_second_smaller(pa):
    from paged_kv_attention_29_amd import runner
    cases = [
        (W.decode_batch(num_splits=8), 8),
        (W.custom("noalloc_small", 31, [700, 33, 1500], [1, 1, 1], 16, 2, 128, 16,
                  torch.bfloat16, "decode", window_left=511, softcap=30.0, alibi=True), 5),
    ]
    for w, S in cases:
        print(f"\n[gpu-case] noalloc decode {w.name} splits={S}", flush=True)
        cb, out, lse = _existing_and_noalloc(pa, runner, w, S)
        assert torch.equal(out.view(torch.int16), cb.out.view(torch.int16)), w.name
        assert torch.equal(lse, cb.lse), w.name
        kc, vc = oracle_cache(w, 0)
        ref = oracle_call(w, kc, vc, w.steps[0].calls[0], S)
        assert_attn_close(out, ref[0], f"noalloc {w.name}")
        assert_lse_close(lse, ref[1], f"noalloc {w.name} lse")


def test_noalloc_rejects_what_does_not_fit(pa):
    q = torch.zeros(2048, 64, 256, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(16, 16, 8, 256, dtype=torch.bfloat16, device="cuda")
    lens = torch.ones(2048, dtype=torch.int32, device="cuda")
    bt = torch.zeros(2048, 1, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(pa.PagedAttnError, match="scratch"):
        pa.paged_attn_decode_noalloc(out, q, kc, kc, lens, bt, 16, 0.0625, num_splits=64)
