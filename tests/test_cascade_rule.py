"""pa_use_cascade (host only, no GPU): the page's support checks and
thresholds one by one [vLLM flash_attn.py (e2f56c3), use_cascade_attention],
and the MI355X time model against the measured crossover of cascade vs
split decode committed under profiles/."""
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILE = os.path.join(ROOT, "profiles", "cascade_crossover_decode_batches.md")


@pytest.fixture(scope="module")
def pa():
    import paged_kv_attention_29_amd as pa
    return pa


def _decode_batch(B, P, suffix=100):
    return np.ones(B, np.int32), np.full(B, P + suffix, np.int32)


def _use(pa, P, ql, sl, **kw):
    args = dict(num_heads=32, num_kv_heads=8, head_size=128)
    args.update(kw)
    return pa.use_cascade(P, ql, sl, **args)


def test_prefix_threshold_256(pa):
    ql, sl = _decode_batch(128, 255)
    assert not _use(pa, 255, ql, sl)
    ql, sl = _decode_batch(128, 256, suffix=1)
    assert _use(pa, 256, ql, sl)          # 128 requests re-reading 256 keys: cascade


def test_alibi_window_local_attention_disable(pa):
    ql, sl = _decode_batch(128, 8192)
    assert _use(pa, 8192, ql, sl)
    for kw in (dict(use_alibi=True), dict(use_sliding_window=True), dict(use_local_attention=True)):
        assert not _use(pa, 8192, ql, sl, **kw), kw


def test_request_threshold_8(pa):
    ql, sl = _decode_batch(7, 8192, suffix=1)
    assert not _use(pa, 8192, ql, sl)
    ql, sl = np.full(8, 4, np.int32), np.full(8, 8196, np.int32)
    assert _use(pa, 8192, ql, sl)        # 8 requests, not a decode batch: cascade


def test_dcp_disables(pa):
    ql, sl = _decode_batch(128, 8192)
    assert not _use(pa, 8192, ql, sl, dcp_world_size=2)


def test_non_decode_batches_take_the_cascade(pa):
    """As on the page: without split-KV decode (a request with several
    queries, or one query head per KV head) the cascade is chosen; so is a
    small decode batch, where it was measured faster too."""
    ql = np.ones(8, np.int32)
    sl = np.full(8, 300, np.int32)
    assert _use(pa, 256, ql, sl)
    ql2 = ql.copy()
    ql2[3] = 2
    assert _use(pa, 256, ql2, sl)
    assert _use(pa, 256, ql, sl, num_heads=8, num_kv_heads=8)


def test_fp8_cache_counts_half_the_bytes(pa):
    """With fp8 codes the K/V bytes halve while the prefix pass's MFMA work
    stays: near the crossover the fp8 decision can only lean to split
    decode."""
    for B in (16, 24, 32, 48):
        for P in (512, 1024, 2048):
            ql, sl = _decode_batch(B, P, 200)
            if _use(pa, P, ql, sl, kv_elem_bytes=1):
                assert _use(pa, P, ql, sl, kv_elem_bytes=2), (B, P)


def test_invalid_arguments(pa):
    with pytest.raises(pa.PagedAttnError):
        _use(pa, 256, np.ones(8, np.int32), np.ones(8, np.int32), num_kv_heads=3)
    with pytest.raises(pa.PagedAttnError):
        _use(pa, 256, np.ones(8, np.int32), np.ones(8, np.int32), kv_elem_bytes=4)


def test_measured_crossover(pa):
    """On the measured decode batches (32/8/128 bf16, requests 8..128,
    prefixes 256..8192, suffix ranges 1-64 and 64-1024) the rule picks the
    path that was faster, up to a few near-ties: the time lost by its
    choice averages under 2% and is at most 25% at any point."""
    rows = []
    for line in open(PROFILE):
        m = re.match(r"\| (\d+) \| (\d+) \| (\d+)-(\d+) \| (\d+) \| (\d+) \| ([\d.]+) \| ([\d.]+) \|", line)
        if m:
            rows.append(tuple(float(x) for x in m.groups()))
    assert len(rows) == 60
    lost, agree = [], 0
    for B, P, lo, hi, ssum, smax, t_cas, t_plain in rows:
        B, P = int(B), int(P)
        rng = np.random.Generator(np.random.PCG64(6))
        suf = rng.integers(int(lo), int(hi), size=B, endpoint=True)
        assert suf.sum() == ssum and suf.max() == smax
        pick = _use(pa, P, np.ones(B, np.int32), (P + suf).astype(np.int32))
        agree += pick == (t_cas < t_plain)
        lost.append((t_cas if pick else t_plain) / min(t_cas, t_plain) - 1)
    assert agree >= 55
    assert np.mean(lost) < 0.02 and max(lost) < 0.25
