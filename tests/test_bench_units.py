"""The algorithmic work bench.py divides by (CPU only): the prefill FLOP
count and the decode K/V bytes, counted from the oracle's own visibility
mask key by key; the digest guard on committed counter traffic; and the
per-CU folding of the timeline trace tool on synthetic records."""
import importlib.util
import json
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle.paged_attention import _visible

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load(name, path):
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def bench():
    return _load("bench_under_test", os.path.join(ROOT, "bench.py"))


def _pairs_by_mask(w, call):
    """Visible (query, key) pairs of a call, from the oracle's mask."""
    n = 0
    for nq, L in zip(call.query_lens, call.seq_lens):
        nq, L = int(nq), int(L)
        if nq == 0:
            continue
        q_pos = (L - nq) + torch.arange(nq, dtype=torch.long)
        n += int(_visible(q_pos, L, True, w.window_left, None).sum())
    return n


@pytest.mark.parametrize("make", [
    lambda: W.custom("units_causal", 3, [0, 17, 300], [40, 1, 129], 8, 2, 64, 16),
    lambda: W.custom("units_window", 4, [500, 0, 64], [90, 70, 3], 8, 2, 64, 16, window_left=63),
    lambda: W.prefill_batch(),
], ids=["causal", "window", "prefill_batch"])
def test_prefill_flops_counts_every_visible_pair(bench, make):
    w = make()
    call = w.steps[0].calls[0]
    assert bench.prefill_flops(w, call) == 4 * w.head_size * w.num_heads * _pairs_by_mask(w, call)


@pytest.mark.parametrize("make,elem", [
    (lambda: W.decode_batch(), 2),
    (lambda: W.decode_batch(), 1),
    (lambda: W.custom("units_dwin", 5, [0, 9, 2000], [1, 1, 1], 8, 2, 128, 16, kind="decode",
                      window_left=100), 2),
], ids=["decode_batch", "decode_batch_fp8", "window"])
def test_decode_bytes_count_each_visible_key_once(bench, make, elem):
    w = make()
    call = w.steps[0].calls[0]
    keys = 0
    for L in call.seq_lens:
        L = int(L)
        keys += int(_visible(torch.tensor([L - 1]), L, True, w.window_left, None).sum())
    assert bench.decode_bytes(w, call, elem) == keys * w.num_kv_heads * w.head_size * 2 * elem


def test_traffic_is_reported_only_for_the_source_it_was_taken_with(bench, tmp_path, monkeypatch):
    rec = {"k": {"source_digest": "abc", "hbm_bytes_per_launch": 1234}}
    (tmp_path / "traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.traffic_from_profile("k", "abc") == 1234
    assert bench.traffic_from_profile("k", "abd") is None
    assert bench.traffic_from_profile("missing", "abc") is None


def test_timeline_folds_records_per_cu():
    """Two CUs, one workgroup each at a time: phase medians, the share of
    time at each occupancy, and the clock from the two counters.  (Loading
    the tool loads no library: it imports the package only to run.)"""
    tt = _load("trace_timeline_under_test",
               os.path.join(ROOT, "paged_kv_attention_29_amd", "trace_timeline.py"))
    rows = []
    for cu in range(2):
        for k in range(3):  # back to back on the CU: [1000 k, 1000 k + 900)
            r = np.zeros(tt.SLOTS, np.int64)
            t0 = 1000 * k + 1
            r[tt.ENTRY], r[tt.ITEM], r[tt.LOOP0] = t0, t0 + 100, t0 + 300
            r[tt.LOOP1], r[tt.END] = t0 + 800, t0 + 900
            r[tt.WAVE_END:tt.WAVE_END + 4] = t0 + 900
            r[tt.UNITS] = 5
            r[tt.HWID] = cu << 8
            r[tt.REAL_ENTRY], r[tt.REAL_END] = 10 * k + 1, 10 * k + 10  # 900 ticks in 90 ns
            rows.append(r)
    w = W.custom("units_tl", 1, [10], [1], 8, 2, 64, 16, kind="decode")
    text = tt.summarise("decode", w, (1.0, 1.0), np.stack(rows))
    assert "| entry -> item known | 100 | 100 |" in text
    assert "| key loop | 500 | 500 |" in text
    assert "| key loop per tile / step | 100 | 100 |" in text
    assert "| a workgroup's end -> the next start on its CU | 100 | 100 |" in text
    assert "median 10.00 GHz" in text
    # each CU holds one workgroup except in the two 100-cycle gaps of its
    # 2 900-cycle span
    share = text.split("more workgroups: ")[1].split()
    assert abs(float(share[0]) - 200 / 2900) < 0.01 and abs(float(share[2]) - 2700 / 2900) < 0.01
    assert float(share[4]) == 0.0
