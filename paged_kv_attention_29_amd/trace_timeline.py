"""Per-workgroup timeline of one prefill or decode launch, from the trace
build of the library (python paged_kv_attention_29_amd/build.py --trace).

    python paged_kv_attention_29_amd/trace_timeline.py --workload decode
    python paged_kv_attention_29_amd/trace_timeline.py --workload prefill

(run as a script: PA_TRACE=1 must be set before the package loads its
library, which `python -m` would do first; run() sets it)

Runs the workload's call a few times, then once with pa_trace_set on (after
reading a 512 MiB buffer, so the caches start cold as in bench.py), and
prints a markdown summary: the per-workgroup phases (lookup, first K/V data,
key loop, epilogue), how many workgroups each CU held over the launch, and
the ramp and tail of the launch per CU.  Times are shader-clock cycles
(s_memtime); the clock is not shared by all shader engines, so every
quantity is taken within one CU and then summarised over the CUs.
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

SLOTS = 16
ENTRY, ITEM, LOOP0, LOOP1, END, HWID, XCC, UNITS, WHO, WAVE_END = range(10)
REAL_ENTRY, REAL_END = 13, 14  # 100 MHz clock


def run(workload: str, splits: int, max_wgs: int):
    os.environ["PA_TRACE"] = "1"  # before the package loads its library
    import torch
    import paged_kv_attention_29_amd as pa
    from paged_kv_attention_29_amd import runner
    if workload == "decode":
        w = W.decode_batch(num_splits=splits)
        call = w.steps[0].calls[0]
    else:
        w = W.prefill_batch()
        call = w.steps[0].calls[0]
    cache = runner.PagedCache(w)
    cache.fill_context()
    k, v, s = cache.step_inputs(w.steps[0])
    cache.write(k, v, s)
    cb = cache.call_buffers(call)
    # every workgroup of the launch writes its record: the buffer must hold
    # the largest grid the call can have
    T = int(call.q.shape[0])
    tok = 128 // (w.num_heads // w.num_kv_heads)  # query tokens per prefill tile
    bound = (w.num_heads * call.num_seqs * cb.num_splits if workload == "decode"
             else w.num_kv_heads * (T // tok + call.num_seqs))
    if bound > max_wgs:
        raise ValueError(f"the launch may have {bound} workgroups; raise --max-wgs")
    buf = torch.zeros(max_wgs * SLOTS, dtype=torch.int64, device="cuda")
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    for _ in range(10):
        cache.run(cb)
    torch.cuda.synchronize()
    rc = pa.lib.pa_trace_set(buf.data_ptr())
    if rc != 0:
        raise RuntimeError(pa.lib.pa_last_error().decode())

    def launch():
        float(flush.sum())
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if workload == "decode" and cb.num_splits > 1:
            # the decode launch alone (no merge), the trace's subject
            pa.paged_attn_decode(None, cb.q, cache.key_cache, cache.value_cache, cb.seq_lens,
                                 cb.block_table, cb.max_seqlen_k, w.scale, w.window_left,
                                 w.softcap, cache.alibi, cb.num_splits, part_out=cb.part_out,
                                 part_lse=cb.part_lse)
        else:
            cache.run(cb)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    ms = launch()
    pa.lib.pa_trace_set(None)
    ms_plain = launch()  # the same launch with the trace off, for comparison
    t = buf.view(max_wgs, SLOTS).cpu().numpy().astype(np.int64)
    return w, (ms, ms_plain), t[t[:, ENTRY] != 0]


def cu_key(rec):
    hw = rec[:, HWID]
    cu, sh, se = (hw >> 8) & 0xF, (hw >> 12) & 1, (hw >> 13) & 0x7
    return (rec[:, XCC] & 0xF) * 1000 + se * 100 + sh * 16 + cu


def summarise(workload, w, ms, t):
    real = t[:, UNITS] > 0
    r = t[real]
    key = cu_key(t)
    wave_end = t[:, WAVE_END:WAVE_END + 4].max(axis=1)
    end = np.where(real, np.maximum(t[:, END], wave_end), t[:, END])
    med = lambda x: int(np.median(x)) if len(x) else 0
    lines = [f"## {workload}: {w.name}", "",
             f"launch {ms[0] * 1e3:.1f} us traced, {ms[1] * 1e3:.1f} us with the trace off "
             f"(HIP events, after a 512 MiB read); "
             f"{len(t)} workgroups with a record, {int(real.sum())} with work", "",
             "| phase (shader-clock cycles, per workgroup) | median | mean |",
             "|---|---|---|"]
    phases = [("entry -> item known", r[:, ITEM] - r[:, ENTRY]),
              ("item known -> first K/V landed", r[:, LOOP0] - r[:, ITEM]),
              ("key loop", r[:, LOOP1] - r[:, LOOP0]),
              ("key loop per tile / step", (r[:, LOOP1] - r[:, LOOP0]) / r[:, UNITS]),
              ("loop end -> last wave done", end[real] - r[:, LOOP1])]
    for name, x in phases:
        lines.append(f"| {name} | {med(x)} | {int(np.mean(x))} |")
    lines.append(f"| tiles or steps per workgroup | {med(r[:, UNITS])} | {np.mean(r[:, UNITS]):.1f} |")
    # the shader clock's rate: its ticks over the constant 100 MHz clock's,
    # per workgroup, from entry to wave 0's end
    dr = r[:, REAL_END] - r[:, REAL_ENTRY]
    ok = dr > 0
    ghz = (r[ok, END] - r[ok, ENTRY]) / dr[ok] * 0.1
    if ok.any():
        span = (r[ok, REAL_END].max() - r[ok, REAL_ENTRY].min()) / 100.0
        lines += ["", f"first workgroup entry -> last workgroup end (100 MHz clock, "
                  f"workgroups with work): {span:.1f} us"]
    if len(ghz):
        lines += ["", f"shader clock over the launch (s_memtime ticks per 10 ns of s_memrealtime, "
                  f"per workgroup): median {np.median(ghz):.2f} GHz, "
                  f"10th-90th percentile {np.percentile(ghz, 10):.2f}-{np.percentile(ghz, 90):.2f} GHz"]
    # per CU: occupancy, ramp, tail
    occ = np.zeros(4)
    tot = 0
    ramps, tails, spans, gaps = [], [], [], []
    for kcu in np.unique(key):
        m = key == kcu
        st, en = t[m, ENTRY], end[m]
        lo, hi = st.min(), en.max()
        spans.append(hi - lo)
        ts = np.linspace(lo, hi, 1000)
        n = ((st[None, :] <= ts[:, None]) & (ts[:, None] < en[None, :])).sum(1)
        peak = n.max()
        for c in range(3):
            occ[c] += (n == c).sum()
        occ[3] += (n > 2).sum()
        tot += len(ts)
        full = np.nonzero(n >= peak)[0]
        ramps.append(ts[full[0]] - lo)
        tails.append(hi - ts[full[-1]])
        ss = np.sort(st)
        for x in en:
            nxt = ss[ss > x]
            if len(nxt):
                gaps.append(nxt[0] - x)
    lines += ["", "| per CU (shader-clock cycles) | median | max |", "|---|---|---|",
              f"| first entry -> last end | {med(spans)} | {int(np.max(spans))} |",
              f"| ramp: first entry -> the CU first holds its most workgroups | "
              f"{med(ramps)} | {int(np.max(ramps))} |",
              f"| tail: the CU last holds its most -> its last end | {med(tails)} | "
              f"{int(np.max(tails))} |",
              f"| a workgroup's end -> the next start on its CU | {med(gaps)} | "
              f"{int(np.max(gaps)) if gaps else 0} |",
              "", f"share of CU time holding 0 / 1 / 2 / more workgroups: "
              f"{occ[0] / tot:.2f} / {occ[1] / tot:.2f} / {occ[2] / tot:.2f} / {occ[3] / tot:.2f}"]
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", choices=["decode", "prefill"], default="decode")
    ap.add_argument("--splits", type=int, default=8)
    ap.add_argument("--max-wgs", type=int, default=1 << 16)
    args = ap.parse_args()
    w, ms, t = run(args.workload, args.splits, args.max_wgs)
    print(summarise(args.workload, w, ms, t), flush=True)


if __name__ == "__main__":
    main()
