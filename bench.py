"""Benchmark of the paged-KV attention hot path on one MI355X.

One step = one decode step of the batch: reshape_and_cache of the new tokens,
split-KV paged_attn_decode, merge_attn_states.  The headline `value` is the
decode KV-read bandwidth (algorithmic bytes: the K and V rows each query
must see, counted once) over the whole step.  The causal prefill workload is
measured in the same run and reported as attention TFLOP/s under "prefill".

Inputs are seeded synthetic data resident in HBM before timing starts.  Each
step uses the next of `--layers` independent caches (as consecutive layers of
a model would) so no step re-reads K/V another step left in the caches.

`--kv-fp8` runs the workloads over an fp8 (e4m3) cache with per-tensor
scales and an fp8 query (`--fp8-q16` keeps the 16-bit query); the bytes then
count one byte per element.

Prints ONE JSON line.  `--gpus N` with N > 1 is refused: the hot path here
runs on a single GPU (no collectives).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "decode KV-read GB/s + prefill attn TFLOP/s, bf16 paged KV, 1×MI355X"
WARM_SECONDS = 0.3  # untimed warm-up after --warmup steps, before each timed region
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
# written between timed repetitions (outside the timed region) so that no
# repetition finds the previous one's data in the 256 MB Infinity Cache or
# the 8 x 4 MB L2
SCRATCH_MIB = 512
CSRC = os.path.join(ROOT, "paged_kv_attention_29_amd", "csrc")


def visible_keys(L: int, pos: int, causal: bool, window_left: int) -> int:
    hi = min(L, pos + 1) if causal else L
    lo = max(0, pos - window_left) if window_left >= 0 else 0
    return max(0, hi - lo)


# per-tensor scales of the fp8 (e4m3) cache in --kv-fp8 runs: the largest
# |x| of N(0,1) data over a few million draws (about 5.6) maps to 448
FP8_SCALES = (5.6 / 448.0, 5.6 / 448.0)
# --kv-fp8 quantises the query too (per-tensor scale, scaled_fp8_quant), the
# pages' default fp8 flow; --fp8-q16 keeps the 16-bit query
Q_FP8_SCALE = 5.6 / 448.0


def set_fp8_query(args, cache):
    if args.kv_fp8 and not args.fp8_q16:
        cache.q_scale = torch.tensor([Q_FP8_SCALE], dtype=torch.float32, device="cuda")


def decode_bytes(w, call, elem: int = 2) -> int:
    """K and V bytes every decode query must see: visible keys x Hkv x D x 2 x elem."""
    keys = sum(visible_keys(int(L), int(L) - 1, True, w.window_left) for L in call.seq_lens)
    return keys * w.num_kv_heads * w.head_size * 2 * elem


def prefill_flops(w, call) -> int:
    """4 * D * Hq per visible (query, key) pair (QK^T and PV, 2 flops per MAC)."""
    pairs = 0
    for nq, L in zip(call.query_lens, call.seq_lens):
        nq, L = int(nq), int(L)
        ctx = L - nq
        if w.window_left < 0:
            pairs += nq * ctx + nq * (nq + 1) // 2
        else:
            pairs += sum(visible_keys(L, ctx + t, True, w.window_left) for t in range(nq))
    return 4 * w.head_size * w.num_heads * pairs


def source_digest(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(CSRC, n), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel_key: str, digest: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if the
    kernel source is unchanged since they were taken."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel_key)
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


class Timed:
    """HIP events around each launch of one kernel on the current stream
    (the stream the library's calls are enqueued on)."""

    def __init__(self):
        self.pairs = []

    def __enter__(self):
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()
        self.pairs.append((self.a, self.b))

    def times_ms(self):
        return sorted(a.elapsed_time(b) for a, b in self.pairs)

    def median_ms(self) -> float:
        return statistics.median(self.times_ms()) if self.pairs else 0.0

    def min_ms(self) -> float:
        return min(self.times_ms()) if self.pairs else 0.0

    def summary(self, work: float, unit_div: float) -> dict:
        """median / min time and the rate of `work` at the median (work /
        unit_div per second)."""
        med, mn = self.median_ms(), self.min_ms()
        return {"median_ms": round(med, 4), "min_ms": round(mn, 4), "reps": len(self.pairs),
                "rate": round(work / (med * 1e-3) / unit_div, 2)}


class Flush:
    """A 512 MiB device buffer streamed through between timed repetitions,
    outside the timed region.  It is READ (pa_probe_stream), not written: a
    write leaves up to L2 + Infinity Cache worth of dirty lines (about
    290 MB) whose write-back then competes with the next timed kernel's own
    traffic, while a read evicts with clean lines."""

    def __init__(self, pa):
        import ctypes
        self.f = pa.lib.pa_probe_stream
        self.f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                           ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        self.f.restype = ctypes.c_int
        self.buf = torch.ones(SCRATCH_MIB << 18, dtype=torch.float32, device="cuda")
        self.sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()

    def __call__(self):
        rc = self.f(0, self.buf.data_ptr(), self.sink.data_ptr(), self.buf.numel() * 4, 2048, 4,
                    torch.cuda.current_stream().cuda_stream)
        assert rc == 0, rc


def run_decode(args, pa, runner, w, merged=True):
    """The decode step over `layers` caches: reshape_and_cache, then the
    split decode with its splits merged in the same launch
    (paged_attn_decode_merged), or (merged=False) paged_attn_decode followed
    by merge_attn_states."""
    call = w.steps[0].calls[0]
    base = runner.PagedCache(w, kv_scales=FP8_SCALES if args.kv_fp8 else None)
    set_fp8_query(args, base)
    base.fill_context()
    caches = [base]
    for _ in range(args.layers - 1):
        c = runner.PagedCache.__new__(runner.PagedCache)
        c.__dict__.update(base.__dict__)
        c.key_cache = base.key_cache.clone()
        c.value_cache = base.value_cache.clone()
        caches.append(c)
    for c in caches:
        c.sinks = bench_sinks(args, w)
    k, v, s = base.step_inputs(w.steps[0])
    bufs = [c.call_buffers(call, args.splits, merged=merged) for c in caches]
    torch.cuda.synchronize()

    dec_t, rac_t, merge_t = Timed(), Timed(), Timed()

    def step(i, timed):
        c, cb = caches[i % len(caches)], bufs[i % len(caches)]
        if timed:
            with rac_t:
                c.write(k, v, s)
        else:
            c.write(k, v, s)
        if cb.num_splits == 1 or merged:
            if timed:
                with dec_t:
                    c.run(cb)
            else:
                c.run(cb)
            return
        kw = dict(part_out=cb.part_out, part_lse=cb.part_lse, k_scale=c.k_scale,
                  v_scale=c.v_scale, q_scale=c.q_scale, out_dtype=w.dtype)
        if timed:
            with dec_t:
                pa.paged_attn_decode(None, cb.q, c.key_cache, c.value_cache, cb.seq_lens,
                                     cb.block_table, cb.max_seqlen_k, w.scale, w.window_left,
                                     w.softcap, c.alibi, cb.num_splits, sinks=c.sinks, **kw)
            with merge_t:
                pa.merge_attn_states(cb.out, cb.part_out, cb.part_lse, out_lse=cb.lse)
        else:
            pa.paged_attn_decode(None, cb.q, c.key_cache, c.value_cache, cb.seq_lens,
                                 cb.block_table, cb.max_seqlen_k, w.scale, w.window_left,
                                 w.softcap, c.alibi, cb.num_splits, sinks=c.sinks, **kw)
            pa.merge_attn_states(cb.out, cb.part_out, cb.part_lse, out_lse=cb.lse)

    for i in range(args.warmup):
        step(i, False)
    spin_up(lambda: step(0, False))
    # whole-step wall time without the per-kernel events
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, False)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # the same steps again with HIP events around each kernel
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    nbytes = decode_bytes(w, call, 1 if args.kv_fp8 else 2)
    return dict(ms_per_step=wall_ms, decode_ms=dec_t.median_ms(), decode_min_ms=dec_t.min_ms(),
                rac_ms=rac_t.median_ms(),
                merge_ms=merge_t.median_ms() if merge_t.pairs else 0.0, bytes=nbytes,
                tokens=int(s.numel()))


def fp8_suffix(args):
    if not args.kv_fp8:
        return ""
    return "_kvfp8" if args.fp8_q16 else "_kvfp8_qfp8"


def bench_sinks(args, w):
    """--sinks: seeded fp32 attention-sink logits, one per query head."""
    if not args.sinks:
        return None
    g = torch.Generator().manual_seed(77)
    return (torch.randn(w.num_heads, generator=g) * 2.0).to("cuda")


def spin_up(fn, seconds: float = WARM_SECONDS):
    """More untimed warm-up: repeat fn until `seconds` of GPU work have run,
    so the timed region sees steady-state clocks."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def run_prefill(args, pa, runner, flush, w=None, call_index=0, write=True):
    """Time reshape_and_cache of the step's new tokens and the prefill call
    (the cache is written once more before every prefill rep, so each rep
    runs on exactly the inputs of the first), with the scratch write
    between repetitions."""
    w = W.prefill_batch() if w is None else w
    call = w.steps[0].calls[call_index]
    cache = runner.PagedCache(w, kv_scales=FP8_SCALES if args.kv_fp8 else None)
    set_fp8_query(args, cache)
    if any(int(c) > 0 for c in w.context_lens):
        fill_cache_on_gpu(cache, seed=w.seed)
    cache.sinks = bench_sinks(args, w)
    k, v, s = cache.step_inputs(w.steps[0])
    cb = cache.call_buffers(call)
    pre_t, rac_t = Timed(), Timed()
    for _ in range(args.warmup):
        cache.write(k, v, s)
        cache.run(cb)
    spin_up(lambda: (cache.write(k, v, s), cache.run(cb)))
    for _ in range(max(args.steps, 20)):
        flush()
        with rac_t:
            cache.write(k, v, s)
        flush()
        with pre_t:
            cache.run(cb)
    torch.cuda.synchronize()
    flops = prefill_flops(w, call)
    ms = pre_t.median_ms()
    tflops = flops / (ms * 1e-3) / 1e12
    # rows read (16-bit) and written (cache element)
    rac_bytes = 2 * int(s.numel()) * w.num_kv_heads * w.head_size * (2 + (1 if args.kv_fp8 else 2))
    digest = source_digest("prefill.hip", "common.h")
    key = "prefill" + ("" if w.name.startswith("prefill") else ":" + w.name)
    out = {
        "value": round(tflops, 2), "unit": "TFLOP/s",
        "workload": w.name + fp8_suffix(args),
        "ms_per_call": round(ms, 4), "min_ms": round(pre_t.min_ms(), 4),
        "reps": len(pre_t.pairs), "flops": flops, "query_tokens": int(call.q.shape[0]),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic_from_profile(key + fp8_suffix(args),
                                                     digest)},
    }
    if write:
        out["reshape_and_cache"] = {
            "ms": round(rac_t.median_ms(), 4), "min_ms": round(rac_t.min_ms(), 4),
            "GB/s": round(rac_bytes / (rac_t.median_ms() * 1e-3) / 1e9, 1),
            "bytes": rac_bytes}
    return out


def fill_cache_on_gpu(cache, seed: int):
    """Fill every slot of a cache with seeded N(0,1) values drawn on the GPU
    (timing runs only: the bytes do not have to match the host-drawn ones
    the parity tests use, and an 8 GB cache is drawn in a moment)."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    for c in (cache.key_cache, cache.value_cache):
        for i in range(0, c.shape[0], 16384):
            part = c[i:i + 16384]
            if c.dtype == torch.uint8:
                x = torch.randn(part.shape, generator=g, device="cuda", dtype=torch.float32)
                part.copy_((x / FP8_SCALES[0]).clamp(-448, 448).to(torch.float8_e4m3fn)
                           .view(torch.uint8))
            else:
                part.normal_(generator=g)
    torch.cuda.synchronize()


def run_decode_call(args, pa, runner, flush, w, call_index=0):
    """One decode call (splits merged in the launch, or with --merge separate
    a split decode then merge_attn_states) with the scratch read between
    repetitions: kernel and whole-call times (median, min)."""
    call = w.steps[0].calls[call_index]
    cache = runner.PagedCache(w, kv_scales=FP8_SCALES if args.kv_fp8 else None)
    set_fp8_query(args, cache)
    fill_cache_on_gpu(cache, seed=w.seed)
    cache.sinks = bench_sinks(args, w)
    merged = args.merge == "merged"
    cb = cache.call_buffers(call, merged=merged)
    S = cb.num_splits
    dec_t, mer_t, all_t = Timed(), Timed(), Timed()

    def decode():
        if merged or S == 1:
            cache.run(cb)
            return
        pa.paged_attn_decode(None, cb.q, cache.key_cache, cache.value_cache,
                             cb.seq_lens, cb.block_table, cb.max_seqlen_k, w.scale, w.window_left,
                             w.softcap, cache.alibi, S, part_out=cb.part_out,
                             part_lse=cb.part_lse, sinks=cache.sinks, k_scale=cache.k_scale,
                             v_scale=cache.v_scale, q_scale=cache.q_scale, out_dtype=w.dtype)

    def merge():
        if S > 1 and not merged:
            pa.merge_attn_states(cb.out, cb.part_out, cb.part_lse, out_lse=cb.lse)

    for _ in range(args.warmup):
        decode()
        merge()
    spin_up(lambda: (decode(), merge()))
    for _ in range(max(args.steps, 20)):
        flush()
        with all_t:
            with dec_t:
                decode()
            with mer_t:
                merge()
    torch.cuda.synchronize()
    nbytes = decode_bytes(w, call, 1 if args.kv_fp8 else 2)
    kern = nbytes / (dec_t.median_ms() * 1e-3) / 1e9
    whole = nbytes / (all_t.median_ms() * 1e-3) / 1e9
    digest = source_digest("decode.hip", "common.h")
    return {
        "workload": w.name + fp8_suffix(args), "num_splits": S,
        "splits_merged_in_kernel": merged and S > 1,
        "bytes": nbytes, "decode_ms": round(dec_t.median_ms(), 4),
        "decode_min_ms": round(dec_t.min_ms(), 4), "merge_ms": round(mer_t.median_ms(), 4),
        "call_ms": round(all_t.median_ms(), 4), "reps": len(dec_t.pairs),
        "call_GB/s": round(whole, 1),
        "roofline": {"bound": "hbm", "achieved": round(kern, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kern / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile(
                         f"decode:{w.name}{fp8_suffix(args)}:S{S}", digest),
                     "kernel": "paged_attn_decode_merged" if merged and S > 1 else "paged_attn_decode"},
    }


def measured_peaks(pa):
    """Measured-achievable ceilings beside the vendor peaks: the best of a
    small sweep of plain streaming read / copy kernels over 4 GiB
    (pa_probe_stream), and a large bf16 GEMM through torch (hipBLASLt)."""
    import ctypes
    lib = pa.lib
    lib.pa_probe_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.pa_probe_stream.restype = ctypes.c_int
    n = 4 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty(n // 8, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def best(mode, nbytes, moved):
        res = {}
        for wgs in (1024, 2048, 4096, 8192):
            for unroll in (4, 8):
                t = Timed()
                for r in range(8):
                    with t:
                        rc = lib.pa_probe_stream(mode, src.data_ptr(), dst.data_ptr(), nbytes, wgs,
                                                 unroll, stream)
                    assert rc == 0, rc
                torch.cuda.synchronize()
                res[(wgs, unroll)] = moved / (t.median_ms() * 1e-3) / 1e9
        k = max(res, key=res.get)
        return round(res[k], 1), {"workgroups": k[0], "loads_per_lane": k[1]}

    rd, rd_cfg = best(0, n, n)
    cp, cp_cfg = best(1, n // 2, n)       # 2 GiB read + 2 GiB written
    del src, dst
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    c = a @ b
    t = Timed()
    for _ in range(10):
        with t:
            torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    gemm = 2 * 8192 ** 3 / (t.median_ms() * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return {"hbm_stream_read_GB/s": rd, "read_probe": rd_cfg,
            "hbm_copy_GB/s": cp, "copy_probe": cp_cfg,
            "bf16_gemm_TFLOP/s": round(gemm, 1), "gemm": "8192^3 bf16 torch.matmul (hipBLASLt)"}


def cpu_baseline(w, seconds: float = 10.0, max_passes: int = 100, sinks=None):
    """The oracle (float64 PyTorch on the host) on the same decode batch:
    every sequence's K/V is placed in a cache of its own once, then whole
    passes over the batch are timed until about `seconds` of work."""
    import oracle
    call = w.steps[0].calls[0]
    threads = torch.get_num_threads()
    setups = []
    for b in range(call.num_seqs):
        L = int(call.seq_lens[b])
        nblk = -(-L // w.block_size)
        kc = torch.full((nblk, w.block_size, w.num_kv_heads, w.head_size), float("nan"),
                        dtype=w.dtype)
        vc = kc.clone()
        kk, vv = w.sequence_kv(b, 0, L)
        pos = np.arange(L)
        slots = torch.from_numpy((pos // w.block_size) * w.block_size + pos % w.block_size)
        oracle.scatter(kk, vv, slots, kc, vc)
        table = torch.arange(nblk, dtype=torch.int32)[None]
        nbytes = visible_keys(L, L - 1, True, w.window_left) * w.num_kv_heads * w.head_size * 4
        setups.append((b, L, kc, vc, table, nbytes))
    done_bytes, elapsed, passes = 0, 0.0, 0
    while elapsed < seconds and passes < max_passes:
        for b, L, kc, vc, table, nbytes in setups:
            t0 = time.perf_counter()
            oracle.decode(call.q[b:b + 1], kc, vc, [L], table, w.scale, w.window_left,
                          w.softcap, w.alibi_slopes, sinks=sinks)
            elapsed += time.perf_counter() - t0
            done_bytes += nbytes
        passes += 1
    return {"value": round(done_bytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"oracle decode of all {call.num_seqs} sequences (all heads), {passes} "
                      f"passes, {elapsed:.1f} s of CPU time, float64"}


LOCAL_METRIC = "chunked local attention prefill (virtual batches): TFLOP/s, bf16 paged KV, 1xMI355X"


def run_local(args, pa, runner, chunk: int = 512):
    """The prefill batch (16 x 256-2048 causal, 32/8/128, block 16) under
    chunked local attention with attn_chunk_size 512: the host rewriting
    gives the virtual batch, and the prefill kernel runs over it.  TFLOP/s
    counts 4 * D * Hq per visible (query, key) pair of the chunked mask."""
    w = W.prefill_batch()
    call = w.steps[0].calls[0]
    cache = runner.PagedCache(w)
    k, v, s = cache.step_inputs(w.steps[0])
    pa.reshape_and_cache(k, v, cache.key_cache, cache.value_cache, s)
    cu = np.concatenate([[0], np.cumsum(call.query_lens)]).astype(np.int32)
    table = w.block_table[np.asarray(call.seq_ids)]
    q_loc, cu_loc, k_loc, bt_loc = pa.local_virtual_batches(chunk, cu, call.seq_lens, table,
                                                            w.block_size)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    cu_d, k_d, bt_d = dev(cu_loc), dev(k_loc), dev(bt_loc)
    q = call.q.cuda()
    out = torch.empty_like(q)
    mq, mk = int(q_loc.max()), int(k_loc.max())

    def run():
        pa.paged_attn_prefill(out, q, cache.key_cache, cache.value_cache, cu_d, k_d, bt_d, mq, mk,
                              w.scale, True)

    for _ in range(args.warmup):
        run()
    spin_up(run)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # causal within each virtual sequence (its queries are its last positions)
    pairs = sum(nq * (nk - nq) + nq * (nq + 1) // 2 for nq, nk in zip(q_loc.tolist(), k_loc.tolist()))
    flops = 4 * w.head_size * w.num_heads * pairs
    tflops = flops / (ms * 1e-3) / 1e12
    return {
        "metric": LOCAL_METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}_local{chunk}", "attn_chunk_size": chunk,
                   "num_seqs": call.num_seqs, "virtual_seqs": int(q_loc.size),
                   "query_tokens": int(cu[-1]), "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_size": w.head_size,
                   "block_size": w.block_size},
        "flops": flops,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "paged_attn_prefill over the virtual batch"},
    }


CASCADE_METRIC = "cascade decode over a shared prefix: effective KV GB/s, bf16 paged KV, 1xMI355X"


def run_cascade(args, pa, B=64, P=4096, suffix_range=(64, 1024)):
    """A decode step of 64 requests that share a 4096-token prefix (the
    shape the cascade is for: many requests, a long common prompt), each
    with its own 64-1024 tokens of history; 32 query / 8 KV heads of 128,
    block 16, bf16.  Times paged_attn_cascade and, on the same inputs, the
    plain split decode + merge.  `value` is the plain path's K/V bytes (every
    key of every sequence) over the cascade's time; the roofline counts the
    bytes the cascade must read (the prefix once, each suffix once)."""
    Hq, Hkv, D, bs, S = 32, 8, 128, 16, 8
    rng = np.random.Generator(np.random.PCG64(6))
    suffix = rng.integers(suffix_range[0], suffix_range[1], size=B, endpoint=True)
    lens = P + suffix
    n = P // bs
    own = [-(-int(x) // bs) for x in suffix]
    nb = n + sum(own)
    perm = rng.permutation(nb).astype(np.int32)
    table = np.zeros((B, n + max(own)), np.int32)
    table[:, :n] = perm[:n]
    at = n
    for b in range(B):
        table[b, n:n + own[b]] = perm[at:at + own[b]]
        at += own[b]
    g = torch.Generator(device="cuda").manual_seed(6)
    # four independent caches used in turn (about 320 MB): more than the
    # 256 MB Infinity Cache, so no call finds the previous call's K/V there
    caches = [(torch.randn(nb, bs, Hkv, D, generator=g, device="cuda", dtype=torch.bfloat16),
               torch.randn(nb, bs, Hkv, D, generator=g, device="cuda", dtype=torch.bfloat16))
              for _ in range(4)]
    q = torch.randn(B, Hq, D, generator=g, device="cuda", dtype=torch.bfloat16)
    bt = torch.from_numpy(table).cuda()
    seq_lens = torch.from_numpy(lens.astype(np.int32)).cuda()
    cu = torch.arange(B + 1, dtype=torch.int32, device="cuda")
    scale = D ** -0.5
    out_c = torch.empty(B, Hq, D, dtype=torch.bfloat16, device="cuda")
    out_d = torch.empty_like(out_c)
    ws = (torch.empty(17, B, Hq, D, dtype=torch.bfloat16, device="cuda"),
          torch.empty(17, Hq, B, dtype=torch.float32, device="cuda"))
    po = torch.empty(S, B, Hq, D, dtype=torch.float32, device="cuda")
    pl = torch.empty(S, Hq, B, dtype=torch.float32, device="cuda")
    mx = int(lens.max())

    turn = [0]

    def next_cache():
        turn[0] += 1
        return caches[turn[0] % len(caches)]

    def cascade():
        kc, vc = next_cache()
        pa.paged_attn_cascade(out_c, q, kc, vc, cu, seq_lens, bt, 1, mx, scale, P,
                              max_prefix_splits=16, workspace=ws)

    def plain():
        kc, vc = next_cache()
        pa.paged_attn_decode(None, q, kc, vc, seq_lens, bt, mx, scale, num_splits=S,
                             part_out=po, part_lse=pl)
        pa.merge_attn_states(out_d, po, pl)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        spin_up(fn)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    t_c, t_d = timed(cascade), timed(plain)
    turn[0] = -1
    cascade()
    turn[0] = -1
    plain()  # both on the same cache for the comparison below
    row = Hkv * D * 2 * 2  # K and V bytes of one key, all KV heads
    plain_bytes = int(lens.sum()) * row
    cascade_bytes = (P + int(suffix.sum())) * row
    diff = (out_c.float() - out_d.float()).abs().max().item()
    ach = cascade_bytes / (t_c * 1e-3) / 1e9
    return {
        "metric": CASCADE_METRIC, "value": round(plain_bytes / (t_c * 1e-3) / 1e9, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(t_c, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"cascade_decode_b{B}_prefix{P}_suffix{suffix_range[0]}-"
                               f"{suffix_range[1]}_h32-8-128_bs16",
                   "num_seqs": B, "common_prefix_len": P, "context_tokens": int(lens.sum()),
                   "num_heads": Hq, "num_kv_heads": Hkv, "head_size": D, "block_size": bs,
                   "step": "paged_attn_cascade (prefix prefill + suffix prefill + merge)"},
        "plain_decode": {"ms": round(t_d, 4), "num_splits": S,
                         "GB/s": round(plain_bytes / (t_d * 1e-3) / 1e9, 1),
                         "step": "paged_attn_decode + merge_attn_states"},
        "speedup_vs_plain": round(t_d / t_c, 2),
        "max_abs_diff_vs_plain": round(diff, 5),
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "paged_attn_cascade (whole call)",
                     "bytes_per_launch": cascade_bytes},
    }


def run_cascade_sweep(args, pa):
    """Cascade vs plain split decode over a grid of batch sizes, shared
    prefix lengths and suffix ranges (the measurements behind the cascade
    decision rule, pa_use_cascade).  One JSON object per point."""
    rows = []
    for B in (8, 16, 32, 64, 128):
        for P in (256, 512, 1024, 2048, 4096, 8192):
            for suf in ((1, 64), (64, 1024)):
                r = run_cascade(args, pa, B=B, P=P, suffix_range=suf)
                rows.append({"B": B, "P": P, "suffix": list(suf),
                             "cascade_ms": r["ms_per_step"], "plain_ms": r["plain_decode"]["ms"]})
                print(json.dumps(rows[-1]), flush=True)
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "mixed", "long", "cascade", "cascade-sweep", "local"])
    ap.add_argument("--splits", type=int, default=None)
    ap.add_argument("--layers", type=int, default=2)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="default run: skip the mixed and long-context workloads and the probes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sinks", action="store_true",
                    help="decode/mixed/long: pass per-head attention-sink logits")
    ap.add_argument("--kv-fp8", action="store_true",
                    help="decode/mixed/long: fp8 (e4m3) K/V cache with per-tensor scales")
    ap.add_argument("--fp8-q16", action="store_true",
                    help="with --kv-fp8: keep the query in 16 bits (not quantised)")
    ap.add_argument("--merge", choices=["merged", "separate"], default="separate",
                    help="split decode: decode then merge_attn_states (the faster on MI355X), "
                         "or the splits merged in the decode launch (paged_attn_decode_merged)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the hot path here is single-GPU "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import paged_kv_attention_29_amd as pa
    from paged_kv_attention_29_amd import runner

    if args.workload == "cascade":
        print(json.dumps(run_cascade(args, pa)), flush=True)
        return
    if args.workload == "cascade-sweep":
        run_cascade_sweep(args, pa)
        return
    if args.workload == "local":
        print(json.dumps(run_local(args, pa, runner)), flush=True)
        return
    if args.workload == "decode":
        w = W.decode_batch() if args.splits is None else W.decode_batch(num_splits=args.splits)
    elif args.workload == "mixed":
        w = W.mixed_batch() if args.splits is None else W.mixed_batch(num_splits=args.splits)
    else:
        w = W.long_decode()
        args.layers = 1
    if args.splits is None:
        args.splits = w.steps[0].calls[0].num_splits
    call = w.steps[0].calls[0]

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    merged = args.merge == "merged" and args.splits > 1
    r = run_decode(args, pa, runner, w, merged=merged)
    gbs = r["bytes"] / (r["ms_per_step"] * 1e-3) / 1e9
    kern_gbs = r["bytes"] / (r["decode_ms"] * 1e-3) / 1e9
    digest = source_digest("decode.hip", "common.h")
    out = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": (("fp8_e4m3 K/V cache, bf16 q" if args.fp8_q16 else "fp8_e4m3 K/V cache and q")
                  if args.kv_fp8 else "bf16"),
        "data": "synthetic",
        "config": {"workload": w.name + fp8_suffix(args),
                   "num_seqs": call.num_seqs,
                   "context_tokens": int(call.seq_lens.sum()), "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_size": w.head_size,
                   "block_size": w.block_size, "num_splits": args.splits,
                   "layers": args.layers,
                   "step": ("reshape_and_cache + decode with the splits merged in the launch"
                            if merged else "reshape_and_cache + decode + merge"),
                   "attention_sinks": bool(args.sinks)},
        "kernels_ms": {"reshape_and_cache": round(r["rac_ms"], 4),
                       ("paged_attn_decode_merged" if merged else "paged_attn_decode"):
                           round(r["decode_ms"], 4),
                       "decode_min": round(r["decode_min_ms"], 4),
                       "merge_attn_states": round(r["merge_ms"], 4),
                       "statistic": f"median over {args.steps} launches (HIP events)"},
        "roofline": {"bound": "hbm", "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile(
                         f"decode:{w.name}{fp8_suffix(args)}:S{args.splits}",
                         digest),
                     "kernel": "paged_attn_decode_merged" if merged else "paged_attn_decode",
                     "bytes_per_launch": r["bytes"]},
    }
    if args.splits > 1 and not args.no_extra:
        # the same step with the other way of merging the splits
        rs = run_decode(args, pa, runner, w, merged=not merged)
        out["merged_in_kernel" if not merged else "separate_merge"] = {
            "ms_per_step": round(rs["ms_per_step"], 4),
            "GB/s": round(rs["bytes"] / (rs["ms_per_step"] * 1e-3) / 1e9, 1),
            "decode_ms": round(rs["decode_ms"], 4), "merge_ms": round(rs["merge_ms"], 4)}
    flush = Flush(pa)
    if not args.no_prefill and args.workload == "decode":
        out["prefill"] = run_prefill(args, pa, runner, flush)
    if not args.no_extra and args.workload == "decode":
        # the other configured workloads, each call timed on its own
        wm = W.mixed_batch()
        out["mixed"] = {"decode": run_decode_call(args, pa, runner, flush, wm, 0),
                        "prefill": run_prefill(args, pa, runner, flush, wm, 1, write=False)}
        torch.cuda.empty_cache()
        out["long"] = run_decode_call(args, pa, runner, flush, W.long_decode(), 0)
        torch.cuda.empty_cache()
        peaks = measured_peaks(pa)
        out["measured_peaks"] = peaks
        out["roofline"]["frac_of_measured_read"] = round(
            kern_gbs / peaks["hbm_stream_read_GB/s"], 4)
        if "prefill" in out:
            out["prefill"]["roofline"]["frac_of_measured_gemm"] = round(
                out["prefill"]["value"] / peaks["bf16_gemm_TFLOP/s"], 4)
    if not args.no_cpu_baseline and not args.kv_fp8:
        sk = bench_sinks(args, w)
        out["cpu_baseline"] = cpu_baseline(w, sinks=None if sk is None else sk.cpu())
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
