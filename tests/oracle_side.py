"""Oracle-side replay of a workload on the CPU, and the comparison bar
(test helpers; the oracle never sees anything the GPU computed)."""
import math

import numpy as np
import torch

import oracle

NAN = float("nan")
MAX_ABS = 2e-2    # attention outputs, bf16/fp16 (fp32 accumulation)
MEAN_ABS = 2e-3


def oracle_cache(w, through_step: int = -1):
    """Oracle K/V cache after the context and steps [0, through_step]."""
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_size)
    kc = torch.full(shape, NAN, dtype=w.dtype)
    vc = torch.full(shape, NAN, dtype=w.dtype)
    for _, k, v, s in w.context_tokens():
        oracle.scatter(k, v, s, kc, vc)
    for i in range(through_step + 1):
        k, v, s = w.step_tokens(w.steps[i])
        oracle.scatter(k, v, s, kc, vc)
    return kc, vc


def oracle_call(w, kc, vc, call, num_splits=1):
    """(out, lse) in float64; split decode returns the merged result and the parts."""
    bt = torch.from_numpy(w.block_table[np.asarray(call.seq_ids)])
    if call.kind == "prefill":
        return oracle.attend(call.q, kc, vc, call.cu_seqlens_q.tolist(), call.seq_lens.tolist(),
                             bt, w.scale, call.causal, w.window_left, w.softcap, w.alibi_slopes)
    if num_splits == 1:
        return oracle.decode(call.q, kc, vc, call.seq_lens.tolist(), bt, w.scale, w.window_left,
                             w.softcap, w.alibi_slopes)
    po, pl = oracle.decode_splits(call.q, kc, vc, call.seq_lens.tolist(), bt, w.scale, num_splits,
                                  w.window_left, w.softcap, w.alibi_slopes)
    o, l = oracle.merge(po, pl)
    return o, l, po, pl


def oracle_sampled(w, call, i: int, g: int):
    """Reference for sequence i of a call and the query heads of KV head g,
    computed on a compact cache holding only that sequence's blocks of that
    KV head (built with the oracle's own scatter, shuffled block ids).
    Returns (out [nq, G, D], lse [G, nq], rows, heads)."""
    b = int(call.seq_ids[i])
    L = int(call.seq_lens[i])
    bs, D = w.block_size, w.head_size
    G = w.num_heads // w.num_kv_heads
    nblk = -(-L // bs)
    perm = np.random.default_rng(1000 * b + g).permutation(nblk + 2)
    table = torch.from_numpy(perm[:nblk].astype(np.int32))[None]
    kc = torch.full((nblk + 2, bs, 1, D), NAN, dtype=w.dtype)
    vc = torch.full((nblk + 2, bs, 1, D), NAN, dtype=w.dtype)
    k, v = w.sequence_kv(b, 0, L, kv_heads=[g])
    pos = np.arange(L)
    slots = torch.from_numpy(perm[pos // bs].astype(np.int64) * bs + pos % bs)
    oracle.scatter(k, v, slots, kc, vc)
    cu = call.cu_seqlens_q
    r0, r1 = int(cu[i]), int(cu[i + 1])
    heads = list(range(g * G, (g + 1) * G))
    q = call.q[r0:r1, heads]
    slopes = None if w.alibi_slopes is None else w.alibi_slopes[heads]
    out, lse = oracle.attend(q, kc, vc, [0, r1 - r0], [L], table, w.scale, True, w.window_left,
                             w.softcap, slopes)
    return out, lse, (r0, r1), heads


def oracle_sequence(w, call, i: int):
    """Reference for every query head of sequence i of a call, computed on a
    compact cache that holds only that sequence's blocks (all KV heads; built
    with the oracle's own scatter, shuffled block ids).  Used where the whole
    workload's cache is too large to replay at once on the host.
    Returns (out [nq, Hq, D], lse [Hq, nq], rows)."""
    b = int(call.seq_ids[i])
    L = int(call.seq_lens[i])
    bs = w.block_size
    nblk = -(-L // bs)
    perm = np.random.default_rng(7000 + b).permutation(nblk + 2)
    table = torch.from_numpy(perm[:nblk].astype(np.int32))[None]
    shape = (nblk + 2, bs, w.num_kv_heads, w.head_size)
    kc = torch.full(shape, NAN, dtype=w.dtype)
    vc = torch.full(shape, NAN, dtype=w.dtype)
    k, v = w.sequence_kv(b, 0, L)
    pos = np.arange(L)
    slots = torch.from_numpy(perm[pos // bs].astype(np.int64) * bs + pos % bs)
    oracle.scatter(k, v, slots, kc, vc)
    del k, v
    cu = call.cu_seqlens_q
    r0, r1 = int(cu[i]), int(cu[i + 1])
    out, lse = oracle.attend(call.q[r0:r1], kc, vc, [0, r1 - r0], [L], table, w.scale, True,
                             w.window_left, w.softcap, w.alibi_slopes)
    return out, lse, (r0, r1)


def assert_attn_close(gpu_out, ref_out, what="out", max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    g = gpu_out.detach().to("cpu", torch.float64)
    assert torch.isfinite(g).all(), f"{what}: non-finite values in the GPU result"
    err = (g - ref_out).abs()
    assert err.max().item() <= max_abs, f"{what}: max abs err {err.max().item():.3e}"
    assert err.mean().item() <= mean_abs, f"{what}: mean abs err {err.mean().item():.3e}"


def assert_lse_close(gpu_lse, ref_lse, what="lse"):
    g = gpu_lse.detach().to("cpu", torch.float64)
    both_inf = torch.isneginf(g) & torch.isneginf(ref_lse)
    tol = 1e-2 * torch.clamp(ref_lse.abs() * 1e-3, min=1.0)
    bad = ~both_inf & ~((g - ref_lse).abs() <= tol)
    assert not bad.any(), f"{what}: {int(bad.sum())} entries off, e.g. gpu {g[bad][:4].tolist()} ref {ref_lse[bad][:4].tolist()}"
