"""GPU-side invariants of the paged attention path, bit for bit:

* paging: moving every physical block (cache and block table together) to
  another block id leaves prefill and split-decode outputs and LSEs
  bit-identical (the kernels' arithmetic follows logical key positions only);
* causality: overwriting the K/V of positions at or after P leaves every
  causal prefill row of a position below P bit-identical (masked keys add
  exact zeros), while rows at or after P change.

These complement the oracle comparisons: they hold exactly, so they catch a
kernel that reads a wrong block or a key it must not see even where the
effect would hide inside the tolerance."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_attention_29_amd as pa
    return pa


@pytest.fixture(scope="module")
def runner(pa):
    from paged_kv_attention_29_amd import runner
    return runner


def _fresh(cb, **kw):
    """The same call with new (NaN-filled) result buffers."""
    nan = float("nan")
    repl = dict(out=torch.full_like(cb.out, nan), lse=torch.full_like(cb.lse, nan))
    if cb.part_out is not None:
        repl.update(part_out=torch.full_like(cb.part_out, nan),
                    part_lse=torch.full_like(cb.part_lse, nan))
    repl.update(kw)
    return dataclasses.replace(cb, **repl)


def _results(cb):
    return [cb.out, cb.lse] + ([cb.part_out, cb.part_lse] if cb.part_out is not None else [])


def _permuted(runner, cache, perm):
    """The same cache with block i stored at block id perm[i]."""
    c = runner.PagedCache.__new__(runner.PagedCache)
    c.__dict__.update(cache.__dict__)
    c.key_cache = torch.empty_like(cache.key_cache)
    c.value_cache = torch.empty_like(cache.value_cache)
    c.key_cache[perm] = cache.key_cache
    c.value_cache[perm] = cache.value_cache
    return c


@pytest.mark.parametrize("kind", ["prefill", "decode_splits"])
def test_block_permutation_is_bitwise_invisible(pa, runner, kind):
    print(f"\n[gpu-case] block permutation {kind}", flush=True)
    if kind == "prefill":
        w = W.custom("perm_p", 51, [100, 37, 0, 700], [70, 129, 50, 1], 16, 4, 128, 16,
                     torch.bfloat16, "prefill", window_left=300, softcap=20.0)
        S = None
    else:
        w = W.custom("perm_d", 52, [1, 17, 300, 1024, 4000, 63], [1] * 6, 32, 8, 128, 16,
                     torch.bfloat16, "decode", num_splits=4)
        S = 4
    cache, res = runner.run_workload(w, num_splits=S)
    cb = res[0][0]
    g = torch.Generator().manual_seed(7)
    perm = torch.randperm(w.num_blocks, generator=g).cuda()
    moved = _permuted(runner, cache, perm)
    a = _fresh(cb)
    b = _fresh(cb, block_table=perm[cb.block_table.long()].to(torch.int32).contiguous())
    cache.run(a)
    moved.run(b)
    torch.cuda.synchronize()
    for x, y in zip(_results(a), _results(b)):
        assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x.view(torch.int16),
                           y.view(torch.int32) if y.dtype == torch.float32 else y.view(torch.int16))


def test_future_keys_are_bitwise_invisible(pa, runner):
    print("\n[gpu-case] causal perturbation", flush=True)
    ctx, q = [100, 37, 0], [70, 129, 50]
    w = W.custom("causal_p", 53, ctx, q, 32, 8, 128, 16, torch.bfloat16, "prefill")
    cache, res = runner.run_workload(w)
    cb = res[0][0]
    base = _fresh(cb)
    cache.run(base)
    # overwrite K and V of sequence 1 from position P on (finite values)
    b, P = 1, 37 + 60
    L = ctx[b] + q[b]
    slots = torch.from_numpy(w.slots(b, np.arange(P, L))).cuda()
    g = torch.Generator().manual_seed(9)
    shape = (L - P, w.num_kv_heads, w.head_size)
    kflat = cache.key_cache.view(-1, w.num_kv_heads, w.head_size)
    vflat = cache.value_cache.view(-1, w.num_kv_heads, w.head_size)
    kflat[slots] = (torch.randn(shape, generator=g) * 3).to(w.dtype).cuda()
    vflat[slots] = (torch.randn(shape, generator=g) * 3).to(w.dtype).cuda()
    pert = _fresh(cb)
    cache.run(pert)
    torch.cuda.synchronize()
    cu = np.concatenate([[0], np.cumsum(q)])
    pos = np.concatenate([np.arange(c, c + n) for c, n in zip(ctx, q)])
    seq = np.concatenate([np.full(n, i) for i, n in enumerate(q)])
    same = torch.from_numpy(~((seq == b) & (pos >= P)))
    o0, o1 = base.out.cpu().view(torch.int16), pert.out.cpu().view(torch.int16)
    l0, l1 = base.lse.cpu().view(torch.int32), pert.lse.cpu().view(torch.int32)
    assert torch.equal(o0[same], o1[same])
    assert torch.equal(l0[:, same], l1[:, same])
    changed = ~same
    assert not torch.equal(o0[changed], o1[changed])   # the perturbation is seen where it may be
    assert int(cu[-1]) == o0.shape[0]
