"""Plain CPU definition of attention over a paged KV cache (float64).

TEST INFRASTRUCTURE ONLY — see the package docstring.  No blocking, fusion
or reordering beyond the definitions below; one library primitive (matrix
product) is used per contraction.

Notation (as on the pages):
  key_cache / value_cache : [num_blocks, block_size, num_kv_heads, head_size],
      the two halves of the (2, num_blocks, block_size, num_kv_heads,
      head_size) cache  [vLLM flash_attn.py (e2f56c3),
      FlashAttentionBackend.get_kv_cache_shape; FlashAttentionImpl.forward
      "kv_cache.unbind(0)"].
  block_table[b, i] : physical block holding logical block i of sequence b
      [Aphrodite flash_attn.py, FlashAttentionMetadata "block_tables"].
  seq_len L_b = context_len C_b + query_len; the query tokens are the last
      query_len positions of the sequence  [vLLM flash_attn.py (e2f56c3),
      FlashAttentionMetadata context_len/seq_len/query_len diagram].
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import torch

_F64 = torch.float64
_NEG_INF = float("-inf")


def scatter(key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor,
            key_cache: torch.Tensor, value_cache: torch.Tensor) -> None:
    """Write token rows of K and V into their cache slots (bitwise copy).

    For every i < len(slot_mapping): slot s = slot_mapping[i]; a negative s is
    padding and is skipped; otherwise row i lands at
    (block s // block_size, offset s % block_size).  The number of tokens is
    the length of slot_mapping, not of key/value, which may be padded.
    [vLLM flash_attn.py (e2f56c3), FlashAttentionImpl.forward, the
    reshape_and_cache_flash call and its padding note; vLLM 0.9.0.1 flash_attn
    API docs, FlashAttentionMetadataBuilder.build, slot_mapping filled with -1
    past the actual tokens.]
    """
    bs = key_cache.shape[1]
    for i, s in enumerate(slot_mapping.tolist()):
        if s < 0:
            continue
        blk, off = divmod(int(s), bs)
        key_cache[blk, off] = key[i]
        value_cache[blk, off] = value[i]


def gather_sequence(cache: torch.Tensor, block_table_row: torch.Tensor,
                    seq_len: int) -> torch.Tensor:
    """Logical rows [0, seq_len) of one sequence: key j sits at
    (block_table_row[j // block_size], j % block_size).  Returns
    [seq_len, num_kv_heads, head_size] widened exactly to float64.
    [Aphrodite flash_attn.py, FlashAttentionMetadata "block_tables" note.]
    """
    bs = cache.shape[1]
    j = torch.arange(seq_len, dtype=torch.long)
    blocks = block_table_row.to(torch.long)[j // bs]
    return cache[blocks, j % bs].to(_F64)


def _visible(q_pos: torch.Tensor, seq_len: int, causal: bool, window_left: int,
             key_range: Optional[Sequence[int]], attn_chunk_size: int = 0) -> torch.Tensor:
    """Boolean [n_queries, seq_len]: may query at position p see key j?

    * j < seq_len always;
    * causal: j <= p (queries are the last positions, so the mask is
      bottom-right aligned);
    * window_left >= 0: j >= p - window_left, i.e. at most window_left + 1
      keys including the query itself (a window w is passed as w - 1)
      [vLLM flash_attn.py (e2f56c3), FlashAttentionImpl.__init__,
      sliding_window -> (sliding_window - 1, 0)];
    * key_range (lo, hi): lo <= j < hi — the key partition of one split;
    * attn_chunk_size > 0 (chunked local attention): j lies in p's chunk,
      (p // attn_chunk_size) * attn_chunk_size <= j — the positions are cut
      into chunks of that many tokens and a query sees only its own chunk
      [vLLM flash_attn.py (v0.9.0.1 docs), make_local_attention_virtual_
      batches: each query's keys start at its local attention block].
    """
    j = torch.arange(seq_len, dtype=torch.long)[None, :]
    p = q_pos[:, None]
    vis = torch.ones(q_pos.numel(), seq_len, dtype=torch.bool)
    if causal:
        vis &= j <= p
    if window_left >= 0:
        vis &= j >= p - window_left
    if key_range is not None:
        lo, hi = key_range
        vis &= (j >= lo) & (j < hi)
    if attn_chunk_size > 0:
        vis &= j >= torch.div(p, attn_chunk_size, rounding_mode="floor") * attn_chunk_size
    return vis


def attend(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
           cu_seqlens_q: Sequence[int], seq_lens: Sequence[int],
           block_table: torch.Tensor, scale: float, causal: bool = True,
           window_left: int = -1, softcap: float = 0.0,
           alibi_slopes: Optional[torch.Tensor] = None,
           key_ranges: Optional[Sequence[Sequence[int]]] = None,
           attn_chunk_size: int = 0, sinks: Optional[torch.Tensor] = None):
    """Varlen attention over the paged cache; returns (out, lse) in float64.
    attn_chunk_size > 0 restricts each query to its own chunk of positions
    (chunked local attention, see ``_visible``).

    sinks (attention sinks, one fp32 logit per query head): the pages pass
    them to the kernels as ``s_aux`` and note that they can be folded into
    a log-sum-exp [vLLM flash_attn.py (e2f56c3), FlashAttentionImpl.__init__
    sinks of shape [num_heads]; cascade_attention, s_aux incorporated into
    the prefix LSE], without printing the formula.  Reading used here: the
    sink of head h is one more logit in the softmax denominator that carries
    no value,
        out = sum_j e^{s_j} V_j / (sum_j e^{s_j} + e^{sink_h}),
        lse = ln(sum_j e^{s_j} + e^{sink_h}),
    so a query that sees no key gets out = 0 and lse = sink_h.

    q : [total_q, num_heads, head_size]; queries of sequence b are rows
        cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (cu_seqlens_q is the running
        sum of query lengths)  [Aphrodite flash_attn.py,
        FlashAttentionMetadata "query_start_loc"].
    seq_lens[b] : keys of sequence b (= seqused_k)  [vLLM flash_attn.py
        (e2f56c3), FlashAttentionImpl.forward, flash_attn_varlen_func call].

    For query row t of sequence b at position p = C_b + t and query head h,
    using KV head g = h // (num_heads // num_kv_heads)  (consecutive groups of
    num_queries_per_kv query heads share one KV head):
        s_j = scale * <q, K_j>
        s_j = softcap * tanh(s_j / softcap)           if softcap > 0
        s_j = s_j - slope_h * |p - j|                 if ALiBi slopes given
        softmax over the visible j (see _visible), out = sum_j P_j V_j,
        lse = m + ln(sum_j exp(s_j - m))  (natural log).
    A query that sees no key gets out = 0 and lse = -inf.
    softcap 0 means off  [vLLM flash_attn.py (e2f56c3), FlashAttentionImpl
    .__init__ logits_soft_cap note]; alibi_slopes are one fp32 slope per
    query head [same, alibi_slopes]; LSE is natural-log with layout
    [num_heads, total_q]  [vLLM flash_attn.py (e2f56c3), _forward_with_dcp
    "LSE in shape [H, B]"; FlashInfer flashinfer.py (Nvidia-Optimization-
    Stack-VLLM), log2_lse_to_ln conversion before merge_attn_states].
    """
    total_q, num_heads, head_size = q.shape
    num_kv_heads = key_cache.shape[2]
    assert num_heads % num_kv_heads == 0
    group = num_heads // num_kv_heads
    out = torch.zeros(total_q, num_heads, head_size, dtype=_F64)
    lse = torch.full((num_heads, total_q), _NEG_INF, dtype=_F64)
    for b in range(len(seq_lens)):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        n_q, L = q1 - q0, int(seq_lens[b])
        if n_q == 0 or L == 0:
            # no keys: the rows keep out = 0 and lse = -inf (or the sink)
            if sinks is not None:
                for h in range(num_heads):
                    lse[h, q0:q1] = float(sinks[h])
            continue
        ctx = L - n_q
        q_pos = ctx + torch.arange(n_q, dtype=torch.long)
        vis = _visible(q_pos, L, causal, window_left,
                       None if key_ranges is None else key_ranges[b], attn_chunk_size)
        K = gather_sequence(key_cache, block_table[b], L)
        V = gather_sequence(value_cache, block_table[b], L)
        dist = (q_pos[:, None] - torch.arange(L)[None, :]).abs().to(_F64)
        any_vis = vis.any(dim=1)
        for h in range(num_heads):
            g = h // group
            s = scale * (q[q0:q1, h].to(_F64) @ K[:, g].T)
            if softcap > 0:
                s = softcap * torch.tanh(s / softcap)
            if alibi_slopes is not None:
                s = s - float(alibi_slopes[h]) * dist
            s = torch.where(vis, s, torch.full_like(s, _NEG_INF))
            if sinks is not None:
                sk = torch.full((n_q, 1), float(sinks[h]), dtype=_F64)
                mt = torch.maximum(s.max(dim=1, keepdim=True).values, sk)
                mt = torch.where(torch.isfinite(mt), mt, torch.zeros_like(mt))
                w = torch.exp(s - mt)
                den = w.sum(dim=1, keepdim=True) + torch.exp(sk - mt)
                o = (w @ V[:, g]) / torch.where(den > 0, den, torch.ones_like(den))
                out[q0:q1, h] = torch.where(den > 0, o, torch.zeros_like(o))
                lse[h, q0:q1] = torch.where(den > 0, mt + torch.log(den),
                                            torch.full_like(den, _NEG_INF))[:, 0]
                continue
            m = s.max(dim=1, keepdim=True).values
            m = torch.where(torch.isfinite(m), m, torch.zeros_like(m))
            w = torch.exp(s - m)                      # exp(-inf) = 0
            l = w.sum(dim=1, keepdim=True)
            o = (w @ V[:, g]) / torch.where(l > 0, l, torch.ones_like(l))
            out[q0:q1, h] = torch.where(any_vis[:, None], o, torch.zeros_like(o))
            lse[h, q0:q1] = torch.where(any_vis, (m + torch.log(l))[:, 0],
                                        torch.full((n_q,), _NEG_INF, dtype=_F64))
    return out, lse


def decode(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
           seq_lens: Sequence[int], block_table: torch.Tensor, scale: float,
           window_left: int = -1, softcap: float = 0.0,
           alibi_slopes: Optional[torch.Tensor] = None,
           key_ranges=None, sinks: Optional[torch.Tensor] = None):
    """Single-token decode: q [num_seqs, num_heads, head_size], one query per
    sequence at position L_b - 1, which sees every key up to itself.
    [Aphrodite flash_attn.py, FlashAttentionImpl.forward, decode through
    flash_attn_with_kvcache with cache_seqlens.]  Returns (out, lse)."""
    B = len(seq_lens)
    cu = list(range(B + 1))
    return attend(q, key_cache, value_cache, cu, seq_lens, block_table, scale,
                  causal=True, window_left=window_left, softcap=softcap,
                  alibi_slopes=alibi_slopes, key_ranges=key_ranges, sinks=sinks)


def split_bounds(seq_len: int, num_splits: int, block_size: int,
                 max_seq_len: Optional[int] = None):
    """Key partition of one sequence for split-KV decode.

    The pages give the partial-result buffers and their shape
    [num_splits, num_heads, num_tokens, head_size] but not the boundaries
    [vLLM flash_attn.py (e2f56c3), FlashAttentionMetadataBuilder, the
    max_num_splits note], and another backend sizes its KV splits by a
    fixed number of keys [vLLM flashinfer.py, FlashInferMetadataBuilder,
    decode_fixed_split_size / fixed_split_size].  Reading used here: every
    sequence of a batch is cut into the same fixed-size, block-aligned
    chunks sized from the batch bound max_seq_len,
        chunk = block_size * ceil(ceil(max_seq_len / S) / block_size),
    split p covers [p * chunk, min((p + 1) * chunk, L)) (possibly empty),
    and the last split also takes any keys past S * chunk (a loose bound
    still covers the sequence).  With max_seq_len = L this is the even
    division of one sequence.
    """
    if max_seq_len is None:
        max_seq_len = seq_len
    per = -(-max_seq_len // num_splits)
    chunk = block_size * (-(-per // block_size))
    out = []
    for p in range(num_splits):
        lo = min(p * chunk, seq_len)
        hi = seq_len if p == num_splits - 1 else min((p + 1) * chunk, seq_len)
        out.append((lo, hi))
    return out


def decode_splits(q, key_cache, value_cache, seq_lens, block_table, scale,
                  num_splits: int, window_left: int = -1, softcap: float = 0.0,
                  alibi_slopes=None, max_seq_len: Optional[int] = None, sinks=None):
    """Partial decode results for each split: parts_out
    [S, num_seqs, num_heads, head_size] and parts_lse [S, num_heads, num_seqs]
    (float64).  An empty split yields out = 0 and lse = -inf.  The splits
    are sized from max_seq_len (default: the longest sequence).  Attention
    sinks, if any, join split 0 only, so the merged result counts each
    once (as the cascade folds them into its prefix part)."""
    block_size = key_cache.shape[1]
    if max_seq_len is None:
        max_seq_len = max(int(L) for L in seq_lens)
    bounds = [split_bounds(int(L), num_splits, block_size, max_seq_len) for L in seq_lens]
    outs, lses = [], []
    for p in range(num_splits):
        o, l = decode(q, key_cache, value_cache, seq_lens, block_table, scale,
                      window_left, softcap, alibi_slopes,
                      key_ranges=[bounds[b][p] for b in range(len(seq_lens))],
                      sinks=sinks if p == 0 else None)
        outs.append(o)
        lses.append(l)
    return torch.stack(outs), torch.stack(lses)


def merge(parts_out: torch.Tensor, parts_lse: torch.Tensor):
    """Combine S partial attention states by their log-sum-exp.

    parts_out [S, T, H, D], parts_lse [S, H, T] (natural log).  Per (t, h):
        M = max_p lse_p,  w_p = exp(lse_p - M),
        out = sum_p w_p out_p / sum_p w_p,  lse = M + ln(sum_p w_p).
    If every part is -inf (nothing visible anywhere) out = 0, lse = -inf.
    The pages call the two-part case merge_attn_states(out, a_out, a_lse,
    b_out, b_lse)  [vLLM flash_attn.py (e2f56c3), cascade_attention and
    _forward_with_dcp]; the S-part form is the same weighted average.
    """
    o = parts_out.to(_F64)
    l = parts_lse.to(_F64)
    S, T, H, D = o.shape
    M = l.max(dim=0).values                                 # [H, T]
    finite = torch.isfinite(M)
    Msafe = torch.where(finite, M, torch.zeros_like(M))
    w = torch.exp(l - Msafe[None])                          # [S, H, T]
    wsum = w.sum(dim=0)                                     # [H, T]
    wt = w.permute(0, 2, 1)[..., None]                      # [S, T, H, 1]
    num = (wt * o).sum(dim=0)                               # [T, H, D]
    den = torch.where(finite, wsum, torch.ones_like(wsum)).T[..., None]
    out = torch.where(finite.T[..., None], num / den, torch.zeros_like(num))
    lse = torch.where(finite, Msafe + torch.log(torch.where(finite, wsum, torch.ones_like(wsum))),
                      torch.full_like(M, _NEG_INF))
    return out, lse


def cascade(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
            cu_seqlens_q: Sequence[int], seq_lens: Sequence[int], block_table: torch.Tensor,
            scale: float, common_prefix_len: int, softcap: float = 0.0, sinks=None):
    """Causal varlen attention of a batch whose sequences share their first
    common_prefix_len keys, taken the cascade way [vLLM flash_attn.py
    (e2f56c3), cascade_attention]:

    1. every query of the batch against the shared prefix keys, as one
       sequence of all the queries over block_table[:1], non-causal (the
       queries all come after the prefix, so none of its keys is masked);
    2. each sequence's queries against the keys after the prefix, causal,
       with seq_lens - common_prefix_len keys through
       block_table[:, common_prefix_len / block_size:];
    3. the two partial states merged by their log-sum-exp (``merge``).

    The page asserts no ALiBi and no sliding window for it, a prefix that is
    a positive multiple of the block size, and (implicitly) that every
    query comes after the prefix; those preconditions are asserted here.
    Returns (out, lse) like ``attend``.
    """
    block_size = key_cache.shape[1]
    assert common_prefix_len > 0 and common_prefix_len % block_size == 0
    n = common_prefix_len // block_size
    total_q = q.shape[0]
    for b in range(len(seq_lens)):
        q_len = int(cu_seqlens_q[b + 1]) - int(cu_seqlens_q[b])
        assert int(seq_lens[b]) - q_len >= common_prefix_len, "queries must follow the prefix"
        assert torch.equal(block_table[b, :n], block_table[0, :n]), "prefix blocks must be shared"
    # attention sinks join the prefix part (the page folds s_aux into the
    # prefix LSE)
    pre_out, pre_lse = attend(q, key_cache, value_cache, [0, total_q], [common_prefix_len],
                              block_table[:1], scale, causal=False, softcap=softcap, sinks=sinks)
    suf_out, suf_lse = attend(q, key_cache, value_cache, cu_seqlens_q,
                              [int(L) - common_prefix_len for L in seq_lens], block_table[:, n:],
                              scale, causal=True, softcap=softcap)
    return merge(torch.stack([pre_out, suf_out]), torch.stack([pre_lse, suf_lse]))
