// paged_attn_cascade: causal varlen attention of a batch whose sequences
// share their first common_prefix_len keys, computed the cascade way (vLLM
// flash_attn.py (e2f56c3), cascade_attention): the shared prefix is read
// once for the whole batch instead of once per sequence.
//
//   1. all T queries as one sequence over the prefix keys (block_table row
//      0), non-causal — every query comes after the prefix — split over the
//      prefix keys when there are few queries;
//   2. each sequence's queries over its keys after the prefix, causal,
//      through block_table + prefix_blocks with lengths seq_lens - prefix,
//      split over those keys when there are few sequences;
//   3. merge_attn_states of the prefix parts and the suffix parts.
//
// Steps 1-2 are one launch of the prefill kernel (two problems in one grid)
// and step 3 the merge kernel.  The prefix pass reads its one sequence's
// bounds as cu_seqlens_q[0], cu_seqlens_q[B] and min(seq_lens[0], prefix);
// the suffix pass subtracts the prefix from seq_lens as it reads them; so
// no device-side lengths are prepared.
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

size_t elem_bytes(Dtype t) { return t == kF32 ? 4 : 2; }

// Keys per split (a multiple of 64) when a pass over up to `keys` keys is
// split into at most `max_parts` parts so that its grid of `wgs` workgroups
// grows to about 512; 0 = no split.  *parts receives the number of parts.
int key_split_for(int64_t wgs, int keys, int max_parts, int* parts) {
  const int tiles = (keys + 63) / 64;
  int s = static_cast<int>((512 + wgs - 1) / wgs);
  s = s > max_parts ? max_parts : s;
  s = s > tiles ? tiles : s;
  s = s < 1 ? 1 : s;
  const int ks = 64 * ((tiles + s - 1) / s);
  *parts = (keys + ks - 1) / ks;
  return *parts > 1 ? ks : 0;
}

}  // namespace

int launch_cascade(const AttnParams& p, int prefix, int max_prefix_splits, void* parts_out,
                   float* parts_lse, hipStream_t stream) {
  const int64_t T = p.total_q;
  const int budget = max_prefix_splits + 1;  // parts the workspaces hold
  const int tok_per_tile = 128 / (p.num_heads / p.num_kv_heads);  // 128 MFMA rows per tile

  // Suffix pass: with few sequences its grid has only Hkv * (T / tokens-per-
  // tile + B) workgroups, each walking its sequence's whole suffix one tile
  // at a time, so the longest suffix sets the pass's time; its keys are then
  // split too, into at most 4 parts (more measured slower: the extra parts
  // cost the merge and the prefix pass more than they save), leaving the
  // prefix at least one.
  const int suf_keys = p.max_seqlen_k - prefix;
  int suf_parts = 1;
  const int suf_split = key_split_for((int64_t)p.num_kv_heads * (T / tok_per_tile + p.num_seqs),
                                      suf_keys, budget - 1 < 4 ? budget - 1 : 4, &suf_parts);

  // Prefix pass: every query over the shared prefix, non-causal.  With few
  // queries (a decode batch) its grid would have only Hkv * T / tokens-per-
  // tile workgroups, so the prefix keys are split (in 64-key tiles) until
  // the pass has about 512 workgroups, in the parts the suffix left.
  int pre_parts = 1;
  const int pre_split = key_split_for((int64_t)p.num_kv_heads * ((T + tok_per_tile - 1) / tok_per_tile),
                                      prefix, budget - suf_parts, &pre_parts);

  AttnParams pre = p;
  pre.out = parts_out;
  pre.lse = parts_lse;
  // one sequence: queries [cu[0], cu[B]) = [0, T), keys min(seq_lens[0],
  // prefix) = prefix
  pre.cu_step = p.num_seqs;
  pre.len_cap = prefix;
  pre.num_seqs = 1;
  pre.max_seqlen_q = static_cast<int>(T);
  pre.max_seqlen_k = prefix;
  pre.causal = 0;
  pre.key_split = pre_split;  // sinks (if any) join split 0

  // Suffix pass: each sequence over its own keys after the prefix, causal,
  // into parts pre_parts ..
  AttnParams suf = p;
  suf.out = static_cast<char*>(parts_out) + pre_parts * T * p.num_heads * p.head_size * elem_bytes(p.dtype);
  suf.lse = parts_lse + pre_parts * T * p.num_heads;
  suf.len_sub = prefix;
  suf.block_table = p.block_table + prefix / p.block_size;
  suf.bt_cols = p.block_table_stride - prefix / p.block_size;
  suf.max_seqlen_k = suf_keys;
  suf.causal = 1;
  suf.key_split = suf_split;
  suf.sinks = nullptr;  // counted once, in the prefix part

  // Both passes in one launch, the suffix pass's workgroups first: the
  // prefix pass's short workgroups then fill the slots the suffix pass's
  // uneven ones free (one launch by one when they cannot share a grid).
  int rc = launch_prefill_pair(suf, pre, stream);
  if (rc == 1) {
    rc = launch_prefill(pre, stream);
    if (rc == 0) rc = launch_prefill(suf, stream);
  }
  if (rc != 0) return rc;

  return launch_merge(p.out, p.lse, parts_out, parts_lse, pre_parts + suf_parts, T, p.num_heads,
                      p.head_size, p.dtype, p.dtype, stream);
}

// Cascade decision for a decode batch (one query per request), from time
// models of the two paths calibrated on one MI355X (32 query / 8 KV heads of
// 128, bf16, block 16; requests 8..128, shared prefixes 256..8192 keys, own
// suffixes 1..1024 keys; non-negative least squares on relative error).
// Bytes are K and V of every KV head; times in microseconds.
//   plain split decode + merge: a fixed cost, the K/V bytes each key is
//     read for once (HBM), and the re-reads of the shared prefix by the
//     other requests (served mostly by the caches);
//   cascade: a fixed cost (two launches), the prefix pass's MFMA work,
//     the prefix bytes, the suffix bytes, and a cost per request (the
//     suffix pass's workgroups, the merge's rows).  The longest suffix per
//     suffix part was a candidate term too; the fit gives it no weight in
//     the measured range (the suffix split and the prefix pass sharing the
//     launch hide it).
// On every measured batch the cascade was the faster path, so within that
// range the decision is the support checks'.  Returns true when the
// modelled cascade time is the lower one.
bool cascade_beats_split_decode(int prefix, const int32_t* seq_lens, int num_reqs, int num_heads,
                                int num_kv_heads, int head_size, int kv_elem_bytes) {
  const double row = (double)num_kv_heads * head_size * 2 * kv_elem_bytes;  // bytes per key
  double suf_sum = 0;
  for (int b = 0; b < num_reqs; ++b) suf_sum += seq_lens[b] > prefix ? seq_lens[b] - prefix : 0;
  const double MB = 1e6;
  const double unique = (prefix + suf_sum) * row / MB;
  const double reread = (double)(num_reqs - 1) * prefix * row / MB;
  const double gflop = 4.0 * head_size * num_heads * (double)num_reqs * prefix / 1e9;
  const double t_plain = 15.585 + 0.17556 * unique + 0.10298 * reread;
  const double t_cascade = 14.157 + 0.95417 * gflop + 0.17501 * suf_sum * row / MB +
                           0.17287 * prefix * row / MB + 0.066596 * num_reqs;
  return t_cascade < t_plain;
}

}  // namespace pa
