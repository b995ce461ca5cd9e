// paged_attn_cascade: causal varlen attention of a batch whose sequences
// share their first common_prefix_len keys, computed the cascade way (vLLM
// flash_attn.py (e2f56c3), cascade_attention): the shared prefix is read
// once for the whole batch instead of once per sequence.
//
//   1. all T queries as one sequence over the prefix keys (block_table row
//      0), non-causal — every query comes after the prefix — split over the
//      prefix keys when there are few queries;
//   2. each sequence's queries over its keys after the prefix, causal,
//      through block_table + prefix_blocks with lengths seq_lens - prefix;
//   3. merge_attn_states of the prefix parts and the suffix part.
//
// Steps 1-2 are the prefill kernel and step 3 the merge kernel; a small
// kernel first writes the device-side lengths the two prefill launches
// read (cu = {0, T}, {prefix}, and the suffix lengths) into the caller's
// integer workspace.
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

__global__ __launch_bounds__(256) void cascade_setup_kernel(const int32_t* seq_lens, int num_seqs,
                                                            int total_q, int prefix,
                                                            int32_t* ints) {
  const int i0 = blockIdx.x * blockDim.x + threadIdx.x;
  if (i0 == 0) {
    ints[0] = 0;
    ints[1] = total_q;
    ints[2] = prefix;
  }
  for (int i = i0; i < num_seqs; i += gridDim.x * blockDim.x) ints[3 + i] = seq_lens[i] - prefix;
}

size_t elem_bytes(Dtype t) { return t == kF32 ? 4 : 2; }

}  // namespace

int launch_cascade(const AttnParams& p, int prefix, int max_prefix_splits, void* parts_out,
                   float* parts_lse, int32_t* ints, hipStream_t stream) {
  const int64_t T = p.total_q;
  const unsigned grid = static_cast<unsigned>(p.num_seqs / 256 + 1 > 1024 ? 1024 : p.num_seqs / 256 + 1);
  hipLaunchKernelGGL(cascade_setup_kernel, dim3(grid), dim3(256), 0, stream, p.seq_lens,
                     p.num_seqs, static_cast<int>(T), prefix, ints);
  if (hipGetLastError() != hipSuccess) return -3;

  // Prefix pass: every query over the shared prefix, non-causal.  With few
  // queries (a decode batch) its grid would have only Hkv * T / tokens-per-
  // tile workgroups, so the prefix keys are split (in 64-key tiles) until
  // the pass has about 512 workgroups; split z writes part z.
  const int tok_per_tile = 128 / (p.num_heads / p.num_kv_heads);  // 128 MFMA rows per tile
  const int64_t wgs = (int64_t)p.num_kv_heads * ((T + tok_per_tile - 1) / tok_per_tile);
  const int tiles = (prefix + 63) / 64;
  int splits = static_cast<int>((512 + wgs - 1) / wgs);
  splits = splits < 1 ? 1 : splits;
  splits = splits > max_prefix_splits ? max_prefix_splits : splits;
  splits = splits > tiles ? tiles : splits;
  const int key_split = 64 * ((tiles + splits - 1) / splits);
  splits = (prefix + key_split - 1) / key_split;

  AttnParams pre = p;
  pre.out = parts_out;
  pre.lse = parts_lse;
  pre.cu_seqlens_q = ints;
  pre.seq_lens = ints + 2;
  pre.num_seqs = 1;
  pre.max_seqlen_q = static_cast<int>(T);
  pre.max_seqlen_k = prefix;
  pre.causal = 0;
  pre.key_split = splits > 1 ? key_split : 0;  // sinks (if any) join split 0
  int rc = launch_prefill(pre, stream);
  if (rc != 0) return rc;

  // Suffix pass: each sequence over its own keys after the prefix, causal,
  // into part `splits`
  AttnParams suf = p;
  suf.out = static_cast<char*>(parts_out) + splits * T * p.num_heads * p.head_size * elem_bytes(p.dtype);
  suf.lse = parts_lse + splits * T * p.num_heads;
  suf.seq_lens = ints + 3;
  suf.block_table = p.block_table + prefix / p.block_size;
  suf.max_seqlen_k = p.max_seqlen_k - prefix;
  suf.causal = 1;
  suf.key_split = 0;
  suf.sinks = nullptr;  // counted once, in the prefix part
  rc = launch_prefill(suf, stream);
  if (rc != 0) return rc;

  return launch_merge(p.out, p.lse, parts_out, parts_lse, splits + 1, T, p.num_heads,
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
//   cascade: a fixed cost (four launches), the prefix pass's MFMA work,
//     the prefix bytes, the suffix bytes, and the longest suffix (the suffix
//     pass runs one query per sequence, so its time follows its longest
//     item).
// Returns true when the modelled cascade time is the lower one.
bool cascade_beats_split_decode(int prefix, const int32_t* seq_lens, int num_reqs, int num_heads,
                                int num_kv_heads, int head_size, int kv_elem_bytes) {
  const double row = (double)num_kv_heads * head_size * 2 * kv_elem_bytes;  // bytes per key
  double suf_sum = 0, suf_max = 0;
  for (int b = 0; b < num_reqs; ++b) {
    const double s = seq_lens[b] > prefix ? seq_lens[b] - prefix : 0;
    suf_sum += s;
    suf_max = s > suf_max ? s : suf_max;
  }
  const double MB = 1e6;
  const double unique = (prefix + suf_sum) * row / MB;
  const double reread = (double)(num_reqs - 1) * prefix * row / MB;
  const double gflop = 4.0 * head_size * num_heads * (double)num_reqs * prefix / 1e9;
  const double t_plain = 14.702 + 0.17726 * unique + 0.10315 * reread;
  const double t_cascade = 20.284 + 1.1570 * gflop + 0.15095 * suf_sum * row / MB +
                           3.3735 * suf_max * row / MB + 0.14465 * prefix * row / MB;
  return t_cascade < t_plain;
}

}  // namespace pa
