// Host-side launchers of the gfx950 kernels.  Arguments are validated by the
// C-ABI layer before these are called; each returns 0 or -3 (HIP error).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum Dtype { kF16 = 0, kBF16 = 1, kF32 = 2 };

int launch_reshape_and_cache(const void* key, const void* value, int64_t key_stride,
                             int64_t value_stride, void* key_cache, void* value_cache,
                             const int64_t* slots, int64_t num_tokens, int row_elems,
                             hipStream_t stream);

// fp8 (e4m3) cache: in_dtype kF16 / kBF16 inputs, device fp32 scales
int launch_reshape_and_cache_fp8(const void* key, const void* value, int64_t key_stride,
                                 int64_t value_stride, void* key_cache, void* value_cache,
                                 const int64_t* slots, int64_t num_tokens, int row_elems,
                                 Dtype in_dtype, const float* k_scale, const float* v_scale,
                                 hipStream_t stream);

// the query quantiser: out[i] = e4m3 code of input[i] / *scale
int launch_scaled_fp8_quant(void* out, const void* input, const float* scale, int64_t n,
                            Dtype in_dtype, hipStream_t stream);

int launch_merge(void* out, float* out_lse, const void* parts, const float* parts_lse,
                 int num_parts, int64_t num_tokens, int num_heads, int head_size,
                 Dtype parts_dtype, Dtype out_dtype, hipStream_t stream);

struct AttnParams {
  void* out;                    // [T, Hq, D] dtype   (decode S == 1 / prefill)
  float* lse;                   // [Hq, T] or null
  float* part_out;              // decode S > 1: [S, B, Hq, D]
  float* part_lse;              // decode S > 1: [S, Hq, B]
  const void* q;                // [T, Hq, D]
  const void* key_cache;        // [nb, bs, Hkv, D]
  const void* value_cache;
  const int32_t* cu_seqlens_q;  // prefill: [B + 1]
  const int32_t* seq_lens;      // [B]
  const int32_t* block_table;
  int64_t block_table_stride;
  int num_seqs;
  int64_t total_q;
  int max_seqlen_q;
  int max_seqlen_k;
  int num_heads;
  int num_kv_heads;
  int head_size;
  int block_size;
  float scale;
  int causal;
  int window_left;
  float softcap;
  const float* alibi_slopes;
  const float* sinks;  // [Hq] fp32 attention-sink logits or null; split 0 only
  int kv_fp8;          // nonzero: the caches hold fp8 (e4m3) codes
  const float* k_scale;  // fp8 cache: device fp32 scales
  const float* v_scale;
  const float* q_scale;  // non-null: q holds fp8 (e4m3) codes and this is their descale
  // decode with num_splits > 1: non-null merges the splits in the kernel
  // (one int per (sequence, query head), zero on entry, left zero) and
  // writes out / lse; null writes the partials only
  int32_t* split_counters = nullptr;
  int num_splits;
  int key_split;  // prefill only: keys per split (a multiple of 64), 0 = none
  // prefill only: sequence b's queries are [cu[b], cu[b + cu_step]) (0 =
  // step 1) and its key count min(seq_lens[b] - len_sub, len_cap) (len_cap
  // 0 = no cap); bt_cols > 0 bounds the block-table columns read from
  // block_table (which may point into the rows), else block_table_stride
  // does
  int cu_step = 0;
  int len_sub = 0;
  int len_cap = 0;
  int64_t bt_cols = 0;
  Dtype dtype;
};

int launch_decode(const AttnParams& p, hipStream_t stream);

// Fixed per-device scratch of the no-allocation decode entry point: split
// partial results (fp32 outputs, then their LSEs), at most this many bytes.
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
// Device address of the calling thread's current device's scratch array
// (looked up once per device).  Returns 0, or -3 when HIP reports an error.
int noalloc_scratch(void** ptr);

// The timeline trace buffer the kernels write (trace library only; null:
// no tracing).  Set by pa_trace_set, read by the launchers.
uint64_t* trace_buffer();

// host-side rewriting for chunked local attention; returns the number of
// virtual sequences (outputs NULL: count only)
int local_virtual_batches(int chunk, int block_size, const int32_t* qsl, const int32_t* seq_lens,
                          int num_seqs, const int32_t* block_table, int64_t bt_stride,
                          int bt_cols, int32_t* q_local, int32_t* cu_q_local, int32_t* k_local,
                          int32_t* bt_local);

int launch_check_indices(const int64_t* slot_mapping, int64_t num_tokens,
                         const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens,
                         int num_seqs, int64_t num_blocks, int block_size, int32_t* counts,
                         hipStream_t stream);
int launch_prefill(const AttnParams& p, hipStream_t stream);
// two independent prefill problems of the same variant (dtype, head size,
// cache and query types, softcap; no ALiBi) in one launch, p0's workgroups
// first; returns 1 without launching when they cannot share one (the
// caller then launches them one by one), else 0 or a negative code
int launch_prefill_pair(const AttnParams& p0, const AttnParams& p1, hipStream_t stream);
// prefix-shared causal prefill (p.causal, no window / ALiBi): parts_out
// [max_prefix_splits + 1, T, Hq, D] in p.dtype, parts_lse
// [max_prefix_splits + 1, Hq, T], shared by the prefix and suffix passes
// host: the calibrated time comparison behind pa_use_cascade (decode batches)
bool cascade_beats_split_decode(int prefix, const int32_t* seq_lens, int num_reqs, int num_heads,
                                int num_kv_heads, int head_size, int kv_elem_bytes);
int launch_cascade(const AttnParams& p, int prefix, int max_prefix_splits, void* parts_out,
                   float* parts_lse, hipStream_t stream);

}  // namespace pa
