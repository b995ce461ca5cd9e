// C ABI of libpagedattn.so (declared in include/paged_attn.h): host-side
// argument validation, then one kernel launch on the caller's stream.
// Validation mirrors the checks the backends make before calling their
// kernels (vLLM flash_attn.py (e2f56c3): block_size multiple of 16 in
// get_kv_cache_shape, fp16/bf16 in supported_dtypes, output buffer required
// in FlashAttentionImpl.forward; vLLM 0.9.0.1 flash_attn API docs:
// num_heads divisible by num_kv_heads).  Nothing is enqueued when a check
// fails.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include <atomic>

#include "../../include/paged_attn.h"
#include "common.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return PA_OK;
}

int hip_result(int rc, const char* what) {
  if (rc == 0) return ok();
  return fail(PA_ERR_HIP, "%s: kernel launch failed: %s", what,
              hipGetErrorString(hipGetLastError()));
}

bool is_16bit(pa_dtype_t t) { return t == PA_F16 || t == PA_BF16; }

// shape checks shared by every entry point that touches the cache
int check_cache_shape(const char* fn, int block_size, int num_kv_heads, int head_size,
                      pa_dtype_t dtype) {
  if (!is_16bit(dtype))
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype must be PA_F16 or PA_BF16 (got %d)", fn, (int)dtype);
  if (block_size <= 0 || block_size % 16 != 0)
    return fail(PA_ERR_INVALID, "%s: block_size must be a positive multiple of 16 (got %d)", fn,
                block_size);
  if (block_size > 256)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size above 256 is not supported (got %d)", fn,
                block_size);
  if (num_kv_heads <= 0)
    return fail(PA_ERR_INVALID, "%s: num_kv_heads must be positive (got %d)", fn, num_kv_heads);
  if (head_size != 64 && head_size != 128 && head_size != 256)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_size must be 64, 128 or 256 (got %d)", fn, head_size);
  return PA_OK;
}

int check_attn_common(const char* fn, int num_seqs, int num_heads, int num_kv_heads,
                      int head_size, int block_size, int64_t num_blocks, float scale,
                      int window_left, float softcap, pa_dtype_t dtype, const void* q,
                      const void* kc, const void* vc, const int32_t* seq_lens,
                      const int32_t* block_table, int64_t bt_stride) {
  int rc = check_cache_shape(fn, block_size, num_kv_heads, head_size, dtype);
  if (rc != PA_OK) return rc;
  if (num_seqs < 0) return fail(PA_ERR_INVALID, "%s: num_seqs must be >= 0", fn);
  if (num_heads <= 0 || num_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID, "%s: num_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                fn, num_heads, num_kv_heads);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID, "%s: scale must be finite", fn);
  if (window_left < -1) return fail(PA_ERR_INVALID, "%s: window_left must be >= -1", fn);
  if (!(softcap >= 0.0f) || !std::isfinite(softcap))
    return fail(PA_ERR_INVALID, "%s: softcap must be finite and >= 0 (0 = off)", fn);
  if (num_seqs > 0) {
    if (q == nullptr || kc == nullptr || vc == nullptr || seq_lens == nullptr ||
        block_table == nullptr)
      return fail(PA_ERR_INVALID, "%s: NULL input pointer", fn);
    if (bt_stride <= 0) return fail(PA_ERR_INVALID, "%s: block_table_stride must be positive", fn);
    if (num_blocks <= 0) return fail(PA_ERR_INVALID, "%s: num_blocks must be positive", fn);
  }
  return PA_OK;
}

// the cache element type: the 16-bit dtype itself, or fp8 codes with their
// device scales
int check_kv(const char* fn, pa_dtype_t dtype, pa_dtype_t kv_cache_dtype, const float* k_scale,
             const float* v_scale, bool fp8_supported) {
  if (kv_cache_dtype == dtype) return PA_OK;
  if (kv_cache_dtype != PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "%s: kv_cache_dtype must be dtype or PA_FP8_E4M3 (got %d)",
                fn, (int)kv_cache_dtype);
  if (!fp8_supported)
    return fail(PA_ERR_UNSUPPORTED, "%s: an fp8 cache is not supported by this entry point", fn);
  if (k_scale == nullptr || v_scale == nullptr)
    return fail(PA_ERR_INVALID, "%s: an fp8 cache needs k_scale and v_scale", fn);
  return PA_OK;
}

// An fp8 query (q_scale non-null: q holds e4m3 codes, q_scale their
// descale) comes with an fp8 cache, as on the pages: the query is quantised
// only when the cache is.
int check_q8(const char* fn, pa_dtype_t kv_cache_dtype, const float* q_scale) {
  if (q_scale != nullptr && kv_cache_dtype != PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "%s: an fp8 query (q_scale) needs an fp8 cache", fn);
  return PA_OK;
}

// Checks shared by the decode entry points (paged_attn_decode and its
// no-allocation variant).
int check_decode(const char* fn, int num_seqs, int max_seq_len, int num_heads, int num_kv_heads,
                 int head_size, int block_size, int64_t num_blocks, float scale, int window_left,
                 float softcap, int num_splits, pa_dtype_t dtype, pa_dtype_t kv_cache_dtype,
                 const float* k_scale, const float* v_scale, const float* q_scale, const void* q,
                 const void* key_cache, const void* value_cache, const int32_t* seq_lens,
                 const int32_t* block_table, int64_t block_table_stride) {
  int rc = check_attn_common(fn, num_seqs, num_heads, num_kv_heads, head_size, block_size,
                             num_blocks, scale, window_left, softcap, dtype, q, key_cache,
                             value_cache, seq_lens, block_table, block_table_stride);
  if (rc != PA_OK) return rc;
  rc = check_kv(fn, dtype, kv_cache_dtype, k_scale, v_scale, true);
  if (rc != PA_OK) return rc;
  rc = check_q8(fn, kv_cache_dtype, q_scale);
  if (rc != PA_OK) return rc;
  if (num_splits < 1 || num_splits > 256)
    return fail(PA_ERR_INVALID, "%s: num_splits must be in [1, 256] (got %d)", fn, num_splits);
  if (num_heads / num_kv_heads > 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: more than 128 query heads per KV head", fn);
  // work items (KV heads x groups of 16 query heads x sequences x splits)
  // form a one-dimensional grid
  if ((int64_t)num_kv_heads * ((num_heads / num_kv_heads + 15) / 16) * num_seqs * num_splits >
      INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "%s: too many work items for one grid", fn);
  if (max_seq_len < 0) return fail(PA_ERR_INVALID, "%s: max_seq_len must be >= 0", fn);
  if (max_seq_len >= (1 << 24))
    return fail(PA_ERR_UNSUPPORTED, "%s: sequences of 2^24 keys or more are not supported", fn);
  return PA_OK;
}

pa::AttnParams decode_params(void* out, float* lse, float* part_out, float* part_lse,
                             const void* q, const void* key_cache, const void* value_cache,
                             const int32_t* seq_lens, const int32_t* block_table,
                             int64_t block_table_stride, int num_seqs, int max_seq_len,
                             int num_heads, int num_kv_heads, int head_size, int block_size,
                             float scale, int window_left, float softcap,
                             const float* alibi_slopes, const float* sinks, int num_splits,
                             pa_dtype_t dtype, pa_dtype_t kv_cache_dtype, const float* k_scale,
                             const float* v_scale, const float* q_scale) {
  pa::AttnParams p{};
  p.out = out;
  p.lse = lse;
  p.part_out = part_out;
  p.part_lse = part_lse;
  p.q = q;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.seq_lens = seq_lens;
  p.block_table = block_table;
  p.block_table_stride = block_table_stride;
  p.num_seqs = num_seqs;
  p.total_q = num_seqs;
  p.max_seqlen_q = 1;
  p.max_seqlen_k = max_seq_len;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_size = head_size;
  p.block_size = block_size;
  p.scale = scale;
  p.causal = 1;
  p.window_left = window_left;
  p.softcap = softcap;
  p.alibi_slopes = alibi_slopes;
  p.sinks = sinks;
  p.num_splits = num_splits;
  p.dtype = static_cast<pa::Dtype>(dtype);
  p.kv_fp8 = kv_cache_dtype == PA_FP8_E4M3;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.q_scale = q_scale;
  return p;
}

}  // namespace

// the trace buffer the launchers hand to the kernels (see pa_trace_set)
namespace pa {
std::atomic<uint64_t*> g_trace_buf{nullptr};
uint64_t* trace_buffer() { return g_trace_buf.load(); }
}  // namespace pa

extern "C" {

const char* pa_last_error(void) { return g_last_error.c_str(); }

int pa_trace_set(void* buffer) {
  if (!pa::kTrace)
    return fail(PA_ERR_UNSUPPORTED, "pa_trace_set: this library is built without tracing "
                                    "(build.py --trace builds libpagedattn_trace.so)");
  pa::g_trace_buf.store(static_cast<uint64_t*>(buffer));
  return ok();
}

int reshape_and_cache(const void* key, const void* value, int64_t key_token_stride,
                      int64_t value_token_stride, void* key_cache, void* value_cache,
                      const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                      int block_size, int num_kv_heads, int head_size, pa_dtype_t dtype,
                      pa_dtype_t kv_cache_dtype, const float* k_scale, const float* v_scale,
                      void* stream) {
  const char* fn = "reshape_and_cache";
  int rc = check_cache_shape(fn, block_size, num_kv_heads, head_size, dtype);
  if (rc != PA_OK) return rc;
  rc = check_kv(fn, dtype, kv_cache_dtype, k_scale, v_scale, true);
  if (rc != PA_OK) return rc;
  if (num_tokens < 0) return fail(PA_ERR_INVALID, "%s: num_tokens must be >= 0", fn);
  if (num_tokens == 0) return ok();
  if (key == nullptr || value == nullptr || key_cache == nullptr || value_cache == nullptr ||
      slot_mapping == nullptr)
    return fail(PA_ERR_INVALID, "%s: NULL pointer", fn);
  const int64_t row = (int64_t)num_kv_heads * head_size;
  if (key_token_stride < row || value_token_stride < row)
    return fail(PA_ERR_INVALID, "%s: token strides (%lld, %lld) must be >= num_kv_heads*head_size (%lld)",
                fn, (long long)key_token_stride, (long long)value_token_stride, (long long)row);
  if (num_blocks <= 0) return fail(PA_ERR_INVALID, "%s: num_blocks must be positive", fn);
  if (kv_cache_dtype == PA_FP8_E4M3)
    return hip_result(pa::launch_reshape_and_cache_fp8(
                          key, value, key_token_stride, value_token_stride, key_cache,
                          value_cache, slot_mapping, num_tokens, static_cast<int>(row),
                          static_cast<pa::Dtype>(dtype), k_scale, v_scale,
                          static_cast<hipStream_t>(stream)),
                      fn);
  return hip_result(pa::launch_reshape_and_cache(key, value, key_token_stride, value_token_stride,
                                                 key_cache, value_cache, slot_mapping, num_tokens,
                                                 static_cast<int>(row),
                                                 static_cast<hipStream_t>(stream)),
                    fn);
}

int paged_attn_prefill(void* out, float* lse, const void* q, const void* key_cache,
                       const void* value_cache, const int32_t* cu_seqlens_q,
                       const int32_t* seq_lens, const int32_t* block_table,
                       int64_t block_table_stride, int num_seqs, int64_t total_q,
                       int max_seqlen_q, int max_seqlen_k, int num_heads, int num_kv_heads,
                       int head_size, int block_size, int64_t num_blocks, float scale, int causal,
                       int window_left, float softcap, const float* alibi_slopes,
                       const float* sinks, pa_dtype_t dtype, pa_dtype_t kv_cache_dtype,
                       const float* k_scale, const float* v_scale, const float* q_scale,
                       void* stream) {
  const char* fn = "paged_attn_prefill";
  int rc = check_attn_common(fn, num_seqs, num_heads, num_kv_heads, head_size, block_size,
                             num_blocks, scale, window_left, softcap, dtype, q, key_cache,
                             value_cache, seq_lens, block_table, block_table_stride);
  if (rc != PA_OK) return rc;
  rc = check_kv(fn, dtype, kv_cache_dtype, k_scale, v_scale, true);
  if (rc != PA_OK) return rc;
  rc = check_q8(fn, kv_cache_dtype, q_scale);
  if (rc != PA_OK) return rc;
  if (out == nullptr) return fail(PA_ERR_INVALID, "%s: output buffer must be provided", fn);
  if (total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(PA_ERR_INVALID, "%s: total_q / max_seqlen_q / max_seqlen_k must be >= 0", fn);
  if (num_seqs > 0 && cu_seqlens_q == nullptr)
    return fail(PA_ERR_INVALID, "%s: NULL cu_seqlens_q", fn);
  if (num_heads / num_kv_heads > 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: more than 128 query heads per KV head", fn);
  if (max_seqlen_k >= (1 << 24))
    return fail(PA_ERR_UNSUPPORTED, "%s: sequences of 2^24 keys or more are not supported", fn);
  if (num_seqs > 65535)
    return fail(PA_ERR_UNSUPPORTED, "%s: more than 65535 sequences in one call", fn);
  if ((int64_t)num_kv_heads * max_seqlen_q > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "%s: num_kv_heads * max_seqlen_q must be below 2^31", fn);
  if ((int64_t)num_kv_heads * (total_q + num_seqs) > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "%s: num_kv_heads * (total_q + num_seqs) must be below 2^31",
                fn);
  if (num_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return ok();
  pa::AttnParams p{};
  p.out = out;
  p.lse = lse;
  p.q = q;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.cu_seqlens_q = cu_seqlens_q;
  p.seq_lens = seq_lens;
  p.block_table = block_table;
  p.block_table_stride = block_table_stride;
  p.num_seqs = num_seqs;
  p.total_q = total_q;
  p.max_seqlen_q = max_seqlen_q;
  p.max_seqlen_k = max_seqlen_k;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_size = head_size;
  p.block_size = block_size;
  p.scale = scale;
  p.causal = causal != 0;
  p.window_left = window_left;
  p.softcap = softcap;
  p.alibi_slopes = alibi_slopes;
  p.sinks = sinks;
  p.num_splits = 1;
  p.dtype = static_cast<pa::Dtype>(dtype);
  p.kv_fp8 = kv_cache_dtype == PA_FP8_E4M3;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.q_scale = q_scale;
  return hip_result(pa::launch_prefill(p, static_cast<hipStream_t>(stream)), fn);
}

int paged_attn_decode(void* out, float* lse, float* part_out, float* part_lse, const void* q,
                      const void* key_cache, const void* value_cache, const int32_t* seq_lens,
                      const int32_t* block_table, int64_t block_table_stride, int num_seqs,
                      int max_seq_len, int num_heads, int num_kv_heads, int head_size,
                      int block_size, int64_t num_blocks, float scale, int window_left,
                      float softcap, const float* alibi_slopes, const float* sinks,
                      int num_splits, pa_dtype_t dtype, pa_dtype_t kv_cache_dtype,
                      const float* k_scale, const float* v_scale, const float* q_scale,
                      void* stream) {
  const char* fn = "paged_attn_decode";
  int rc = check_decode(fn, num_seqs, max_seq_len, num_heads, num_kv_heads, head_size, block_size,
                        num_blocks, scale, window_left, softcap, num_splits, dtype,
                        kv_cache_dtype, k_scale, v_scale, q_scale, q, key_cache, value_cache,
                        seq_lens, block_table, block_table_stride);
  if (rc != PA_OK) return rc;
  if (num_splits == 1 && out == nullptr)
    return fail(PA_ERR_INVALID, "%s: output buffer must be provided", fn);
  if (num_splits > 1 && (part_out == nullptr || part_lse == nullptr))
    return fail(PA_ERR_INVALID, "%s: num_splits > 1 needs part_out and part_lse", fn);
  if (num_seqs == 0) return ok();
  pa::AttnParams p = decode_params(out, lse, part_out, part_lse, q, key_cache, value_cache,
                                   seq_lens, block_table, block_table_stride, num_seqs,
                                   max_seq_len, num_heads, num_kv_heads, head_size, block_size,
                                   scale, window_left, softcap, alibi_slopes, sinks, num_splits,
                                   dtype, kv_cache_dtype, k_scale, v_scale, q_scale);
  return hip_result(pa::launch_decode(p, static_cast<hipStream_t>(stream)), fn);
}

int paged_attn_decode_merged(void* out, float* lse, float* part_out, float* part_lse,
                             int32_t* split_counters, const void* q, const void* key_cache,
                             const void* value_cache, const int32_t* seq_lens,
                             const int32_t* block_table, int64_t block_table_stride, int num_seqs,
                             int max_seq_len, int num_heads, int num_kv_heads, int head_size,
                             int block_size, int64_t num_blocks, float scale, int window_left,
                             float softcap, const float* alibi_slopes, const float* sinks,
                             int num_splits, pa_dtype_t dtype, pa_dtype_t kv_cache_dtype,
                             const float* k_scale, const float* v_scale, const float* q_scale,
                             void* stream) {
  const char* fn = "paged_attn_decode_merged";
  int rc = check_decode(fn, num_seqs, max_seq_len, num_heads, num_kv_heads, head_size, block_size,
                        num_blocks, scale, window_left, softcap, num_splits, dtype,
                        kv_cache_dtype, k_scale, v_scale, q_scale, q, key_cache, value_cache,
                        seq_lens, block_table, block_table_stride);
  if (rc != PA_OK) return rc;
  if (out == nullptr) return fail(PA_ERR_INVALID, "%s: output buffer must be provided", fn);
  if (num_splits > 1 && (part_out == nullptr || part_lse == nullptr || split_counters == nullptr))
    return fail(PA_ERR_INVALID, "%s: num_splits > 1 needs part_out, part_lse and split_counters",
                fn);
  if (num_seqs == 0) return ok();
  pa::AttnParams p = decode_params(out, lse, part_out, part_lse, q, key_cache, value_cache,
                                   seq_lens, block_table, block_table_stride, num_seqs,
                                   max_seq_len, num_heads, num_kv_heads, head_size, block_size,
                                   scale, window_left, softcap, alibi_slopes, sinks, num_splits,
                                   dtype, kv_cache_dtype, k_scale, v_scale, q_scale);
  p.split_counters = split_counters;
  return hip_result(pa::launch_decode(p, static_cast<hipStream_t>(stream)), fn);
}

int paged_attn_decode_noalloc(void* out, float* lse, const void* q, const void* key_cache,
                              const void* value_cache, const int32_t* seq_lens,
                              const int32_t* block_table, int64_t block_table_stride,
                              int num_seqs, int max_seq_len, int num_heads, int num_kv_heads,
                              int head_size, int block_size, int64_t num_blocks, float scale,
                              int window_left, float softcap, const float* alibi_slopes,
                              const float* sinks, int num_splits, pa_dtype_t dtype,
                              pa_dtype_t kv_cache_dtype, const float* k_scale,
                              const float* v_scale, const float* q_scale, void* stream) {
  const char* fn = "paged_attn_decode_noalloc";
  int rc = check_decode(fn, num_seqs, max_seq_len, num_heads, num_kv_heads, head_size, block_size,
                        num_blocks, scale, window_left, softcap, num_splits, dtype,
                        kv_cache_dtype, k_scale, v_scale, q_scale, q, key_cache, value_cache,
                        seq_lens, block_table, block_table_stride);
  if (rc != PA_OK) return rc;
  if (out == nullptr) return fail(PA_ERR_INVALID, "%s: output buffer must be provided", fn);
  // partial results [S, B, Hq, D] fp32, then their LSEs [S, Hq, B] at a
  // 256-byte boundary
  const size_t parts = (size_t)num_splits * num_seqs * num_heads * head_size * 4;
  const size_t lse_off = (parts + 255) / 256 * 256;
  const size_t need = num_splits > 1 ? lse_off + (size_t)num_splits * num_heads * num_seqs * 4 : 0;
  if (need > pa::kNoallocScratchBytes)
    return fail(PA_ERR_UNSUPPORTED,
                "%s: %d splits x %d sequences x %d heads x %d need %zu bytes of partial results; "
                "the fixed scratch holds %zu",
                fn, num_splits, num_seqs, num_heads, head_size, need, pa::kNoallocScratchBytes);
  if (num_seqs == 0) return ok();
  float* part_out = nullptr;
  float* part_lse = nullptr;
  if (num_splits > 1) {
    void* base = nullptr;
    if (pa::noalloc_scratch(&base) != 0)
      return fail(PA_ERR_HIP, "%s: the device address of the scratch array is unavailable: %s",
                  fn, hipGetErrorString(hipGetLastError()));
    part_out = static_cast<float*>(base);
    part_lse = reinterpret_cast<float*>(static_cast<char*>(base) + lse_off);
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  pa::AttnParams p = decode_params(num_splits > 1 ? nullptr : out, num_splits > 1 ? nullptr : lse,
                                   part_out, part_lse, q, key_cache, value_cache, seq_lens,
                                   block_table, block_table_stride, num_seqs, max_seq_len,
                                   num_heads, num_kv_heads, head_size, block_size, scale,
                                   window_left, softcap, alibi_slopes, sinks, num_splits, dtype,
                                   kv_cache_dtype, k_scale, v_scale, q_scale);
  rc = pa::launch_decode(p, st);
  if (rc == 0 && num_splits > 1)
    rc = pa::launch_merge(out, lse, part_out, part_lse, num_splits, num_seqs, num_heads,
                          head_size, pa::kF32, static_cast<pa::Dtype>(dtype), st);
  return hip_result(rc, fn);
}

int merge_attn_states(void* out, float* out_lse, const void* parts_out, const float* parts_lse,
                      int num_parts, int64_t num_tokens, int num_heads, int head_size,
                      pa_dtype_t parts_dtype, pa_dtype_t out_dtype, void* stream) {
  const char* fn = "merge_attn_states";
  auto dtype_ok = [](pa_dtype_t t) { return t == PA_F16 || t == PA_BF16 || t == PA_F32; };
  if (!dtype_ok(parts_dtype) || !dtype_ok(out_dtype))
    return fail(PA_ERR_UNSUPPORTED, "%s: dtypes must be PA_F32, PA_F16 or PA_BF16", fn);
  if (head_size != 64 && head_size != 128 && head_size != 256)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_size must be 64, 128 or 256 (got %d)", fn, head_size);
  if (num_parts < 1 || num_parts > 256)
    return fail(PA_ERR_INVALID, "%s: num_parts must be in [1, 256] (got %d)", fn, num_parts);
  if (num_tokens < 0 || num_heads <= 0)
    return fail(PA_ERR_INVALID, "%s: num_tokens must be >= 0 and num_heads > 0", fn);
  if (num_tokens == 0) return ok();
  if (out == nullptr || parts_out == nullptr || parts_lse == nullptr)
    return fail(PA_ERR_INVALID, "%s: NULL pointer", fn);
  return hip_result(pa::launch_merge(out, out_lse, parts_out, parts_lse, num_parts, num_tokens,
                                     num_heads, head_size, static_cast<pa::Dtype>(parts_dtype),
                                     static_cast<pa::Dtype>(out_dtype),
                                     static_cast<hipStream_t>(stream)),
                    fn);
}

int paged_attn_cascade(void* out, float* lse, const void* q, const void* key_cache,
                       const void* value_cache, const int32_t* cu_seqlens_q,
                       const int32_t* seq_lens, const int32_t* block_table,
                       int64_t block_table_stride, int num_seqs, int64_t total_q,
                       int max_seqlen_q, int max_seqlen_k, int num_heads, int num_kv_heads,
                       int head_size, int block_size, int64_t num_blocks, float scale,
                       float softcap, const float* sinks, int common_prefix_len,
                       int max_prefix_splits,
                       void* parts_out, float* parts_lse, int32_t* work_ints, pa_dtype_t dtype,
                       pa_dtype_t kv_cache_dtype, const float* k_scale, const float* v_scale,
                       const float* q_scale, void* stream) {
  const char* fn = "paged_attn_cascade";
  int rc = check_attn_common(fn, num_seqs, num_heads, num_kv_heads, head_size, block_size,
                             num_blocks, scale, -1, softcap, dtype, q, key_cache, value_cache,
                             seq_lens, block_table, block_table_stride);
  if (rc != PA_OK) return rc;
  rc = check_kv(fn, dtype, kv_cache_dtype, k_scale, v_scale, true);
  if (rc != PA_OK) return rc;
  rc = check_q8(fn, kv_cache_dtype, q_scale);
  if (rc != PA_OK) return rc;
  if (out == nullptr) return fail(PA_ERR_INVALID, "%s: output buffer must be provided", fn);
  if (total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(PA_ERR_INVALID, "%s: total_q / max_seqlen_q / max_seqlen_k must be >= 0", fn);
  if (common_prefix_len <= 0 || common_prefix_len % block_size != 0)
    return fail(PA_ERR_INVALID,
                "%s: common_prefix_len must be a positive multiple of block_size (got %d)", fn,
                common_prefix_len);
  if (common_prefix_len >= max_seqlen_k && num_seqs > 0)
    return fail(PA_ERR_INVALID, "%s: common_prefix_len (%d) must be below max_seqlen_k (%d)", fn,
                common_prefix_len, max_seqlen_k);
  if (max_prefix_splits < 1 || max_prefix_splits > 255)
    return fail(PA_ERR_INVALID, "%s: max_prefix_splits must be in [1, 255] (got %d)", fn,
                max_prefix_splits);
  (void)work_ints;  // reserved: the passes need no device-side lengths
  if (num_seqs > 0 && (cu_seqlens_q == nullptr || parts_out == nullptr || parts_lse == nullptr))
    return fail(PA_ERR_INVALID, "%s: NULL cu_seqlens_q or workspace", fn);
  if (num_heads / num_kv_heads > 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: more than 128 query heads per KV head", fn);
  if (max_seqlen_k >= (1 << 24))
    return fail(PA_ERR_UNSUPPORTED, "%s: sequences of 2^24 keys or more are not supported", fn);
  if (num_seqs > 65535)
    return fail(PA_ERR_UNSUPPORTED, "%s: more than 65535 sequences in one call", fn);
  // the prefix pass takes every query as one sequence; the suffix pass's
  // grid has up to total_q + num_seqs query tiles per KV head
  if ((int64_t)num_kv_heads * (total_q + num_seqs) > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "%s: num_kv_heads * (total_q + num_seqs) must be below 2^31",
                fn);
  if (num_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return ok();
  pa::AttnParams p{};
  p.out = out;
  p.lse = lse;
  p.q = q;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.cu_seqlens_q = cu_seqlens_q;
  p.seq_lens = seq_lens;
  p.block_table = block_table;
  p.block_table_stride = block_table_stride;
  p.num_seqs = num_seqs;
  p.total_q = total_q;
  p.max_seqlen_q = max_seqlen_q;
  p.max_seqlen_k = max_seqlen_k;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_size = head_size;
  p.block_size = block_size;
  p.scale = scale;
  p.causal = 1;
  p.window_left = -1;
  p.softcap = softcap;
  p.alibi_slopes = nullptr;
  p.sinks = sinks;
  p.num_splits = 1;
  p.dtype = static_cast<pa::Dtype>(dtype);
  p.kv_fp8 = kv_cache_dtype == PA_FP8_E4M3;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.q_scale = q_scale;
  return hip_result(pa::launch_cascade(p, common_prefix_len, max_prefix_splits, parts_out,
                                       parts_lse, static_cast<hipStream_t>(stream)),
                    fn);
}

int scaled_fp8_quant(void* out, const void* input, const float* scale, int64_t num_elems,
                     pa_dtype_t dtype, void* stream) {
  const char* fn = "scaled_fp8_quant";
  if (!is_16bit(dtype))
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype must be PA_F16 or PA_BF16 (got %d)", fn, (int)dtype);
  if (num_elems < 0) return fail(PA_ERR_INVALID, "%s: num_elems must be >= 0", fn);
  if (num_elems > 0 && (out == nullptr || input == nullptr || scale == nullptr))
    return fail(PA_ERR_INVALID, "%s: NULL out, input or scale", fn);
  if (num_elems == 0) return ok();
  return hip_result(pa::launch_scaled_fp8_quant(out, input, scale, num_elems,
                                                static_cast<pa::Dtype>(dtype),
                                                static_cast<hipStream_t>(stream)),
                    fn);
}

int pa_use_cascade(int common_prefix_len, const int32_t* query_lens, const int32_t* seq_lens,
                   int num_reqs, int num_heads, int num_kv_heads, int head_size,
                   int kv_elem_bytes, int use_alibi, int use_sliding_window,
                   int use_local_attention, int dcp_world_size) {
  const char* fn = "pa_use_cascade";
  if (num_reqs < 0) return fail(PA_ERR_INVALID, "%s: num_reqs must be >= 0", fn);
  if (num_reqs > 0 && (query_lens == nullptr || seq_lens == nullptr))
    return fail(PA_ERR_INVALID, "%s: NULL query_lens or seq_lens", fn);
  if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 || head_size <= 0 ||
      (kv_elem_bytes != 1 && kv_elem_bytes != 2))
    return fail(PA_ERR_INVALID, "%s: bad head counts, head_size or kv_elem_bytes", fn);
  ok();
  // the page's support checks, in its order
  if (common_prefix_len < 256) return 0;
  if (use_alibi || use_sliding_window || use_local_attention) return 0;
  if (num_reqs < 8) return 0;
  if (dcp_world_size > 1) return 0;
  // not a split-decode batch (several queries per request, or one query
  // head per KV head): the cascade saves the prefix re-reads
  bool all_decode = true;
  for (int b = 0; b < num_reqs; ++b) all_decode = all_decode && query_lens[b] == 1;
  if (!(num_heads / num_kv_heads > 1 && all_decode)) return 1;
  // a decode batch: the calibrated time models of the two paths
  return pa::cascade_beats_split_decode(common_prefix_len, seq_lens, num_reqs, num_heads,
                                        num_kv_heads, head_size, kv_elem_bytes)
             ? 1
             : 0;
}

int pa_local_virtual_batches(int attn_chunk_size, int block_size, const int32_t* query_start_loc,
                             const int32_t* seq_lens, int num_seqs, const int32_t* block_table,
                             int64_t block_table_stride, int block_table_cols, int max_virtual,
                             int32_t* seqlens_q_local, int32_t* cu_seqlens_q_local,
                             int32_t* seqlens_k_local, int32_t* block_table_local) {
  const char* fn = "pa_local_virtual_batches";
  if (attn_chunk_size <= 0 || block_size <= 0 || attn_chunk_size % block_size != 0)
    return fail(PA_ERR_INVALID,
                "%s: attn_chunk_size (%d) must be a positive multiple of block_size (%d)", fn,
                attn_chunk_size, block_size);
  if (num_seqs < 0) return fail(PA_ERR_INVALID, "%s: num_seqs must be >= 0", fn);
  if (num_seqs > 0 && (query_start_loc == nullptr || seq_lens == nullptr))
    return fail(PA_ERR_INVALID, "%s: NULL query_start_loc or seq_lens", fn);
  for (int b = 0; b < num_seqs; ++b) {
    const int64_t q_len = (int64_t)query_start_loc[b + 1] - query_start_loc[b];
    if (q_len < 0 || seq_lens[b] < q_len)
      return fail(PA_ERR_INVALID, "%s: sequence %d has %lld queries and %d keys", fn, b,
                  (long long)q_len, seq_lens[b]);
  }
  const bool count_only = seqlens_q_local == nullptr && cu_seqlens_q_local == nullptr &&
                          seqlens_k_local == nullptr && block_table_local == nullptr;
  const int v = pa::local_virtual_batches(attn_chunk_size, block_size, query_start_loc, seq_lens,
                                          num_seqs, nullptr, 0, 0, nullptr, nullptr, nullptr,
                                          nullptr);
  if (count_only) {
    ok();
    return v;
  }
  if (seqlens_q_local == nullptr || cu_seqlens_q_local == nullptr || seqlens_k_local == nullptr ||
      block_table_local == nullptr)
    return fail(PA_ERR_INVALID, "%s: outputs must be all NULL (count) or all given", fn);
  if (v > max_virtual)
    return fail(PA_ERR_INVALID, "%s: %d virtual sequences exceed max_virtual (%d)", fn, v,
                max_virtual);
  if (num_seqs > 0 && (block_table == nullptr || block_table_cols <= 0 ||
                       block_table_stride < block_table_cols))
    return fail(PA_ERR_INVALID, "%s: block_table needs cols > 0 and a stride >= cols", fn);
  pa::local_virtual_batches(attn_chunk_size, block_size, query_start_loc, seq_lens, num_seqs,
                            block_table, block_table_stride, block_table_cols, seqlens_q_local,
                            cu_seqlens_q_local, seqlens_k_local, block_table_local);
  ok();
  return v;
}

int pa_check_indices(const int64_t* slot_mapping, int64_t num_tokens, const int32_t* block_table,
                     int64_t block_table_stride, const int32_t* seq_lens, int num_seqs,
                     int64_t num_blocks, int block_size, int32_t* counts, void* stream) {
  const char* fn = "pa_check_indices";
  if (counts == nullptr) return fail(PA_ERR_INVALID, "%s: NULL counts", fn);
  if (block_size <= 0 || block_size % 16 != 0)
    return fail(PA_ERR_INVALID, "%s: block_size must be a positive multiple of 16 (got %d)", fn,
                block_size);
  if (num_blocks <= 0) return fail(PA_ERR_INVALID, "%s: num_blocks must be positive", fn);
  if (num_tokens < 0 || num_seqs < 0)
    return fail(PA_ERR_INVALID, "%s: num_tokens and num_seqs must be >= 0", fn);
  if (num_tokens > 0 && slot_mapping == nullptr)
    return fail(PA_ERR_INVALID, "%s: NULL slot_mapping", fn);
  if (num_seqs > 0 && (block_table == nullptr || seq_lens == nullptr || block_table_stride <= 0))
    return fail(PA_ERR_INVALID, "%s: num_seqs > 0 needs block_table, seq_lens and a positive stride",
                fn);
  return hip_result(pa::launch_check_indices(slot_mapping, num_tokens, block_table,
                                             block_table_stride, seq_lens, num_seqs, num_blocks,
                                             block_size, counts, static_cast<hipStream_t>(stream)),
                    fn);
}

}  // extern "C"
