// reshape_and_cache: scatter the K/V rows of new tokens into their cache
// slots (vLLM flash_attn.py (e2f56c3), FlashAttentionImpl.forward, the
// reshape_and_cache_flash call).  A token's row (num_kv_heads * head_size
// 16-bit elements) is contiguous both in the input and in the cache slot, so
// the copy is a gather of contiguous rows: consecutive lanes move
// consecutive 16-byte pieces of the same row (fully coalesced reads and
// writes); a negative slot skips the row.  Memory-bound by construction.
#include "common.h"
#include "launch.h"

namespace pa {

// VEC = 16-bit elements moved per lane-access (8 -> 16 bytes, 1 -> 2 bytes).
// A token needs 2 * row_elems / VEC lane-accesses (K row, then V row); a
// 256-lane workgroup takes as many whole tokens as fit, or loops over one
// token's accesses when a token needs more than 256.
template <int VEC>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    int64_t key_stride, int64_t value_stride, uint16_t* __restrict__ key_cache,
    uint16_t* __restrict__ value_cache, const int64_t* __restrict__ slots,
    int64_t num_tokens, int row_elems) {
  typedef uint16_t vec_t __attribute__((ext_vector_type(VEC)));
  const int vpr = row_elems / VEC;
  const int per_tok = 2 * vpr;
  const bool big = per_tok >= static_cast<int>(blockDim.x);
  const int tpb = big ? 1 : blockDim.x / per_tok;
  const int sub = big ? 0 : threadIdx.x / per_tok;
  const int first = big ? threadIdx.x : threadIdx.x % per_tok;
  const int step = big ? blockDim.x : per_tok;
  if (sub >= tpb) return;
  for (int64_t tok = (int64_t)blockIdx.x * tpb + sub; tok < num_tokens;
       tok += (int64_t)gridDim.x * tpb) {
    const int64_t slot = slots[tok];
    if (slot < 0) continue;
    for (int v = first; v < per_tok; v += step) {
      const bool is_v = v >= vpr;
      const int c = is_v ? v - vpr : v;
      const uint16_t* src = is_v ? value + tok * value_stride : key + tok * key_stride;
      uint16_t* dst = (is_v ? value_cache : key_cache) + slot * row_elems;
      reinterpret_cast<vec_t*>(dst)[c] = reinterpret_cast<const vec_t*>(src)[c];
    }
  }
}

int launch_reshape_and_cache(const void* key, const void* value, int64_t key_stride,
                             int64_t value_stride, void* key_cache, void* value_cache,
                             const int64_t* slots, int64_t num_tokens, int row_elems,
                             hipStream_t stream) {
  const bool aligned = ((reinterpret_cast<uintptr_t>(key) | reinterpret_cast<uintptr_t>(value) |
                         reinterpret_cast<uintptr_t>(key_cache) |
                         reinterpret_cast<uintptr_t>(value_cache)) % 16 == 0) &&
                       key_stride % 8 == 0 && value_stride % 8 == 0 && row_elems % 8 == 0;
  const int vec = aligned ? 8 : 1;
  const int per_tok = 2 * (row_elems / vec);
  const int64_t tpb = per_tok >= 256 ? 1 : 256 / per_tok;
  int64_t blocks = (num_tokens + tpb - 1) / tpb;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  if (aligned)
    hipLaunchKernelGGL(reshape_and_cache_kernel<8>, dim3(blocks), dim3(256), 0, stream,
                       (const uint16_t*)key, (const uint16_t*)value, key_stride, value_stride,
                       (uint16_t*)key_cache, (uint16_t*)value_cache, slots, num_tokens, row_elems);
  else
    hipLaunchKernelGGL(reshape_and_cache_kernel<1>, dim3(blocks), dim3(256), 0, stream,
                       (const uint16_t*)key, (const uint16_t*)value, key_stride, value_stride,
                       (uint16_t*)key_cache, (uint16_t*)value_cache, slots, num_tokens, row_elems);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace pa
