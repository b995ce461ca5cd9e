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

// ---------------------------------------------------------------------------
// fp8 (OCP e4m3) cache: each element is divided by its tensor's scale in
// fp32 (correctly rounded) and rounded to the nearest e4m3 code, ties to the
// even code, saturating at +-448 (infinities too); NaN gives 0x7F with its
// sign and the sign of zero is kept (vLLM flash_attn.py (e2f56c3),
// FlashAttentionImpl.forward: reshape_and_cache_flash with kv_cache_dtype
// "fp8" and the per-tensor k/v scales; float8_e4m3fn from
// get_fp8_dtype_for_flashattn).  Integer rounding, so the result does not
// depend on how a hardware conversion treats overflow.
__device__ __forceinline__ uint32_t e4m3_code(float t) {
  const uint32_t u = __float_as_uint(t);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;  // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;  // |t| >= 448, inf: saturate
  if (a < 0x3c800000u) {
    // below 2^-6: subnormal codes m * 2^-9, m = rne(|t| * 512) in 0..8 (the
    // scaling is exact; m = 8 is the code of 2^-6)
    return sign | static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.0f));
  }
  // normal: keep 3 of the 23 mantissa bits, ties to even; a carry moves the
  // exponent up (at most to 448, since |t| < 448 here)
  const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
  return sign | (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
}

// Same token/lane mapping as above; VEC 16-bit inputs -> VEC code bytes.
template <typename T, int VEC>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    int64_t key_stride, int64_t value_stride, uint8_t* __restrict__ key_cache,
    uint8_t* __restrict__ value_cache, const int64_t* __restrict__ slots,
    int64_t num_tokens, int row_elems, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale) {
  typedef uint16_t in_t __attribute__((ext_vector_type(VEC)));
  const float ks = *k_scale, vs = *v_scale;
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
      uint8_t* dst = (is_v ? value_cache : key_cache) + slot * row_elems + c * VEC;
      const float s = is_v ? vs : ks;
      const in_t x = reinterpret_cast<const in_t*>(src)[c];
      if constexpr (VEC == 8) {
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e >> 2] |= e4m3_code(T::to_float(x[e]) / s) << (8 * (e & 3));
        *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
      } else {
        *dst = static_cast<uint8_t>(e4m3_code(T::to_float(x[0]) / s));
      }
    }
  }
}

template <typename T>
void launch_rac_fp8(bool aligned, dim3 grid, hipStream_t stream, const void* key,
                    const void* value, int64_t key_stride, int64_t value_stride,
                    void* key_cache, void* value_cache, const int64_t* slots,
                    int64_t num_tokens, int row_elems, const float* k_scale,
                    const float* v_scale) {
  if (aligned)
    hipLaunchKernelGGL((reshape_and_cache_fp8_kernel<T, 8>), grid, dim3(256), 0, stream,
                       (const uint16_t*)key, (const uint16_t*)value, key_stride, value_stride,
                       (uint8_t*)key_cache, (uint8_t*)value_cache, slots, num_tokens, row_elems,
                       k_scale, v_scale);
  else
    hipLaunchKernelGGL((reshape_and_cache_fp8_kernel<T, 1>), grid, dim3(256), 0, stream,
                       (const uint16_t*)key, (const uint16_t*)value, key_stride, value_stride,
                       (uint8_t*)key_cache, (uint8_t*)value_cache, slots, num_tokens, row_elems,
                       k_scale, v_scale);
}

int launch_reshape_and_cache_fp8(const void* key, const void* value, int64_t key_stride,
                                 int64_t value_stride, void* key_cache, void* value_cache,
                                 const int64_t* slots, int64_t num_tokens, int row_elems,
                                 Dtype in_dtype, const float* k_scale, const float* v_scale,
                                 hipStream_t stream) {
  const bool aligned =
      ((reinterpret_cast<uintptr_t>(key) | reinterpret_cast<uintptr_t>(value)) % 16 == 0) &&
      ((reinterpret_cast<uintptr_t>(key_cache) | reinterpret_cast<uintptr_t>(value_cache)) % 8 ==
       0) &&
      key_stride % 8 == 0 && value_stride % 8 == 0 && row_elems % 8 == 0;
  const int vec = aligned ? 8 : 1;
  const int per_tok = 2 * (row_elems / vec);
  const int64_t tpb = per_tok >= 256 ? 1 : 256 / per_tok;
  int64_t blocks = (num_tokens + tpb - 1) / tpb;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  if (in_dtype == kBF16)
    launch_rac_fp8<BF16>(aligned, dim3(blocks), stream, key, value, key_stride, value_stride,
                         key_cache, value_cache, slots, num_tokens, row_elems, k_scale, v_scale);
  else
    launch_rac_fp8<F16>(aligned, dim3(blocks), stream, key, value, key_stride, value_stride,
                        key_cache, value_cache, slots, num_tokens, row_elems, k_scale, v_scale);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// The query quantiser (scaled_fp8_quant with a static per-tensor scale; vLLM
// flash_attn.py (v0.9.0.1 docs), FlashAttentionImpl.forward, the fp8
// branch): each element divided by the scale, then e4m3_code, as for the
// cache.  VEC consecutive elements per lane, grid-stride.
template <typename T, int VEC>
__global__ __launch_bounds__(256) void scaled_fp8_quant_kernel(const uint16_t* __restrict__ in,
                                                               uint8_t* __restrict__ out,
                                                               const float* __restrict__ scale,
                                                               int64_t n_vec) {
  typedef uint16_t in_t __attribute__((ext_vector_type(VEC)));
  const float s = *scale;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_vec;
       i += (int64_t)gridDim.x * blockDim.x) {
    const in_t x = reinterpret_cast<const in_t*>(in)[i];
    if constexpr (VEC == 8) {
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e >> 2] |= e4m3_code(T::to_float(x[e]) / s) << (8 * (e & 3));
      reinterpret_cast<u32x2*>(out)[i] = u32x2{w[0], w[1]};
    } else {
      out[i] = static_cast<uint8_t>(e4m3_code(T::to_float(x[0]) / s));
    }
  }
}

int launch_scaled_fp8_quant(void* out, const void* input, const float* scale, int64_t n,
                            Dtype in_dtype, hipStream_t stream) {
  const bool aligned = n % 8 == 0 && reinterpret_cast<uintptr_t>(input) % 16 == 0 &&
                       reinterpret_cast<uintptr_t>(out) % 8 == 0;
  const int64_t n_vec = aligned ? n / 8 : n;
  int64_t blocks = (n_vec + 255) / 256;
  if (blocks > (1 << 16)) blocks = 1 << 16;
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  const uint16_t* in = static_cast<const uint16_t*>(input);
  uint8_t* o = static_cast<uint8_t*>(out);
  if (in_dtype == kBF16) {
    if (aligned) hipLaunchKernelGGL((scaled_fp8_quant_kernel<BF16, 8>), grid, block, 0, stream, in, o, scale, n_vec);
    else hipLaunchKernelGGL((scaled_fp8_quant_kernel<BF16, 1>), grid, block, 0, stream, in, o, scale, n_vec);
  } else {
    if (aligned) hipLaunchKernelGGL((scaled_fp8_quant_kernel<F16, 8>), grid, block, 0, stream, in, o, scale, n_vec);
    else hipLaunchKernelGGL((scaled_fp8_quant_kernel<F16, 1>), grid, block, 0, stream, in, o, scale, n_vec);
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
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
