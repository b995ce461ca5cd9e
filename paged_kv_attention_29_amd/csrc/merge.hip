// merge_attn_states: combine partial attention states by log-sum-exp
// (vLLM flash_attn.py (e2f56c3), cascade_attention / _forward_with_dcp,
// merge_attn_states).  One wave per (token, head); each lane owns
// head_size / 64 consecutive output elements, so every part row is read
// as one coalesced 64-lane access.  Memory-bound: it reads
// num_parts * (head_size * elem + 4) bytes per (token, head).
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace pa {

template <int T> struct Elem;
template <> struct Elem<kF32> {
  static __device__ __forceinline__ float ld(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  static __device__ __forceinline__ void st(void* p, int64_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
};
template <> struct Elem<kBF16> {
  static __device__ __forceinline__ float ld(const void* p, int64_t i) {
    return BF16::to_float(static_cast<const uint16_t*>(p)[i]);
  }
  static __device__ __forceinline__ void st(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = BF16::from_float(v);
  }
};
template <> struct Elem<kF16> {
  static __device__ __forceinline__ float ld(const void* p, int64_t i) {
    return F16::to_float(static_cast<const uint16_t*>(p)[i]);
  }
  static __device__ __forceinline__ void st(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = F16::from_float(v);
  }
};

template <int PT, int OT, int D>
__global__ __launch_bounds__(256) void merge_kernel(void* __restrict__ out,
                                                    float* __restrict__ out_lse,
                                                    const void* __restrict__ parts,
                                                    const float* __restrict__ parts_lse,
                                                    int S, int64_t T, int H) {
  constexpr int EPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= T * H) return;
  const int64_t t = pair / H;
  const int h = static_cast<int>(pair - t * H);
  const int64_t lse_stride = (int64_t)H * T;
  const int64_t lse_off = (int64_t)h * T + t;

  const int64_t row = pair * D + lane * EPL;  // (t * H + h) * D
  const int64_t part_stride = T * H * D;
  // The LSEs of parts [0, 64) (lane p holds part p's) and the rows of the
  // first batch of parts go out together: the row loads do not wait for the
  // maximum, so up to eight parts cost one memory latency.
  constexpr int NB = 8;
  const int nb0 = S < NB ? S : NB;
  const float lse_l = lane < S ? parts_lse[lane * lse_stride + lse_off] : kNegInf;
  float x0[NB][EPL];
#pragma unroll
  for (int j = 0; j < NB; ++j)
    if (j < nb0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) x0[j][e] = Elem<PT>::ld(parts, j * part_stride + row + e);
    }
  float m = lse_l;
  for (int p = 64 + lane; p < S; p += 64) m = fmaxf(m, parts_lse[p * lse_stride + lse_off]);
  m = wave_max(m);

  if (m == kNegInf) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) Elem<OT>::st(out, row + e, 0.0f);
    if (out_lse != nullptr && lane == 0) out_lse[lse_off] = kNegInf;
    return;
  }
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
  float wsum = 0.0f;
  // weight of part p (p wave-uniform): with at most 64 parts every LSE is
  // in a lane already; the choice is made once, outside the loops, so each
  // batch's row loads stay together
  auto accumulate = [&](auto lse_in_lanes) {
    constexpr bool IN_LANES = decltype(lse_in_lanes)::value;
    auto weight = [&](int p) {
      const float l = IN_LANES ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lse_l), p))
                               : parts_lse[p * lse_stride + lse_off];
      return fast_exp2((l - m) * kLog2e);
    };
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (j < nb0) {
        const float w = weight(j);
        wsum += w;
        // an empty part (w = 0) may hold anything, finite or not; each part
        // adds w * x with one fused multiply-add
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = w != 0.0f ? __builtin_fmaf(w, x0[j][e], acc[e]) : acc[e];
      }
    // the other parts in batches of 8: the loads of a batch are independent
    // and go out together
    int p = nb0;
    for (; p + 8 <= S; p += 8) {
      float w[8], x[8][EPL];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        w[j] = weight(p + j);
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[j][e] = Elem<PT>::ld(parts, (p + j) * part_stride + row + e);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        wsum += w[j];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = w[j] != 0.0f ? __builtin_fmaf(w[j], x[j][e], acc[e]) : acc[e];
      }
    }
    for (; p < S; ++p) {
      const float w = weight(p);
      wsum += w;
      if (w == 0.0f) continue;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(w, Elem<PT>::ld(parts, p * part_stride + row + e), acc[e]);
    }
  };
  if (S <= 64) accumulate(std::true_type{});
  else accumulate(std::false_type{});
  const float inv = 1.0f / wsum;
#pragma unroll
  for (int e = 0; e < EPL; ++e) Elem<OT>::st(out, row + e, acc[e] * inv);
  if (out_lse != nullptr && lane == 0) out_lse[lse_off] = m + __logf(wsum);
}

template <int PT, int OT>
static int merge_dispatch_d(void* out, float* out_lse, const void* parts, const float* parts_lse,
                            int S, int64_t T, int H, int D, hipStream_t stream) {
  const int64_t pairs = T * H;
  const dim3 grid(static_cast<unsigned>((pairs + 3) / 4));
  switch (D) {
    case 64:
      hipLaunchKernelGGL((merge_kernel<PT, OT, 64>), grid, dim3(256), 0, stream, out, out_lse,
                         parts, parts_lse, S, T, H);
      break;
    case 128:
      hipLaunchKernelGGL((merge_kernel<PT, OT, 128>), grid, dim3(256), 0, stream, out, out_lse,
                         parts, parts_lse, S, T, H);
      break;
    default:
      hipLaunchKernelGGL((merge_kernel<PT, OT, 256>), grid, dim3(256), 0, stream, out, out_lse,
                         parts, parts_lse, S, T, H);
      break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

template <int PT>
static int merge_dispatch_out(void* out, float* out_lse, const void* parts,
                              const float* parts_lse, int S, int64_t T, int H, int D,
                              Dtype out_dtype, hipStream_t stream) {
  switch (out_dtype) {
    case kF32: return merge_dispatch_d<PT, kF32>(out, out_lse, parts, parts_lse, S, T, H, D, stream);
    case kBF16: return merge_dispatch_d<PT, kBF16>(out, out_lse, parts, parts_lse, S, T, H, D, stream);
    default: return merge_dispatch_d<PT, kF16>(out, out_lse, parts, parts_lse, S, T, H, D, stream);
  }
}

int launch_merge(void* out, float* out_lse, const void* parts, const float* parts_lse,
                 int num_parts, int64_t num_tokens, int num_heads, int head_size,
                 Dtype parts_dtype, Dtype out_dtype, hipStream_t stream) {
  if (num_tokens == 0) return 0;
  switch (parts_dtype) {
    case kF32:
      return merge_dispatch_out<kF32>(out, out_lse, parts, parts_lse, num_parts, num_tokens,
                                      num_heads, head_size, out_dtype, stream);
    case kBF16:
      return merge_dispatch_out<kBF16>(out, out_lse, parts, parts_lse, num_parts, num_tokens,
                                       num_heads, head_size, out_dtype, stream);
    default:
      return merge_dispatch_out<kF16>(out, out_lse, parts, parts_lse, num_parts, num_tokens,
                                      num_heads, head_size, out_dtype, stream);
  }
}

}  // namespace pa
