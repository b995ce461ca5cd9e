// Shared device helpers for the gfx950 paged-attention kernels: 16-bit
// storage types, fp32 conversions, MFMA wrappers and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// 16-bit element types.  Storage is always the raw 16-bit pattern.
// ---------------------------------------------------------------------------
struct BF16 {
  static __device__ __forceinline__ float to_float(uint16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
  }
  // round to nearest even (hardware conversion); NaN stays NaN
  static __device__ __forceinline__ uint16_t from_float(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
  }
  // two floats -> packed pair (lo in bits 0..15), one v_cvt_pk_bf16_f32
  // (round to nearest even)
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{lo, hi}), bf2));
  }
  // four fp8 (OCP e4m3) codes, byte i -> element i; exact (every e4m3
  // value is a bf16 value); one v_cvt_scalef32_pk_bf16_fp8 per pair, scale 1
  static __device__ __forceinline__ v4s from_fp8x4(uint32_t w) {
    const bf2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const bf2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    // (whole registers: extracting the 16-bit lanes one by one made the
    // compiler duplicate the low lane)
    return __builtin_bit_cast(
        v4s, (u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)}));
  }
  // acc + lo + hi of a packed pair (v_dot2c_f32_bf16 with (1, 1))
  static __device__ __forceinline__ float sum2(uint32_t pair, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, pair),
                                           __builtin_bit_cast(bf2, 0x3f803f80u), acc, false);
  }
  // D[16x16] += A[16x32] * B[32x16]; operands are 8 elements per lane
  static __device__ __forceinline__ v4f mfma16x16x32(v8s a, v8s b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                   __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
  }
  // D[32x32] += A[32x16] * B[16x32]
  static __device__ __forceinline__ v16f mfma32x32x16(v8s a, v8s b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a),
                                                   __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
  }
  // D[16x16] += A[16x16] * B[16x16]; 4 elements per lane
  static __device__ __forceinline__ v4f mfma16x16x16(v4s a, v4s b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
};

struct F16 {
  static __device__ __forceinline__ float to_float(uint16_t x) {
    return static_cast<float>(__builtin_bit_cast(_Float16, x));
  }
  // four fp8 (OCP e4m3) codes, byte i -> element i; exact (every e4m3
  // value is an fp16 value); one v_cvt_scalef32_pk_f16_fp8 per pair, scale 1
  static __device__ __forceinline__ v4s from_fp8x4(uint32_t w) {
    const h2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
    const h2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
    // (whole registers: extracting the 16-bit lanes one by one made the
    // compiler duplicate the low lane)
    return __builtin_bit_cast(
        v4s, (u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)}));
  }
  static __device__ __forceinline__ uint16_t from_float(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
  }
  // one v_cvt_pk_f16_f32 (round to nearest even)
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{lo, hi}), h2));
  }
  static __device__ __forceinline__ float sum2(uint32_t pair, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, pair), __builtin_bit_cast(h2, 0x3c003c00u),
                                  acc, false);
  }
  static __device__ __forceinline__ v4f mfma16x16x32(v8s a, v8s b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a),
                                                  __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ v16f mfma32x32x16(v8s a, v8s b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a),
                                                  __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ v4f mfma16x16x16(v4s a, v4s b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(v4h, a),
                                                 __builtin_bit_cast(v4h, b), c, 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// Timeline tracing.  Built with -DPA_TRACE=1 (the separate trace library),
// the prefill and decode kernels record per workgroup kTraceSlots 64-bit
// words at trace + workgroup * kTraceSlots: shader-clock times of their
// phases, the CU's HW_ID and XCC_ID and the work done.  Otherwise the
// trace points compile to nothing.  The clock (s_memtime) is not shared by
// all shader engines: compare times within one CU only.
// ---------------------------------------------------------------------------
#ifndef PA_TRACE
#define PA_TRACE 0
#endif
constexpr bool kTrace = PA_TRACE != 0;
constexpr int kTraceSlots = 16;
enum TraceSlot {
  kTrEntry = 0,    // kernel entry
  kTrItem = 1,     // work item known (after the lookup / ranking)
  kTrLoop0 = 2,    // first K/V data landed: the key loop starts
  kTrLoop1 = 3,    // key loop done
  kTrEnd = 4,      // results stored (wave 0)
  kTrHwId = 5,     // HW_ID register (CU, SH, SE)
  kTrXcc = 6,      // XCC_ID register
  kTrUnits = 7,    // key tiles (prefill) or key steps (decode) of the item
  kTrWho = 8,      // item: sequence << 32 | query tile (prefill) or split (decode)
  kTrWaveEnd = 9,  // .. 12: each wave's end time
  kTrRealEntry = 13,  // constant-rate (100 MHz) clock at entry
  kTrRealEnd = 14,    // and when wave 0 stored its results
};
__device__ __forceinline__ uint64_t trace_clock() { return __builtin_amdgcn_s_memtime(); }
__device__ __forceinline__ uint64_t trace_realclock() { return __builtin_amdgcn_s_memrealtime(); }
// lane 0 of the calling wave stores v into slot k of this workgroup's record
__device__ __forceinline__ void trace_put(uint64_t* trace, int k, uint64_t v) {
  if constexpr (kTrace) {
    if (trace != nullptr && (threadIdx.x & 63) == 0)
      __builtin_nontemporal_store(v, trace + (uint64_t)blockIdx.x * kTraceSlots + k);
  }
}
__device__ __forceinline__ void trace_hw(uint64_t* trace) {
  if constexpr (kTrace) {
    trace_put(trace, kTrHwId, __builtin_amdgcn_s_getreg((4 << 0) | (0 << 6) | (31 << 11)));
    trace_put(trace, kTrXcc, __builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (31 << 11)));
  }
}

// ---------------------------------------------------------------------------
// wave64 cross-lane helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float shfl_xor(float v, int mask) {
  int lane = __lane_id();
  int src = lane ^ mask;
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}

// exp2 of a finite-or--inf argument (v_exp_f32); exp2(-inf) = 0
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Soft-capped logit in log2 units, cap * tanh(scale * s / cap) * log2(e),
// with tanh(x) = 1 - 2 / (1 + e^{2x}) on the hardware exp2 and reciprocal:
// the limits are exact (exp2 overflows to inf and its reciprocal to 0 for
// large x; it underflows to 0 for very negative x), and the absolute error
// of tanh is a few ulp of 1.  Five instructions: mul, exp2, add, rcp, fma.
// k2 = 2 * log2(e) * scale / cap, cap_log2 = cap * log2(e).
__device__ __forceinline__ float softcap_log2(float s, float k2, float cap_log2) {
  const float r = __builtin_amdgcn_rcpf(1.0f + fast_exp2(s * k2));
  return fmaf(r, -2.0f * cap_log2, cap_log2);
}

// floor(j / d) for 0 <= j < 2^24 and 16 <= d <= 256, with
// magic = ceil(2^32 / d) computed on the host (exact in that range).
__device__ __forceinline__ int div_magic(int j, uint32_t magic) {
  return static_cast<int>(__umulhi(static_cast<uint32_t>(j), magic));
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane j supplies the address of 4 consecutive 16-bit elements; lane i of
// the group receives element i of the four 16-element rows those 16 pieces
// form when laid end to end in lane order (row e = pieces of lanes 4e..4e+3).
// So if lane j points at M[r0 + j/4][c0 + 4*(j%4)] of a row-major matrix M,
// lane i receives M[r0 + e][c0 + i] for e = 0..3: four rows of one column.
__device__ __forceinline__ v4s lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(p));
}

// any lane of the wave
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Order LDS writes before later LDS reads of other lanes of the same wave
// (LDS accesses of one wave are executed in order; this only stops the
// compiler from moving memory operations across the point).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace pa
