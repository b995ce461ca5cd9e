// Bandwidth probe (include/pa_probe.h): plain streaming read, copy and write
// kernels over a flat device buffer, used only to measure what HBM delivers
// to a simple access pattern on this part.  Each lane moves 16-byte pieces;
// the grid strides over the buffer in steps of (workgroups x 256 lanes x U
// pieces), so every workgroup keeps U independent 16-byte loads per lane in
// flight.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

template <int U>
__global__ __launch_bounds__(kThreads) void probe_read(const u32x4* __restrict__ src, int64_t n,
                                                       uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads * U;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * kThreads * U + threadIdx.x;
  for (; i + (U - 1) * kThreads < n; i += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * kThreads];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (int u = 0; u < U; ++u) {  // ragged tail
    const int64_t j = i + u * kThreads;
    if (j < n) {
      const u32x4 v = src[j];
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  // a value no test buffer produces: keeps the loads without writing
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

template <int U>
__global__ __launch_bounds__(kThreads) void probe_copy(const u32x4* __restrict__ src, int64_t n,
                                                       u32x4* __restrict__ dst) {
  const int64_t stride = (int64_t)gridDim.x * kThreads * U;
  for (int64_t i = (int64_t)blockIdx.x * kThreads * U + threadIdx.x; i < n; i += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + u * kThreads;
      v[u] = j < n ? src[j] : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + u * kThreads;
      if (j < n) dst[j] = v[u];
    }
  }
}

template <int U>
__global__ __launch_bounds__(kThreads) void probe_write(int64_t n, u32x4* __restrict__ dst) {
  const int64_t stride = (int64_t)gridDim.x * kThreads * U;
  for (int64_t i = (int64_t)blockIdx.x * kThreads * U + threadIdx.x; i < n; i += stride) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + u * kThreads;
      if (j < n) dst[j] = u32x4{0, 0, 0, 0};
    }
  }
}

template <int U>
int launch(int mode, const void* src, void* dst, int64_t n, int wgs, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(wgs)), block(kThreads);
  if (mode == 0)
    hipLaunchKernelGGL(probe_read<U>, grid, block, 0, s, static_cast<const u32x4*>(src), n,
                       static_cast<uint32_t*>(dst));
  else if (mode == 1)
    hipLaunchKernelGGL(probe_copy<U>, grid, block, 0, s, static_cast<const u32x4*>(src), n,
                       static_cast<u32x4*>(dst));
  else
    hipLaunchKernelGGL(probe_write<U>, grid, block, 0, s, n, static_cast<u32x4*>(dst));
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace

extern "C" int pa_probe_stream(int mode, const void* src, void* dst, int64_t bytes,
                               int workgroups, int unroll, void* stream) {
  if (mode < 0 || mode > 2 || bytes <= 0 || bytes % 16 != 0 || workgroups < 1 ||
      workgroups > 65535 || dst == nullptr || (mode != 2 && src == nullptr) ||
      (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0)
    return -1;
  const int64_t n = bytes / 16;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  switch (unroll) {
    case 1: return launch<1>(mode, src, dst, n, workgroups, s);
    case 2: return launch<2>(mode, src, dst, n, workgroups, s);
    case 4: return launch<4>(mode, src, dst, n, workgroups, s);
    case 8: return launch<8>(mode, src, dst, n, workgroups, s);
    default: return -1;
  }
}
