// pa_check_indices: debug validation of the device index arrays the other
// entry points trust (slot ids of reshape_and_cache; block ids and sequence
// lengths of the attention calls).  Not on the hot path.  A slot addresses
// (slot / block_size, slot % block_size) and a sequence of length L reads
// the first ceil(L / block_size) entries of its block-table row [vLLM
// flash_attn.py (e2f56c3), FlashAttentionImpl.forward, slot_mapping and
// block_table; Aphrodite flash_attn.py, FlashAttentionMetadata].
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

__global__ __launch_bounds__(64) void check_zero_kernel(int32_t* counts) {
  if (threadIdx.x < 3) counts[threadIdx.x] = 0;
}

// Grid-stride over the slots, then over the sequences (one wave per
// sequence at a time).  Each wave adds its counts with one atomic per
// counter that is not zero.
__global__ __launch_bounds__(256) void check_kernel(const int64_t* slot_mapping, int64_t num_tokens,
                                                    const int32_t* block_table, int64_t bt_stride,
                                                    const int32_t* seq_lens, int num_seqs,
                                                    int64_t num_blocks, int block_size,
                                                    int32_t* counts) {
  const int lane = threadIdx.x & 63;
  const int64_t n_slots = num_blocks * block_size;
  int bad_slot = 0, bad_id = 0, bad_len = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < num_tokens; i += stride)
    bad_slot += slot_mapping[i] >= n_slots ? 1 : 0;
  const int waves = gridDim.x * (blockDim.x / 64);
  for (int b = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6); b < num_seqs; b += waves) {
    const int L = seq_lens[b];
    const int64_t used = L > 0 ? ((int64_t)L + block_size - 1) / block_size : 0;
    if (L < 0 || used > bt_stride) {
      // a negative length, or one whose blocks cannot fit in a row
      bad_len += lane == 0 ? 1 : 0;
      continue;
    }
    const int32_t* row = block_table + (int64_t)b * bt_stride;
    for (int64_t j = lane; j < used; j += 64) {
      const int32_t id = row[j];
      bad_id += (id < 0 || id >= num_blocks) ? 1 : 0;
    }
  }
  const int s = static_cast<int>(wave_sum(static_cast<float>(bad_slot)));
  const int d = static_cast<int>(wave_sum(static_cast<float>(bad_id)));
  const int l = static_cast<int>(wave_sum(static_cast<float>(bad_len)));
  if (lane == 0) {
    if (s) atomicAdd(&counts[0], s);
    if (d) atomicAdd(&counts[1], d);
    if (l) atomicAdd(&counts[2], l);
  }
}

}  // namespace

int launch_check_indices(const int64_t* slot_mapping, int64_t num_tokens,
                         const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens,
                         int num_seqs, int64_t num_blocks, int block_size, int32_t* counts,
                         hipStream_t stream) {
  hipLaunchKernelGGL(check_zero_kernel, dim3(1), dim3(64), 0, stream, counts);
  const int64_t work = num_tokens > (int64_t)num_seqs * 64 ? num_tokens : (int64_t)num_seqs * 64;
  const int64_t blocks = (work + 255) / 256;
  const unsigned grid = static_cast<unsigned>(blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks));
  hipLaunchKernelGGL(check_kernel, dim3(grid), dim3(256), 0, stream, slot_mapping, num_tokens,
                     block_table, bt_stride, seq_lens, num_seqs, num_blocks, block_size, counts);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace pa
