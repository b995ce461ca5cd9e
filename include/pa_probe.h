/*
 * pa_probe.h — measurement probe exported by libpagedattn.so.  Not part of
 * the attention path: it gives a measured-achievable HBM bandwidth to set
 * beside the vendor peak when the attention kernels are reported as a
 * fraction of their roofline.
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pa_probe_stream — one streaming pass over device memory.
 *   mode 0: read `bytes` of src (16-byte loads, `unroll` independent loads
 *           per lane in flight); nothing is written unless the data sum to a
 *           value the caller's buffers never hold (dst then takes one word).
 *   mode 1: copy `bytes` from src to dst (16-byte loads and stores).
 *   mode 2: write `bytes` of dst (16-byte stores of zero).
 * src / dst: device pointers, 16-byte aligned; bytes a positive multiple of
 * 16; workgroups 1..65535 (256 threads each) sizes the grid; unroll one of
 * 1, 2, 4, 8.  Enqueued on `stream`; returns 0, PA_ERR_INVALID (-1) or
 * PA_ERR_HIP (-3).  The caller owns both buffers (dst needs 4 bytes in mode 0).
 */
int pa_probe_stream(int mode, const void* src, void* dst, int64_t bytes, int workgroups,
                    int unroll, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */
