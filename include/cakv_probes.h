/* cakv_probes.h -- attainable peaks of the GPU, for pricing measurements.
 *
 * libcakv_probes.so (built beside libcakv.so) holds two measurement kernels
 * that are not part of the attention path: a streaming read of a large
 * buffer (the HBM read bandwidth a kernel can reach) and a loop of
 * independent bf16 MFMAs (the matrix throughput a kernel can reach).  The
 * benchmark reports each roofline fraction against these beside the
 * published peaks.  Both calls are asynchronous on the given stream,
 * allocate nothing and keep no pointer after they return.
 */
#ifndef CAKV_PROBES_H
#define CAKV_PROBES_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read.  Every 16-byte word of buf[0, bytes) is loaded exactly
 * once, with nontemporal loads, by `blocks` workgroups of 256 threads, each
 * taking a contiguous range (eight 16-byte loads in flight per thread);
 * workgroup g writes the XOR of the 32-bit words it read to sink[g], so the
 * reads cannot be dropped and the result can be checked (the XOR of
 * sink[0 .. blocks) is the XOR of the buffer).
 *   buf:    device memory, 16-byte aligned; read only
 *   bytes:  a multiple of 16 (0 reads nothing, each sink word becomes 0)
 *   sink:   device memory of `blocks` uint32, overwritten
 *   blocks: 1 .. 65535, or 0 for 2048
 * Returns 0; -1 for a bad argument (nothing is launched); -4 when the launch
 * fails. */
int cakv_probe_read(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks, hipStream_t stream);

/* bf16 MFMA throughput.  `blocks` workgroups of four waves; every wave
 * issues `iters` rounds of four independent v_mfma_f32_32x32x16_bf16
 * (32,768 flops each), so one call performs blocks * 4 * iters * 4 * 32,768
 * flops.  Each wave writes one float (a sum of its accumulators) to
 * sink[4 * workgroup + wave].
 *   iters:  >= 0
 *   blocks: 1 .. 65535
 *   sink:   device memory of 4 * blocks floats, overwritten
 * Returns 0; -1 for a bad argument (nothing is launched); -4 when the launch
 * fails. */
int cakv_probe_mfma_bf16(int64_t iters, int32_t blocks, float* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CAKV_PROBES_H */
