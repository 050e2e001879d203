/*
 * mdlm_probe.h -- measurement kernels for the roofline of the loss path.
 *
 * Not part of the loss path: these two kernels give the achievable peaks that
 * the loss-path kernels are compared with on the machine at hand (the
 * datasheet peaks assume a clock that power limits may not allow).
 *
 * Both take a HIP stream (NULL = default stream) and return 0 on success or
 * a nonzero HIP error code from the launch; nothing is validated beyond the
 * documented preconditions, which the caller must meet.
 */
#ifndef MDLM_PROBE_H
#define MDLM_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Streaming copy: dst[i] = src[i] for n16 16-byte elements, one element per
 * thread (a one-pass grid of ceil(n16 / 256) blocks of 256 threads).
 *   src, dst  device buffers of n16 * 16 bytes, 16-byte aligned, disjoint.
 *   n16       element count, 0 <= n16 < 2^40.
 */
int mdlm_probe_copy(const void* src, void* dst, int64_t n16, void* stream);

/*
 * MFMA issue loop: `blocks` workgroups of 512 threads (8 waves); each wave
 * runs `iters` iterations of 8 independent v_mfma_f32_32x32x16_bf16 on
 * register operands and writes one float (the sum of its accumulators) to
 * out[block * 8 + wave].  Work: blocks * 8 * iters * 8 * 32768 flops.
 *   out     device buffer of blocks * 8 floats.
 *   blocks  1 .. 65535;  iters  >= 1.
 */
int mdlm_probe_mfma(float* out, int32_t blocks, int32_t iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MDLM_PROBE_H */
