/*
 * zs_host.h -- C ABI of libzs_host: the ZeRO-Offload form of one rank's
 * shard step, run by the host CPU over optimizer state kept in host memory.
 *
 * Source: "Chapter 9: Distributed Training and Data Parallelism", section
 * 9.4.3 (ZeRO-Offload: the optimizer state lives in CPU memory; after the
 * backward pass the gradients go to the CPU over PCIe, the CPU runs the Adam
 * update on its state, and the updated parameters return to the GPU).
 *
 * The step computes exactly what zs_shard_step of include/zs.h computes (the
 * same reduce, AdamW, decay reading and bf16 cast, binary32 one operation at
 * a time, no fused multiply-add, IEEE divide and square root, denormals
 * kept), so its results are bitwise equal to the GPU path on the same
 * inputs.  Buffers are HOST memory owned by the caller.
 */
#ifndef ZS_HOST_H_
#define ZS_HOST_H_

#include <stdint.h>

#include "zs.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * One shard step on the host, synchronous, using `nthreads` threads
 * (0 = the OpenMP default).
 *
 *   master, m, v : HOST fp32 [n], read and updated in place
 *   param_bf16   : HOST bf16 [n], written only
 *   grads        : k HOST pointers, each bf16 [n], read only (left fold
 *                  j = 0 .. k-1)
 *   segs, nseg   : HOST segment table (same layout and lookup rule as the
 *                  device table of zs.h); here its order IS checked
 *   hparams, step: as zs_shard_step
 *
 * No alignment is required.  Returns ZS_OK, ZS_ERR_INVALID_ARGUMENT (null
 * pointer, k or n out of range, step < 1, bad hparams, unsorted table or a
 * first start other than 0, nthreads < 0), ZS_ERR_TOO_MANY_SEGMENTS or
 * ZS_ERR_ALIASING (an output range overlaps another buffer); nothing is
 * written on error.  The flush-to-zero and denormals-are-zero bits of the
 * calling threads' MXCSR are cleared during the call and restored after it.
 * HBM-free: traffic is n * (26 + 2k) bytes of host DRAM.
 */
int zs_host_shard_step(float *master, float *m, float *v, uint16_t *param_bf16,
                       const uint16_t *const *grads, int k, int64_t n, const zs_segment *segs,
                       int32_t nseg, const zs_hparams *hparams, int64_t step, int nthreads);

/* Threads a call with nthreads = 0 uses. */
int zs_host_max_threads(void);

/* "avx512" when the 16-wide vector path runs on this CPU, else "scalar". */
const char *zs_host_isa(void);

#ifdef __cplusplus
}
#endif

#endif /* ZS_HOST_H_ */
