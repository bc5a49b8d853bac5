/*
 * ubs_bench.h -- measurement helpers of libubs.so.
 *
 * Not part of the method: two small kernels that measure what the GPU sustains, so that
 * the method's kernels can be read against a measured ceiling beside the published one
 * (the roofline figures of bench.py). Same conventions as ubs.h: device pointers, the
 * current device, work enqueued on `stream`, UBS_OK or a negative UBS_ERR_* code.
 */
#ifndef UBS_BENCH_H
#define UBS_BENCH_H

#include "ubs.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * ubs_bench_read -- reads `bytes` of device memory once (16-byte loads, each of 8
 * work-groups per CU streaming one contiguous share) and writes nothing, except in the
 * case where the xor of everything read equals a fixed constant, when it writes that
 * value to sink[0]. Time it with events to get the plain read rate.
 *   buf    device memory, 16-byte aligned, `bytes` >= 16 (a tail shorter than 16 bytes
 *          is not read)
 *   sink   device memory of at least 4 bytes
 * Errors: UBS_ERR_INVALID_ARGUMENT (NULL, misaligned, too small), UBS_ERR_HIP.
 */
int ubs_bench_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

/*
 * ubs_bench_mfma -- ubs_bench_mfma_waves() waves (two per SIMD) each run `iters` rounds of
 * four independent 32x32x16 bf16 MFMAs on register operands: 4 * 32768 flops per round
 * and wave, no memory traffic. out[0] is written only if a result equals a fixed value
 * it does not take. Time it with events for the matrix cores' rate at the clock the
 * GPU holds under that load.
 *   iters  > 0
 *   out    device memory of at least 4 bytes
 * Errors: UBS_ERR_INVALID_ARGUMENT, UBS_ERR_HIP.
 */
int ubs_bench_mfma(int32_t iters, float* out, hipStream_t stream);
int64_t ubs_bench_mfma_waves(void); /* 0 if the device cannot be queried */

#ifdef __cplusplus
}
#endif

#endif /* UBS_BENCH_H */
