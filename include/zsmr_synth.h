/*
 * zsmr_synth.h -- C ABI of synth/libzsmr_synth.so, the GPU side of the seeded
 * synthetic-input generator (not part of the method).
 *
 * Definition (identical to synth/__init__.py, which is the reference for it):
 * key = splitmix64(seed ^ tag<<56 ^ rank<<40 ^ step<<32); for parameter index
 * p the draws are d_j = splitmix64(key + 4p + j); d_0..d_2 give twelve 16-bit
 * integers whose sum minus 393210, times 2^-16, is an Irwin-Hall(12) normal z
 * (exact in fp32); x = fl32(z * sigma); with outliers, x = fl32(x * 100) when
 * d_3 mod 10000 < outlier_permyriad.  16-bit values are x truncated toward
 * zero.  splitmix64 is the SplitMix64 output function (Steele, Lea and Flood,
 * OOPSLA 2014).
 *
 * Layout rule of both fills: position k of row r holds the value for
 * parameter p0 + k of rank rank0 + r when k < p_valid, and 0 otherwise (the
 * zero pad).  Returns 0, or 1 for a bad argument, or 6 for a HIP error.
 * Asynchronous on `stream`; the caller owns `dst`.
 */
#ifndef ZSMR_SYNTH_H
#define ZSMR_SYNTH_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZSMR_SYNTH_FP16 1
#define ZSMR_SYNTH_BF16 2

/* rows x n 16-bit values at dst + r*row_stride (elements). */
int32_t zsmr_synth_fill16(void* dst, int32_t rows, int64_t row_stride, int64_t n, int64_t p0,
                          int64_t p_valid, uint32_t seed, int32_t tag, int32_t rank0,
                          int32_t step, float sigma, int32_t dtype, int32_t outlier_permyriad,
                          hipStream_t stream);

/* n fp32 values (no truncation). */
int32_t zsmr_synth_fill32(float* dst, int64_t n, int64_t p0, int64_t p_valid, uint32_t seed,
                          int32_t tag, int32_t rank, int32_t step, float sigma,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* ZSMR_SYNTH_H */
