// GPU side of the seeded synthetic-input generator (synth/__init__.py holds
// the reference definition; the two agree bit for bit, which a GPU test
// checks).  This is input preparation, not part of the method: no reduce,
// no Adam and no round-to-nearest cast.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zsmr_synth.h"

#pragma clang fp contract(off)

namespace {

constexpr int kThreads = 256;

__host__ __device__ inline uint64_t splitmix64(uint64_t x) {
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ inline float normal_at(uint64_t key, int64_t p, float sigma, int32_t outlier) {
    const uint64_t base = key + 4ull * static_cast<uint64_t>(p);
    int32_t s = 0;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const uint64_t d = splitmix64(base + static_cast<uint64_t>(j));
        s += static_cast<int32_t>(d & 0xffffu) + static_cast<int32_t>((d >> 16) & 0xffffu) +
             static_cast<int32_t>((d >> 32) & 0xffffu) + static_cast<int32_t>(d >> 48);
    }
    const float z = static_cast<float>(s - 393210) * 0x1p-16f;   // exact
    float x = z * sigma;
    if (outlier) {
        const uint64_t d3 = splitmix64(base + 3ull);
        if (d3 % 10000ull < static_cast<uint64_t>(outlier)) x = x * 100.0f;
    }
    return x;
}

__device__ inline uint16_t trunc16(float x, int32_t dtype) {
    const uint32_t u = __float_as_uint(x);
    if (dtype == ZSMR_SYNTH_BF16) return static_cast<uint16_t>(u >> 16);
    const uint32_t sign = (u >> 16) & 0x8000u;
    const int32_t e = static_cast<int32_t>((u >> 23) & 0xffu);
    const uint32_t mant = u & 0x7fffffu;
    const int32_t big = e - 127 + 15;
    if (big >= 31) return static_cast<uint16_t>(sign | 0x7bffu);
    if (big >= 1) return static_cast<uint16_t>(sign | (static_cast<uint32_t>(big) << 10) | (mant >> 13));
    if (e == 0) return static_cast<uint16_t>(sign);
    const int32_t sh = 126 - e;
    return static_cast<uint16_t>(sign | (sh < 32 ? ((mant | 0x800000u) >> sh) : 0u));
}

__global__ __launch_bounds__(kThreads) void fill16_kernel(uint16_t* dst, int64_t row_stride,
                                                          int64_t n, int64_t p0, int64_t p_valid,
                                                          uint32_t seed, int32_t tag, int32_t rank0,
                                                          int32_t step, float sigma, int32_t dtype,
                                                          int32_t outlier) {
    const int32_t r = blockIdx.y;
    const uint64_t key = splitmix64(static_cast<uint64_t>(seed) ^ (static_cast<uint64_t>(tag) << 56) ^
                                    (static_cast<uint64_t>(rank0 + r) << 40) ^
                                    (static_cast<uint64_t>(step) << 32));
    uint16_t* row = dst + static_cast<int64_t>(r) * row_stride;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t k = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; k < n; k += stride)
        row[k] = k < p_valid ? trunc16(normal_at(key, p0 + k, sigma, outlier), dtype) : 0;
}

__global__ __launch_bounds__(kThreads) void fill32_kernel(float* dst, int64_t n, int64_t p0,
                                                          int64_t p_valid, uint64_t key, float sigma) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t k = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; k < n; k += stride)
        dst[k] = k < p_valid ? normal_at(key, p0 + k, sigma, 0) : 0.0f;
}

bool ids_ok(uint32_t, int32_t tag, int32_t rank, int32_t step) {
    return tag >= 0 && tag < 256 && rank >= 0 && rank < 65536 && step >= 0 && step < 256;
}

unsigned blocks_for(int64_t n, int64_t cap) {
    int64_t b = (n + kThreads - 1) / kThreads;
    if (b > cap) b = cap;
    return static_cast<unsigned>(b < 1 ? 1 : b);
}

}  // namespace

extern "C" int32_t zsmr_synth_fill16(void* dst, int32_t rows, int64_t row_stride, int64_t n,
                                     int64_t p0, int64_t p_valid, uint32_t seed, int32_t tag,
                                     int32_t rank0, int32_t step, float sigma, int32_t dtype,
                                     int32_t outlier_permyriad, hipStream_t stream) {
    if (!dst || rows < 1 || rows > 65535 || n < 0 || p0 < 0 || row_stride < (rows > 1 ? n : 0))
        return 1;
    if (!ids_ok(seed, tag, rank0, step) || rank0 + rows > 65536) return 1;
    if ((dtype != ZSMR_SYNTH_BF16 && dtype != ZSMR_SYNTH_FP16) || outlier_permyriad < 0) return 1;
    if (reinterpret_cast<uintptr_t>(dst) % 2) return 1;
    if (n == 0) return 0;
    const dim3 grid(blocks_for(n, 4096), static_cast<unsigned>(rows));
    hipLaunchKernelGGL(fill16_kernel, grid, dim3(kThreads), 0, stream, static_cast<uint16_t*>(dst),
                       row_stride, n, p0, p_valid, seed, tag, rank0, step, sigma, dtype,
                       outlier_permyriad);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}

extern "C" int32_t zsmr_synth_fill32(float* dst, int64_t n, int64_t p0, int64_t p_valid,
                                     uint32_t seed, int32_t tag, int32_t rank, int32_t step,
                                     float sigma, hipStream_t stream) {
    if (!dst || n < 0 || p0 < 0 || !ids_ok(seed, tag, rank, step)) return 1;
    if (reinterpret_cast<uintptr_t>(dst) % 4) return 1;
    if (n == 0) return 0;
    const uint64_t key = splitmix64(static_cast<uint64_t>(seed) ^ (static_cast<uint64_t>(tag) << 56) ^
                                    (static_cast<uint64_t>(rank) << 40) ^
                                    (static_cast<uint64_t>(step) << 32));
    hipLaunchKernelGGL(fill32_kernel, dim3(blocks_for(n, 4096)), dim3(kThreads), 0, stream, dst, n,
                       p0, p_valid, key, sigma);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}
