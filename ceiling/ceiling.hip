// Pure-read and pure-write reference streams for gfx950 (C ABI in
// include/zsmr_ceiling.h).  Measurement only: they bound what a kernel that
// reads R bytes and writes W bytes can take on this device.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zsmr_ceiling.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kBurst = 32;         // vectors per lane per burst: 32 KB per wave
constexpr int kRegionBurst = 8;    // contiguous-region reads: 8 KB per wave per burst
constexpr int64_t kChunk = int64_t(kBurst) * 64;
constexpr int64_t kRegionChunk = int64_t(kRegionBurst) * 64;

// the read streams store only if the XOR of what they read equals this value
__device__ __forceinline__ void keep(u32x4 acc, u32x4* sink) {
    if (acc[0] == 0x9e3779b9u && acc[1] == 0x7f4a7c15u && acc[2] == 0xf39cc060u &&
        acc[3] == 0x5ced1e2bu)
        sink[0] = acc;
}

// Wave w reads vectors [w * kChunk, (w + 1) * kChunk) as one burst; the last,
// partial chunk goes vector by vector.
__global__ __launch_bounds__(kThreads) void read_bursts(const u32x4* src, int64_t nvec, u32x4* sink) {
    const int64_t lane = threadIdx.x & 63;
    const int64_t first = ((int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6)) * kChunk;
    u32x4 acc = {0u, 0u, 0u, 0u};
    if (first + kChunk <= nvec) {
        u32x4 r[kBurst];
#pragma unroll
        for (int i = 0; i < kBurst; ++i) r[i] = __builtin_nontemporal_load(src + first + lane + i * 64);
        __builtin_amdgcn_sched_barrier(0);   // the whole burst is issued before any is used
#pragma unroll
        for (int i = 0; i < kBurst; ++i) acc ^= r[i];
    } else {
        for (int64_t v = first + lane; v < nvec; v += 64) acc ^= __builtin_nontemporal_load(src + v);
    }
    keep(acc, sink);
}

// Wave w reads the contiguous region [w * per, min((w + 1) * per, nvec)) in
// bursts of kRegionChunk vectors (per is a multiple of kRegionChunk).
__global__ __launch_bounds__(kThreads) void read_regions(const u32x4* src, int64_t nvec, int64_t per,
                                                         u32x4* sink) {
    const int64_t lane = threadIdx.x & 63;
    const int64_t lo = ((int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6)) * per;
    const int64_t hi = lo + per < nvec ? lo + per : nvec;
    u32x4 acc = {0u, 0u, 0u, 0u};
    int64_t c = lo;
    for (; c + kRegionChunk <= hi; c += kRegionChunk) {
        u32x4 r[kRegionBurst];
#pragma unroll
        for (int i = 0; i < kRegionBurst; ++i) r[i] = __builtin_nontemporal_load(src + c + lane + i * 64);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kRegionBurst; ++i) acc ^= r[i];
    }
    for (int64_t v = c + lane; v < hi; v += 64) acc ^= __builtin_nontemporal_load(src + v);
    keep(acc, sink);
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void write_bursts(u32x4* dst, int64_t nvec, uint32_t value) {
    const int64_t lane = threadIdx.x & 63;
    const int64_t first = ((int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6)) * kChunk;
    const u32x4 x = {value, value, value, value};
    if (first + kChunk <= nvec) {
#pragma unroll
        for (int i = 0; i < kBurst; ++i) {
            if constexpr (NT)
                __builtin_nontemporal_store(x, dst + first + lane + i * 64);
            else
                dst[first + lane + i * 64] = x;
        }
    } else {
        for (int64_t v = first + lane; v < nvec; v += 64) {
            if constexpr (NT)
                __builtin_nontemporal_store(x, dst + v);
            else
                dst[v] = x;
        }
    }
}

int cu_count() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    return cus;
}

// workgroups of kWaves waves for `waves` waves (0 if it does not fit a grid)
unsigned blocks_for(int64_t waves) {
    const int64_t b = (waves + kWaves - 1) / kWaves;
    return b < 1 ? 1u : (b > 0x7fffffff ? 0u : static_cast<unsigned>(b));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int32_t zsmr_ceiling_read(const void* src, int64_t bytes, int32_t shape, void* sink,
                                     hipStream_t stream) {
    if (bytes < 0 || bytes % 16 != 0) return 1;
    if (shape != ZSMR_CEILING_BURSTS && shape != ZSMR_CEILING_REGIONS) return 1;
    const int64_t nvec = bytes / 16;
    if (nvec == 0) return 0;   // nothing is touched, whatever the pointers
    if (!src || !sink) return 1;
    if (!aligned16(src) || !aligned16(sink)) return 5;
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* k = static_cast<u32x4*>(sink);
    if (shape == ZSMR_CEILING_BURSTS) {
        const unsigned grid = blocks_for((nvec + kChunk - 1) / kChunk);
        if (!grid) return 1;
        hipLaunchKernelGGL(read_bursts, dim3(grid), dim3(kThreads), 0, stream, s, nvec, k);
    } else {
        const int64_t waves = int64_t(cu_count()) * kWaves;
        const int64_t each = (nvec + waves - 1) / waves;
        const int64_t per = (each + kRegionChunk - 1) / kRegionChunk * kRegionChunk;
        hipLaunchKernelGGL(read_regions, dim3(static_cast<unsigned>(cu_count())), dim3(kThreads), 0, stream,
                           s, nvec, per, k);
    }
    return hipGetLastError() == hipSuccess ? 0 : 6;
}

extern "C" int32_t zsmr_ceiling_write(void* dst, int64_t bytes, int32_t shape, uint32_t value,
                                      hipStream_t stream) {
    if (bytes < 0 || bytes % 16 != 0) return 1;
    if (shape != ZSMR_CEILING_BURSTS && shape != ZSMR_CEILING_PLAIN) return 1;
    const int64_t nvec = bytes / 16;
    if (nvec == 0) return 0;
    if (!dst) return 1;
    if (!aligned16(dst)) return 5;
    u32x4* d = static_cast<u32x4*>(dst);
    const unsigned grid = blocks_for((nvec + kChunk - 1) / kChunk);
    if (!grid) return 1;
    if (shape == ZSMR_CEILING_BURSTS)
        hipLaunchKernelGGL(write_bursts<true>, dim3(grid), dim3(kThreads), 0, stream, d, nvec, value);
    else
        hipLaunchKernelGGL(write_bursts<false>, dim3(grid), dim3(kThreads), 0, stream, d, nvec, value);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}
