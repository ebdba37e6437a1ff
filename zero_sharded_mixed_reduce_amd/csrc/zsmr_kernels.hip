// gfx950 kernels of the ZeRO shard step.
//
// One streaming pass per launch.  The path is bound by HBM bandwidth (about
// 0.3-0.6 flop per byte), so there is no MFMA: every lane owns 8 elements of
// a 512-element wave tile, reads each 16-bit gradient row and the fp32
// master/m/v once, and writes each output once.  LDS only holds the results
// whose stores are deferred (the fused step).  The same device code, selected
// by the MODE bits, gives the fused step and the unfused reduce-only,
// Adam-only, cast-only and init launches, so the fused and unfused results
// are the same bits.
//
// Arithmetic (the pages: "The four schemes", Base._adam and the schemes'
// reduce_scatter_mean / astype casts; "ZeRO and FSDP", ZeroAdam.step):
//  - reduce: fp32 accumulation strictly in rank order 0..N-1, then / N;
//  - Adam: one IEEE fp32 rounding per operation, no contraction into FMA
//    (the file is compiled with contraction off and the pragma below),
//    correctly rounded division and square root;
//  - cast: round to nearest even (bf16 by the integer carry rule; fp16 by
//    v_cvt_f16_f32 in the default round-to-nearest-even mode).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "zsmr.h"
#include "zsmr_launch.h"

#pragma clang fp contract(off)

// Compile-time shape of the streaming loops (tuned on MI355X; results never
// depend on them).
#ifndef ZSMR_NT_LOAD
#define ZSMR_NT_LOAD 1          // non-temporal loads of streamed data
#endif
#ifndef ZSMR_NT_STORE
#define ZSMR_NT_STORE 1         // non-temporal stores
#endif
// Gradient rows per double-buffered load batch.  Measured on MI355X,
// alternating processes on one box: the deferred-write kernel on share64
// (tuned windows) 2.694-2.730 ms with 4 against 2.742-2.769 with 8 (154
// against 184 VGPRs).  The direct kernel takes 8 or 12 by row count (the
// measurements are beside direct_row_batch below).
#ifndef ZSMR_ROW_BATCH
#define ZSMR_ROW_BATCH 8        // direct kernel's default batch
#endif
#ifndef ZSMR_DEFER_BATCH
#define ZSMR_DEFER_BATCH 4      // deferred-write kernel
#endif
#ifndef ZSMR_COPY_UNROLL
#define ZSMR_COPY_UNROLL 1      // vectors in flight per lane in the 2-byte copy
#endif
#ifndef ZSMR_COPY_BURST_BYTES
#define ZSMR_COPY_BURST_BYTES 512   // copies: bytes per lane per register burst (32 KB per wave)
#endif

namespace zsmr {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRowBatch = ZSMR_ROW_BATCH;
constexpr int kRowBatchWide = 12;
constexpr int kDeferBatch = ZSMR_DEFER_BATCH;
constexpr int kCopyUnroll = ZSMR_COPY_UNROLL;
// Grids.  0 = one unit of work per thread (a wave tile per wave for the step
// kernels, a 32 KB burst per wave for the copies), as many workgroups as the
// launch needs, handed out by the hardware in order as earlier ones finish:
// the work in flight stays one contiguous window and no waves straggle at
// the end.  k > 0 = a grid-stride grid of k workgroups per CU.
// The direct step kernel, measured on MI355X (each pair on one box), one
// tile per wave against 2 per CU grid-stride: 4 rows 5.89 against 5.28
// TB/s, 8 rows 5.87-5.91 against 5.53, 12 rows 6.14-6.19 against 5.45;
// GPT-2 small's 15.5M-element shard at 8 rows 6.05-6.09 against 5.62-5.69.
std::atomic<int> g_step_bpc{0};
constexpr int kNarrowCopyBpc = 4;   // the 2-byte copies: 4 per CU
// The burst copies (receive and ZeRO-3 gather), measured the same way: a
// 14.77 GB copy between fresh buffers, one burst per wave 6.22 TB/s against
// 6.07 grid-stride at 1 per CU; the share64 receive 6.00-6.03 against
// 5.82-5.84 (2 per CU 5.84-5.86, 4 per CU 5.94-5.96).
std::atomic<int> g_copy_bpc{0};
// The copies' share of regions for each even-numbered XCD against each odd
// one, in thousandths (the measurements are beside XcdSplit below).
std::atomic<int> g_xcd_even_permille{1200};
// the fused step's deferred-write kernel: tiles kept in LDS per wave with
// write windows (0 = write at once with step_vec8_kernel).  With windows and
// a ring of at most 3 tiles (72 KB per workgroup), two workgroups run per CU
// (two waves per SIMD): one wave's loads stay in flight while the other runs
// its Adam tail.  Measured on MI355X, share64, per step: 3 tiles x 2
// workgroups 2.78 ms, 2 x 2 2.85 ms, 5 x 1 3.07 ms; without windows one
// workgroup per CU is 5% faster (16-24 rows).
std::atomic<int> g_defer_tiles{3};
constexpr int kRingTwoPerCu = 3;
// ... used when a step reduces at least this many rows.  Measured on MI355X,
// one box, 97,375,000 elements, against the direct kernel with one tile per
// wave: 16 rows 5.57-5.62 against 5.74-5.81 TB/s, 20 rows 5.62-5.64 against
// 5.90-5.99, 24 rows 5.99-6.09 against 5.66-5.69, 32 rows 6.12-6.15 against
// 5.48-5.50, 64 rows 6.05 against 5.29; the 1.558e9-element, 16-rank world
// 16.94 against 15.96-15.99 ms per step.
std::atomic<int> g_defer_min_rows{24};
// without windows the ring holds at most this many tiles: smaller bursts at
// ring-full beat larger ones (8-24 rows: 2 tiles up to 5% faster than 5)
constexpr int kRingWithoutWindows = 2;
// Its write windows, in ns (cycle 0: none), converted to clock ticks per
// device.  Measured on MI355X, share64, 3 tiles x 2 workgroups per CU:
// 74 / 12 / 1 / 2 us (cycle, write, margin, lead) gave 2.779 ms per step.
// The read phase, ~63 us, is about the time two waves per SIMD take to fill
// their 3-tile rings: a longer cycle idles until its window, a shorter one
// pays the window more often; +-4 us cost 3-5%.  The best window follows
// the device's read rate, so callers that can time the step may tune it;
// the default is the window a tuning over 31 candidates picked on three
// boxes of three (72 / 11 / 1 / 4 us, 2.70-2.72 ms per step).
struct WindowNs {
    int64_t cycle, write, margin, lead;
};
WindowNs g_window_ns{72000, 11000, 1000, 4000};
// the four values change together: a launch reads them under this lock, so
// it never sees half of a new window
std::mutex g_window_lock;
// The cycle as set is the one for 64 rows of 16-bit gradients.  A wave's
// ring fills in a time proportional to the bytes its tiles move per element
// (2 * rows + 26: the gradient rows, master, m and v read and written, the
// 16-bit copy written), so a step of other row counts scales the cycle by
// (2 * rows + 26) / 154; the write window, margin and lead stay as set.
// Measured on MI355X, 97,375,000 elements, 3 tiles x 2 workgroups per CU
// (no windows / scaled / the 64-row cycle unscaled): 16 rows 1.007 / 1.008
// (x1.1: 0.988) ms, 24 rows 1.292 / 1.190, 32 rows 1.577 / 1.421 / 2.260,
// 48 rows 2.186 / 1.858 / 2.276.
constexpr int64_t kWindowRefBytes = 2 * 64 + 26;
constexpr int64_t kMaxCycleTicks = int64_t(1) << 30;
// Windows pay from 16 rows on; with 8 the ring fills so fast that the
// windowed kernel ran 19% slower than the direct one (4-13% with windows
// sized for 8 rows).
constexpr int kWindowMinRows = 16;

// Streamed data is touched once per step: non-temporal loads and stores keep
// it from displacing anything useful in L2 and the MALL.
template <typename T>
__device__ __forceinline__ T ld(const T* p) {
#if ZSMR_NT_LOAD
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}
template <typename T>
__device__ __forceinline__ void st(T* p, T v) {
#if ZSMR_NT_STORE
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

// ---------------------------------------------------------------- formats --
template <int DT>
__device__ __forceinline__ float widen(uint32_t h);
template <>
__device__ __forceinline__ float widen<ZSMR_BF16>(uint32_t h) {
    return __uint_as_float(h << 16);
}
template <>
__device__ __forceinline__ float widen<ZSMR_FP16>(uint32_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

template <int DT>
__device__ __forceinline__ uint32_t narrow(float x);
template <>
__device__ __forceinline__ uint32_t narrow<ZSMR_BF16>(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;   // quiet NaN
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
template <>
__device__ __forceinline__ uint32_t narrow<ZSMR_FP16>(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

template <int DT>
__device__ __forceinline__ void unpack8(u32x4 w, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = widen<DT>(w[i] & 0xffffu);
        f[2 * i + 1] = widen<DT>(w[i] >> 16);
    }
}

// The rank-order sum divided by N.  For N a power of two the quotient is
// exact up to the one rounding both forms share, so multiplying by 1/N gives
// the same bits as dividing, and is cheaper.
__device__ __forceinline__ float mean_of(const StepArgs& a, float sum) {
    return a.inv_pow2 ? sum * a.inv_nf : sum / a.nf;
}

// ------------------------------------------------------------------- Adam --
__device__ __forceinline__ void adam1(const AdamK& k, float g, float& w, float& m, float& v) {
    m = k.c1 * m + k.c1m * g;
    v = k.c2 * v + (k.c2m * g) * g;
    const float mh = m / k.bc1;
    const float vh = v / k.bc2;
    const float d = __builtin_sqrtf(vh) + k.eps;
    const float u = (k.lr * mh) / d;
    w = w - u;
}

// -------------------------------------------------- 16-bit group store --
// Four 16-bit results at p (DV: widest store the address allows).
template <int DV>
__device__ __forceinline__ void store4x16(uint16_t* p, const uint32_t* h) {
    if constexpr (DV >= 4) {
        u32x2 w;
        w[0] = h[0] | (h[1] << 16);
        w[1] = h[2] | (h[3] << 16);
        st(reinterpret_cast<u32x2*>(p), w);
    } else if constexpr (DV == 2) {
        st(reinterpret_cast<uint32_t*>(p), h[0] | (h[1] << 16));
        st(reinterpret_cast<uint32_t*>(p + 2), h[2] | (h[3] << 16));
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) st(p + i, static_cast<uint16_t>(h[i]));
    }
}

// ------------------------------------------- two 4-element groups per lane --
// A lane owns elements e0..e0+3 and e1..e1+3.  The store map, which every
// kernel uses for its stores and the direct kernels for everything: a wave
// owns 512 consecutive elements, lane l the groups at 4l and 256+4l
// (e1 = e0 + 256), so every load and store instruction of the wave covers one
// contiguous run (1 KB of fp32, 512 B of 16-bit data).  The deferred kernel
// computes in the contiguous map, e1 = e0 + 4: 8 consecutive elements per
// lane, one 16-byte load per gradient row.
struct Groups {
    // the 8 raw 16-bit words of one row in the store map, packed two per dword
    __device__ static __forceinline__ u32x4 load16raw(const uint16_t* p, uint32_t e0, uint32_t e1) {
        const u32x2 a = ld(reinterpret_cast<const u32x2*>(p + e0));
        const u32x2 b = ld(reinterpret_cast<const u32x2*>(p + e1));
        u32x4 r;
        r[0] = a[0];
        r[1] = a[1];
        r[2] = b[0];
        r[3] = b[1];
        return r;
    }
    template <int DV>
    __device__ static __forceinline__ void store16(uint16_t* p, uint32_t e0, uint32_t e1, const uint32_t* h) {
        store4x16<DV>(p + e0, h);
        store4x16<DV>(p + e1, h + 4);
    }
    __device__ static __forceinline__ void load32(const float* p, uint32_t e0, uint32_t e1, float* f) {
        const f32x4 a = ld(reinterpret_cast<const f32x4*>(p + e0));
        const f32x4 b = ld(reinterpret_cast<const f32x4*>(p + e1));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[i] = a[i];
            f[4 + i] = b[i];
        }
    }
    __device__ static __forceinline__ void store32(float* p, uint32_t e0, uint32_t e1, const float* f) {
        f32x4 a, b;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[i] = f[i];
            b[i] = f[4 + i];
        }
        st(reinterpret_cast<f32x4*>(p + e0), a);
        st(reinterpret_cast<f32x4*>(p + e1), b);
    }
};

template <int RB>
__device__ __forceinline__ void load_rows(const StepArgs& a, int r, uint32_t e0, uint32_t e1, u32x4* buf) {
    // Rows past the last one are clamped to it: every load is issued (so the
    // compiler can count them) and add_rows() skips the extra ones.  Those
    // re-reads are plain loads, which the L2 keeps and merges; as
    // non-temporal loads about one in 25 of them went to DRAM again
    // (measured on MI355X, 16 rows in 12-row batches: DRAM reads 1.020x the
    // algorithmic bytes against 1.000x, and the launch 1.5% slower).
#pragma unroll
    for (int k = 0; k < RB; ++k) {
        if (r + k < a.nrows) {
            buf[k] = Groups::load16raw(a.grads + (int64_t)(r + k) * a.row_stride, e0, e1);
        } else {
            const uint16_t* p = a.grads + (int64_t)(a.nrows - 1) * a.row_stride;
            const u32x2 x = *reinterpret_cast<const u32x2*>(p + e0);
            const u32x2 y = *reinterpret_cast<const u32x2*>(p + e1);
            buf[k] = u32x4{x[0], x[1], y[0], y[1]};
        }
    }
}

template <int GDT, int RB>
__device__ __forceinline__ void add_rows(const StepArgs& a, int r, const u32x4* buf, float* g) {
#pragma unroll
    for (int k = 0; k < RB; ++k) {
        if (r + k < a.nrows) {
            float t[8];
            unpack8<GDT>(buf[k], t);
#pragma unroll
            for (int j = 0; j < 8; ++j) g[j] = g[j] + t[j];
        }
    }
}

// One lane's 8 elements (groups at e0 and e1) of the launch's MODE; RB
// gradient rows per load batch.
template <int GDT, int PDT, int MODE, int DV, int RB>
__device__ __forceinline__ void body8(const StepArgs& a, uint32_t e0, uint32_t e1) {
    typedef Groups G;
    float g[8];
    float w[8], m[8], v[8];
    if constexpr ((MODE & M_REDUCE) != 0) {
        // rows 1..N-1 in batches, double-buffered so that one batch is in
        // flight while the previous one is added; the sum itself runs
        // strictly in rank order 0, 1, ..., N-1
        u32x4 bufA[RB], bufB[RB];
        const u32x4 row0 = G::load16raw(a.grads, e0, e1);
        int r = 1;
        if (a.nrows > 1) load_rows<RB>(a, r, e0, e1, bufA);
        unpack8<GDT>(row0, g);
        while (r < a.nrows) {
            if (r + RB >= a.nrows) {
                add_rows<GDT, RB>(a, r, bufA, g);
                break;
            }
            load_rows<RB>(a, r + RB, e0, e1, bufB);
            add_rows<GDT, RB>(a, r, bufA, g);
            r += RB;
            if (r + RB >= a.nrows) {
                add_rows<GDT, RB>(a, r, bufB, g);
                break;
            }
            load_rows<RB>(a, r + RB, e0, e1, bufA);
            add_rows<GDT, RB>(a, r, bufB, g);
            r += RB;
        }
        if (a.mean) {
#pragma unroll
            for (int j = 0; j < 8; ++j) g[j] = mean_of(a, g[j]);
        }
        if constexpr ((MODE & M_GOUT) != 0) G::store32(a.g_out, e0, e1, g);
    } else if constexpr ((MODE & (M_ADAM | M_INIT)) != 0) {
        G::load32(a.g_in, e0, e1, g);
    }

    if constexpr ((MODE & M_ADAM) != 0) {
        G::load32(a.master, e0, e1, w);
        G::load32(a.m, e0, e1, m);
        G::load32(a.v, e0, e1, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) adam1(a.k, g[j], w[j], m[j], v[j]);
        G::store32(a.master, e0, e1, w);
        G::store32(a.m, e0, e1, m);
        G::store32(a.v, e0, e1, v);
    } else if constexpr ((MODE & M_INIT) != 0) {
        const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = g[j];
        G::store32(a.master, e0, e1, w);
        G::store32(a.m, e0, e1, z);
        G::store32(a.v, e0, e1, z);
    } else if constexpr ((MODE & M_CAST) != 0) {
        G::load32(a.master, e0, e1, w);
    }

    if constexpr ((MODE & M_CAST) != 0) {
        uint32_t h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) h[j] = narrow<PDT>(w[j]);
        G::template store16<DV>(a.p16, e0, e1, h);
    }
}

// ------------------------------------------------------- one element -----
template <int GDT, int PDT, int MODE>
__device__ __forceinline__ void body1(const StepArgs& a, int64_t e) {
    float g = 0.f;
    if constexpr ((MODE & M_REDUCE) != 0) {
        const uint16_t* p = a.grads + e;
        g = widen<GDT>(p[0]);
        for (int r = 1; r < a.nrows; ++r) g = g + widen<GDT>(p[(int64_t)r * a.row_stride]);
        if (a.mean) g = mean_of(a, g);
        if constexpr ((MODE & M_GOUT) != 0) a.g_out[e] = g;
    } else if constexpr ((MODE & (M_ADAM | M_INIT)) != 0) {
        g = a.g_in[e];
    }
    float w = 0.f;
    if constexpr ((MODE & M_ADAM) != 0) {
        float m = a.m[e], v = a.v[e];
        w = a.master[e];
        adam1(a.k, g, w, m, v);
        a.master[e] = w;
        a.m[e] = m;
        a.v[e] = v;
    } else if constexpr ((MODE & M_INIT) != 0) {
        w = g;
        a.master[e] = w;
        a.m[e] = 0.f;
        a.v[e] = 0.f;
    } else if constexpr ((MODE & M_CAST) != 0) {
        w = a.master[e];
    }
    if constexpr ((MODE & M_CAST) != 0) a.p16[e] = static_cast<uint16_t>(narrow<PDT>(w));
}

// ---------------------------------------------------------------- kernels --
// elements the vector path covers: whole 512-element wave tiles
__host__ __device__ constexpr int64_t vec_elems(int64_t n) { return n / 512 * 512; }

// The elements outside whole tiles, one per lane of workgroup 0: those past
// the last tile and the head before the first.
template <int GDT, int PDT, int MODE>
__device__ __forceinline__ void edges1(const StepArgs& a) {
    if (blockIdx.x != 0) return;
    for (int64_t e = vec_elems(a.n) + threadIdx.x; e < a.n; e += kThreads) body1<GDT, PDT, MODE>(a, e);
    for (int64_t e = (int64_t)threadIdx.x - a.head; e < 0; e += kThreads) body1<GDT, PDT, MODE>(a, e);
}

// Aligned path over vector index i (8 elements each, grid-stride); the
// elements outside whole tiles go one per lane to workgroup 0.
template <int GDT, int PDT, int MODE, int DV, int RB>
__global__ __launch_bounds__(kThreads) void step_vec8_kernel(StepArgs a) {
    // a launch covers fewer than 2^31 elements (the host splits larger
    // pieces), so in-launch offsets are 32-bit
    const uint32_t nv = static_cast<uint32_t>(vec_elems(a.n) >> 3);
    const uint32_t stride = gridDim.x * kThreads;
    for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < nv; i += stride) {
        const uint32_t e0 = (i >> 6) * 512u + (i & 63u) * 4u;   // wave tile, lane group
        body8<GDT, PDT, MODE, DV, RB>(a, e0, e0 + 256u);
    }
    edges1<GDT, PDT, MODE>(a);
}

// Write windows of the deferred-write kernel, in ticks of the chip's
// constant-rate clock (s_memrealtime, 100 MHz; on MI355X the eight XCDs read
// it within a microsecond of each other): in every
// cycle of `cycle` ticks the last `write` ticks are the write window; a wave
// stops issuing loads `margin` ticks before it and resumes `lead` ticks
// before it ends.  cycle == 0: no windows.
struct Window {
    uint32_t cycle, write, margin, lead;
};

__device__ __forceinline__ uint64_t clock_now() { return __builtin_amdgcn_s_memrealtime(); }

// Sleeps until the clock reaches t.  The spin count bounds the wait (about
// 30 ms), so a wave always goes on even if the clock stood still.
__device__ __forceinline__ void wait_clock(uint64_t t) {
    for (int i = 0; i < (1 << 20); ++i) {
        if (clock_now() >= t) break;
        __builtin_amdgcn_s_sleep(1);
    }
}

// The fused step with deferred, windowed writes.  A write stream mixed into
// the 2N-row read stream costs HBM throughput out of proportion to its bytes,
// so each wave keeps the results of its completed wave tiles (master, m and
// v: 96 B per lane per tile; the 16-bit copy is cast from the master when
// the tile is stored) in a ring of KD tiles in LDS
// and writes them only in the write windows, which every wave of the chip
// takes at the same time from the shared clock: HBM then sees long read-only
// stretches and short write-only bursts.  Between windows a wave streams its
// tiles' gradient rows as one double-buffered sequence of row batches, across
// tile boundaries; a tile whose rows straddle a window keeps its partial sum
// in registers.  Wave w owns tiles w, w + W, w + 2W, ... (W waves in the
// grid).  While computing, lane l holds the tile's 8 consecutive elements
// [8l, 8l+8): one 16-byte load per gradient row.  The ring keeps each tile in
// element order, and the flush reads it back in the store map (lane l:
// [4l, 4l+4) and [256+4l, 256+4l+4)), so that every store instruction covers
// one contiguous run; the ring is a wave's own, and a wave's LDS operations
// complete in order, so waves never synchronise.  Results are the same bits
// as step_vec8_kernel's: only the time at which they are stored changes.
// Any number of rows; rows 16-byte aligned (the host checks); a row stride of
// fewer than 2^63 bytes.
template <int GDT, int PDT, int DV, int KD>
__global__ __launch_bounds__(kThreads, KD <= kRingTwoPerCu ? 2 : 1) void step_deferred_kernel(StepArgs a, Window win) {
    constexpr int kWaves = kThreads / 64;
    __shared__ float s_w[kWaves][KD][512];      // a tile's results in element order
    __shared__ float s_m[kWaves][KD][512];
    __shared__ float s_v[kWaves][KD][512];
    const uint32_t lane = threadIdx.x & 63u, wv = threadIdx.x >> 6;
    const uint32_t tiles = static_cast<uint32_t>(vec_elems(a.n) / 512);
    const uint32_t nw = gridDim.x * kWaves;
    const uint32_t wid = blockIdx.x * kWaves + wv;
    const uint32_t mine = wid < tiles ? (tiles - 1 - wid) / nw + 1 : 0;
    const uint32_t bps = (static_cast<uint32_t>(a.nrows) + kDeferBatch - 1) / kDeferBatch;
    const uint32_t nb = mine * bps;
    auto tile_of = [&](uint32_t j) { return (wid + j * nw) * 512u; };

    // the ring: tiles [flushed, done) of this wave are in LDS, not yet stored
    uint32_t done = 0, flushed = 0;
    auto flush = [&]() {
        // the ring holds other lanes' values: release this lane's ring stores
        // (consume) and acquire the other lanes' before reading them back
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        for (uint32_t j = flushed; j < done; ++j) {
            const uint32_t k = j % KD, e0 = tile_of(j) + lane * 4u;
            float w[8], m[8], v[8];
            uint32_t h[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                w[q] = s_w[wv][k][lane * 4u + q];
                w[4 + q] = s_w[wv][k][256u + lane * 4u + q];
                m[q] = s_m[wv][k][lane * 4u + q];
                m[4 + q] = s_m[wv][k][256u + lane * 4u + q];
                v[q] = s_v[wv][k][lane * 4u + q];
                v[4 + q] = s_v[wv][k][256u + lane * 4u + q];
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) h[q] = narrow<PDT>(w[q]);   // the cast, at store time
            Groups::store32(a.master, e0, e0 + 256u, w);
            Groups::store32(a.m, e0, e0 + 256u, m);
            Groups::store32(a.v, e0, e0 + 256u, v);
            Groups::template store16<DV>(a.p16, e0, e0 + 256u, h);
        }
        flushed = done;
    };

    // the clock: cyc = start of the current cycle; used = cycle whose window
    // this wave has already taken
    uint64_t cyc = 0, used = ~0ull;
    auto phase_at = [&](uint64_t now) -> uint64_t {
        if (now - cyc >= win.cycle) cyc = now - now % win.cycle;
        return now - cyc;
    };
    auto phase = [&]() -> uint64_t { return phase_at(clock_now()); };
    // decided on a clock value read one row batch earlier, right after that
    // batch's loads were issued, so the read's latency never delays an issue
    auto near_window = [&](uint64_t seen) -> bool {
        if (!win.cycle) return false;
        return phase_at(seen) + win.write + win.margin >= win.cycle && cyc != used;
    };
    // flush in the window of cycle `want` (waiting for it to open) unless it
    // was taken already or has passed, then idle to the end of the cycle
    auto take_window = [&](uint64_t want) {
        const uint64_t ph = phase();
        if (cyc != want || cyc == used) return;
        if (ph + win.write < win.cycle) wait_clock(cyc + win.cycle - win.write);
        flush();
        used = cyc;
        wait_clock(cyc + win.cycle - win.lead);
    };
    // the ring is full: flush in the next window not yet taken
    auto make_room = [&]() {
        if (win.cycle) {
            phase();
            if (cyc == used) wait_clock(cyc + win.cycle);
            phase();
            take_window(cyc);
        }
        if (done - flushed == KD) flush();   // no window (or the clock stood still)
    };

    // The row streams.  Issue and consume each walk rows 0..N-1 of one tile
    // after another with a running row counter (no division); the issue side
    // also keeps a running row address, and past the last row it keeps
    // re-reading that row (every load is issued unconditionally, so the
    // compiler can count them; consume skips the extra rows).
    const char* const grads = reinterpret_cast<const char*>(a.grads);
    const uint64_t stride_b = static_cast<uint64_t>(a.row_stride) * 2u;
    const uint32_t nrows = static_cast<uint32_t>(a.nrows);
    uint32_t i_tile = 0, i_row = 0, c_row = 0;
    const char* i_ptr = grads;
    // two row buffers, each with the master/m/v of the tile whose last batch
    // it holds: a buffer is consumed before it is issued again, so a tile's
    // state is never overwritten before its Adam step, whatever N
    struct State {
        float w[8], m[8], v[8];
    };
    u32x4 bufA[kDeferBatch], bufB[kDeferBatch];
    State stA, stB;
    float g[8];
    auto issue = [&](u32x4* buf, State& st) {
        const uint32_t e0 = tile_of(i_tile) + lane * 8u, off = e0 * 2u;
#pragma unroll
        for (int k = 0; k < kDeferBatch; ++k) {
            buf[k] = ld(reinterpret_cast<const u32x4*>(i_ptr + off));
            if (i_row + k + 1 < nrows) i_ptr += stride_b;
        }
        i_row += kDeferBatch;
        if (i_row >= nrows) {      // the tile's last batch: its master/m/v come with it
            Groups::load32(a.master, e0, e0 + 4u, st.w);   // contiguous map
            Groups::load32(a.m, e0, e0 + 4u, st.m);
            Groups::load32(a.v, e0, e0 + 4u, st.v);
            ++i_tile;
            i_row = 0;
            i_ptr = grads;
        }
    };
    auto consume = [&](const u32x4* buf, State& st) {
        // rows in rank order; the tile's sum starts from row 0 itself (for
        // N <= kDeferBatch a tile's one batch is both its first and its last)
        const bool full = c_row + kDeferBatch <= nrows;
#pragma unroll
        for (int k = 0; k < kDeferBatch; ++k) {
            if (full || c_row + k < nrows) {
                float t[8];
                unpack8<GDT>(buf[k], t);
                if (k == 0 && c_row == 0) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) g[e] = t[e];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) g[e] = g[e] + t[e];
                }
            }
        }
        c_row += kDeferBatch;
        if (c_row < nrows) return;
        c_row = 0;
        if (a.mean) {
#pragma unroll
            for (int e = 0; e < 8; ++e) g[e] = mean_of(a, g[e]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) adam1(a.k, g[e], st.w[e], st.m[e], st.v[e]);
        if (done - flushed == KD) make_room();
        const uint32_t k = done % KD;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            s_w[wv][k][lane * 8u + e] = st.w[e];
            s_m[wv][k][lane * 8u + e] = st.m[e];
            s_v[wv][k][lane * 8u + e] = st.v[e];
        }
        ++done;
    };

    uint64_t seen = win.cycle ? clock_now() : 0;
    if (nb) issue(bufA, stA);
    for (uint32_t b = 0; b < nb; b += 2) {
        bool hold = near_window(seen);
        uint64_t want = cyc;
        if (!hold && b + 1 < nb) issue(bufB, stB);
        if (win.cycle) seen = clock_now();
        consume(bufA, stA);
        if (hold) {
            take_window(want);
            if (b + 1 < nb) issue(bufB, stB);
            seen = clock_now();
        }
        if (b + 1 >= nb) break;
        hold = near_window(seen);
        want = cyc;
        if (!hold && b + 2 < nb) issue(bufA, stA);
        if (win.cycle) seen = clock_now();
        consume(bufB, stB);
        if (hold) {
            take_window(want);
            if (b + 2 < nb) issue(bufA, stA);
            seen = clock_now();
        }
    }
    flush();
    edges1<GDT, PDT, M_REDUCE | M_ADAM | M_CAST>(a);
}

// Any-alignment path: one element per lane.
template <int GDT, int PDT, int MODE>
__global__ __launch_bounds__(kThreads) void step_scalar_kernel(StepArgs a) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < a.n; e += stride)
        body1<GDT, PDT, MODE>(a, e);
}

// ------------------------------------------------------------ 16-bit copy --
template <int W>
struct VecOf;
template <>
struct VecOf<16> { typedef u32x4 T; };
template <>
struct VecOf<8> { typedef u32x2 T; };
template <>
struct VecOf<4> { typedef uint32_t T; };
template <>
struct VecOf<2> { typedef uint16_t T; };

// The hardware hands workgroup i of a launch to XCD i % 8.  A copy's
// regions (one workgroup's work each) are split between the XCDs in
// contiguous runs, XCD x taking regions [start[x], start[x] + count[x]) in
// order: workgroup i is the (i / 8)-th of XCD i % 8, and one past its XCD's
// count has nothing to do.  Measured on MI355X, a 14 GB copy with one 32 KB
// burst per wave: one contiguous eighth per XCD 6.21 TB/s against 6.05-6.06
// with workgroup i on region i; the share64 receive 4.68-4.69 ms against
// 4.78.  (The direct step kernel ran 4-10% slower remapped, and the deferred
// kernel no faster, so only the copies use it.)
//
// The counts are not equal.  On MI355X the even-numbered XCDs move data
// faster than the odd ones: with equal eighths of the share64 receive the
// even XCDs finished 450-490 us (10%) before the odd ones, whichever
// addresses each copied (eighths swapped between neighbours, or interleaved,
// gave the same split).  The odd XCDs then speed up, so most of that comes
// back on its own, but not all: giving each even XCD r times an odd one's
// regions, the receive took 4.689 ms at r = 1.0, 4.652 at 1.1, 4.603 at 1.2,
// 4.621 at 1.25, 4.645 at 1.3 and 4.732 at 0.9 (three passes, one box).
constexpr uint32_t kXcds = 8;
struct XcdSplit {
    int64_t start[kXcds];
    int64_t count[kXcds];
};
__device__ __forceinline__ int64_t split_region(const XcdSplit& sp, int64_t i) {
    const int64_t x = i % kXcds, j = i / kXcds;
    return j < sp.count[x] ? sp.start[x] + j : -1;
}

// Copy n elements: `head` scalar elements bring dst (and src, which has the
// same alignment modulo W) to a W-byte boundary, then W-byte vectors, then
// the scalar tail.  Region `region` of `regions` takes its share of the
// vectors.  The burst copies lay their chunks out from `pre` vectors before
// the vector body (the body's offset from dst's last 128 KB boundary), so
// that every whole chunk, and every workgroup's four, sits on that grid.
template <int W>
__device__ __forceinline__ void copy_range(const uint16_t* src, uint16_t* dst, int64_t n,
                                           int64_t head, int64_t pre, int64_t region,
                                           int64_t regions) {
    typedef typename VecOf<W>::T V;
    constexpr int E = W / 2;
    const int64_t nb = (n - head) / E;
    const int64_t body_end = head + nb * E;
    const V* s = reinterpret_cast<const V*>(src + head);
    V* d = reinterpret_cast<V*>(dst + head);
    if constexpr (W >= 4) {
        // Register bursts: each wave loads kBurst vectors per lane (32 KB per
        // wave) before it stores any, so every wave alternates a read burst
        // and a write burst; wave w of the regions' waves takes chunks w,
        // w + waves, ... (neighbouring waves, neighbouring chunks).  Chunk c covers body
        // vectors [c * chunk - pre, (c + 1) * chunk - pre); the partial first
        // and last chunks go one guarded vector at a time.
        constexpr int kBurst = ZSMR_COPY_BURST_BYTES / W;
        constexpr int64_t chunk = (int64_t)kBurst * 64;
        const int64_t lane = threadIdx.x & 63u;
        const int64_t waves = regions * (kThreads / 64);
        const int64_t wid = region * (kThreads / 64) + (threadIdx.x >> 6);
        const int64_t nv = nb;
        for (int64_t c = wid; c * chunk < nv + pre; c += waves) {
            const int64_t first = c * chunk - pre;   // the chunk's first body vector (may be < 0)
            const int64_t base = first + lane;
            if (first >= 0 && first + chunk <= nv) {
                V r[kBurst];
#pragma unroll
                for (int i = 0; i < kBurst; ++i) r[i] = ld(s + base + i * 64);
                __builtin_amdgcn_sched_barrier(0);   // the whole read burst is issued first
#pragma unroll
                for (int i = 0; i < kBurst; ++i) st(d + base + i * 64, r[i]);
            } else {
                for (int i = 0; i < kBurst; ++i) {
                    const int64_t v = base + i * 64;
                    if (v >= 0 && v < nv) st(d + v, ld(s + v));
                }
            }
        }
    } else {
        // 2-byte elements (source and destination an odd number of elements
        // apart): one contiguous chunk per region; kCopyUnroll consecutive
        // groups of kThreads elements are loaded before any is stored
        constexpr int64_t group = (int64_t)kThreads * kCopyUnroll;
        const int64_t chunk = ((nb + regions - 1) / regions + group - 1) / group * group;
        const int64_t lo = region * chunk;
        const int64_t hi = lo + chunk < nb ? lo + chunk : nb;
        for (int64_t i = lo + threadIdx.x; i < hi; i += group) {
            V tmp[kCopyUnroll];
#pragma unroll
            for (int k = 0; k < kCopyUnroll; ++k)
                if (i + k * kThreads < hi) tmp[k] = ld(s + i + k * kThreads);
#pragma unroll
            for (int k = 0; k < kCopyUnroll; ++k)
                if (i + k * kThreads < hi) st(d + i + k * kThreads, tmp[k]);
        }
    }
    if (region == 0) {
        const int t = static_cast<int>(threadIdx.x);
        if (t < head) dst[t] = src[t];
        const int64_t tail = n - body_end;
        if (t >= 64 && t - 64 < tail) dst[body_end + (t - 64)] = src[body_end + (t - 64)];
    }
}

// Widest copy vector (bytes) for source and destination addresses a and b:
// the vectors need both equally aligned, so the width divides b - a.
__host__ __device__ inline int copy_width(uintptr_t a, uintptr_t b) {
    const uintptr_t d = a > b ? a - b : b - a;
    if (d % 16 == 0) return 16;
    if (d % 8 == 0) return 8;
    if (d % 4 == 0) return 4;
    return 2;
}

// Elements copied one by one before the vector body.  W-byte vectors need dst
// (and src, equal to it modulo W) W-aligned; the burst copies (W >= 4) also
// start their body on a 128-byte line of dst: HBM writes that cover part of a
// line cost far more than their bytes (measured on MI355X: a copy whose
// destination starts 16-96 bytes into a line runs about 8% slower, whatever
// the source's offset).  At most 63 elements, within one workgroup.
__host__ __device__ inline int64_t head_for(const void* dst, int w, int64_t n) {
    const uintptr_t align = w >= 4 ? 128 : static_cast<uintptr_t>(w);
    const uintptr_t mis = reinterpret_cast<uintptr_t>(dst) % align;
    int64_t h = mis ? static_cast<int64_t>((align - mis) / 2) : 0;
    return h < n ? h : n;
}

// Vectors between dst's last 128 KB boundary and the burst copy's vector body
// (dst + head), where the chunk grid starts (0 for the 2-byte copy).  128 KB
// is one workgroup's four 32 KB bursts.  Measured on MI355X, a 14.77 GB copy
// with source and destination shifted alike: 6.22-6.25 TB/s at multiples of
// 128 KB, 6.15-6.19 at 4-8 KB past one, 6.01-6.04 at 18 KB, 5.87-5.91 at 32-64
// KB (destination alone at 64 KB: 5.99; source alone: 6.13).
__host__ __device__ inline int64_t pre_for(const void* dst, int w, int64_t head) {
    constexpr uintptr_t kGrid = 128 * 1024;
    if (w < 4) return 0;
    const uintptr_t body = reinterpret_cast<uintptr_t>(dst) + static_cast<uintptr_t>(head) * 2;
    return static_cast<int64_t>(body % kGrid / static_cast<uintptr_t>(w));
}

template <int W>
__global__ __launch_bounds__(kThreads) void copy16_kernel(const uint16_t* src, uint16_t* dst,
                                                          int64_t n, int64_t head, int64_t pre,
                                                          XcdSplit sp, int64_t regions) {
    const int64_t r = split_region(sp, blockIdx.x);
    if (r < 0) return;
    copy_range<W>(src, dst, n, head, pre, r, regions);
}

// Block k of `count` (blockIdx.y): n elements from src + k * stride to
// dst + k * stride, each block with the head and chunk grid a copy of its own
// would have (the blocks' destinations need not share their alignment).
template <int W>
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(const uint16_t* src, uint16_t* dst,
                                                               int64_t n, int64_t stride,
                                                               XcdSplit sp, int64_t regions) {
    const int64_t r = split_region(sp, blockIdx.x);
    if (r < 0) return;
    const int64_t k = blockIdx.y;
    const uint16_t* s = src + k * stride;
    uint16_t* d = dst + k * stride;
    const int64_t head = head_for(d, W, n);
    copy_range<W>(s, d, n, head, pre_for(d, W, head), r, regions);
}

constexpr int kMaxGather = 64;
struct GatherArgs {
    const uint16_t* src[kMaxGather];
    int64_t head[kMaxGather];
    int64_t pre[kMaxGather];
    uint16_t* dst;
    int64_t each;
};

template <int W>
__global__ __launch_bounds__(kThreads) void gather16_kernel(GatherArgs g, XcdSplit sp,
                                                            int64_t regions) {
    const int64_t reg = split_region(sp, blockIdx.x);
    if (reg < 0) return;
    const int r = blockIdx.y;
    copy_range<W>(g.src[r], g.dst + (int64_t)r * g.each, g.each, g.head[r], g.pre[r], reg, regions);
}

// ------------------------------------------------------------------ host --
int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (dev >= 0 && dev < 64 && cache[dev].load(std::memory_order_relaxed))
        return cache[dev].load(std::memory_order_relaxed);
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// Workgroups for `work_items` threads' worth of work: all of them (bpc 0),
// or at most bpc per CU, each thread then striding over several items.
unsigned grid_for(int64_t work_items, int bpc) {
    int64_t blocks = (work_items + kThreads - 1) / kThreads;
    if (bpc > 0 && blocks > (int64_t)cu_count() * bpc) blocks = (int64_t)cu_count() * bpc;
    if (blocks < 1) blocks = 1;
    return static_cast<unsigned>(blocks);
}

// `regions` split between the XCDs, each even one weighted
// g_xcd_even_permille / 1000 against 1 for each odd one (floors, then the
// remainder one region at a time from XCD 0 on); *grid receives the
// workgroups that cover the largest share on every XCD.
XcdSplit xcd_split(int64_t regions, unsigned* grid) {
    XcdSplit sp{};
    const int64_t we = g_xcd_even_permille.load(std::memory_order_relaxed), wo = 1000, wsum = (kXcds / 2) * (we + wo);
    int64_t given = 0;
    for (uint32_t x = 0; x < kXcds; ++x) {
        sp.count[x] = regions * (x % 2 == 0 ? we : wo) / wsum;
        given += sp.count[x];
    }
    for (uint32_t x = 0; given < regions; x = (x + 1) % kXcds, ++given) sp.count[x] += 1;
    int64_t at = 0, most = 0;
    for (uint32_t x = 0; x < kXcds; ++x) {
        sp.start[x] = at;
        at += sp.count[x];
        most = sp.count[x] > most ? sp.count[x] : most;
    }
    *grid = static_cast<unsigned>(most * kXcds);
    return sp;
}

inline bool al(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// 16-bit elements per store the destination allows (a lane's groups are 4
// elements, so at most 4)
int dst_vec(const void* p) {
    if (al(p, 8)) return 4;
    if (al(p, 4)) return 2;
    return 1;
}

// ticks of the s_memrealtime clock per second on the current device (0 if
// the runtime does not say: then no windows)
int64_t clock_hz() {
    static std::atomic<int64_t> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (dev >= 0 && dev < 64) {
        const int64_t c = cache[dev].load(std::memory_order_relaxed);
        if (c) return c > 0 ? c : 0;
    }
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) khz = 0;
    const int64_t hz = khz > 0 ? (int64_t)khz * 1000 : -1;
    if (dev >= 0 && dev < 64) cache[dev].store(hz, std::memory_order_relaxed);
    return hz > 0 ? hz : 0;
}

// the windows of a step reducing `rows` rows (the cycle scaled to its bytes
// per element, at most 2^30 ticks)
Window window_ticks(int32_t rows) {
    Window w{0, 0, 0, 0};
    WindowNs ns;
    {
        std::lock_guard<std::mutex> hold(g_window_lock);
        ns = g_window_ns;
    }
    const int64_t hz = clock_hz();
    if (!ns.cycle || !hz || rows < 1) return w;
    auto ticks = [&](int64_t t) { return static_cast<uint32_t>(t * hz / 1000000000); };
    const int64_t cycle = int64_t(ticks(ns.cycle)) * (2 * int64_t(rows) + 26) / kWindowRefBytes;
    w.cycle = static_cast<uint32_t>(cycle < kMaxCycleTicks ? cycle : kMaxCycleTicks);
    w.write = ticks(ns.write);
    w.margin = ticks(ns.margin);
    w.lead = ticks(ns.lead);
    if (w.write < 1 || w.write + w.margin >= w.cycle || w.lead >= w.write) w = Window{0, 0, 0, 0};
    return w;
}

// Which kernel a launch runs, and its shape (every launch of one call runs
// the same plan: the host's cuts keep every operand's alignment).
enum : int { K_SCALAR = 0, K_DIRECT = 1, K_DEFERRED = 2 };
struct Plan {
    int kernel;   // K_*
    int dv;       // 16-bit elements per store of the 16-bit output (4, 2 or 1)
    int kd;       // K_DEFERRED: tiles in each wave's LDS ring
    Window win;   // K_DEFERRED: write windows (cycle 0: none)
    int rb;       // K_DIRECT, launches that reduce: gradient rows per load batch
};

template <int GDT, int PDT, int DV>
hipError_t launch_deferred(const StepArgs& a, const Plan& p, hipStream_t s) {
    const Window w = p.win;
    const int kd = p.kd;
    const int bpc = w.cycle && kd <= kRingTwoPerCu ? 2 : 1;
    const dim3 grid(grid_for(vec_elems(a.n) >> 3, bpc));   // one wave per tile at most
    switch (kd) {
        case 1: hipLaunchKernelGGL((step_deferred_kernel<GDT, PDT, DV, 1>), grid, dim3(kThreads), 0, s, a, w); break;
        case 2: hipLaunchKernelGGL((step_deferred_kernel<GDT, PDT, DV, 2>), grid, dim3(kThreads), 0, s, a, w); break;
        case 3: hipLaunchKernelGGL((step_deferred_kernel<GDT, PDT, DV, 3>), grid, dim3(kThreads), 0, s, a, w); break;
        case 4: hipLaunchKernelGGL((step_deferred_kernel<GDT, PDT, DV, 4>), grid, dim3(kThreads), 0, s, a, w); break;
        default: hipLaunchKernelGGL((step_deferred_kernel<GDT, PDT, DV, 5>), grid, dim3(kThreads), 0, s, a, w); break;
    }
    return hipGetLastError();
}

template <int GDT, int PDT, int MODE>
hipError_t launch_mode(const StepArgs& a, const Plan& p, hipStream_t s) {
    if constexpr (MODE == (M_REDUCE | M_ADAM | M_CAST)) {
        if (p.kernel == K_DEFERRED) {
            switch (p.dv) {
                case 4: return launch_deferred<GDT, PDT, 4>(a, p, s);
                case 2: return launch_deferred<GDT, PDT, 2>(a, p, s);
                default: return launch_deferred<GDT, PDT, 1>(a, p, s);
            }
        }
    }
    if (p.kernel == K_SCALAR) {
        hipLaunchKernelGGL((step_scalar_kernel<GDT, PDT, MODE>), dim3(grid_for(a.n, g_step_bpc.load(std::memory_order_relaxed))), dim3(kThreads),
                           0, s, a);
        return hipGetLastError();
    }
    const dim3 grid(grid_for(vec_elems(a.n) >> 3, g_step_bpc.load(std::memory_order_relaxed)));
    if constexpr ((MODE & M_REDUCE) != 0) {
        if (p.rb == kRowBatchWide) {
            switch (p.dv) {
                case 4: hipLaunchKernelGGL((step_vec8_kernel<GDT, PDT, MODE, 4, kRowBatchWide>), grid, dim3(kThreads), 0, s, a); break;
                case 2: hipLaunchKernelGGL((step_vec8_kernel<GDT, PDT, MODE, 2, kRowBatchWide>), grid, dim3(kThreads), 0, s, a); break;
                default: hipLaunchKernelGGL((step_vec8_kernel<GDT, PDT, MODE, 1, kRowBatchWide>), grid, dim3(kThreads), 0, s, a); break;
            }
            return hipGetLastError();
        }
    }
    switch (p.dv) {
        case 4: hipLaunchKernelGGL((step_vec8_kernel<GDT, PDT, MODE, 4, kRowBatch>), grid, dim3(kThreads), 0, s, a); break;
        case 2: hipLaunchKernelGGL((step_vec8_kernel<GDT, PDT, MODE, 2, kRowBatch>), grid, dim3(kThreads), 0, s, a); break;
        default: hipLaunchKernelGGL((step_vec8_kernel<GDT, PDT, MODE, 1, kRowBatch>), grid, dim3(kThreads), 0, s, a); break;
    }
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_dt(int gdt, int pdt, const StepArgs& a, const Plan& p, hipStream_t s) {
    const bool gb = gdt == ZSMR_BF16, pb = pdt == ZSMR_BF16;
    if (gb && pb) return launch_mode<ZSMR_BF16, ZSMR_BF16, MODE>(a, p, s);
    if (gb) return launch_mode<ZSMR_BF16, ZSMR_FP16, MODE>(a, p, s);
    if (pb) return launch_mode<ZSMR_FP16, ZSMR_BF16, MODE>(a, p, s);
    return launch_mode<ZSMR_FP16, ZSMR_FP16, MODE>(a, p, s);
}

}  // namespace

void set_xcd_balance(int32_t even_permille) { g_xcd_even_permille.store(even_permille, std::memory_order_relaxed); }

void set_launch_shape(int32_t step_bpc, int32_t copy_bpc, int32_t defer_tiles,
                      int32_t defer_min_rows) {
    g_step_bpc.store(step_bpc, std::memory_order_relaxed);
    g_copy_bpc.store(copy_bpc, std::memory_order_relaxed);
    g_defer_tiles.store(defer_tiles, std::memory_order_relaxed);
    g_defer_min_rows.store(defer_min_rows, std::memory_order_relaxed);
}

void set_write_window(int64_t cycle_ns, int64_t write_ns, int64_t margin_ns, int64_t lead_ns) {
    std::lock_guard<std::mutex> hold(g_window_lock);
    g_window_ns = WindowNs{cycle_ns, write_ns, margin_ns, lead_ns};
}

namespace {
// whether the operands a launch of `mode` uses allow the vector path
bool vec_ok(int mode, const StepArgs& a) {
    bool vec = true;
    if (mode & M_REDUCE)
        vec = vec && al(a.grads, 8) && (a.row_stride % 4) == 0;
    if (mode & (M_ADAM | M_CAST | M_INIT)) vec = vec && al(a.master, 16);
    if (mode & (M_ADAM | M_INIT)) vec = vec && al(a.m, 16) && al(a.v, 16);
    if ((mode & M_INIT) || ((mode & M_ADAM) && !(mode & M_REDUCE))) vec = vec && al(a.g_in, 16);
    if (mode & M_GOUT) vec = vec && al(a.g_out, 16);
    return vec;
}

// a's operands `d` elements further on, with n - d elements and head `head`
StepArgs advanced(const StepArgs& a, int64_t d, int64_t n, int32_t head) {
    StepArgs b = a;
    b.n = n;
    b.head = head;
    if (b.grads) b.grads += d;
    if (b.g_in) b.g_in += d;
    if (b.g_out) b.g_out += d;
    if (b.master) b.master += d;
    if (b.m) b.m += d;
    if (b.v) b.v += d;
    if (b.p16) b.p16 += d;
    return b;
}

// Elements to run one by one before the vector body so that its tiles start
// on a 128-byte line of the operand read most: the gradient rows when the
// launch reduces, else the fp32 master.  A slice at an offset that is not a
// multiple of 64 elements (a rank's shard in a vector that N cuts into
// shards whose size is not such a multiple) otherwise has every wave's
// loads and stores straddle one line more than they cover; measured on
// MI355X, 16 rows, 97,375,000 elements: 1.09-1.23 ms per launch at a
// straddling offset against 0.98-1.01 ms on a line.  0 where the piece is
// shorter than a tile past the head, or where the shift would cost an
// operand its vector alignment.
int64_t line_head(int mode, const StepArgs& a) {
    const bool red = (mode & M_REDUCE) != 0;
    const uintptr_t p = red ? reinterpret_cast<uintptr_t>(a.grads) : reinterpret_cast<uintptr_t>(a.master);
    const uintptr_t es = red ? 2 : 4;
    if (!p || p % es || !vec_ok(mode, a)) return 0;
    const int64_t h = static_cast<int64_t>((128 - p % 128) % 128 / es);
    if (h == 0 || a.n - h < 512) return 0;
    return vec_ok(mode, advanced(a, h, a.n - h, 0)) ? h : 0;
}

// The kernel a launch of `mode` over a's operands runs: the one-element
// kernel unless every operand allows the vector path; for the fused step the
// deferred-write kernel when it is on, the step has at least
// g_defer_min_rows rows and its rows are 16-byte aligned (one 16-byte load
// per row per lane), else the direct kernel.
// Gradient rows per load batch of the direct kernel for a step of `rows`
// rows: 12 where one batch of 12 holds rows 1..N-1 (9-13 rows) or the
// batches stay mostly full (16-23 rows), else 8.  Measured on MI355X, one
// launch of 60M elements, ms with 12 / 8 rows per batch: 9 rows 0.434 /
// 0.458, 10 0.446 / 0.465, 11 0.466 / 0.480, 12 0.490 / 0.499, 14 0.567 /
// 0.548, 16 (97M elements) 0.953 / 0.980, 18 0.624 / 0.624, 20 0.668 /
// 0.679; the 1.558e9-element 16-rank world 15.37 / 15.92 ms per step; 8 rows
// (GPT-2 small, Llama-3-8B shape) within 1% either way, 8 kept.
int direct_row_batch(int rows) {
    return (rows >= 9 && rows <= 13) || (rows >= 16 && rows <= 23) ? kRowBatchWide : kRowBatch;
}

Plan plan_for(int mode, const StepArgs& a) {
    Plan p{K_DIRECT, (mode & M_CAST) ? dst_vec(a.p16) : 4, 0, Window{0, 0, 0, 0},
           (mode & M_REDUCE) ? direct_row_batch(a.nrows) : kRowBatch};
    if (!vec_ok(mode, a)) {
        p.kernel = K_SCALAR;
        return p;
    }
    const int tiles = g_defer_tiles.load(std::memory_order_relaxed);
    if (mode == (M_REDUCE | M_ADAM | M_CAST) && tiles > 0 &&
        a.nrows >= g_defer_min_rows.load(std::memory_order_relaxed) && al(a.grads, 16) &&
        a.row_stride % 8 == 0) {
        p.kernel = K_DEFERRED;
        p.win = a.nrows >= kWindowMinRows ? window_ticks(a.nrows) : Window{0, 0, 0, 0};
        p.kd = p.win.cycle || tiles < kRingWithoutWindows ? tiles : kRingWithoutWindows;
    }
    return p;
}

hipError_t launch_step_one(int mode, int gdt, int pdt, const StepArgs& a, hipStream_t s) {
    const Plan p = plan_for(mode, a);
    if (p.kernel == K_SCALAR && a.head) return hipErrorInvalidValue;   // the host gives a head to vector launches only
    switch (mode) {
        case M_REDUCE | M_ADAM | M_CAST: return launch_dt<M_REDUCE | M_ADAM | M_CAST>(gdt, pdt, a, p, s);
        case M_REDUCE | M_GOUT: return launch_dt<M_REDUCE | M_GOUT>(gdt, ZSMR_BF16, a, p, s);
        case M_ADAM: return launch_mode<ZSMR_BF16, ZSMR_BF16, M_ADAM>(a, p, s);
        case M_CAST: return launch_dt<M_CAST>(ZSMR_BF16, pdt, a, p, s);
        case M_INIT | M_CAST: return launch_dt<M_INIT | M_CAST>(ZSMR_BF16, pdt, a, p, s);
        default: return hipErrorInvalidValue;
    }
}
}  // namespace

// A piece's head (the elements before its first 128-byte line) runs with the
// first launch; the rest is cut into launches of at most 2^30 elements (a
// multiple of every vector width and of the line, so alignment is kept).
hipError_t launch_step(int mode, int gdt, int pdt, const StepArgs& a0, hipStream_t s) {
    constexpr int64_t kMaxLaunch = int64_t(1) << 30;
    const int64_t h = line_head(mode, a0);
    for (int64_t c = h; c < a0.n; c += kMaxLaunch) {
        const int64_t n = a0.n - c < kMaxLaunch ? a0.n - c : kMaxLaunch;
        const hipError_t e = launch_step_one(mode, gdt, pdt, advanced(a0, c, n, c == h ? (int32_t)h : 0), s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

void describe_step(int mode, const StepArgs& a0, StepPlan* out) {
    constexpr int64_t kMaxLaunch = int64_t(1) << 30;
    const int64_t h = line_head(mode, a0);
    const int64_t n = a0.n - h < kMaxLaunch ? a0.n - h : kMaxLaunch;
    const Plan p = plan_for(mode, advanced(a0, h, n, (int32_t)h));
    out->kernel = p.kernel;
    out->ring_tiles = p.kernel == K_DEFERRED ? p.kd : 0;
    out->windowed = p.win.cycle != 0;
    out->store_elems = p.dv;
    out->launches = a0.n > h ? (int32_t)((a0.n - h + kMaxLaunch - 1) / kMaxLaunch) : 0;
    out->head = h;
    out->row_batch = p.kernel == K_DIRECT && (mode & M_REDUCE) ? p.rb : 0;
}

hipError_t launch_copy16(const uint16_t* src, uint16_t* dst, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int w = copy_width(reinterpret_cast<uintptr_t>(src), reinterpret_cast<uintptr_t>(dst));
    const int64_t head = head_for(dst, w, n);
    const int64_t pre = pre_for(dst, w, head);
    const int64_t vecs = (n - head) / (w / 2) + 1;
    const int64_t regions = w >= 4 ? grid_for((vecs + pre) / (ZSMR_COPY_BURST_BYTES / w) + 1, g_copy_bpc.load(std::memory_order_relaxed))
                                   : grid_for(vecs, kNarrowCopyBpc);
    unsigned gx = 0;
    const XcdSplit sp = xcd_split(regions, &gx);
    const dim3 grid(gx);
    switch (w) {
        case 16: hipLaunchKernelGGL(copy16_kernel<16>, grid, dim3(kThreads), 0, s, src, dst, n, head, pre, sp, regions); break;
        case 8: hipLaunchKernelGGL(copy16_kernel<8>, grid, dim3(kThreads), 0, s, src, dst, n, head, pre, sp, regions); break;
        case 4: hipLaunchKernelGGL(copy16_kernel<4>, grid, dim3(kThreads), 0, s, src, dst, n, head, pre, sp, regions); break;
        default: hipLaunchKernelGGL(copy16_kernel<2>, grid, dim3(kThreads), 0, s, src, dst, n, head, pre, sp, regions); break;
    }
    return hipGetLastError();
}

hipError_t launch_copy_blocks(const uint16_t* src, uint16_t* dst, int64_t n, int32_t count,
                              int64_t stride, hipStream_t s) {
    if (n <= 0 || count <= 0) return hipSuccess;
    // src - dst is the same for every block, and so is the vector width
    const int w = copy_width(reinterpret_cast<uintptr_t>(src), reinterpret_cast<uintptr_t>(dst));
    const int64_t pre_max = w >= 4 ? int64_t(128 * 1024) / w : 0;   // a block's chunk-grid offset
    const int64_t per = n / (w / 2) + 1 + pre_max;
    const int64_t units = w >= 4 ? per / (ZSMR_COPY_BURST_BYTES / w) + 1 : per;   // lanes' work
    int64_t regions = (units + kThreads - 1) / kThreads;   // of each block
    const int bpc = w >= 4 ? g_copy_bpc.load(std::memory_order_relaxed) : kNarrowCopyBpc;
    if (bpc > 0) {   // a grid-stride grid: bpc workgroups per CU over all blocks
        const int64_t cap = (int64_t)cu_count() * bpc;
        const int64_t lim = cap / count > 0 ? cap / count : 1;
        if (regions > lim) regions = lim;
    }
    if (regions < 1) regions = 1;
    unsigned gx = 0;   // a multiple of 8: each block's row starts on XCD 0
    const XcdSplit sp = xcd_split(regions, &gx);
    const dim3 grid(gx, static_cast<unsigned>(count));
    switch (w) {
        case 16: hipLaunchKernelGGL(copy_blocks_kernel<16>, grid, dim3(kThreads), 0, s, src, dst, n, stride, sp, regions); break;
        case 8: hipLaunchKernelGGL(copy_blocks_kernel<8>, grid, dim3(kThreads), 0, s, src, dst, n, stride, sp, regions); break;
        case 4: hipLaunchKernelGGL(copy_blocks_kernel<4>, grid, dim3(kThreads), 0, s, src, dst, n, stride, sp, regions); break;
        default: hipLaunchKernelGGL(copy_blocks_kernel<2>, grid, dim3(kThreads), 0, s, src, dst, n, stride, sp, regions); break;
    }
    return hipGetLastError();
}

hipError_t launch_gather16(const uint16_t* const* srcs, int32_t nsrc, int64_t each, uint16_t* dst,
                           hipStream_t s) {
    if (each <= 0 || nsrc <= 0) return hipSuccess;
    for (int32_t r0 = 0; r0 < nsrc; r0 += kMaxGather) {
        const int32_t cnt = nsrc - r0 < kMaxGather ? nsrc - r0 : kMaxGather;
        GatherArgs g{};
        g.dst = dst + (int64_t)r0 * each;
        g.each = each;
        int w = 16;
        for (int32_t i = 0; i < cnt; ++i) {
            const int wi = copy_width(reinterpret_cast<uintptr_t>(srcs[r0 + i]),
                                      reinterpret_cast<uintptr_t>(g.dst + (int64_t)i * each));
            if (wi < w) w = wi;
        }
        int64_t pre_max = 0;
        for (int32_t i = 0; i < cnt; ++i) {
            g.src[i] = srcs[r0 + i];
            g.head[i] = head_for(g.dst + (int64_t)i * each, w, each);
            g.pre[i] = pre_for(g.dst + (int64_t)i * each, w, g.head[i]);
            if (g.pre[i] > pre_max) pre_max = g.pre[i];
        }
        const int64_t per = each / (w / 2) + 1 + pre_max;
        const int64_t units = w >= 4 ? per / (ZSMR_COPY_BURST_BYTES / w) + 1 : per;   // lanes' work
        int64_t regions = (units + kThreads - 1) / kThreads;   // of each source
        const int bpc = w >= 4 ? g_copy_bpc.load(std::memory_order_relaxed) : kNarrowCopyBpc;
        if (bpc > 0) {   // a grid-stride grid: bpc workgroups per CU over all sources
            const int64_t cap = (int64_t)cu_count() * bpc;
            const int64_t lim = cap / cnt > 0 ? cap / cnt : 1;
            if (regions > lim) regions = lim;
        }
        if (regions < 1) regions = 1;
        unsigned gx = 0;   // a multiple of 8: each source's row starts on XCD 0
        const XcdSplit sp = xcd_split(regions, &gx);
        const dim3 grid(gx, static_cast<unsigned>(cnt));
        switch (w) {
            case 16: hipLaunchKernelGGL(gather16_kernel<16>, grid, dim3(kThreads), 0, s, g, sp, regions); break;
            case 8: hipLaunchKernelGGL(gather16_kernel<8>, grid, dim3(kThreads), 0, s, g, sp, regions); break;
            case 4: hipLaunchKernelGGL(gather16_kernel<4>, grid, dim3(kThreads), 0, s, g, sp, regions); break;
            default: hipLaunchKernelGGL(gather16_kernel<2>, grid, dim3(kThreads), 0, s, g, sp, regions); break;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace zsmr
