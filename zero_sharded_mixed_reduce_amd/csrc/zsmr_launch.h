// Internal interface between the C-ABI host code (zsmr_api.cpp) and the
// gfx950 kernels (zsmr_kernels.hip).  Not part of the public ABI.
#pragma once
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace zsmr {

// fp32 constants of one Adam step, rounded once from double on the host.
struct AdamK {
    float c1, c1m, c2, c2m, bc1, bc2, lr, eps;
};

// Which parts of the step a launch performs.
enum : int {
    M_REDUCE = 1,   // read N 16-bit rows, fp32 rank-order sum (/N if mean)
    M_ADAM = 2,     // Adam on master/m/v with g (reduced, or read from g_in)
    M_CAST = 4,     // write RNE16(master) to p16
    M_GOUT = 8,     // write the reduced g to g_out
    M_INIT = 16,    // master = g_in (theta0), m = v = 0
};

struct StepArgs {
    const uint16_t* grads;  // row 0 at the piece's first element
    int64_t row_stride;     // elements between rows
    int32_t nrows;          // N
    int32_t mean;           // divide the sum by N
    float nf;               // (float)N
    float inv_nf;           // 1/N when N is a power of two (then exact)
    int32_t inv_pow2;       // N is a power of two: the mean multiplies by inv_nf
    const float* g_in;      // Adam-only input gradient, or theta0 for init
    float* g_out;           // reduce-only output
    float* master;
    float* m;
    float* v;
    uint16_t* p16;
    int64_t n;              // elements from the pointers on
    int32_t head;           // elements just before the pointers that also
                            // belong to the piece (the vector path's tiles
                            // then start on a 128-byte line); run one per
                            // lane by workgroup 0, with the tail
    AdamK k;
};

hipError_t launch_step(int mode, int grad_dtype, int param_dtype, const StepArgs& a,
                       hipStream_t stream);
// what launch_step(mode, ..., a) would launch (no launch; the write windows
// need the current device's clock rate)
struct StepPlan {
    int32_t kernel, ring_tiles, windowed, store_elems, launches, row_batch;
    int64_t head;
};
void describe_step(int mode, const StepArgs& a, StepPlan* out);
hipError_t launch_copy16(const uint16_t* src, uint16_t* dst, int64_t n, hipStream_t stream);
// dst[k*stride + j] = src[k*stride + j], j < n, k < count (count <= 65535)
hipError_t launch_copy_blocks(const uint16_t* src, uint16_t* dst, int64_t n, int32_t count,
                              int64_t stride, hipStream_t stream);
// dst[r*each + j] = srcs[r][j], r < nsrc
hipError_t launch_gather16(const uint16_t* const* srcs, int32_t nsrc, int64_t each,
                           uint16_t* dst, hipStream_t stream);
void set_launch_shape(int32_t step_bpc, int32_t copy_bpc, int32_t defer_tiles,
                      int32_t defer_min_rows);
// each even XCD's share of a copy's regions against an odd one's, in thousandths
void set_xcd_balance(int32_t even_permille);
// write windows of the fused step's deferred-write kernel (cycle_ns 0: none)
void set_write_window(int64_t cycle_ns, int64_t write_ns, int64_t margin_ns, int64_t lead_ns);

}  // namespace zsmr
