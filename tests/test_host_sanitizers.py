"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

``csrc/zsmr_api.cpp`` (layout, accounting, the ZeRO-3 schedule, every
argument check) is built with g++ for the CPU together with a stand-in for
the kernel launch layer (``zsmr_launch.h``) that records each launch instead
of running it.  A C++ driver then calls every entry point of ``include/zsmr.h``
with placeholder device addresses and checks, without a GPU:

* the partition: for every stage, world, size, pad and unit split the pieces
  of all ranks tile the padded vector, local offsets add up, owners are
  unique, and the accounting's bands sum to its totals;
* what each device entry point launches: the operand addresses, the length,
  the rows and their stride, the mode and the Adam constants follow from its
  arguments and the layout, so a kernel never receives a range outside the
  piece it was asked for;
* argument, alignment, state and size-limit errors return their codes and
  launch nothing; a failing launch returns ZSMR_ERR_HIP and changes no
  counter or schedule state;
* no memory error, leak, signed overflow or other undefined behaviour
  happens on the way (the sanitizers abort the run on the first one).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "zero_sharded_mixed_reduce_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

DRIVER = r"""
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <vector>

#include "zsmr.h"
#include "zsmr_launch.h"

#define CHECK(c) do { if (!(c)) { std::printf("CHECK failed line %d: %s\n", __LINE__, #c); \
                                   std::exit(1); } } while (0)

// ---- the launch layer, recorded instead of run
struct Launch {
    int kind;                        // 0 step, 1 copy16, 2 copy_blocks, 3 gather16
    int mode, gdt, pdt;
    zsmr::StepArgs a;
    const uint16_t* src;
    uint16_t* dst;
    int64_t n, stride, each;
    int32_t count;
    std::vector<const uint16_t*> srcs;
};
static std::vector<Launch> g_launch;
static hipError_t g_result = hipSuccess;

namespace zsmr {
hipError_t launch_step(int mode, int gdt, int pdt, const StepArgs& a, hipStream_t) {
    Launch l{};
    l.kind = 0; l.mode = mode; l.gdt = gdt; l.pdt = pdt; l.a = a;
    g_launch.push_back(l);
    return g_result;
}
hipError_t launch_copy16(const uint16_t* s, uint16_t* d, int64_t n, hipStream_t) {
    Launch l{};
    l.kind = 1; l.src = s; l.dst = d; l.n = n;
    g_launch.push_back(l);
    return g_result;
}
hipError_t launch_copy_blocks(const uint16_t* s, uint16_t* d, int64_t n, int32_t count,
                              int64_t stride, hipStream_t) {
    Launch l{};
    l.kind = 2; l.src = s; l.dst = d; l.n = n; l.count = count; l.stride = stride;
    g_launch.push_back(l);
    return g_result;
}
hipError_t launch_gather16(const uint16_t* const* srcs, int32_t nsrc, int64_t each, uint16_t* dst,
                           hipStream_t) {
    Launch l{};
    l.kind = 3; l.srcs.assign(srcs, srcs + nsrc); l.each = each; l.dst = dst;
    g_launch.push_back(l);
    return g_result;
}
static int32_t g_shape[4];
static int64_t g_window[4];
void set_launch_shape(int32_t a, int32_t b, int32_t c, int32_t d) {
    g_shape[0] = a; g_shape[1] = b; g_shape[2] = c; g_shape[3] = d;
}
void set_write_window(int64_t a, int64_t b, int64_t c, int64_t d) {
    g_window[0] = a; g_window[1] = b; g_window[2] = c; g_window[3] = d;
}
static int32_t g_balance;
void set_xcd_balance(int32_t even_permille) { g_balance = even_permille; }
static StepArgs g_described;
void describe_step(int mode, const StepArgs& a, StepPlan* out) {
    g_described = a;
    out->kernel = mode;                 // echoed so that the driver can see the mode
    out->ring_tiles = 3;
    out->windowed = 1;
    out->store_elems = 4;
    out->launches = 1;
    out->row_batch = 12;
    out->head = 5;
}
}  // namespace zsmr

const char* hipGetErrorString(hipError_t) { return "launch refused by the stand-in"; }

// placeholder device addresses: never dereferenced, only compared
template <class T> static T* at(uint64_t addr) { return reinterpret_cast<T*>(addr); }
static const uint64_t G = 0x100000000ull, M = 0x200000000ull, MM = 0x300000000ull,
                      V = 0x400000000ull, P = 0x500000000ull, O = 0x600000000ull,
                      TH = 0x700000000ull;

static zsmr_ctx* make(int64_t numel, int32_t world, int32_t stage, int32_t pad,
                      const std::vector<int64_t>& units, int32_t* st) {
    zsmr_ctx* c = nullptr;
    *st = zero_init_shards(&c, numel, world, stage, ZSMR_BF16, ZSMR_BF16, pad,
                           units.empty() ? nullptr : units.data(), (int32_t)units.size());
    CHECK((*st == ZSMR_OK) == (c != nullptr));
    return c;
}

// ---- the partition and the accounting over many shapes
static void layout_sweep() {
    const int64_t sizes[] = {1, 7, 64, 1000, 1000003};
    const int32_t worlds[] = {1, 2, 3, 5, 8, 64};
    int checked = 0;
    for (int32_t stage = 0; stage <= 4; ++stage)
    for (int64_t numel : sizes)
    for (int32_t world : worlds)
    for (int32_t pad = 0; pad <= 1; ++pad)
    for (int split = 0; split <= 2; ++split) {
        std::vector<int64_t> units;
        if (split == 1 && numel >= 3) units = {numel / 3, numel / 3, numel - 2 * (numel / 3)};
        if (split == 2 && numel >= 7) units = {1, numel - 5, 4};
        if (split && units.empty()) continue;
        int32_t st;
        zsmr_ctx* c = make(numel, world, stage, pad, units, &st);
        if (!c) {
            CHECK(st == ZSMR_ERR_INDIVISIBLE && !pad && (stage == 1 || stage == 2 || stage == 3));
            continue;
        }
        zsmr_layout_info li;
        CHECK(zero_layout_info(c, &li) == ZSMR_OK);
        CHECK(li.numel == numel && li.world == world && li.stage == stage);
        const int32_t U = li.n_units;
        const int32_t pieces = (stage == 3 || stage == 4) ? U : 1;
        std::vector<std::pair<int64_t, int64_t>> iv;
        std::vector<int64_t> held(world, 0);
        for (int32_t u = 0; u < pieces; ++u) {
            int owners = 0;
            for (int32_t r = 0; r < world; ++r) {
                int64_t off, len, loc;
                CHECK(zero_layout(c, r, u, &off, &len, &loc) == ZSMR_OK);
                CHECK(off >= 0 && len >= 0 && off + len <= li.padded_numel);
                if (stage == 0) {
                    CHECK(off == 0 && len == numel && loc == 0);
                    continue;
                }
                if (len == 0) continue;
                CHECK(loc == held[r]);              // a rank's pieces follow one another
                held[r] += len;
                iv.push_back({off, len});
                ++owners;
            }
            if (stage == 4) {
                int32_t o;
                CHECK(zero_unit_owner(c, u, &o) == ZSMR_OK && o >= 0 && o < world);
                CHECK(owners == 1);
            }
        }
        if (stage != 0) {                           // pieces tile [0, padded)
            std::sort(iv.begin(), iv.end());
            int64_t at_ = 0;
            for (auto& p : iv) {
                CHECK(p.first == at_);
                at_ += p.second;
            }
            CHECK(at_ == li.padded_numel);
            CHECK(*std::max_element(held.begin(), held.end()) == li.shard_numel);
        }
        CHECK(zero_layout(c, world, 0, nullptr, nullptr, nullptr) == ZSMR_ERR_ARG);
        CHECK(zero_layout(c, 0, pieces, nullptr, nullptr, nullptr) == ZSMR_ERR_ARG);
        for (int32_t gb : {0, 2, 4, 8})
        for (int32_t ml : {0, 1, 2, 5}) {
            zsmr_bytes b, worst{};
            for (int32_t r = 0; r < world; ++r) {
                CHECK(zero_bytes_of_rank(c, r, gb, ml, &b) == ZSMR_OK);
                CHECK(b.resident == b.res_p16 + b.res_grad + b.res_master + b.res_m + b.res_v);
                CHECK(b.peak == b.resident + b.gathered);
                CHECK(b.traffic_elems == b.rs_elems + b.ag_elems + b.ar_elems);
                CHECK(b.traffic_bytes == 2 * b.traffic_elems);
                if (r == 0 || b.peak > worst.peak) worst = b;
            }
            CHECK(zero_bytes_per_rank(c, gb, ml, &b) == ZSMR_OK);
            CHECK(b.peak == worst.peak && b.resident == worst.resident);
        }
        zero_destroy(c);
        ++checked;
    }
    std::printf("layouts checked: %d\n", checked);
    CHECK(checked > 300);
}

// ---- what the device entry points launch
static void launches() {
    // stage 3, 4 ranks, units of 10 and 6 padded to shards of 3 and 2
    int32_t st;
    zsmr_ctx* c = make(16, 4, 3, 1, {10, 6}, &st);
    CHECK(c);
    int64_t off, len, loc;
    CHECK(zero_layout(c, 2, 1, &off, &len, &loc) == ZSMR_OK);
    CHECK(off == 12 + 2 * 2 && len == 2 && loc == 3);
    zsmr_adam hp{1e-3, 0.9, 0.999, 1e-8};

    g_launch.clear();
    CHECK(zero_fused_step_range(c, 2, 1, 1, 1, at<void>(G), 100, 14, at<float>(M), at<float>(MM),
                                at<float>(V), at<void>(P), 3, &hp, nullptr) == ZSMR_OK);
    CHECK(g_launch.size() == 1);
    const Launch& f = g_launch[0];
    CHECK(f.kind == 0 && f.mode == (zsmr::M_REDUCE | zsmr::M_ADAM | zsmr::M_CAST));
    CHECK(f.a.grads == at<const uint16_t>(G) + 14 + 1 && f.a.row_stride == 100);
    CHECK(f.a.nrows == 4 && f.a.mean == 1 && f.a.inv_pow2 == 1 && f.a.inv_nf == 0.25f);
    CHECK(f.a.master == at<float>(M) + 1 && f.a.m == at<float>(MM) + 1);
    CHECK(f.a.v == at<float>(V) + 1 && f.a.p16 == at<uint16_t>(P) + 1 && f.a.n == 1);
    CHECK(f.a.k.bc1 == (float)(1.0 - std::pow(0.9, 3.0)));
    CHECK(f.a.k.bc2 == (float)(1.0 - std::pow(0.999, 3.0)));
    CHECK(f.a.k.c1m == (float)(1.0 - 0.9) && f.a.k.lr == (float)1e-3 && f.a.k.eps == (float)1e-8);
    CHECK(f.gdt == ZSMR_BF16 && f.pdt == ZSMR_BF16);
    zsmr_counters k;
    CHECK(zero_counters(c, 2, &k) == ZSMR_OK && k.rs_elems == 3 && k.ag_elems == 0);

    // the whole piece; a sub-range past the piece; an empty one
    g_launch.clear();
    CHECK(zero_fused_step(c, 2, 1, at<void>(G), 8, 4, at<float>(M), at<float>(MM), at<float>(V),
                          at<void>(P), 1, &hp, nullptr) == ZSMR_OK);
    CHECK(g_launch.size() == 1 && g_launch[0].a.n == 2 && g_launch[0].a.grads == at<const uint16_t>(G) + 4);
    CHECK(zero_fused_step_range(c, 2, 1, 1, 2, at<void>(G), 8, 4, at<float>(M), at<float>(MM),
                                at<float>(V), at<void>(P), 1, &hp, nullptr) == ZSMR_ERR_ARG);
    CHECK(zero_fused_step_range(c, 2, 1, 2, 0, at<void>(G), 8, 4, at<float>(M), at<float>(MM),
                                at<float>(V), at<void>(P), 1, &hp, nullptr) == ZSMR_OK);
    CHECK(zero_fused_step_range(c, 2, 1, -1, 1, at<void>(G), 8, 4, at<float>(M), at<float>(MM),
                                at<float>(V), at<void>(P), 1, &hp, nullptr) == ZSMR_ERR_ARG);
    // rows that would overlap, a misaligned row, bad Adam constants
    CHECK(zero_fused_step(c, 2, 1, at<void>(G), 1, 4, at<float>(M), at<float>(MM), at<float>(V),
                          at<void>(P), 1, &hp, nullptr) == ZSMR_ERR_ARG);
    CHECK(zero_fused_step(c, 2, 1, at<void>(G + 1), 8, 4, at<float>(M), at<float>(MM),
                          at<float>(V), at<void>(P), 1, &hp, nullptr) == ZSMR_ERR_ALIGN);
    CHECK(zero_fused_step(c, 2, 1, at<void>(G), 8, 4, at<float>(M + 2), at<float>(MM),
                          at<float>(V), at<void>(P), 1, &hp, nullptr) == ZSMR_ERR_ALIGN);
    zsmr_adam bad[] = {{NAN, 0.9, 0.999, 1e-8}, {1e-3, 1.0, 0.999, 1e-8}, {1e-3, 0.9, -0.1, 1e-8},
                       {1e-3, 0.9, 0.999, -1.0}, {-1.0, 0.9, 0.999, 1e-8}, {INFINITY, 0.9, 0.999, 0}};
    for (auto& h : bad)
        CHECK(zero_fused_step(c, 2, 1, at<void>(G), 8, 4, at<float>(M), at<float>(MM),
                              at<float>(V), at<void>(P), 1, &h, nullptr) == ZSMR_ERR_ARG);
    CHECK(zero_fused_step(c, 2, 1, at<void>(G), 8, 4, at<float>(M), at<float>(MM), at<float>(V),
                          at<void>(P), 0, &hp, nullptr) == ZSMR_ERR_ARG);
    CHECK(zero_fused_step(c, 2, 1, at<void>(G), 8, 4, at<float>(M), at<float>(MM), at<float>(V),
                          at<void>(P), 1, nullptr, nullptr) == ZSMR_ERR_ARG);
    CHECK(zero_fused_step(c, 4, 0, at<void>(G), 8, 4, at<float>(M), at<float>(MM), at<float>(V),
                          at<void>(P), 1, &hp, nullptr) == ZSMR_ERR_ARG);
    CHECK(g_launch.size() == 1);                    // none of the refused calls launched

    // reduce only, Adam only, cast only, init
    g_launch.clear();
    CHECK(zero_reduce_shard(c, 1, 0, at<void>(G), 12, 3, 0, at<float>(O), nullptr) == ZSMR_OK);
    CHECK(zero_adam_step(at<float>(M), at<float>(MM), at<float>(V), at<float>(O), 5, 2, &hp,
                         nullptr) == ZSMR_OK);
    CHECK(zero_adam_step(at<float>(M), at<float>(MM), at<float>(V), at<float>(O), 0, 2, &hp,
                         nullptr) == ZSMR_OK);
    CHECK(zero_gather_cast(c, 3, 0, at<float>(M), at<void>(P), nullptr) == ZSMR_OK);
    CHECK(zero_init_state(c, 0, 1, at<float>(TH), at<float>(M), at<float>(MM), at<float>(V),
                          at<void>(P), nullptr) == ZSMR_OK);
    CHECK(g_launch.size() == 4);
    CHECK(g_launch[0].mode == (zsmr::M_REDUCE | zsmr::M_GOUT) && g_launch[0].a.mean == 0);
    CHECK(g_launch[0].a.grads == at<const uint16_t>(G) + 3 && g_launch[0].a.n == 3);
    CHECK(g_launch[0].a.g_out == at<float>(O) && g_launch[0].a.nf == 4.0f);
    CHECK(g_launch[1].mode == zsmr::M_ADAM && g_launch[1].a.n == 5 && g_launch[1].a.g_in == at<float>(O));
    CHECK(g_launch[1].a.k.bc1 == (float)(1.0 - 0.9 * 0.9));
    CHECK(g_launch[2].mode == zsmr::M_CAST && g_launch[2].a.n == 3 && g_launch[2].a.master == at<float>(M));
    CHECK(g_launch[3].mode == (zsmr::M_INIT | zsmr::M_CAST) && g_launch[3].a.n == 2);
    CHECK(g_launch[3].a.g_in == at<float>(TH));

    // the ZeRO-3 schedule and its gathers
    g_launch.clear();
    const void* sh[4] = {at<void>(P), at<void>(P + 100), at<void>(P + 200), at<void>(P + 300)};
    CHECK(zero_stage3_unit_gather(c, 0, sh, at<void>(O), nullptr) == ZSMR_OK);
    CHECK(g_launch.size() == 1 && g_launch[0].kind == 3 && g_launch[0].each == 3);
    CHECK(g_launch[0].srcs.size() == 4 && g_launch[0].srcs[3] == at<const uint16_t>(P + 300));
    CHECK(zero_stage3_unit_gather(c, 0, sh, at<void>(O), nullptr) == ZSMR_ERR_STATE);
    CHECK(zero_stage3_unit_gather(c, 1, sh, at<void>(O + 64), nullptr) == ZSMR_ERR_STATE);
    CHECK(zero_stage3_set_max_live(c, 2) == ZSMR_ERR_STATE);
    CHECK(zero_stage3_unit_release(c, 0) == ZSMR_OK);
    CHECK(zero_stage3_unit_release(c, 0) == ZSMR_ERR_STATE);
    CHECK(zero_stage3_set_max_live(c, 2) == ZSMR_OK);
    CHECK(zero_stage3_unit_gather(c, 0, sh, at<void>(O), nullptr) == ZSMR_OK);
    CHECK(zero_stage3_unit_gather(c, 1, sh, at<void>(O + 64), nullptr) == ZSMR_OK);
    CHECK(zero_counters(c, 1, &k) == ZSMR_OK && k.live_units == 2);
    CHECK(k.live_bytes == 2 * 12 + 2 * 8 && k.peak_live_bytes == k.live_bytes);
    CHECK(zero_stage3_unit_release(c, 0) == ZSMR_OK && zero_stage3_unit_release(c, 1) == ZSMR_OK);
    // a shard at its own slot of the unit buffer; one overlapping another slot
    const void* inplace[4] = {at<void>(O), at<void>(O + 6), at<void>(P + 200), at<void>(P + 300)};
    CHECK(zero_stage3_unit_gather(c, 0, inplace, at<void>(O), nullptr) == ZSMR_OK);
    CHECK(zero_stage3_unit_release(c, 0) == ZSMR_OK);
    const void* clash[4] = {at<void>(O + 2), at<void>(P + 100), at<void>(P + 200), at<void>(P + 300)};
    CHECK(zero_stage3_unit_gather(c, 0, clash, at<void>(O), nullptr) == ZSMR_ERR_ARG);
    const void* odd[4] = {at<void>(P + 1), at<void>(P + 100), at<void>(P + 200), at<void>(P + 300)};
    CHECK(zero_stage3_unit_gather(c, 0, odd, at<void>(O), nullptr) == ZSMR_ERR_ALIGN);
    const void* nul[4] = {at<void>(P), nullptr, at<void>(P + 200), at<void>(P + 300)};
    CHECK(zero_stage3_unit_gather(c, 0, nul, at<void>(O), nullptr) == ZSMR_ERR_ARG);
    CHECK(zero_stage3_unit_gather(c, 2, sh, at<void>(O), nullptr) == ZSMR_ERR_ARG);
    int32_t live;
    int64_t gathers, releases;
    CHECK(zero_stage3_unit_state(c, 0, &live, &gathers, &releases) == ZSMR_OK);
    CHECK(live == 0 && gathers == 3 && releases == 3);

    // a launch that fails changes no counter and no schedule state
    CHECK(zero_counters(c, 2, &k) == ZSMR_OK);
    const zsmr_counters before = k;
    g_result = hipErrorInvalidValue;
    CHECK(zero_fused_step(c, 2, 1, at<void>(G), 8, 4, at<float>(M), at<float>(MM), at<float>(V),
                          at<void>(P), 1, &hp, nullptr) == ZSMR_ERR_HIP);
    CHECK(std::strcmp(zsmr_last_hip_error(), "launch refused by the stand-in") == 0);
    CHECK(zero_stage3_unit_gather(c, 0, sh, at<void>(O), nullptr) == ZSMR_ERR_HIP);
    CHECK(zero_stage3_unit_state(c, 0, &live, &gathers, nullptr) == ZSMR_OK && live == 0 && gathers == 3);
    CHECK(zero_counters(c, 2, &k) == ZSMR_OK);
    CHECK(k.rs_elems == before.rs_elems && k.ag_elems == before.ag_elems && k.live_units == 0);
    g_result = hipSuccess;
    CHECK(zero_reset_counters(c) == ZSMR_OK && zero_counters(c, 2, &k) == ZSMR_OK);
    CHECK(k.traffic_elems == 0 && k.stage3_gathers == 0);
    zero_destroy(c);

    // owner broadcast: one source, the whole unit
    c = make(30, 3, 4, 0, {10, 5, 15}, &st);
    CHECK(c);
    int32_t own;
    CHECK(zero_unit_owner(c, 2, &own) == ZSMR_OK && own == 2);
    g_launch.clear();
    const void* one[1] = {at<void>(P + 30)};
    CHECK(zero_stage3_unit_gather(c, 2, one, at<void>(O), nullptr) == ZSMR_OK);
    CHECK(g_launch.size() == 1 && g_launch[0].srcs.size() == 1 && g_launch[0].each == 15);
    CHECK(zero_counters(c, 0, &k) == ZSMR_OK && k.ag_elems == 15 && k.live_bytes == 30);
    CHECK(zero_counters(c, 2, &k) == ZSMR_OK && k.ag_elems == 0 && k.live_bytes == 0);
    CHECK(zero_fused_step(c, 0, 2, at<void>(G), 15, 0, at<float>(M), at<float>(MM), at<float>(V),
                          at<void>(P), 1, &hp, nullptr) == ZSMR_OK);
    CHECK(g_launch.size() == 1);                    // a rank that owns nothing of it: no launch
    CHECK(zero_set_unit_owners(c, (const int32_t[]){0, 1, 2}, 3) == ZSMR_ERR_STATE);   // used
    zero_destroy(c);

    // owner broadcast with owners chosen by the caller
    c = make(30, 3, 4, 0, {10, 5, 15}, &st);
    const int32_t map[3] = {1, 1, 0}, out_of_range[3] = {1, 3, 0}, negative[3] = {1, -1, 0};
    CHECK(zero_set_unit_owners(c, map, 2) == ZSMR_ERR_ARG);
    CHECK(zero_set_unit_owners(c, out_of_range, 3) == ZSMR_ERR_ARG);
    CHECK(zero_set_unit_owners(c, negative, 3) == ZSMR_ERR_ARG);
    CHECK(zero_set_unit_owners(c, nullptr, 3) == ZSMR_ERR_ARG);
    CHECK(zero_set_unit_owners(nullptr, map, 3) == ZSMR_ERR_ARG);
    CHECK(zero_unit_owner(c, 0, &own) == ZSMR_OK && own == 0);   // unchanged by the refusals
    CHECK(zero_set_unit_owners(c, map, 3) == ZSMR_OK);
    for (int32_t u = 0; u < 3; ++u) CHECK(zero_unit_owner(c, u, &own) == ZSMR_OK && own == map[u]);
    CHECK(zero_layout(c, 1, 1, &off, &len, &loc) == ZSMR_OK && off == 10 && len == 5 && loc == 10);
    CHECK(zero_layout(c, 0, 2, &off, &len, &loc) == ZSMR_OK && off == 15 && len == 15 && loc == 0);
    CHECK(zero_layout(c, 2, 0, &off, &len, &loc) == ZSMR_OK && len == 0);
    zsmr_layout_info oi;
    CHECK(zero_layout_info(c, &oi) == ZSMR_OK && oi.shard_numel == 15);
    zsmr_bytes ob;
    CHECK(zero_bytes_of_rank(c, 2, 0, 1, &ob) == ZSMR_OK && ob.resident == 0);
    CHECK(ob.rs_elems == 30 && ob.ag_elems == 60 && ob.gathered == 2 * 15);
    CHECK(zero_bytes_of_rank(c, 1, 0, 2, &ob) == ZSMR_OK && ob.resident == 16 * 15);
    CHECK(ob.gathered == 2 * 15);                  // a borrowed pair: units 1 (own) and 2
    g_launch.clear();
    CHECK(zero_stage3_unit_gather(c, 0, one, at<void>(O), nullptr) == ZSMR_OK);
    CHECK(zero_counters(c, 1, &k) == ZSMR_OK && k.ag_elems == 0 && k.live_bytes == 0);
    CHECK(zero_counters(c, 0, &k) == ZSMR_OK && k.ag_elems == 10 && k.live_bytes == 20);
    CHECK(zero_set_unit_owners(c, map, 3) == ZSMR_ERR_STATE);    // a unit is live
    CHECK(zero_stage3_unit_release(c, 0) == ZSMR_OK);
    CHECK(zero_set_unit_owners(c, map, 3) == ZSMR_ERR_STATE);    // counters moved
    CHECK(zero_reset_counters(c) == ZSMR_OK);
    const int32_t back[3] = {2, 2, 2};
    CHECK(zero_set_unit_owners(c, back, 3) == ZSMR_OK);
    CHECK(zero_layout_info(c, &oi) == ZSMR_OK && oi.shard_numel == 30);
    CHECK(zero_layout(c, 2, 2, &off, &len, &loc) == ZSMR_OK && len == 15 && loc == 15);
    zero_destroy(c);
    c = make(16, 4, 3, 1, {10, 6}, &st);
    CHECK(zero_set_unit_owners(c, map, 2) == ZSMR_ERR_ARG);     // not an owner-broadcast context
    zero_destroy(c);

    // data parallel: a replica's all-reduce covers the whole vector, so a
    // fused range must be the whole vector (counted once per step)
    c = make(8, 2, 0, 0, {}, &st);
    g_launch.clear();
    CHECK(zero_fused_step_range(c, 1, 0, 0, 4, at<void>(G), 8, 0, at<float>(M), at<float>(MM),
                                at<float>(V), at<void>(P), 1, &hp, nullptr) == ZSMR_ERR_ARG);
    CHECK(zero_fused_step_range(c, 1, 0, 0, 8, at<void>(G), 8, 0, at<float>(M), at<float>(MM),
                                at<float>(V), at<void>(P), 1, &hp, nullptr) == ZSMR_OK);
    CHECK(g_launch.size() == 1 && g_launch[0].a.n == 8);
    CHECK(zero_counters(c, 1, &k) == ZSMR_OK && k.ar_elems == 2 * 1 * 4 && k.rs_elems == 0);
    zero_destroy(c);

    // the plan query: the fused step's checks, the first launch's arguments, no launch
    c = make(16, 4, 3, 1, {10, 6}, &st);
    g_launch.clear();
    zsmr_plan pl;
    CHECK(zsmr_fused_step_plan(c, 2, 1, at<void>(G), 8, 4, at<float>(M), at<float>(MM),
                               at<float>(V), at<void>(P), &pl) == ZSMR_OK);
    CHECK(pl.kernel == (zsmr::M_REDUCE | zsmr::M_ADAM | zsmr::M_CAST) && pl.ring_tiles == 3);
    CHECK(pl.windowed == 1 && pl.store_elems == 4 && pl.launches == 1 && pl.head == 5);
    CHECK(pl.row_batch == 12);
    CHECK(zsmr::g_described.grads == at<const uint16_t>(G) + 4 && zsmr::g_described.n == 2);
    CHECK(zsmr::g_described.nrows == 4 && zsmr::g_described.p16 == at<uint16_t>(P));
    CHECK(zsmr_fused_step_plan(c, 2, 1, at<void>(G + 1), 8, 4, at<float>(M), at<float>(MM),
                               at<float>(V), at<void>(P), &pl) == ZSMR_ERR_ALIGN);
    CHECK(zsmr_fused_step_plan(c, 2, 1, at<void>(G), 1, 4, at<float>(M), at<float>(MM),
                               at<float>(V), at<void>(P), &pl) == ZSMR_ERR_ARG);
    CHECK(zsmr_fused_step_plan(c, 2, 1, at<void>(G), 8, 4, at<float>(M), at<float>(MM),
                               at<float>(V), at<void>(P), nullptr) == ZSMR_ERR_ARG);
    CHECK(zsmr_fused_step_plan(c, 4, 1, at<void>(G), 8, 4, at<float>(M), at<float>(MM),
                               at<float>(V), at<void>(P), &pl) == ZSMR_ERR_ARG);
    CHECK(g_launch.empty());
    CHECK(zero_counters(c, 2, &k) == ZSMR_OK && k.traffic_elems == 0);
    zero_destroy(c);

    // copies: the receive and the block receive
    c = make(64, 4, 2, 0, {}, &st);
    g_launch.clear();
    CHECK(zero_gather_copy(c, 1, at<void>(P), at<void>(O), 7, nullptr) == ZSMR_OK);
    CHECK(g_launch.size() == 1 && g_launch[0].kind == 1 && g_launch[0].n == 7);
    CHECK(zero_gather_copy(c, 1, at<void>(P), at<void>(P + 12), 7, nullptr) == ZSMR_ERR_ARG);
    CHECK(zero_gather_copy(c, 1, at<void>(P + 1), at<void>(O), 7, nullptr) == ZSMR_ERR_ALIGN);
    CHECK(zero_gather_copy(c, 1, nullptr, nullptr, 0, nullptr) == ZSMR_OK);
    CHECK(zero_gather_copy_blocks(c, 1, at<void>(P), at<void>(O), 5, 3, 16, nullptr) == ZSMR_OK);
    CHECK(g_launch.size() == 2 && g_launch[1].kind == 2 && g_launch[1].count == 3);
    CHECK(g_launch[1].stride == 16 && g_launch[1].n == 5);
    CHECK(zero_gather_copy_blocks(c, 1, at<void>(P), at<void>(O), 5, 65536, 16, nullptr) == ZSMR_ERR_ARG);
    CHECK(zero_gather_copy_blocks(c, 1, at<void>(P), at<void>(O), 5, 3, 4, nullptr) == ZSMR_ERR_ARG);
    CHECK(zero_gather_copy_blocks(c, 1, at<void>(P), at<void>(O), 5, 3, INT64_MAX / 2, nullptr) == ZSMR_ERR_ARG);
    CHECK(zero_gather_copy_blocks(c, 1, at<void>(P), at<void>(P + 60), 5, 3, 16, nullptr) == ZSMR_ERR_ARG);
    CHECK(zero_gather_copy_blocks(c, 1, at<void>(P), at<void>(O), 5, 1, 0, nullptr) == ZSMR_OK);
    CHECK(zero_gather_copy_blocks(c, 1, at<void>(P), at<void>(O), 0, 3, 0, nullptr) == ZSMR_OK);
    CHECK(g_launch.size() == 3);
    CHECK(zero_counters(c, 1, &k) == ZSMR_OK && k.ag_elems == 7 + 15 + 5);
    zero_destroy(c);
}

// ---- sizes and codes at and past the documented limits
static void limits() {
    int32_t st;
    zsmr_ctx* c = nullptr;
    CHECK(zero_init_shards(nullptr, 8, 2, 1, ZSMR_BF16, ZSMR_BF16, 0, nullptr, 0) == ZSMR_ERR_ARG);
    const int64_t big[] = {ZSMR_MAX_NUMEL + 1, INT64_MAX, 0, -1};
    for (int64_t n : big)
        for (int32_t stage = 0; stage <= 4; ++stage)
            CHECK(zero_init_shards(&c, n, 3, stage, ZSMR_BF16, ZSMR_BF16, 1, nullptr, 0) == ZSMR_ERR_ARG && !c);
    for (int32_t stage = 0; stage <= 4; ++stage) {
        c = make(ZSMR_MAX_NUMEL, 7, stage, 1, {}, &st);
        CHECK(c);
        zsmr_bytes b;
        CHECK(zero_bytes_per_rank(c, ZSMR_MAX_GATHER_BYTES, 2, &b) == ZSMR_OK);
        CHECK(b.resident > 0 && b.peak >= b.resident && b.traffic_bytes >= 0);
        CHECK(zero_bytes_per_rank(c, ZSMR_MAX_GATHER_BYTES + 1, 1, &b) == ZSMR_ERR_ARG);
        CHECK(zero_bytes_of_rank(c, 0, INT32_MAX, 1, &b) == ZSMR_ERR_ARG);
        CHECK(zero_bytes_of_rank(c, 0, 2, INT32_MAX, &b) == ZSMR_OK);
        zero_destroy(c);
    }
    // the largest world, and many units of one element each padded to it
    c = make(ZSMR_MAX_WORLD, ZSMR_MAX_WORLD, 2, 0, {}, &st);
    CHECK(c);
    zero_destroy(c);
    CHECK(zero_init_shards(&c, 8, ZSMR_MAX_WORLD + 1, 1, ZSMR_BF16, ZSMR_BF16, 1, nullptr, 0) == ZSMR_ERR_ARG);
    std::vector<int64_t> ones(4096, 1);
    c = make(4096, 1 << 20, 3, 1, ones, &st);
    CHECK(c);
    zsmr_layout_info li;
    CHECK(zero_layout_info(c, &li) == ZSMR_OK && li.padded_numel == (int64_t)4096 << 20);
    zero_destroy(c);
    std::vector<int64_t> many(ZSMR_MAX_UNITS + 1, 1);
    CHECK(zero_init_shards(&c, (int64_t)many.size(), 1, 3, ZSMR_BF16, ZSMR_BF16, 0, many.data(),
                           (int32_t)many.size()) == ZSMR_ERR_ARG);
    std::vector<int64_t> sums = {INT64_MAX, 1};
    CHECK(zero_init_shards(&c, 8, 2, 3, ZSMR_BF16, ZSMR_BF16, 1, sums.data(), 2) == ZSMR_ERR_ARG);
    std::vector<int64_t> neg = {9, -1};
    CHECK(zero_init_shards(&c, 8, 2, 3, ZSMR_BF16, ZSMR_BF16, 1, neg.data(), 2) == ZSMR_ERR_ARG);
    CHECK(zero_init_shards(&c, 8, 2, 3, 3, ZSMR_BF16, 1, nullptr, 0) == ZSMR_ERR_DTYPE);
    CHECK(zero_init_shards(&c, 8, 2, 5, ZSMR_BF16, ZSMR_BF16, 1, nullptr, 0) == ZSMR_ERR_ARG);
    CHECK(zero_init_shards(&c, 10, 4, 1, ZSMR_BF16, ZSMR_BF16, 0, nullptr, 0) == ZSMR_ERR_INDIVISIBLE);
    CHECK(zero_init_shards(&c, 8, 2, 1, ZSMR_BF16, ZSMR_BF16, 2, nullptr, 0) == ZSMR_ERR_ARG);
    zero_destroy(nullptr);
    for (int32_t s = -1; s <= 7; ++s) CHECK(zsmr_strerror(s) != nullptr);
    CHECK(zsmr_set_launch_shape(65, 0, 3, 24) == ZSMR_ERR_ARG);
    CHECK(zsmr_set_launch_shape(0, 0, 6, 24) == ZSMR_ERR_ARG);
    CHECK(zsmr_set_launch_shape(0, 0, 3, 0) == ZSMR_ERR_ARG);
    CHECK(zsmr_set_launch_shape(4, 8, 2, 16) == ZSMR_OK && zsmr::g_shape[1] == 8);
    CHECK(zsmr_set_write_window(500, 100, 10, 10) == ZSMR_ERR_ARG);
    CHECK(zsmr_set_write_window(72000, 72000, 0, 0) == ZSMR_ERR_ARG);
    CHECK(zsmr_set_write_window(INT32_MAX, INT32_MAX - 1, INT32_MAX, 0) == ZSMR_ERR_ARG);
    CHECK(zsmr_set_write_window(72000, 11000, 1000, 4000) == ZSMR_OK && zsmr::g_window[0] == 72000);
    CHECK(zsmr_set_write_window(0, 0, 0, 0) == ZSMR_OK && zsmr::g_window[0] == 0);
    CHECK(zsmr_set_xcd_balance(499) == ZSMR_ERR_ARG && zsmr_set_xcd_balance(2001) == ZSMR_ERR_ARG);
    CHECK(zsmr_set_xcd_balance(1000) == ZSMR_OK && zsmr::g_balance == 1000);
    CHECK(zsmr_set_xcd_balance(1200) == ZSMR_OK && zsmr::g_balance == 1200);
}

int main() {
    layout_sweep();
    launches();
    limits();
    std::printf("host checks passed\n");
    return 0;
}
"""


def _compile(tmp_path, extra):
    src = tmp_path / "host_driver.cpp"
    src.write_text(DRIVER)
    exe = tmp_path / "host_driver"
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-Wall", "-Wextra", "-Werror",
           "-Wno-deprecated-declarations", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", os.path.join(ROCM, "include"),
           *extra, os.path.join(CSRC, "zsmr_api.cpp"), str(src), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


def _run(exe, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "host checks passed" in r.stdout
    return r


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_code_plain(tmp_path):
    """The driver's own checks, without sanitizers."""
    _run(_compile(tmp_path, []))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = _compile(tmp_path, ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                              "-fno-omit-frame-pointer"])
    # the sanitizer runtime need not come first among the preloaded libraries
    _run(exe, {"ASAN_OPTIONS": "detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
