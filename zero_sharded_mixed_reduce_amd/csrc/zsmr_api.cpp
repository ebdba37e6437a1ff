// Host side of libzsmr.so: the C ABI declared in include/zsmr.h.
//
// Layout and accounting are integer host code (no HIP call), so they work on
// a machine without a GPU.  Device entry points validate every argument,
// compute the fp32 Adam constants, launch through zsmr_launch.h on the
// caller's stream and only then update the per-rank counters.
#include <algorithm>
#include <cstdint>
#include <cmath>
#include <cstring>
#include <memory>
#include <new>
#include <string>
#include <vector>

#include "zsmr.h"
#include "zsmr_launch.h"

struct zsmr_ctx {
    int64_t numel = 0;
    int32_t world = 0, stage = 0, gdt = 0, pdt = 0, pad = 0;
    std::vector<int64_t> units;        // true unit sizes
    std::vector<int64_t> shard_u;      // S_u (stage 3); {S} stages 1-2; {Psi} DP; P_u (stage 4)
    std::vector<int64_t> unit_pstart;  // padded start Q_u (stage 3); unit start (stage 4); {0} otherwise
    std::vector<int64_t> local_off;    // offset of unit u's piece in its holder's shard
    std::vector<int32_t> owners;       // stage 4: the rank owning each unit
    std::vector<int64_t> own;          // stage 4: elements each rank owns
    int64_t padded = 0, shard_total = 0;
    // counters per rank (elements): all-gathers received; reduce-scatters
    // received = sent at stages 1-3, sent at stage 4; all-reduce
    std::vector<int64_t> rs, ag, ar;
    // ZeRO-3 schedule (live and peak gathered bytes per rank: at stage 4 a
    // rank needs no buffer for its own units)
    std::vector<int64_t> gathers, releases;
    std::vector<char> live;
    int32_t max_live = 1, live_units = 0;
    std::vector<int64_t> live_bytes, peak_live_bytes;
};

namespace {

thread_local std::string g_hip_error;

int32_t hip_fail(hipError_t e) {
    g_hip_error = hipGetErrorString(e);
    return ZSMR_ERR_HIP;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool dtype_ok(int32_t d) { return d == ZSMR_FP16 || d == ZSMR_BF16; }

bool stage3(const zsmr_ctx* c) { return c->stage == ZSMR_ZERO3 || c->stage == ZSMR_ZERO3_OWNER; }

int n_pieces(const zsmr_ctx* c) { return stage3(c) ? (int)c->units.size() : 1; }

int32_t check_piece(const zsmr_ctx* c, int32_t rank, int32_t unit) {
    if (!c) return ZSMR_ERR_ARG;
    if (rank < 0 || rank >= c->world) return ZSMR_ERR_ARG;
    if (unit < 0 || unit >= n_pieces(c)) return ZSMR_ERR_ARG;
    return ZSMR_OK;
}

void piece(const zsmr_ctx* c, int32_t rank, int32_t unit, int64_t* off, int64_t* len, int64_t* loc) {
    int64_t o, l, lo;
    if (c->stage == ZSMR_DP) {
        o = 0;
        l = c->numel;
        lo = 0;
    } else if (c->stage == ZSMR_ZERO3_OWNER) {
        o = c->unit_pstart[unit];
        l = c->owners[unit] == rank ? c->units[unit] : 0;
        lo = c->local_off[unit];
    } else if (c->stage != ZSMR_ZERO3) {
        l = c->shard_u[0];
        o = (int64_t)rank * l;
        lo = 0;
    } else {
        l = c->shard_u[unit];
        o = c->unit_pstart[unit] + (int64_t)rank * l;
        lo = c->local_off[unit];
    }
    if (off) *off = o;
    if (len) *len = l;
    if (loc) *loc = lo;
}

bool al(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int32_t check_adam(const zsmr_adam* hp, int32_t t, zsmr::AdamK* k) {
    if (!hp || t < 1) return ZSMR_ERR_ARG;
    const double lr = hp->lr, b1 = hp->beta1, b2 = hp->beta2, eps = hp->eps;
    if (!std::isfinite(lr) || !std::isfinite(b1) || !std::isfinite(b2) || !std::isfinite(eps))
        return ZSMR_ERR_ARG;
    if (lr < 0 || b1 < 0 || b1 >= 1 || b2 < 0 || b2 >= 1 || eps < 0) return ZSMR_ERR_ARG;
    // Each constant is a double expression rounded to fp32 once ("The four
    // schemes", Base._adam uses Python scalars against fp32 arrays).
    k->c1 = (float)b1;
    k->c1m = (float)(1.0 - b1);
    k->c2 = (float)b2;
    k->c2m = (float)(1.0 - b2);
    k->bc1 = (float)(1.0 - std::pow(b1, (double)t));
    k->bc2 = (float)(1.0 - std::pow(b2, (double)t));
    k->lr = (float)lr;
    k->eps = (float)eps;
    return ZSMR_OK;
}

// Counting of one reduce over (rank, unit) of `len` elements: a data-parallel
// replica takes part in one all-reduce of the whole vector; a sharded rank
// receives (N-1) peers' contributions to its piece (and sends as many); at
// stage 4 every other rank sends its contribution to the owner.
void count_reduce(zsmr_ctx* c, int32_t rank, int64_t len) {
    const int64_t w = c->world;
    if (c->stage == ZSMR_DP) {
        c->ar[rank] += 2 * (w - 1) * ceil_div(c->numel, w);
    } else if (c->stage == ZSMR_ZERO3_OWNER) {
        for (int32_t q = 0; q < c->world; ++q)
            if (q != rank) c->rs[q] += len;
    } else {
        c->rs[rank] += (w - 1) * len;
    }
}

// Stage 4: the owner of each unit is the rank whose equal share of the vector
// holds the unit's midpoint, floor(N * (2 * start + size) / (2 * Psi)).
int32_t midpoint_owner(int64_t start, int64_t size, int64_t numel, int32_t world) {
    const __int128 num = (__int128)world * (2 * (__int128)start + size);
    const int64_t r = (int64_t)(num / (2 * (__int128)numel));
    return r < world - 1 ? (int32_t)r : world - 1;
}

// Stage 4: each unit's offset within its owner's concatenated units, what
// every rank owns, and the most any rank owns, from c->owners (no
// allocation: the vectors are sized when the context is built).
void assign_owners(zsmr_ctx* c) {
    std::fill(c->own.begin(), c->own.end(), 0);
    for (size_t u = 0; u < c->units.size(); ++u) {
        const int32_t o = c->owners[u];
        c->local_off[u] = c->own[o];
        c->own[o] += c->units[u];
    }
    c->shard_total = *std::max_element(c->own.begin(), c->own.end());
}

// The largest sum of size(u) over max_live consecutive units (all of them if
// there are fewer): the most a rank holds gathered at once when units are
// gathered in order and at most max_live are live.  One pass, a running sum
// over the window.
template <typename F>
int64_t most_in_window(int64_t n_units, int64_t max_live, F size) {
    const int64_t k = max_live < n_units ? max_live : n_units;
    int64_t best = 0, sum = 0;
    for (int64_t j = 0; j < n_units; ++j) {
        sum += size(j);
        if (j >= k) sum -= size(j - k);
        if (j >= k - 1 && sum > best) best = sum;
    }
    return best;
}

// Counting of one cast of (rank, unit): at stages 1-2 the all-gather delivers
// the rank's slot to every other rank; DP and stage 3 cast locally.
void count_cast(zsmr_ctx* c, int32_t rank, int64_t len) {
    if (c->stage == ZSMR_ZERO1 || c->stage == ZSMR_ZERO2)
        for (int32_t q = 0; q < c->world; ++q)
            if (q != rank) c->ag[q] += len;
}

// The body of zero_init_shards once the scalar arguments are checked; the
// vectors it fills may throw std::bad_alloc, which the caller turns into a
// status (an exception may not cross the C ABI).
int32_t build_ctx(zsmr_ctx** out, int64_t numel, int32_t world, int32_t stage,
                  int32_t grad_dtype, int32_t param_dtype, int32_t pad,
                  const int64_t* unit_numel, int32_t n_units) {
    std::vector<int64_t> units;
    if (n_units == 0) {
        units.push_back(numel);
    } else {
        int64_t sum = 0;
        for (int32_t i = 0; i < n_units; ++i) {
            if (unit_numel[i] < 1 || unit_numel[i] > numel - sum) return ZSMR_ERR_ARG;
            sum += unit_numel[i];
            units.push_back(unit_numel[i]);
        }
        if (sum != numel) return ZSMR_ERR_ARG;
    }
    std::unique_ptr<zsmr_ctx> c(new zsmr_ctx);
    c->numel = numel;
    c->world = world;
    c->stage = stage;
    c->gdt = grad_dtype;
    c->pdt = param_dtype;
    c->pad = pad;
    c->units = units;
    if (stage == ZSMR_DP) {
        c->shard_u = {numel};
        c->unit_pstart = {0};
        c->local_off = {0};
        c->padded = numel;
        c->shard_total = numel;
    } else if (stage == ZSMR_ZERO3_OWNER) {
        // whole units, natural order, no padding; owners by default from the
        // midpoint rule, replaceable by zero_set_unit_owners()
        int64_t start = 0;
        for (int64_t u : units) {
            c->shard_u.push_back(u);
            c->unit_pstart.push_back(start);
            c->owners.push_back(midpoint_owner(start, u, numel, world));
            start += u;
        }
        c->local_off.assign(units.size(), 0);
        c->own.assign(world, 0);
        assign_owners(c.get());
        c->padded = numel;
    } else if (stage != ZSMR_ZERO3) {
        if (numel % world && !pad) {
            return ZSMR_ERR_INDIVISIBLE;
        }
        const int64_t s = ceil_div(numel, world);
        c->shard_u = {s};
        c->unit_pstart = {0};
        c->local_off = {0};
        c->padded = s * world;
        c->shard_total = s;
    } else {
        int64_t q = 0, loc = 0;
        for (int64_t u : units) {
            if (u % world && !pad) {
                return ZSMR_ERR_INDIVISIBLE;
            }
            const int64_t s = ceil_div(u, world);
            c->shard_u.push_back(s);
            c->unit_pstart.push_back(q);
            c->local_off.push_back(loc);
            q += s * world;
            loc += s;
        }
        c->padded = q;
        c->shard_total = loc;
    }
    c->rs.assign(world, 0);
    c->ag.assign(world, 0);
    c->ar.assign(world, 0);
    c->gathers.assign(units.size(), 0);
    c->releases.assign(units.size(), 0);
    c->live.assign(units.size(), 0);
    c->live_bytes.assign(world, 0);
    c->peak_live_bytes.assign(world, 0);
    *out = c.release();
    return ZSMR_OK;
}

}  // namespace

extern "C" {

const char* zsmr_strerror(int32_t s) {
    switch (s) {
        case ZSMR_OK: return "ok";
        case ZSMR_ERR_ARG: return "invalid argument";
        case ZSMR_ERR_INDIVISIBLE: return "parameter count (or unit) not divisible by world size";
        case ZSMR_ERR_STATE: return "ZeRO-3 gather/release out of order";
        case ZSMR_ERR_DTYPE: return "unknown 16-bit format";
        case ZSMR_ERR_ALIGN: return "pointer not aligned to its element size";
        case ZSMR_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* zsmr_last_hip_error(void) { return g_hip_error.c_str(); }

int32_t zero_init_shards(zsmr_ctx** out, int64_t numel, int32_t world, int32_t stage,
                         int32_t grad_dtype, int32_t param_dtype, int32_t pad,
                         const int64_t* unit_numel, int32_t n_units) {
    if (!out) return ZSMR_ERR_ARG;
    *out = nullptr;
    if (numel < 1 || numel > ZSMR_MAX_NUMEL || world < 1 || world > ZSMR_MAX_WORLD ||
        stage < ZSMR_DP || stage > ZSMR_ZERO3_OWNER || (pad != 0 && pad != 1))
        return ZSMR_ERR_ARG;
    if (!dtype_ok(grad_dtype) || !dtype_ok(param_dtype)) return ZSMR_ERR_DTYPE;
    if (n_units < 0 || n_units > ZSMR_MAX_UNITS || (n_units > 0 && !unit_numel) ||
        (n_units == 0 && unit_numel))
        return ZSMR_ERR_ARG;
    try {
        return build_ctx(out, numel, world, stage, grad_dtype, param_dtype, pad, unit_numel,
                         n_units);
    } catch (const std::bad_alloc&) {
        return ZSMR_ERR_ARG;
    }
}

void zero_destroy(zsmr_ctx* ctx) { delete ctx; }

int32_t zero_layout_info(const zsmr_ctx* c, zsmr_layout_info* out) {
    if (!c || !out) return ZSMR_ERR_ARG;
    out->numel = c->numel;
    out->padded_numel = c->padded;
    out->shard_numel = c->shard_total;
    int64_t mx = 0;
    if (c->stage == ZSMR_ZERO3) {
        for (int64_t s : c->shard_u) mx = s * c->world > mx ? s * c->world : mx;
    } else if (c->stage == ZSMR_ZERO3_OWNER) {
        for (int64_t u : c->units) mx = u > mx ? u : mx;
    } else {
        mx = c->padded;
    }
    out->max_unit_numel = mx;
    out->world = c->world;
    out->stage = c->stage;
    out->n_units = (int32_t)c->units.size();
    out->grad_dtype = c->gdt;
    out->param_dtype = c->pdt;
    out->pad = c->pad;
    return ZSMR_OK;
}

int32_t zero_layout(const zsmr_ctx* c, int32_t rank, int32_t unit, int64_t* offset, int64_t* len,
                    int64_t* local_offset) {
    const int32_t st = check_piece(c, rank, unit);
    if (st) return st;
    piece(c, rank, unit, offset, len, local_offset);
    return ZSMR_OK;
}

namespace {

// Stage 4, one rank: its own units' 16 bytes per element; it receives each
// weight it does not own twice and sends each of those gradients once; its
// peak adds the borrowed units live at once ("One Poem Suffices: ZeRO"
// section 4.1.4; "ZeRO, annotated" section 7).
void owner_bytes(const zsmr_ctx* c, int32_t rank, int64_t gather_bytes, int64_t max_live,
                 zsmr_bytes* o) {
    const int64_t own = c->own[rank];
    std::memset(o, 0, sizeof(*o));
    o->res_p16 = 2 * own;
    o->res_grad = 2 * own;
    o->res_master = 4 * own;
    o->res_m = 4 * own;
    o->res_v = 4 * own;
    o->resident = 16 * own;
    const int64_t nu = (int64_t)c->units.size();
    auto borrowed = [&](int64_t u) { return c->owners[u] == rank ? int64_t(0) : c->units[u]; };
    const int64_t best = most_in_window(nu, max_live, borrowed);
    int64_t widest = 0;
    for (int64_t u : c->units) widest = u > widest ? u : widest;
    o->gathered = gather_bytes * best;
    o->unit_grad = 2 * widest;
    o->peak = o->resident + o->gathered;
    o->rs_elems = c->numel - own;
    o->ag_elems = 2 * (c->numel - own);
    o->traffic_elems = o->rs_elems + o->ag_elems;
    o->traffic_bytes = 2 * o->traffic_elems;
}

// Stages 0-3: every rank holds the same.
void even_bytes(const zsmr_ctx* c, int64_t gather_bytes, int64_t max_live, zsmr_bytes* o) {
    const int64_t n = c->numel, w = c->world;
    const bool shard_opt = c->stage >= ZSMR_ZERO1, shard_grad = c->stage >= ZSMR_ZERO2,
               shard_param = c->stage >= ZSMR_ZERO3;
    const int64_t s = c->shard_total;
    std::memset(o, 0, sizeof(*o));
    // bytes per element of each band: 2 + 2 + 4 + 4 + 4 = 16 ("One Poem
    // Suffices: ZeRO" section 3.1; "The four schemes", per-band constants)
    o->res_p16 = 2 * (shard_param ? s : n);
    o->res_grad = 2 * (shard_grad ? s : n);
    const int64_t opt = shard_opt ? s : n;
    o->res_master = 4 * opt;
    o->res_m = 4 * opt;
    o->res_v = 4 * opt;
    o->resident = o->res_p16 + o->res_grad + o->res_master + o->res_m + o->res_v;
    if (c->stage == ZSMR_ZERO3) {
        const int64_t nu = (int64_t)c->shard_u.size();
        const int64_t best = most_in_window(nu, max_live, [&](int64_t u) { return w * c->shard_u[u]; });
        int64_t widest = 0;
        for (int64_t su : c->shard_u) widest = w * su > widest ? w * su : widest;
        o->gathered = gather_bytes * best;
        o->unit_grad = 2 * widest;
    }
    o->peak = o->resident + o->gathered;
    if (c->stage == ZSMR_DP) {
        o->ar_elems = 2 * (w - 1) * ceil_div(n, w);
    } else if (c->stage != ZSMR_ZERO3) {
        o->rs_elems = (w - 1) * s;
        o->ag_elems = (w - 1) * s;
    } else {
        o->rs_elems = (w - 1) * s;
        o->ag_elems = 2 * (w - 1) * s;
    }
    o->traffic_elems = o->rs_elems + o->ag_elems + o->ar_elems;
    o->traffic_bytes = 2 * o->traffic_elems;
}

}  // namespace

int32_t zero_bytes_of_rank(const zsmr_ctx* c, int32_t rank, int32_t gather_bytes,
                           int32_t max_live, zsmr_bytes* o) {
    if (!c || !o || rank < 0 || rank >= c->world || gather_bytes < 0 ||
        gather_bytes > ZSMR_MAX_GATHER_BYTES || max_live < 0)
        return ZSMR_ERR_ARG;
    if (gather_bytes == 0) gather_bytes = 2;
    if (max_live == 0) max_live = 1;
    if (c->stage == ZSMR_ZERO3_OWNER)
        owner_bytes(c, rank, gather_bytes, max_live, o);
    else
        even_bytes(c, gather_bytes, max_live, o);
    return ZSMR_OK;
}

int32_t zero_bytes_per_rank(const zsmr_ctx* c, int32_t gather_bytes, int32_t max_live,
                            zsmr_bytes* o) {
    if (!c || !o || gather_bytes < 0 || gather_bytes > ZSMR_MAX_GATHER_BYTES || max_live < 0)
        return ZSMR_ERR_ARG;
    if (c->stage != ZSMR_ZERO3_OWNER) return zero_bytes_of_rank(c, 0, gather_bytes, max_live, o);
    // stage 4: the rank with the largest peak (the lowest such rank)
    zsmr_bytes best{}, cur{};
    for (int32_t r = 0; r < c->world; ++r) {
        zero_bytes_of_rank(c, r, gather_bytes, max_live, &cur);
        if (r == 0 || cur.peak > best.peak) best = cur;
    }
    *o = best;
    return ZSMR_OK;
}

int32_t zero_counters(const zsmr_ctx* c, int32_t rank, zsmr_counters* o) {
    if (!c || !o || rank < 0 || rank >= c->world) return ZSMR_ERR_ARG;
    std::memset(o, 0, sizeof(*o));
    o->rs_elems = c->rs[rank];
    o->ag_elems = c->ag[rank];
    o->ar_elems = c->ar[rank];
    o->traffic_elems = o->rs_elems + o->ag_elems + o->ar_elems;
    o->traffic_bytes = 2 * o->traffic_elems;
    for (size_t u = 0; u < c->gathers.size(); ++u) {
        o->stage3_gathers += c->gathers[u];
        o->stage3_releases += c->releases[u];
    }
    o->live_units = c->live_units;
    o->live_bytes = c->live_bytes[rank];
    o->peak_live_bytes = c->peak_live_bytes[rank];
    return ZSMR_OK;
}

int32_t zero_reset_counters(zsmr_ctx* c) {
    if (!c) return ZSMR_ERR_ARG;
    std::fill(c->rs.begin(), c->rs.end(), 0);
    std::fill(c->ag.begin(), c->ag.end(), 0);
    std::fill(c->ar.begin(), c->ar.end(), 0);
    std::fill(c->gathers.begin(), c->gathers.end(), 0);
    std::fill(c->releases.begin(), c->releases.end(), 0);
    c->peak_live_bytes = c->live_bytes;
    return ZSMR_OK;
}

int32_t zero_init_state(const zsmr_ctx* c, int32_t rank, int32_t unit, const float* theta0,
                        float* master, float* m, float* v, void* p16, hipStream_t stream) {
    int32_t st = check_piece(c, rank, unit);
    if (st) return st;
    if (!theta0 || !master || !m || !v || !p16) return ZSMR_ERR_ARG;
    if (!al(theta0, 4) || !al(master, 4) || !al(m, 4) || !al(v, 4) || !al(p16, 2))
        return ZSMR_ERR_ALIGN;
    int64_t len = 0;
    piece(c, rank, unit, nullptr, &len, nullptr);
    zsmr::StepArgs a{};
    a.g_in = theta0;
    a.master = master;
    a.m = m;
    a.v = v;
    a.p16 = static_cast<uint16_t*>(p16);
    a.n = len;
    const hipError_t e = zsmr::launch_step(zsmr::M_INIT | zsmr::M_CAST, c->gdt, c->pdt, a, stream);
    return e == hipSuccess ? ZSMR_OK : hip_fail(e);
}

static int32_t check_grads(const zsmr_ctx* c, const void* grads, int64_t row_stride,
                           int64_t base, int64_t len) {
    if (!grads || base < 0 || row_stride < 0) return ZSMR_ERR_ARG;
    if (c->world > 1 && row_stride < len) return ZSMR_ERR_ARG;   // rows may not overlap
    if (!al(grads, 2)) return ZSMR_ERR_ALIGN;
    return ZSMR_OK;
}

// N as the divisor of the mean; for N a power of two also 1/N, which the
// kernels multiply by instead (the same bits).
static void set_mean_divisor(zsmr::StepArgs& a, int32_t world) {
    a.nf = (float)world;
    a.inv_pow2 = world > 0 && (world & (world - 1)) == 0;
    a.inv_nf = a.inv_pow2 ? 1.0f / (float)world : 0.0f;
}

int32_t zero_reduce_shard(zsmr_ctx* c, int32_t rank, int32_t unit, const void* grads,
                          int64_t row_stride, int64_t base, int32_t mean, float* g_out,
                          hipStream_t stream) {
    int32_t st = check_piece(c, rank, unit);
    if (st) return st;
    int64_t len = 0;
    piece(c, rank, unit, nullptr, &len, nullptr);
    if ((st = check_grads(c, grads, row_stride, base, len))) return st;
    if (!g_out || (mean != 0 && mean != 1)) return ZSMR_ERR_ARG;
    if (!al(g_out, 4)) return ZSMR_ERR_ALIGN;
    zsmr::StepArgs a{};
    a.grads = static_cast<const uint16_t*>(grads) + base;
    a.row_stride = row_stride;
    a.nrows = c->world;
    a.mean = mean;
    set_mean_divisor(a, c->world);
    a.g_out = g_out;
    a.n = len;
    const hipError_t e = zsmr::launch_step(zsmr::M_REDUCE | zsmr::M_GOUT, c->gdt, c->pdt, a, stream);
    if (e != hipSuccess) return hip_fail(e);
    count_reduce(c, rank, len);
    return ZSMR_OK;
}

int32_t zero_adam_step(float* master, float* m, float* v, const float* g, int64_t n, int32_t t,
                       const zsmr_adam* hp, hipStream_t stream) {
    zsmr::AdamK k{};
    int32_t st = check_adam(hp, t, &k);
    if (st) return st;
    if (n < 0) return ZSMR_ERR_ARG;
    if (n == 0) return ZSMR_OK;
    if (!master || !m || !v || !g) return ZSMR_ERR_ARG;
    if (!al(master, 4) || !al(m, 4) || !al(v, 4) || !al(g, 4)) return ZSMR_ERR_ALIGN;
    zsmr::StepArgs a{};
    a.g_in = g;
    a.master = master;
    a.m = m;
    a.v = v;
    a.n = n;
    a.k = k;
    const hipError_t e = zsmr::launch_step(zsmr::M_ADAM, ZSMR_BF16, ZSMR_BF16, a, stream);
    return e == hipSuccess ? ZSMR_OK : hip_fail(e);
}

int32_t zero_gather_cast(zsmr_ctx* c, int32_t rank, int32_t unit, const float* master,
                         void* p16_dst, hipStream_t stream) {
    int32_t st = check_piece(c, rank, unit);
    if (st) return st;
    if (!master || !p16_dst) return ZSMR_ERR_ARG;
    if (!al(master, 4) || !al(p16_dst, 2)) return ZSMR_ERR_ALIGN;
    int64_t len = 0;
    piece(c, rank, unit, nullptr, &len, nullptr);
    zsmr::StepArgs a{};
    a.master = const_cast<float*>(master);
    a.p16 = static_cast<uint16_t*>(p16_dst);
    a.n = len;
    const hipError_t e = zsmr::launch_step(zsmr::M_CAST, c->gdt, c->pdt, a, stream);
    if (e != hipSuccess) return hip_fail(e);
    count_cast(c, rank, len);
    return ZSMR_OK;
}

// The arguments of the fused step over [begin, begin + count) of the
// (rank, unit) piece (whole: the piece), checked as every fused call checks
// them.  *empty is set when there is nothing to launch.
static int32_t fused_args(const zsmr_ctx* c, int32_t rank, int32_t unit, int64_t begin,
                          int64_t count, bool whole, const void* grads, int64_t row_stride,
                          int64_t base, float* master, float* m, float* v, void* p16_dst,
                          int32_t t, const zsmr_adam* hp, zsmr::StepArgs* a) {
    int32_t st = check_piece(c, rank, unit);
    if (st) return st;
    int64_t len = 0;
    piece(c, rank, unit, nullptr, &len, nullptr);
    if (whole) {
        begin = 0;
        count = len;
    }
    if (begin < 0 || count < 0 || begin > len - count) return ZSMR_ERR_ARG;
    // a data-parallel replica's all-reduce covers the whole vector: it is
    // counted once per step, so a range must be the whole vector too
    if (c->stage == ZSMR_DP && count != len) return ZSMR_ERR_ARG;
    if ((st = check_grads(c, grads, row_stride, base, len))) return st;
    zsmr::AdamK k{};
    if ((st = check_adam(hp, t, &k))) return st;
    if (!master || !m || !v || !p16_dst) return ZSMR_ERR_ARG;
    if (!al(master, 4) || !al(m, 4) || !al(v, 4) || !al(p16_dst, 2)) return ZSMR_ERR_ALIGN;
    *a = zsmr::StepArgs{};
    a->grads = static_cast<const uint16_t*>(grads) + base + begin;
    a->row_stride = row_stride;
    a->nrows = c->world;
    a->mean = 1;
    set_mean_divisor(*a, c->world);
    a->master = master + begin;
    a->m = m + begin;
    a->v = v + begin;
    a->p16 = static_cast<uint16_t*>(p16_dst) + begin;
    a->n = count;
    a->k = k;
    return ZSMR_OK;
}

static int32_t fused_range(zsmr_ctx* c, int32_t rank, int32_t unit, int64_t begin, int64_t count,
                           bool whole, const void* grads, int64_t row_stride, int64_t base,
                           float* master, float* m, float* v, void* p16_dst, int32_t t,
                           const zsmr_adam* hp, hipStream_t stream) {
    zsmr::StepArgs a{};
    const int32_t st = fused_args(c, rank, unit, begin, count, whole, grads, row_stride, base,
                                  master, m, v, p16_dst, t, hp, &a);
    if (st) return st;
    if (a.n == 0) return ZSMR_OK;
    const hipError_t e =
        zsmr::launch_step(zsmr::M_REDUCE | zsmr::M_ADAM | zsmr::M_CAST, c->gdt, c->pdt, a, stream);
    if (e != hipSuccess) return hip_fail(e);
    count_reduce(c, rank, a.n);
    count_cast(c, rank, a.n);
    return ZSMR_OK;
}

int32_t zero_fused_step(zsmr_ctx* c, int32_t rank, int32_t unit, const void* grads,
                        int64_t row_stride, int64_t base, float* master, float* m, float* v,
                        void* p16_dst, int32_t t, const zsmr_adam* hp, hipStream_t stream) {
    return fused_range(c, rank, unit, 0, 0, true, grads, row_stride, base, master, m, v, p16_dst, t,
                       hp, stream);
}

int32_t zero_fused_step_range(zsmr_ctx* c, int32_t rank, int32_t unit, int64_t begin,
                              int64_t count, const void* grads, int64_t row_stride,
                              int64_t base, float* master, float* m, float* v, void* p16_dst,
                              int32_t t, const zsmr_adam* hp, hipStream_t stream) {
    return fused_range(c, rank, unit, begin, count, false, grads, row_stride, base, master, m, v,
                       p16_dst, t, hp, stream);
}

int32_t zsmr_fused_step_plan(const zsmr_ctx* c, int32_t rank, int32_t unit, const void* grads,
                             int64_t row_stride, int64_t base, float* master, float* m, float* v,
                             void* p16_dst, zsmr_plan* out) {
    if (!out) return ZSMR_ERR_ARG;
    const zsmr_adam hp{1e-3, 0.9, 0.999, 1e-8};
    zsmr::StepArgs a{};
    const int32_t st = fused_args(c, rank, unit, 0, 0, true, grads, row_stride, base, master, m, v,
                                  p16_dst, 1, &hp, &a);
    if (st) return st;
    zsmr::StepPlan p{};
    zsmr::describe_step(zsmr::M_REDUCE | zsmr::M_ADAM | zsmr::M_CAST, a, &p);
    out->kernel = p.kernel;
    out->ring_tiles = p.ring_tiles;
    out->windowed = p.windowed;
    out->store_elems = p.store_elems;
    out->launches = p.launches;
    out->row_batch = p.row_batch;
    out->head = p.head;
    return ZSMR_OK;
}

int32_t zero_gather_copy(zsmr_ctx* c, int32_t recv_rank, const void* src, void* dst, int64_t n,
                         hipStream_t stream) {
    if (!c || recv_rank < 0 || recv_rank >= c->world || n < 0) return ZSMR_ERR_ARG;
    if (n == 0) return ZSMR_OK;
    if (!src || !dst) return ZSMR_ERR_ARG;
    if (!al(src, 2) || !al(dst, 2)) return ZSMR_ERR_ALIGN;
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    const uintptr_t bytes = static_cast<uintptr_t>(n) * 2;
    if (s < d + bytes && d < s + bytes) return ZSMR_ERR_ARG;
    const hipError_t e = zsmr::launch_copy16(static_cast<const uint16_t*>(src),
                                             static_cast<uint16_t*>(dst), n, stream);
    if (e != hipSuccess) return hip_fail(e);
    c->ag[recv_rank] += n;
    return ZSMR_OK;
}

int32_t zero_gather_copy_blocks(zsmr_ctx* c, int32_t recv_rank, const void* src, void* dst,
                                int64_t n, int32_t count, int64_t stride, hipStream_t stream) {
    if (!c || recv_rank < 0 || recv_rank >= c->world || n < 0 || count < 0 || count > 65535)
        return ZSMR_ERR_ARG;
    if (n == 0 || count == 0) return ZSMR_OK;
    if (count > 1 && (stride < n || stride > (INT64_MAX - n) / (count - 1)))
        return ZSMR_ERR_ARG;   // blocks would overlap, or the span would overflow
    if (!src || !dst) return ZSMR_ERR_ARG;
    if (!al(src, 2) || !al(dst, 2)) return ZSMR_ERR_ALIGN;
    const int64_t span = (int64_t)(count - 1) * (count > 1 ? stride : 0) + n;
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    const uintptr_t bytes = static_cast<uintptr_t>(span) * 2;
    if (s < d + bytes && d < s + bytes) return ZSMR_ERR_ARG;
    const hipError_t e = zsmr::launch_copy_blocks(static_cast<const uint16_t*>(src),
                                                  static_cast<uint16_t*>(dst), n, count, stride, stream);
    if (e != hipSuccess) return hip_fail(e);
    c->ag[recv_rank] += (int64_t)count * n;
    return ZSMR_OK;
}

int32_t zero_stage3_set_max_live(zsmr_ctx* c, int32_t max_live) {
    if (!c || !stage3(c) || max_live < 1) return ZSMR_ERR_ARG;
    if (c->live_units) return ZSMR_ERR_STATE;
    c->max_live = max_live;
    return ZSMR_OK;
}

int32_t zero_stage3_unit_gather(zsmr_ctx* c, int32_t unit, const void* const* shard_ptrs,
                                void* unit_buf, hipStream_t stream) {
    if (!c || !stage3(c) || unit < 0 || unit >= (int32_t)c->units.size()) return ZSMR_ERR_ARG;
    if (!shard_ptrs || !unit_buf) return ZSMR_ERR_ARG;
    const bool owner = c->stage == ZSMR_ZERO3_OWNER;
    const int32_t nsrc = owner ? 1 : c->world;      // stage 4: the owner's copy only
    for (int32_t r = 0; r < nsrc; ++r)
        if (!shard_ptrs[r]) return ZSMR_ERR_ARG;
    for (int32_t r = 0; r < nsrc; ++r)
        if (!al(shard_ptrs[r], 2)) return ZSMR_ERR_ALIGN;
    if (!al(unit_buf, 2)) return ZSMR_ERR_ALIGN;
    if (c->live[unit] || c->live_units >= c->max_live) return ZSMR_ERR_STATE;
    const int64_t each = owner ? c->units[unit] : c->shard_u[unit];
    // A source may not overlap the unit buffer, except a shard that already
    // sits exactly in its own slot (copied onto itself, it stays as it is).
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(unit_buf);
    const uintptr_t slot = static_cast<uintptr_t>(each) * 2;
    const uintptr_t d1 = d0 + slot * static_cast<uintptr_t>(nsrc);
    for (int32_t r = 0; r < nsrc; ++r) {
        const uintptr_t s0 = reinterpret_cast<uintptr_t>(shard_ptrs[r]);
        if (s0 == d0 + slot * static_cast<uintptr_t>(r)) continue;
        if (s0 < d1 && d0 < s0 + slot) return ZSMR_ERR_ARG;
    }
    const hipError_t e = zsmr::launch_gather16(reinterpret_cast<const uint16_t* const*>(shard_ptrs),
                                               nsrc, each, static_cast<uint16_t*>(unit_buf), stream);
    if (e != hipSuccess) return hip_fail(e);
    c->live[unit] = 1;
    c->live_units += 1;
    c->gathers[unit] += 1;
    for (int32_t r = 0; r < c->world; ++r) {
        if (owner && r == c->owners[unit]) continue;       // the owner holds it already
        c->ag[r] += owner ? each : (int64_t)(c->world - 1) * each;
        c->live_bytes[r] += owner ? 2 * each : 2 * (int64_t)c->world * each;
        if (c->live_bytes[r] > c->peak_live_bytes[r]) c->peak_live_bytes[r] = c->live_bytes[r];
    }
    return ZSMR_OK;
}

int32_t zero_stage3_unit_release(zsmr_ctx* c, int32_t unit) {
    if (!c || !stage3(c) || unit < 0 || unit >= (int32_t)c->units.size()) return ZSMR_ERR_ARG;
    if (!c->live[unit]) return ZSMR_ERR_STATE;
    const bool owner = c->stage == ZSMR_ZERO3_OWNER;
    c->live[unit] = 0;
    c->live_units -= 1;
    c->releases[unit] += 1;
    for (int32_t r = 0; r < c->world; ++r) {
        if (owner && r == c->owners[unit]) continue;
        c->live_bytes[r] -= owner ? 2 * c->units[unit] : 2 * (int64_t)c->world * c->shard_u[unit];
    }
    return ZSMR_OK;
}

int32_t zero_stage3_unit_state(const zsmr_ctx* c, int32_t unit, int32_t* live, int64_t* gathers,
                               int64_t* releases) {
    if (!c || !stage3(c) || unit < 0 || unit >= (int32_t)c->units.size()) return ZSMR_ERR_ARG;
    if (live) *live = c->live[unit];
    if (gathers) *gathers = c->gathers[unit];
    if (releases) *releases = c->releases[unit];
    return ZSMR_OK;
}

int32_t zero_set_unit_owners(zsmr_ctx* c, const int32_t* owners, int32_t n_units) {
    if (!c || !owners || c->stage != ZSMR_ZERO3_OWNER || n_units != (int32_t)c->units.size())
        return ZSMR_ERR_ARG;
    for (int32_t u = 0; u < n_units; ++u)
        if (owners[u] < 0 || owners[u] >= c->world) return ZSMR_ERR_ARG;
    // only on a context no call has used yet (or whose counters were reset
    // with no unit live): counters and schedule state follow the owners
    bool used = c->live_units != 0;
    for (int32_t r = 0; r < c->world; ++r)
        used = used || c->rs[r] || c->ag[r] || c->ar[r] || c->live_bytes[r] || c->peak_live_bytes[r];
    for (size_t u = 0; u < c->units.size(); ++u) used = used || c->gathers[u] || c->releases[u];
    if (used) return ZSMR_ERR_STATE;
    std::copy(owners, owners + n_units, c->owners.begin());
    assign_owners(c);
    return ZSMR_OK;
}

int32_t zero_unit_owner(const zsmr_ctx* c, int32_t unit, int32_t* owner) {
    if (!c || !owner || c->stage != ZSMR_ZERO3_OWNER || unit < 0 ||
        unit >= (int32_t)c->units.size())
        return ZSMR_ERR_ARG;
    *owner = c->owners[unit];
    return ZSMR_OK;
}

int32_t zsmr_set_launch_shape(int32_t step_bpc, int32_t copy_bpc, int32_t defer_tiles,
                              int32_t defer_min_rows) {
    if (step_bpc < 0 || step_bpc > 64 || copy_bpc < 0 || copy_bpc > 64 || defer_tiles < 0 ||
        defer_tiles > 5 || defer_min_rows < 1)
        return ZSMR_ERR_ARG;
    zsmr::set_launch_shape(step_bpc, copy_bpc, defer_tiles, defer_min_rows);
    return ZSMR_OK;
}

int32_t zsmr_set_write_window(int32_t cycle_ns, int32_t write_ns, int32_t margin_ns,
                              int32_t lead_ns) {
    if (cycle_ns != 0 && (cycle_ns < 1000 || cycle_ns > 10000000 || write_ns < 1 ||
                          margin_ns < 0 || (int64_t)write_ns + margin_ns >= cycle_ns ||
                          lead_ns < 0 || lead_ns >= write_ns))
        return ZSMR_ERR_ARG;
    if (cycle_ns == 0 && (write_ns < 0 || margin_ns < 0 || lead_ns < 0)) return ZSMR_ERR_ARG;
    zsmr::set_write_window(cycle_ns, write_ns, margin_ns, lead_ns);
    return ZSMR_OK;
}

int32_t zsmr_set_xcd_balance(int32_t even_permille) {
    if (even_permille < 500 || even_permille > 2000) return ZSMR_ERR_ARG;
    zsmr::set_xcd_balance(even_permille);
    return ZSMR_OK;
}

}  // extern "C"
