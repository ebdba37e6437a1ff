/*
 * zsmr.h -- C ABI of libzsmr.so, the ZeRO shard step on one MI355X (gfx950).
 *
 * The library runs the per-rank step of ZeRO data parallelism over a flat
 * parameter vector of Psi elements for a world of N ranks that is simulated in
 * one GPU's HBM:
 *   1. the arithmetic of the gradient reduce-scatter: N 16-bit gradient rows
 *      summed in fp32 in rank order 0..N-1, then divided by N;
 *   2. mixed-precision Adam on the rank's fp32 master, m and v shard;
 *   3. the all-gather side: the updated master cast (round to nearest even)
 *      into the 16-bit working copy, and copies of peers' 16-bit slices;
 *   4. ZeRO-3's per-unit gather -> use -> release -> re-gather schedule,
 *      with exact per-band byte and per-rank traffic accounting for data
 *      parallel and ZeRO stages 1-3.
 * Sources: "The four schemes" (the scheme flags table, Base._adam, the
 * accounting methods and the resident-vs-peak table), "ZeRO and FSDP" (the
 * three-stage table, ZeroAdam, "ZeRO-3 and FSDP"), "ZeRO, annotated"
 * (sections 3.1, 5.1-5.3 and 7), "One Poem Suffices: ZeRO" (sections 3.1 and
 * 4.1, Appendix B) and "Sharding the States.".
 *
 * Conventions for every entry point:
 *  - Return value: ZSMR_OK (0) or one of the ZSMR_ERR_* codes below; no C++
 *    exception crosses the ABI.  zsmr_strerror() names a code.
 *  - Device pointers are owned by the caller (the library never allocates
 *    device memory).  The library allocates only the host-side context.
 *  - Every device operation is enqueued asynchronously on the caller's
 *    hipStream_t (0 = the null stream).  Launch failures are returned at once
 *    (ZSMR_ERR_HIP, text in zsmr_last_hip_error()); faults during execution
 *    surface at the caller's next synchronisation.
 *  - Arguments are checked before anything is launched or counted; a call
 *    that returns an error has no effect.  The caller guarantees that every
 *    buffer covers the elements the call touches (the library cannot see
 *    allocation sizes through raw pointers).
 *  - A context is not thread-safe; calls on one context must be serialised.
 *  - Element counts and offsets are int64 (the 7.5e9-element working copy and
 *    the 2.5e10-element gradient set exceed 2^32).
 *  - fp32 buffers (master, m, v, g, theta0) must be 4-byte aligned; the fast
 *    path wants 16 bytes.  16-bit buffers must be 2-byte aligned.  Any legal
 *    alignment works; the kernel variant is chosen from the pointers.  Where
 *    a piece does not start on a 128-byte line, up to 63 leading elements
 *    run one by one so that the rest is processed in line-aligned tiles
 *    (results do not depend on it).
 */
#ifndef ZSMR_H
#define ZSMR_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define ZSMR_OK              0
#define ZSMR_ERR_ARG         1  /* null/negative/out-of-range argument        */
#define ZSMR_ERR_INDIVISIBLE 2  /* Psi or a unit not divisible by N, pad == 0 */
#define ZSMR_ERR_STATE       3  /* ZeRO-3 gather/release out of order         */
#define ZSMR_ERR_DTYPE       4  /* unknown 16-bit format code                 */
#define ZSMR_ERR_ALIGN       5  /* pointer not aligned to its element size    */
#define ZSMR_ERR_HIP         6  /* a HIP runtime call or launch failed        */

/* Size limits of a context.  Within them every element count, byte count
 * and traffic figure the library computes fits in int64_t with room to
 * spare: 2^56 elements is over 7e16 parameters, a world of 2^20 ranks and
 * 2^20 units exceed anything the pages consider. */
#define ZSMR_MAX_NUMEL ((int64_t)1 << 56)
#define ZSMR_MAX_WORLD (1 << 20)
#define ZSMR_MAX_UNITS (1 << 20)
/* largest bytes per gathered element an accounting call accepts (8: fp64) */
#define ZSMR_MAX_GATHER_BYTES 8

/* 16-bit formats of gradients and of the working copy */
#define ZSMR_FP16 1
#define ZSMR_BF16 2

/* schemes ("The four schemes", the three-flag table) */
#define ZSMR_DP    0  /* nothing sharded; one all-reduce per step          */
#define ZSMR_ZERO1 1  /* optimizer state sharded                            */
#define ZSMR_ZERO2 2  /* + gradients sharded                                */
#define ZSMR_ZERO3 3  /* + parameters sharded, gathered per unit            */
/* stage 3 with owner broadcast ("One Poem Suffices: ZeRO" section 4.1.4, the
 * 64-device, 192-block example; "ZeRO, annotated" section 7, where GPU i owns
 * shard i): every unit belongs whole to one rank, which sends it to the
 * others when it is needed; gradients are summed onto the owner */
#define ZSMR_ZERO3_OWNER 4

typedef struct zsmr_ctx zsmr_ctx;

/* Adam hyper-parameters, in double; the library rounds each constant of a
 * step (beta1, 1-beta1, beta2, 1-beta2, 1-beta1^t, 1-beta2^t, lr, eps) to
 * fp32 once, as the prototype's Python scalars are ("The four schemes",
 * Base._adam).  Requires lr >= 0, 0 <= beta < 1, eps >= 0, all finite. */
typedef struct zsmr_adam {
    double lr, beta1, beta2, eps;
} zsmr_adam;

/* The partition a context describes. */
typedef struct zsmr_layout_info {
    int64_t numel;         /* Psi                                               */
    int64_t padded_numel;  /* flat length including the zero pad (DP: Psi)      */
    int64_t shard_numel;   /* elements of optimizer state one rank keeps (stage 4: the most any rank keeps) */
    int64_t max_unit_numel;/* largest padded unit N*S_u (stage 3), largest unit (stage 4), else padded */
    int32_t world, stage, n_units, grad_dtype, param_dtype, pad;
} zsmr_layout_info;

/* Accounting, bytes per rank ("The four schemes": bytes_per_param and
 * peak_bytes_per_param; "ZeRO and FSDP": the three-stage table).  Sharded
 * bands count the padded shard, unsharded bands the true Psi.  Traffic is
 * the elements one rank sends per step: DP one all-reduce of 2(N-1)
 * chunks of ceil(Psi/N); stages 1-2 one reduce-scatter and one all-gather of
 * (N-1)*S each; stage 3 a reduce-scatter plus two all-gathers of
 * (N-1)*sum(S_u) each ("ZeRO, annotated" section 7).  Stage 4, rank r owning
 * own(r) elements: 16*own(r) resident; it receives the Psi - own(r) elements
 * it does not own twice (ag) and sends their gradients once (rs); its peak
 * counts only borrowed units (its own need no buffer).  Bytes = elements x 2. */
typedef struct zsmr_bytes {
    int64_t res_p16, res_grad, res_master, res_m, res_v;
    int64_t resident;      /* sum of the five bands                             */
    int64_t gathered;      /* stage 3: bytes of the gathered unit(s) live at once */
    int64_t peak;          /* resident + gathered                               */
    int64_t unit_grad;     /* stage 3: full 16-bit gradient of the largest unit */
    int64_t rs_elems, ag_elems, ar_elems;
    int64_t traffic_elems, traffic_bytes;
} zsmr_bytes;

/* What the calls made on a context actually did, for one rank: elements that
 * rank received through each simulated all-gather and all-reduce, and sent
 * through each reduce-scatter (at stages 1-3 the same as it received), plus
 * the ZeRO-3 schedule (live and peak bytes are this rank's). */
typedef struct zsmr_counters {
    int64_t rs_elems, ag_elems, ar_elems;
    int64_t traffic_elems, traffic_bytes;
    int64_t stage3_gathers, stage3_releases;   /* summed over units           */
    int64_t live_units, live_bytes, peak_live_bytes;
} zsmr_counters;

/* Name of a status code (static storage).  Library plumbing: the pages
 * define no error codes; the conditions behind ZSMR_ERR_INDIVISIBLE and
 * ZSMR_ERR_STATE are the prototype's divisibility assertion ("The four
 * schemes", Base.__init__) and ZeRO-3's gather-before-use order ("The four
 * schemes", where the third P comes from). */
const char* zsmr_strerror(int32_t status);

/* Text of the last HIP error seen by this thread, or "" (thread-local).
 * Library plumbing, no passage of the pages. */
const char* zsmr_last_hip_error(void);

/* Build the partition of Psi = numel elements over `world` ranks (host only).
 * stage: ZSMR_DP..ZSMR_ZERO3_OWNER.  grad_dtype/param_dtype: ZSMR_FP16 or
 * ZSMR_BF16.
 * units: n_units sizes summing to numel (ZeRO-3 splits each unit N ways with
 * its own pad, "ZeRO and FSDP", "ZeRO-3 and FSDP"); n_units == 0 with
 * unit_numel == NULL means one unit of numel.  Stages 0-2 ignore the unit
 * split.  pad == 0: Psi (stage 3: every unit) must divide by world, else
 * ZSMR_ERR_INDIVISIBLE (the prototype's assertion in "The four schemes");
 * pad == 1: shards are ceil(./N) and the tail is zero (ZeroAdam in "ZeRO and
 * FSDP").  Rank r of stages 1-2 owns [r*S, (r+1)*S); of stage 3 owns
 * [Q_u + r*S_u, Q_u + (r+1)*S_u) of unit u, Q_u its padded start; a data
 * parallel rank "owns" [0, Psi).  Stage 4 keeps units whole and unpadded in
 * their natural order: unit u goes to the rank whose equal share
 * [r*Psi/N, (r+1)*Psi/N) holds the unit's midpoint (with U = k*N equal units
 * the pages' k consecutive units per rank -- for unequal units this default is
 * a reading no passage fixes; zero_set_unit_owners() sets any other map);
 * pad is ignored.  *out receives a context to free with zero_destroy().  ZSMR_ERR_ARG if numel exceeds
 * ZSMR_MAX_NUMEL, world ZSMR_MAX_WORLD or n_units ZSMR_MAX_UNITS, or if the
 * host allocation of the context fails; *out is then NULL. */
int32_t zero_init_shards(zsmr_ctx** out, int64_t numel, int32_t world, int32_t stage,
                         int32_t grad_dtype, int32_t param_dtype, int32_t pad,
                         const int64_t* unit_numel, int32_t n_units);

/* Free a context (NULL is ignored).  Library plumbing. */
void zero_destroy(zsmr_ctx* ctx);

/* Copy the partition's sizes into *out (host only): Psi, the padded length
 * N*ceil(Psi/N) and the shard ceil(Psi/N) ("ZeRO and FSDP", ZeroAdam.__init__
 * and _flatten), the largest unit ("ZeRO and FSDP", "ZeRO-3 and FSDP"). */
int32_t zero_layout_info(const zsmr_ctx* ctx, zsmr_layout_info* out);

/* Index map (host only): padded flat offset and length of what `rank` owns
 * in `unit` (stages 0-2: unit must be 0), and the offset of that piece inside
 * the rank's own concatenated shard.  The slice a rank keeps is
 * [rank*S, rank*S + S) of the flat vector ("The four schemes", Base.__init__;
 * "ZeRO and FSDP", ZeroAdam.__init__, lo = rank * shard); at stage 3 the same
 * split is made within each unit ("ZeRO and FSDP", "ZeRO-3 and FSDP").  Stage 4: the unit's start and length
 * for its owner, length 0 for every other rank; the local offset is within
 * the owner's units.  Any output pointer may be NULL. */
int32_t zero_layout(const zsmr_ctx* ctx, int32_t rank, int32_t unit,
                    int64_t* offset, int64_t* len, int64_t* local_offset);

/* Stage 4: the rank owning `unit` (host only).  ZSMR_ERR_ARG at other stages.
 * ("One Poem Suffices: ZeRO" section 4.1.4; "ZeRO, annotated" section 7.) */
int32_t zero_unit_owner(const zsmr_ctx* ctx, int32_t unit, int32_t* owner);

/* Stage 4: give unit u to rank owners[u], for every unit (host only).  The
 * pages fix owners only for equal partitions ("One Poem Suffices: ZeRO"
 * section 4.1.4: 192 equal blocks, 3 consecutive ones per device of 64;
 * "ZeRO, annotated" section 7: GPU i owns shard i); for any other unit list
 * the caller chooses, here, which rank holds each unit's master, m and v and
 * broadcasts it.  Offsets within each owner's concatenated units follow the
 * natural unit order.  n_units must equal the context's unit count and every
 * owner lie in [0, world), else ZSMR_ERR_ARG (also at stages 0-3).
 * ZSMR_ERR_STATE if any unit is live or any counter or schedule count is
 * non-zero: call it before the first step (or after zero_reset_counters()
 * with no unit live); the context is then unchanged. */
int32_t zero_set_unit_owners(zsmr_ctx* ctx, const int32_t* owners, int32_t n_units);

/* Accounting for one rank (pure, host only).  gather_bytes: bytes per
 * gathered element of the stage-3 peak (0 = the 16-bit working copy's 2; the
 * prototype's fp32 gather is 4).  max_live: units gathered at once (0 = 1;
 * 2 = prefetch of the next unit).  Ranks are alike at stages 0-3; at stage 4
 * this reports the rank with the largest peak (the lowest such rank).
 * ZSMR_ERR_ARG if gather_bytes is negative or above ZSMR_MAX_GATHER_BYTES,
 * or max_live is negative. */
int32_t zero_bytes_per_rank(const zsmr_ctx* ctx, int32_t gather_bytes, int32_t max_live,
                            zsmr_bytes* out);

/* The same accounting for a given rank (stage 4: ranks owning different
 * amounts hold and move different amounts; "One Poem Suffices: ZeRO"
 * section 4.1.4, the owner's shard plus one borrowed block). */
int32_t zero_bytes_of_rank(const zsmr_ctx* ctx, int32_t rank, int32_t gather_bytes,
                           int32_t max_live, zsmr_bytes* out);

/* Counters of `rank` accumulated by the calls below since creation or the
 * last zero_reset_counters() (host only): the elements each simulated
 * collective moved for that rank, in the same units as zero_bytes_per_rank
 * ("The four schemes", bytes_comm_per_rank and the Comm calls of each
 * scheme's step; "ZeRO, annotated" section 7, the all-gathers of the
 * forward and backward passes and the reduce-scatter), and the ZeRO-3
 * schedule's gathers, releases and live bytes ("The four schemes", where the
 * third P comes from). */
int32_t zero_counters(const zsmr_ctx* ctx, int32_t rank, zsmr_counters* out);
/* Zero every counter of zero_counters() (live units stay live). */
int32_t zero_reset_counters(zsmr_ctx* ctx);

/* Device-side init of one (rank, unit) piece of length len = layout len:
 * master = theta0, m = v = 0, p16 = RNE16(theta0).  theta0 points at the
 * piece's initial values (fp32, len), p16 at where its 16-bit copy lives.
 * ("The four schemes", Base.__init__: the fp32 master copied from theta0,
 * zero moments, the 16-bit working copy cast from it; "ZeRO and FSDP",
 * ZeroAdam.__init__: master = the rank's slice, m = v = 0.) */
int32_t zero_init_state(const zsmr_ctx* ctx, int32_t rank, int32_t unit, const float* theta0,
                        float* master, float* m, float* v, void* p16, hipStream_t stream);

/* Gradient layout shared by the reduce entry points: row r (rank r's
 * 16-bit gradient) starts at grads + r*row_stride elements, and the piece
 * owned by (rank, unit) starts at column base_elem of every row; the call
 * reads N rows x len elements.  In a simulated world of full gradient
 * vectors row_stride is the padded length and base_elem the layout offset;
 * for one rank's received contributions base_elem is 0. */

/* Reduce only: g_out[j] = (sum over r in order of fp32(G_r[base+j])) / N, or
 * the raw sum if mean == 0 ("The four schemes", reduce_scatter_mean; "ZeRO
 * and FSDP", ZeroAdam.step).  fp32 output of len elements. */
int32_t zero_reduce_shard(zsmr_ctx* ctx, int32_t rank, int32_t unit, const void* grads,
                          int64_t row_stride, int64_t base_elem, int32_t mean, float* g_out,
                          hipStream_t stream);

/* Adam only, on n elements ("The four schemes", Base._adam):
 *   m = b1*m + (1-b1)*g;  v = b2*v + ((1-b2)*g)*g;
 *   master -= (lr * (m/(1-b1^t))) / (sqrt(v/(1-b2^t)) + eps)
 * every operation rounded to fp32, no fused multiply-add.  t >= 1. */
int32_t zero_adam_step(float* master, float* m, float* v, const float* g, int64_t n, int32_t t,
                       const zsmr_adam* hp, hipStream_t stream);

/* Cast only: p16_dst[j] = RNE16(master[j]) for the (rank, unit) piece -- the
 * all-gather side of stages 1-2 (into slot r of the working copy) and the
 * rank's own 16-bit shard at stage 3.  ("The four schemes", ZeRO1.step: the
 * gathered masters cast to the 16-bit copy; "ZeRO and FSDP", ZeroAdam.step:
 * all_gather_into_tensor of the updated slice into the full parameters;
 * "Sharding the States.": the all-gather moves the 16-bit weights.)  At
 * stages 1-2 it counts the all-gather that delivers this slot to the other
 * ranks. */
int32_t zero_gather_cast(zsmr_ctx* ctx, int32_t rank, int32_t unit, const float* master,
                         void* p16_dst, hipStream_t stream);

/* The hot path: reduce + Adam + cast in one pass over the (rank, unit)
 * piece, reading each gradient row, master, m and v once and writing master,
 * m, v and the 16-bit copy once.  Bit-identical to zero_reduce_shard(mean=1)
 * + zero_adam_step + zero_gather_cast.  It is the middle of a sharded step as
 * the pages give it: reduce-scatter the gradients, update the rank's own
 * slice, all-gather it ("ZeRO and FSDP", ZeroAdam.step and the remark after
 * the three-stage table; "The four schemes", ZeRO1.step and ZeRO3.step;
 * "ZeRO, annotated" section 5.2).  t >= 1 is the step number (the same
 * for every rank and unit of a step). */
int32_t zero_fused_step(zsmr_ctx* ctx, int32_t rank, int32_t unit, const void* grads,
                        int64_t row_stride, int64_t base_elem, float* master, float* m,
                        float* v, void* p16_dst, int32_t t, const zsmr_adam* hp,
                        hipStream_t stream);

/* The fused step on elements [begin, begin + count) of the (rank, unit)
 * piece only, for gradients that arrive in buckets during the backward pass
 * ("ZeRO and FSDP", the remark that real ZeRO-2 reduce-scatters bucket by
 * bucket during backward; "ZeRO, annotated" section 5.2 and 6.2, buckets and
 * constant-size buffers).  Pointers and base_elem refer to the whole piece,
 * exactly as for zero_fused_step; the call touches only the sub-range.
 * Calls over disjoint sub-ranges that cover the piece, with the same t, give
 * the same bits as one zero_fused_step.  ZSMR_ERR_ARG if begin < 0, count < 0
 * or begin + count exceeds the piece, and at stage ZSMR_DP unless the range
 * is the whole vector (a replica's all-reduce covers the whole vector and is
 * counted once per step).  Counts count elements of traffic. */
int32_t zero_fused_step_range(zsmr_ctx* ctx, int32_t rank, int32_t unit, int64_t begin,
                              int64_t count, const void* grads, int64_t row_stride,
                              int64_t base_elem, float* master, float* m, float* v,
                              void* p16_dst, int32_t t, const zsmr_adam* hp, hipStream_t stream);

/* All-gather receive: copy n 16-bit elements src -> dst (peers' slices into
 * the working copy of recv_rank); counted as all-gather traffic received by
 * recv_rank.  Overlapping src and dst is not allowed.  ("ZeRO and FSDP",
 * ZeroAdam.step: all_gather_into_tensor assembles every rank's slice into
 * the complete parameters; "Sharding the States.": the 16-bit all-gather of
 * (N-1)/N of the weights.) */
int32_t zero_gather_copy(zsmr_ctx* ctx, int32_t recv_rank, const void* src, void* dst,
                         int64_t n, hipStream_t stream);

/* All-gather receive of one bucket: copy `count` blocks of n 16-bit elements,
 * block k from src + k*stride to dst + k*stride (elements).  With buckets
 * over the ranks' shards (see zero_fused_step_range), bucket [b0, b1) of
 * every peer q sits at q*S + b0 of the working copy, so the peers' pieces of
 * one bucket are such blocks with n = b1 - b0 and stride = S, and each
 * bucket's receive can follow its update while the backward pass goes on
 * ("ZeRO, annotated" section 5.2, the bucketed all-gather).  Blocks are
 * copied as zero_gather_copy would copy each (results identical).  Counted
 * as count*n elements of all-gather traffic received by recv_rank.
 * ZSMR_ERR_ARG if count > 65535, if blocks overlap (count > 1 and stride <
 * n), or if the spans [src, src + (count-1)*stride + n) and the same of dst
 * overlap; n == 0 or count == 0 does nothing. */
int32_t zero_gather_copy_blocks(zsmr_ctx* ctx, int32_t recv_rank, const void* src, void* dst,
                                int64_t n, int32_t count, int64_t stride, hipStream_t stream);

/* ZeRO-3 schedule ("The four schemes", where the third P comes from; "ZeRO
 * and FSDP", "ZeRO-3 and FSDP").  Units gathered at once may not exceed
 * max_live (default 1, i.e. no prefetch; 2 allows gathering unit i+1 while
 * unit i is live).  Fails with ZSMR_ERR_STATE if units are live. */
int32_t zero_stage3_set_max_live(zsmr_ctx* ctx, int32_t max_live);

/* Gather unit `unit`: copy the N 16-bit shards shard_ptrs[0..N-1] (a host
 * array of N device pointers, shard r of S_u elements) into unit_buf (N*S_u
 * elements, shard r at r*S_u).  A shard may not overlap unit_buf
 * (ZSMR_ERR_ARG), except one that sits exactly at its own slot r*S_u, which
 * is left as it is.  ZSMR_ERR_STATE if the unit is already live or
 * max_live units are live.  Counts one all-gather of (N-1)*S_u elements
 * received by every rank, and the live/peak gathered bytes.
 * Stage 4 (owner broadcast): shard_ptrs holds one pointer, the owner's 16-bit
 * copy of the whole unit (P_u elements), which is copied to unit_buf (they
 * may not overlap); every rank but the owner receives P_u elements and holds
 * P_u x 2 bytes while the unit is live.  The schedule calls below work the
 * same at stages 3 and 4. */
int32_t zero_stage3_unit_gather(zsmr_ctx* ctx, int32_t unit, const void* const* shard_ptrs,
                                void* unit_buf, hipStream_t stream);

/* Release unit `unit` (host only): the gathered copy is dropped and only
 * the rank's own slice stays ("The four schemes", where the third P comes
 * from: gather, use, release, gather again for backward; "ZeRO and FSDP",
 * "ZeRO-3 and FSDP" steps 1-2).  ZSMR_ERR_STATE if it is not live. */
int32_t zero_stage3_unit_release(zsmr_ctx* ctx, int32_t unit);

/* Schedule state of one unit (host only): live or not, gathers and releases
 * so far ("The four schemes", where the third P comes from).  Any output
 * pointer may be NULL. */
int32_t zero_stage3_unit_state(const zsmr_ctx* ctx, int32_t unit, int32_t* live,
                               int64_t* gathers, int64_t* releases);

/* Diagnostics: the kernel a call of zero_fused_step with these arguments
 * runs, without running it (host only, but the write windows depend on the
 * current device's clock rate).  The arguments are checked exactly as
 * zero_fused_step checks them (the Adam constants aside), with the same
 * errors.  A library query, no passage of the pages: it lets a caller (and
 * the tests) confirm which of the equivalent kernels its buffers select. */
#define ZSMR_KERNEL_SCALAR   0  /* one element per lane: an operand is not vector-aligned  */
#define ZSMR_KERNEL_DIRECT   1  /* 8 elements per lane, results stored at once             */
#define ZSMR_KERNEL_DEFERRED 2  /* 8 elements per lane, results kept in LDS, stored later  */
typedef struct zsmr_plan {
    int32_t kernel;       /* ZSMR_KERNEL_*                                               */
    int32_t ring_tiles;   /* deferred: completed 512-element tiles each wave keeps in LDS */
    int32_t windowed;     /* deferred: stores wait for chip-wide write windows            */
    int32_t store_elems;  /* 16-bit elements per store of the working copy (4, 2, 1)      */
    int32_t launches;     /* launches the piece is cut into (2^30 elements each at most)  */
    int32_t row_batch;    /* direct: gradient rows loaded per batch (8 or 12)              */
    int64_t head;         /* leading elements run one by one to reach a 128-byte line      */
} zsmr_plan;
int32_t zsmr_fused_step_plan(const zsmr_ctx* ctx, int32_t rank, int32_t unit, const void* grads,
                             int64_t row_stride, int64_t base_elem, float* master, float* m,
                             float* v, void* p16_dst, zsmr_plan* out);

/* Launch shape of the kernels behind the calls above.  No passage of the
 * pages concerns it (they run NumPy and gloo on CPUs).  step_bpc, 0..64: the grid of the step kernels (reduce,
 * Adam, cast, and the fused step when it writes at once), where 0 (the
 * default) gives one 512-element wave tile per wave and as many workgroups
 * as the launch needs, and k > 0 a grid-stride grid of k workgroups per
 * compute unit.  copy_bpc, 0..64: the same for the copies (receive and
 * ZeRO-3 gather), 0 giving one 32 KB burst per wave (copies between
 * addresses that differ by an odd number of 2-byte elements run 4 per CU
 * whatever it is).  defer_tiles, 0..5 (default 3): how many completed
 * 512-element tiles of fused-step results each wave keeps in LDS before it
 * must write them (0 = write at once; without write windows, that is below
 * 16 rows or with windows off, at most 2; with windows and at most 3, two
 * workgroups run per CU).  defer_min_rows >= 1 (default 24): the fewest
 * gradient rows for which the fused step defers its writes.
 * Process-wide; safe to call while other threads launch (each value is read
 * atomically, and a launch that overlaps the call may take some values old
 * and some new).  Affects speed only, never results. */
int32_t zsmr_set_launch_shape(int32_t step_bpc, int32_t copy_bpc, int32_t defer_tiles,
                              int32_t defer_min_rows);

/* Write windows of the fused step's deferred writes.  A speed knob of
 * zero_fused_step; no passage of the pages concerns it.  Every cycle_ns, the
 * last write_ns form a window that all waves on the GPU take at the same
 * time, read from the chip's constant-rate clock: deferred results are
 * stored only inside windows, and no gradient loads are issued from
 * margin_ns before a window until lead_ns before its end, so HBM sees long
 * read-only stretches and short write-only bursts.  Windows apply to steps
 * of 16 or more rows.  cycle_ns is the cycle of a 64-row step; a step of R
 * rows uses cycle_ns * (2R + 26) / 154 (its bytes per element against the
 * 64-row step's: the time the rings take to fill scales with them), and runs
 * without windows where that cannot hold write_ns + margin_ns.  cycle_ns = 0
 * turns them off (a wave then stores its tiles whenever its LDS ring is
 * full).
 * Otherwise 1,000 <= cycle_ns <= 10,000,000, write_ns >= 1, margin_ns >= 0,
 * write_ns + margin_ns < cycle_ns and 0 <= lead_ns < write_ns; ZSMR_ERR_ARG
 * if not.  Defaults: 72,000 / 11,000 / 1,000 / 4,000.  The best cycle follows
 * the device's read rate (it is the time the rings take to fill), so a
 * caller that can time the step may tune it.  Process-wide; safe to call
 * while other threads launch, and a launch sees either all four old values
 * or all four new ones.  Affects speed only, never results. */
int32_t zsmr_set_write_window(int32_t cycle_ns, int32_t write_ns, int32_t margin_ns,
                              int32_t lead_ns);

/* Work split of the copies (zero_gather_copy, zero_gather_copy_blocks,
 * zero_stage3_unit_gather); a speed knob, no passage of the pages concerns
 * it: the regions a copy is cut into go to the eight
 * XCDs in contiguous runs, each even-numbered XCD taking even_permille / 1000
 * times the regions of each odd one.  On MI355X the even XCDs move data
 * faster than the odd ones, so equal shares leave them idle at the end of a
 * copy.  500 <= even_permille <= 2000 (1000: equal shares), else
 * ZSMR_ERR_ARG.  Default 1200, the best measured for the 14.77 GB receive of
 * one rank's share of a 64-rank world.  Process-wide; safe to call while
 * other threads launch.  Affects speed only, never results. */
int32_t zsmr_set_xcd_balance(int32_t even_permille);

#ifdef __cplusplus
}
#endif
#endif /* ZSMR_H */
