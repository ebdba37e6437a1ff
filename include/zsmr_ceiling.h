/*
 * zsmr_ceiling.h -- C ABI of ceiling/libzsmr_ceiling.so: pure-read and
 * pure-write reference streams over HBM (measurement only, not part of the
 * method; nothing in libzsmr.so calls them).
 *
 * What they are for: a kernel that reads R bytes and writes W bytes can at
 * best take R / (read rate) + W / (write rate), the two pure rates of the
 * same device, if it lost no time turning HBM between reads and writes.
 * Timing these streams beside the shard step's kernels, on buffers of the
 * same size in the same process, gives that bound for the device at hand,
 * so that a kernel's time can be compared with it as well as with the
 * published 8 TB/s peak.
 *
 * Shapes (the best read and write shapes measured on MI355X; a caller takes
 * the faster of the two for each direction):
 *   ZSMR_CEILING_BURSTS   one 32 KB burst per wave (64 lanes x 32 16-byte
 *                         vectors), one wave per burst in launch order,
 *                         non-temporal loads or stores;
 *   ZSMR_CEILING_REGIONS  reads only: each wave of one workgroup per CU
 *                         streams one contiguous region in 8 KB bursts;
 *   ZSMR_CEILING_PLAIN    writes only: as BURSTS with ordinary stores;
 *   ZSMR_CEILING_BURSTS_BALANCED   as BURSTS (reads or non-temporal writes),
 *                         the chunks split between the eight XCDs in
 *                         contiguous runs, each even-numbered XCD taking
 *                         zsmr_ceiling_set_balance()'s thousandths of an odd
 *                         one's (on MI355X the even XCDs stream faster);
 *   ZSMR_CEILING_PLAIN_BALANCED    writes only: as PLAIN, split the same way.
 *
 * Arguments: `bytes` >= 0 and a multiple of 16; `src` / `dst` 16-byte
 * aligned device pointers covering `bytes`; `sink` a 16-byte aligned device
 * buffer of at least 16 bytes that the read stream may overwrite (it stores
 * there only if the XOR of everything it read equals one fixed 128-bit
 * value, which keeps the compiler from dropping the loads).  The write
 * stream stores `value` into every 32-bit word of [dst, dst + bytes).
 * Returns 0, 1 for a bad argument (negative or non-multiple of 16 size,
 * unknown shape, null pointer), 5 for a misaligned pointer, 6 for a HIP
 * error.  A call with bytes == 0 touches nothing and returns 0 (after the
 * size and shape checks) whatever the pointers.  Asynchronous on `stream`;
 * the caller owns every buffer.
 */
#ifndef ZSMR_CEILING_H
#define ZSMR_CEILING_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZSMR_CEILING_BURSTS 0
#define ZSMR_CEILING_REGIONS 1
#define ZSMR_CEILING_PLAIN 1
#define ZSMR_CEILING_BURSTS_BALANCED 2
#define ZSMR_CEILING_PLAIN_BALANCED 3

/* Read [src, src + bytes) once. */
int32_t zsmr_ceiling_read(const void* src, int64_t bytes, int32_t shape, void* sink,
                          hipStream_t stream);

/* Write `value` to every 32-bit word of [dst, dst + bytes). */
int32_t zsmr_ceiling_write(void* dst, int64_t bytes, int32_t shape, uint32_t value,
                           hipStream_t stream);

/* Weight of each even-numbered XCD against each odd one in the balanced
 * shapes, in thousandths: 500..2000 (default 1200), else 1.  Process-wide. */
int32_t zsmr_ceiling_set_balance(int32_t even_permille);

#ifdef __cplusplus
}
#endif
#endif /* ZSMR_CEILING_H */
