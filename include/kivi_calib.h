/*
 * kivi_calib.h -- measurement aids exported by libkivi next to the hot path.
 *
 * The VeloxQuant-MLX "Benchmarks" page ("KV-Cache Kernel Roofline: What
 * Actually Limits Decode") reports its kernels against a bandwidth ceiling
 * calibrated on the hardware itself rather than the spec sheet.  These
 * streaming kernels are those ceilings on an MI355X, one per traffic shape:
 * a copy (read n, write n), a pure read (the decode attend's shape), a pure
 * write, and a flush-shaped mix (read n, write 3n/8: 2 B in per 0.75 B out,
 * the 4-bit flush's ratio, in the flush's own pattern: per 8 KiB tile read,
 * 2 KiB written to one region and 512 B to each of two others).  Each moves
 * every byte once, with 16-byte accesses, and with the cache hints and the
 * number of workgroups resident per CU that measured fastest for its shape
 * (the nontemporal hint, except plain stores for the pure write; 3 or 4
 * workgroups of 4 waves per CU, held there by LDS each launch reserves and
 * never touches); the bytes/s they reach bound what a kernel with the same
 * read/write mix can reach.
 *
 * Every pointer is device memory, 16-byte aligned; sizes are multiples of
 * 16.  The calls enqueue on `stream` and return KIVI_OK (0) or a negative
 * KIVI_ERR_* code from kivi.h (nothing is launched on error).
 */
#ifndef KIVI_CALIB_H
#define KIVI_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

/* Copy n_bytes (a multiple of 16) of device memory from src to dst on
 * `stream`.  Both pointers 16-byte aligned and non-overlapping.  Returns
 * KIVI_OK (0) or a negative KIVI_ERR_* code from kivi.h. */
int kivi_calib_copy(const void* src, void* dst, size_t n_bytes, hipStream_t stream);

/* Read n_bytes of src.  The loads are folded into one word, stored to sink
 * (at least 4 bytes) only in the unlikely case that it equals a fixed
 * value, so the reads cannot be optimized away. */
int kivi_calib_read(const void* src, size_t n_bytes, void* sink, hipStream_t stream);

/* Write n_bytes of a fixed pattern to dst. */
int kivi_calib_write(void* dst, size_t n_bytes, hipStream_t stream);

/* Read n_bytes of src and write floor(3 n / 8) 16-byte vectors to dst (n =
 * n_bytes / 16; dst must hold that many): vectors [0, floor(n/4)) form the
 * code region, the next floor(n/16) the scale region and the rest the zero
 * region, each written in 8 KiB-source-tile order. */
int kivi_calib_mix(const void* src, size_t n_bytes, void* dst, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KIVI_CALIB_H */
