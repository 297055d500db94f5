/*
 * kivi_calib.h -- measurement aid exported by libkivi next to the hot path.
 *
 * The VeloxQuant-MLX "Benchmarks" page ("KV-Cache Kernel Roofline: What
 * Actually Limits Decode") reports its kernels against a bandwidth ceiling
 * calibrated on the hardware itself rather than the spec sheet.  This copy
 * kernel is that ceiling on an MI355X: a plain streaming device-to-device
 * copy whose achieved bytes/s (read + write) bound what any of the flush,
 * dequantize or attend kernels can reach.
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

#ifdef __cplusplus
}
#endif

#endif /* KIVI_CALIB_H */
