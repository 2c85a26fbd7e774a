/*
 * sv_probe.h -- streaming-read probe for MI355X (gfx950), measurement only.
 *
 * Not part of the verification method: the benchmark reads the same bytes
 * the verification pass reads with no arithmetic but a keep-alive sum, and
 * reports that rate beside the pass's roofline as the machine's empirical
 * ceiling for one read pass (context; the roofline's peak stays the
 * published 8 TB/s).
 */
#ifndef SV_PROBE_H
#define SV_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_PROBE_ONESHOT 0     /* one 256-thread block per 32 KB chunk */
#define SV_PROBE_PERSISTENT 1  /* blocks_per_cu blocks per CU, each striding over the chunks */

/* Blocks of a probe launch over bytes0 + bytes1 bytes (one float of `out`
 * per block), or -1 for an unknown mode or blocks_per_cu outside [1, 8]
 * (persistent mode only; it queries the current device's CU count). */
int64_t sv_probe_blocks(size_t bytes0, size_t bytes1, int32_t mode, int32_t blocks_per_cu);

/* Read buf0[0, bytes0) and buf1[0, bytes1) (device memory, 16-byte aligned,
 * sizes multiples of 16; buf1 may be NULL when bytes1 == 0) once, on
 * `stream` (a hipStream_t), writing one float per block to `out` (device
 * memory of sv_probe_blocks floats).  Returns 0, -1 for invalid arguments,
 * -3 when the launch fails.  Asynchronous like any launch. */
int32_t sv_probe_read(const void* buf0, size_t bytes0, const void* buf1, size_t bytes1, int32_t mode,
                      int32_t blocks_per_cu, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SV_PROBE_H */
