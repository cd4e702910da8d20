/*
 * fp4_phase_clock.h - the phase clock of the one-pass NVFP4 quantize, a
 * profiling aid exported only by libfp4_phase.so (the library built with
 * -DFP4_PHASE_CLOCK by `python -m mxfp4_block_amax_amd.build --phase-clock`),
 * never by libfp4.so.
 *
 * In that build, thread 0 of each workgroup of the one-pass kernel (a bf16
 * tensor that the CUs hold, see fp4_quantize_nvfp4) stamps the device's
 * constant 100 MHz clock (s_memrealtime) into slots 8w + k of a device
 * array: k = 0 at its start, 1 when its loads and partial amax are done, 2
 * after the grid barrier, 3 after the block-scale table is built, 4 after
 * its stores have left.  The stamps are those of the last call.
 */
#ifndef FP4_PHASE_CLOCK_H
#define FP4_PHASE_CLOCK_H
#include <stddef.h>
#include <stdint.h>
#include "fp4.h"
#ifdef __cplusplus
extern "C" {
#endif

/* Copies the first n stamps (at most 8 per workgroup slot of the one-pass
 * grid) into host memory (the caller's, n uint64_t).  Synchronous with the
 * device.  FP4_E_ARG for a NULL pointer, FP4_E_HIP on a runtime error. */
fp4_status fp4_debug_phase_clock(uint64_t *host, size_t n);

#ifdef __cplusplus
}
#endif
#endif
