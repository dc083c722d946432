/*
 * forge_measure.h -- measurement helpers of the library (not part of the method).
 *
 * The fused step is bound by the matrix cores, whose rate scales with the shader clock, and
 * the MI355X lowers that clock under sustained load.  A throughput figure is therefore only
 * comparable together with the clock it ran at; this entry point measures it.
 */
#ifndef FORGE_MEASURE_H
#define FORGE_MEASURE_H

#include <stdint.h>

#include "forge.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * forge_clock_sample -- enqueue, on `stream`, one wave that spins (sleeping between reads)
 * for `seconds` of real time and then writes two counts to the device buffer `out` (2 x
 * uint64, caller-owned): out[0] = shader-clock cycles elapsed (s_memtime), out[1] = real-time
 * counter ticks elapsed (s_memrealtime).  The average shader clock over the interval is
 * out[0] / out[1] * forge_realtime_hz().  Run it on a second stream beside the kernels to be
 * characterised; the wave occupies one SIMD slot of one CU and no LDS.  Errors: FORGE_ERR_ARG
 * if `out` is NULL or `seconds` is not in (0, 10]; FORGE_ERR_LAUNCH from the runtime.
 */
forge_status forge_clock_sample(double seconds, uint64_t* out, void* stream);

/* Frequency of the real-time counter read by forge_clock_sample on the current device (Hz),
 * or 0 if the runtime cannot tell. */
double forge_realtime_hz(void);

#ifdef __cplusplus
}
#endif
#endif /* FORGE_MEASURE_H */
