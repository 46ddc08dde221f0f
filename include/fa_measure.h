/*
 * Measurement utility of libfa.so (not part of the attention method).
 *
 * fa_clock_probe enqueues one wave on `stream` that records n samples into
 * `samples` (device memory, uint64 [n][2], 16-byte aligned): sample i is
 * (shader-clock counter, real-time counter), read back to back, and
 * consecutive samples are about sleep_units x 127 x 64 shader clocks apart.
 * The real-time counter runs at a constant 100 MHz, so for two samples a, b
 *     shader clock = (b.shader - a.shader) / (b.real - a.real) x 100 MHz.
 * Launched on a second stream just before a kernel under test, it gives the
 * shader clock while that kernel runs (the wave occupies one wave slot of
 * one compute unit and sleeps between samples).
 *   n            0 .. 2^20 (0: no-op); sleep_units 0 .. 1024.
 *   Errors       n or sleep_units negative, or a null buffer with n > 0 ->
 *                FA_ERR_INVALID_ARG; a misaligned buffer or a size beyond
 *                the limits -> FA_ERR_UNSUPPORTED; a refused launch ->
 *                FA_ERR_HIP. Asynchronous like every other entry point.
 */
#ifndef FA_MEASURE_H_
#define FA_MEASURE_H_

#include <stdint.h>

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

fa_status_t fa_clock_probe(uint64_t* samples, int n, int sleep_units, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_MEASURE_H_ */
