/*
 * ep_probe.h -- a check hook into libep_mi355x.so's FP8 conversion.
 *
 * ep_dispatch's FP8 path (DeepEP V1 Legacy guide §5.2(6): E4M3FN tokens with
 * one fp32 scale per 128 channels) ends every channel with the same step:
 * clamp to [-448, 448], then round to the nearest E4M3FN code with ties to
 * even.  This entry point applies exactly that step to an array of floats so
 * a test can compare it, value by value, against an independent encoder over
 * every binary32 input the pack can produce.  It is not part of the
 * dispatch/combine path.
 *
 * ep_probe_log2_bf16 applies the LogFMT encoder's logarithm (log2 rounded to
 * the nearest binary32, of a bf16 magnitude) to an array, so a test can check
 * it against the correctly rounded value for every bf16 input.
 */
#ifndef EP_MI355X_PROBE_H
#define EP_MI355X_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* in [n] float (device), out_hw [n] and out_sw [n] uint8 (device, either may
 * be NULL).  out_hw: the gfx950 packed conversion instruction the pack uses;
 * out_sw: the bitwise formulation kept as its cross-check.  n >= 0 and
 * n % 4 == 0, pointers 16-byte aligned.  Enqueued on `stream`; returns
 * EP_OK, EP_ERR_NULL, EP_ERR_SHAPE, EP_ERR_ALIGN or EP_ERR_HIP (ep.h). */
int ep_probe_e4m3fn(const float *in, uint8_t *out_hw, uint8_t *out_sw, int64_t n, void *stream);

/* bits [n] bf16 patterns (device, 2-byte aligned), out [n] float (device,
 * 4-byte aligned): out[i] = log2(|x_i|) rounded to the nearest binary32 as
 * the LogFMT encoder computes it, -inf for a zero.  Inputs must be finite.
 * Returns EP_OK, EP_ERR_NULL, EP_ERR_SHAPE (n < 0), EP_ERR_ALIGN or
 * EP_ERR_HIP. */
int ep_probe_log2_bf16(const uint16_t *bits, float *out, int64_t n, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* EP_MI355X_PROBE_H */
