/*
 * synth.h -- seeded synthetic inputs for the MoE decode stack.
 *
 * A module of its own: it holds none of the decode step's arithmetic and is
 * shared by the GPU path's tests and benchmark and by the oracle's tests.
 *
 * Generator: Philox4x32-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11),
 * written from its published definition.  Element i of a tensor with
 * (seed, stream) uses counter (i/4 low, i/4 high, stream low, stream high)
 * and key (seed low, seed high); the four 32-bit outputs r0..r3 give four
 * values for elements 4*(i/4) .. 4*(i/4)+3:
 *   normal:  Box-Muller on the pairs (r0, r1) and (r2, r3), in double:
 *            u1 = (r0 + 1) * 2^-32, u2 = r1 * 2^-32,
 *            z0 = sqrt(-2 ln u1) cos(2 pi u2), z1 = sqrt(-2 ln u1) sin(2 pi u2);
 *            value = mean + std * z, rounded to binary32 (nearest even),
 *            then to bf16 (nearest even) for bf16 tensors.
 *   uniform: u = (r + 0.5) * 2^-32, value = lo + (hi - lo) * u, rounded as above.
 * The host and device implementations compute the same double expressions;
 * libm and the device math library may differ in the last bit of a double,
 * which the rounding to binary32 absorbs except in rare boundary cases.
 *
 * Layout: dst is a flat array of n elements of the given dtype.
 * Return: 0 on success, -1 bad argument, -2 HIP error (device variants).
 * Device variants are asynchronous on the given stream; dst is device memory.
 */
#ifndef SYNTH_H
#define SYNTH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { SYNTH_F32 = 0, SYNTH_BF16 = 1 };

void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

int synth_fill_normal_host(void* dst, int dtype, uint64_t n, uint64_t seed, uint64_t stream, double mean,
                           double std);
int synth_fill_uniform_host(void* dst, int dtype, uint64_t n, uint64_t seed, uint64_t stream, double lo,
                            double hi);

/* stream: a hipStream_t passed as void* (NULL = the default stream) */
int synth_fill_normal_device(void* dst, int dtype, uint64_t n, uint64_t seed, uint64_t stream, double mean,
                             double std, void* hip_stream);
int synth_fill_uniform_device(void* dst, int dtype, uint64_t n, uint64_t seed, uint64_t stream, double lo,
                              double hi, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif
