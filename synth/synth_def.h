/*
 * Seeded, counter-based synthetic inputs (test and benchmark infrastructure).
 *
 * This header holds only the input generator.  It contains none of the MoGE
 * layer's arithmetic; it is included by the CPU filler (synth_cpu.c, built
 * with gcc) and by the GPU filler (synth_gpu.hip, built with hipcc), so both
 * produce the same bytes for the same (seed, tensor_id, element index).
 *
 * Definition (every step is integer arithmetic or one IEEE-754 binary32
 * multiply, so the result does not depend on the machine that computes it):
 *
 *   mix(z)  : the SplitMix64 output finaliser of Steele, Lea and Flood,
 *             "Fast splittable pseudorandom number generators" (OOPSLA 2014):
 *               z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9
 *               z = (z ^ (z >> 27)) * 0x94D049BB133111EB
 *               z =  z ^ (z >> 31)                        (all mod 2^64)
 *   key     = mix(mix(seed ^ 0x5851F42D4C957F2D) + (tensor_id + 1) * GAMMA)
 *             with GAMMA = 0x9E3779B97F4A7C15 (the SplitMix64 increment)
 *   word_n  = mix(key + (n + 1) * GAMMA)  -- the n-th SplitMix64 output
 *   element i draws the three words n = 3i, 3i+1, 3i+2, splits each into
 *   four 16-bit unsigned integers u_0..u_11 and forms
 *     S = sum(u_j) - 393210         (393210 = 12 * 32767.5; exact int)
 *   an approximately N(0,1) variate with variance (65536^2-1)/65536^2 by the
 *   classic twelve-uniform (Irwin-Hall n=12) construction, scaled:
 *     value = fl32( (float)S * c ),  c = fl32(std) * 2^-16   (c exact)
 *   bf16 outputs round that binary32 value to nearest-even.
 */
#ifndef MOGE_SYNTH_DEF_H
#define MOGE_SYNTH_DEF_H

#include <stdint.h>

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL
#define SYNTH_SEED_SALT 0x5851F42D4C957F2DULL

#define SYNTH_MIX_BODY(z)                         \
  do {                                            \
    (z) = ((z) ^ ((z) >> 30)) * 0xBF58476D1CE4E5B9ULL; \
    (z) = ((z) ^ ((z) >> 27)) * 0x94D049BB133111EBULL; \
    (z) = (z) ^ ((z) >> 31);                      \
  } while (0)

/* sum of the four 16-bit fields of a 64-bit word */
#define SYNTH_SUM16(w) \
  ((int32_t)((w)&0xFFFFu) + (int32_t)(((w) >> 16) & 0xFFFFu) + (int32_t)(((w) >> 32) & 0xFFFFu) + (int32_t)((w) >> 48))

/* binary32 bits -> bf16 bits, round to nearest even (inputs are finite) */
#define SYNTH_BF16_RNE(u) ((uint16_t)(((u) + 0x7FFFu + (((u) >> 16) & 1u)) >> 16))

#endif
