/*
 * CPU filler for the seeded synthetic inputs defined in synth_def.h.
 * Test and benchmark infrastructure: it computes none of the MoGE layer.
 */
#include <stdint.h>
#include "synth_def.h"

static inline uint64_t synth_mix(uint64_t z) {
  SYNTH_MIX_BODY(z);
  return z;
}

uint64_t synth_key(uint64_t seed, uint64_t tensor_id) {
  return synth_mix(synth_mix(seed ^ SYNTH_SEED_SALT) + (tensor_id + 1ULL) * SYNTH_GAMMA);
}

static inline float synth_value(uint64_t key, uint64_t i, float c) {
  int32_t s = 0;
  for (uint64_t j = 0; j < 3; ++j) {
    uint64_t w = synth_mix(key + (3ULL * i + j + 1ULL) * SYNTH_GAMMA);
    s += SYNTH_SUM16(w);
  }
  s -= 393210;
  return (float)s * c;
}

/* out[k] = value of element start+k, k in [0, n) */
void synth_fill_f32(uint64_t seed, uint64_t tensor_id, int64_t start, int64_t n, float stdv, float* out) {
  const uint64_t key = synth_key(seed, tensor_id);
  const float c = stdv * (1.0f / 65536.0f);
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < n; ++k) out[k] = synth_value(key, (uint64_t)(start + k), c);
}

void synth_fill_bf16(uint64_t seed, uint64_t tensor_id, int64_t start, int64_t n, float stdv, uint16_t* out) {
  const uint64_t key = synth_key(seed, tensor_id);
  const float c = stdv * (1.0f / 65536.0f);
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < n; ++k) {
    union { float f; uint32_t u; } v;
    v.f = synth_value(key, (uint64_t)(start + k), c);
    out[k] = SYNTH_BF16_RNE(v.u);
  }
}
