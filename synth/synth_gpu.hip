// GPU filler for the seeded synthetic inputs defined in synth_def.h: the same
// bytes as synth_cpu.c for the same (seed, tensor_id, element index).
// Benchmark and test infrastructure; it computes none of the MoGE layer.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "synth_def.h"

__device__ static inline uint64_t synth_mix_d(uint64_t z) {
  SYNTH_MIX_BODY(z);
  return z;
}

__global__ void synth_fill_kernel(uint64_t key, int64_t start, int64_t n, float c, void* out, int as_bf16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += stride) {
    const uint64_t i = (uint64_t)(start + k);
    int32_t s = 0;
#pragma unroll
    for (uint64_t j = 0; j < 3; ++j) {
      uint64_t w = synth_mix_d(key + (3ULL * i + j + 1ULL) * SYNTH_GAMMA);
      s += SYNTH_SUM16(w);
    }
    s -= 393210;
    const float v = __fmul_rn((float)s, c);
    if (as_bf16) {
      const uint32_t u = __float_as_uint(v);
      ((uint16_t*)out)[k] = SYNTH_BF16_RNE(u);
    } else {
      ((float*)out)[k] = v;
    }
  }
}

static uint64_t synth_key_h(uint64_t seed, uint64_t tensor_id) {
  uint64_t z = seed ^ SYNTH_SEED_SALT;
  SYNTH_MIX_BODY(z);
  z = z + (tensor_id + 1ULL) * SYNTH_GAMMA;
  SYNTH_MIX_BODY(z);
  return z;
}

// Fills out[k] (k in [0,n)) with element start+k of stream (seed, tensor_id).
// as_bf16: 1 -> uint16 bf16 bits, 0 -> float.  Returns a hipError_t value.
extern "C" int synth_fill_device(uint64_t seed, uint64_t tensor_id, int64_t start, int64_t n, float stdv,
                                 void* out, int as_bf16, hipStream_t stream) {
  if (n <= 0) return 0;
  const float c = stdv * (1.0f / 65536.0f);
  const int64_t blocks64 = (n + 255) / 256;
  const unsigned blocks = (unsigned)(blocks64 < 65536 ? blocks64 : 65536);
  hipLaunchKernelGGL(synth_fill_kernel, dim3(blocks), dim3(256), 0, stream, synth_key_h(seed, tensor_id), start, n, c,
                     out, as_bf16);
  return (int)hipGetLastError();
}
