// moge_combine: the gate-weighted sum of each token's expert outputs (gates are
// the global softmax probabilities of the chosen experts; Pangu Pro MoE,
// lsdiaocha.cn summary, section 1), plus the always-on shared expert's output
// (Pangu Ultra MoE digests on reportify.cn: one shared expert).
//
// HBM-bound gather: one wave per token; each lane owns 8 consecutive hidden
// elements per pass, loads the K rows' 16- or 32-byte pieces together and
// accumulates in float32 in slot order (deterministic), then writes 32 bytes of y.
#include "moge_internal.hpp"

namespace moge {

template <typename OT>
__device__ __forceinline__ void load8(const OT* p, float* v);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* v) {
  const u32x4_t u = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(u[i] << 16);
    v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
  const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

template <typename OT>
__global__ __launch_bounds__(256) void combine_kernel(int64_t T, int K, int d, const OT* __restrict__ o,
                                                      const int32_t* __restrict__ inv, const float* __restrict__ gate,
                                                      int64_t rows_cap, const OT* __restrict__ shared_out,
                                                      float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  const int chunks = d >> 3;
  for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += nw) {
    for (int c = lane; c < chunks; c += 64) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < K; ++s) {
        const int r = inv[t * K + s];
        if (r < 0 || (int64_t)r >= rows_cap) continue;
        const float g = gate[t * K + s];
        float v[8];
        load8<OT>(o + (int64_t)r * d + c * 8, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, v[i], acc[i]);
      }
      if (shared_out) {
        float v[8];
        load8<OT>(shared_out + t * d + c * 8, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[i];
      }
      f32x4_t a = {acc[0], acc[1], acc[2], acc[3]}, b = {acc[4], acc[5], acc[6], acc[7]};
      *reinterpret_cast<f32x4_t*>(y + t * d + c * 8) = a;
      *reinterpret_cast<f32x4_t*>(y + t * d + c * 8 + 4) = b;
    }
  }
}

}  // namespace moge

using namespace moge;

extern "C" moge_status_t moge_combine(const moge_shape_t* shape, const void* o, const int32_t* inv, const float* gate,
                                      int64_t rows_cap, const void* shared_out, float* y, hipStream_t stream) {
  moge_status_t st = validate_shape(shape);
  if (st != MOGE_OK) return st;
  const moge_shape_t& s = *shape;
  if (!o || !inv || !gate || !y) return fail(MOGE_ERR_NULL, "o, inv, gate and y are required");
  if (rows_cap < 1) return fail(MOGE_ERR_CAPACITY, "rows_cap must be >= 1");
  const int K = s.M * s.k_per_group;
  int64_t grid = ((int64_t)s.T + 3) / 4;
  if (grid > 8192) grid = 8192;
  if (s.dtype == MOGE_BF16)
    hipLaunchKernelGGL(combine_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, stream, (int64_t)s.T, K, s.d,
                       static_cast<const uint16_t*>(o), inv, gate, rows_cap,
                       static_cast<const uint16_t*>(shared_out), y);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3((unsigned)grid), dim3(256), 0, stream, (int64_t)s.T, K, s.d,
                       static_cast<const float*>(o), inv, gate, rows_cap, static_cast<const float*>(shared_out), y);
  st = check_launch("combine_kernel");
  return st == MOGE_OK ? ok() : st;
}
