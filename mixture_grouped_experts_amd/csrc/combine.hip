// moge_combine: the gate-weighted sum of each token's expert outputs (gates are
// the global softmax probabilities of the chosen experts; Pangu Pro MoE,
// lsdiaocha.cn summary, section 1), plus the always-on shared expert's output
// (Pangu Ultra MoE digests on reportify.cn: one shared expert).
//
// HBM-bound gather.  A wave takes one (token, 512-column block) item, so even a
// few tokens spread over the whole chip; each lane owns 8 consecutive hidden
// elements.  The token's slots are read in batches of 8 whose row loads are all
// in flight together (lane j reads slot j's row index and gate; the contributing
// slots are compacted with a ballot and handed to the whole wave with readlane),
// then accumulated in float32 in slot order (deterministic).  The expert
// rows are read once and y is written once, so both go with the non-temporal hint
// (kept out of the caches' working sets: 287 -> 239 us on 8192 tokens x 8 slots x
// 7680 columns).
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

// 8 elements as loaded (kept raw until every load of a batch is in flight).
template <typename OT>
struct Raw8;
template <>
struct Raw8<uint16_t> {
  u32x4_t u;
  __device__ __forceinline__ void load(const uint16_t* p) {
    u = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  }
  __device__ __forceinline__ void fma_into(float g, float* acc) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(g, __uint_as_float(u[i] << 16), acc[2 * i]);
      acc[2 * i + 1] = fmaf(g, __uint_as_float(u[i] & 0xFFFF0000u), acc[2 * i + 1]);
    }
  }
};
template <>
struct Raw8<float> {
  f32x4_t a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4_t*>(p);
    b = *reinterpret_cast<const f32x4_t*>(p + 4);
  }
  __device__ __forceinline__ void fma_into(float g, float* acc) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] = fmaf(g, a[i], acc[i]);
      acc[4 + i] = fmaf(g, b[i], acc[4 + i]);
    }
  }
};

constexpr int kCombineCols = 512;  // columns per wave item: 64 lanes x 8
constexpr int kCombineBatch = 8;   // slots whose rows are loaded together

template <typename OT>
__global__ __launch_bounds__(256) void combine_kernel(int64_t T, int K, int d, const OT* __restrict__ o,
                                                      const int32_t* __restrict__ inv, const float* __restrict__ gate,
                                                      int64_t rows_cap, const OT* __restrict__ shared_out,
                                                      float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nblk = (d + kCombineCols - 1) / kCombineCols;
  const int64_t items = T * nblk;
  const int64_t nw = (int64_t)gridDim.x * 4;
  for (int64_t it = (int64_t)blockIdx.x * 4 + wave; it < items; it += nw) {
    const int64_t t = it / nblk;
    const int c = (int)(it - t * nblk) * kCombineCols + lane * 8;
    const bool live = c < d;
    const int cl = live ? c : 0;  // lanes past d read (and drop) the row's first columns
    const int32_t* ti = inv + t * K;
    const float* tg = gate + t * K;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < K; s0 += 64) {
      // lane j holds slot s0 + j: its row (-1 when absent or outside the computed experts) and gate
      int rv = -1;
      float gv = 0.f;
      if (s0 + lane < K) {
        rv = ti[s0 + lane];
        gv = tg[s0 + lane];
      }
      if (rv < 0 || (int64_t)rv >= rows_cap) {
        rv = -1;
        gv = 0.f;
      }
      // the slots that contribute, in slot order, 8 at a time: their row loads are all
      // issued before any is used; slots outside the computed experts cost nothing
      uint64_t todo = __builtin_amdgcn_ballot_w64(rv >= 0);
      while (todo) {
        int r[kCombineBatch];
        float g[kCombineBatch];
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j) {
          r[j] = -1;
          g[j] = 0.f;
          if (todo) {
            const int sl = __builtin_ctzll(todo);
            todo &= todo - 1;
            r[j] = __builtin_amdgcn_readlane(rv, sl);
            g[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), sl));
          }
        }
        Raw8<OT> v[kCombineBatch];
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j)
          if (r[j] >= 0) v[j].load(o + (int64_t)r[j] * d + cl);
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j)
          if (r[j] >= 0) v[j].fma_into(g[j], acc);
      }
    }
    if (!live) continue;
    if (shared_out) {
      float v[8];
      load8<OT>(shared_out + t * d + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    f32x4_t a = {acc[0], acc[1], acc[2], acc[3]}, b = {acc[4], acc[5], acc[6], acc[7]};
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4_t*>(y + t * d + c));
    __builtin_nontemporal_store(b, reinterpret_cast<f32x4_t*>(y + t * d + c + 4));
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
  const int64_t items = (int64_t)s.T * ((s.d + kCombineCols - 1) / kCombineCols);
  int64_t grid = (items + 3) / 4;  // 4 waves per workgroup, one item per wave per pass
  if (grid > 4096) grid = 4096;
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
