// moge_imbalance: load per device (= per expert group) and the imbalance score,
// the gap in workload between the busiest and the idlest device in the batch
// (Pangu Pro MoE, lsdiaocha.cn summary, section 1).  Workload counts the
// (token, expert) assignments that land in the group.  One small workgroup.
// moge_imbalance_batches: the same score for each of many batches routed in one
// call (the Monte-Carlo setting in which the pages compare the two routers): one
// workgroup per batch counts its assignments per group in LDS straight from idx.
#include "moge_internal.hpp"

namespace moge {

__global__ __launch_bounds__(256) void imbalance_kernel(int N, int M, int64_t T, const int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ group_load, int32_t* __restrict__ is_raw,
                                                        double* __restrict__ is_norm) {
  __shared__ int load[kMaxExperts];
  const int G = N / M;
  for (int g = threadIdx.x; g < M; g += blockDim.x) {
    int s = 0;
    for (int e = g * G; e < (g + 1) * G; ++e) s += counts[e];
    load[g] = s;
    group_load[g] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int lo = load[0], hi = load[0];
    for (int g = 1; g < M; ++g) {
      lo = load[g] < lo ? load[g] : lo;
      hi = load[g] > hi ? load[g] : hi;
    }
    *is_raw = hi - lo;
    *is_norm = (double)(hi - lo) / (double)T;
  }
}

__global__ __launch_bounds__(256) void imbalance_batches_kernel(int N, int M, int K, int64_t tb,
                                                                const int32_t* __restrict__ idx,
                                                                int32_t* __restrict__ group_load,
                                                                int32_t* __restrict__ is_raw) {
  __shared__ int load[kMaxExperts];
  const int G = N / M;
  const int64_t b = blockIdx.x;
  for (int g = threadIdx.x; g < M; g += blockDim.x) load[g] = 0;
  __syncthreads();
  const int32_t* src = idx + b * tb * K;
  for (int64_t i = threadIdx.x; i < tb * K; i += blockDim.x) {
    const int e = src[i];
    if ((unsigned)e < (unsigned)N) atomicAdd(&load[e / G], 1);
  }
  __syncthreads();
  for (int g = threadIdx.x; g < M; g += blockDim.x) group_load[b * M + g] = load[g];
  if (threadIdx.x == 0) {
    int lo = load[0], hi = load[0];
    for (int g = 1; g < M; ++g) {
      lo = load[g] < lo ? load[g] : lo;
      hi = load[g] > hi ? load[g] : hi;
    }
    is_raw[b] = hi - lo;
  }
}

}  // namespace moge

using namespace moge;

extern "C" moge_status_t moge_imbalance_batches(const moge_shape_t* shape, const int32_t* idx,
                                                int64_t tokens_per_batch, int32_t* group_load, int32_t* is_raw,
                                                hipStream_t stream) {
  moge_status_t st = validate_shape(shape);
  if (st != MOGE_OK) return st;
  if (!idx || !group_load || !is_raw) return fail(MOGE_ERR_NULL, "idx, group_load and is_raw are required");
  if (tokens_per_batch < 1 || shape->T % tokens_per_batch != 0)
    return fail(MOGE_ERR_ARG, "tokens_per_batch must divide T");
  const int64_t B = shape->T / tokens_per_batch;
  if (B > 0x7fffffff) return fail(MOGE_ERR_ARG, "too many batches");
  hipLaunchKernelGGL(imbalance_batches_kernel, dim3((unsigned)B), dim3(256), 0, stream, shape->N, shape->M,
                     shape->M * shape->k_per_group, tokens_per_batch, idx, group_load, is_raw);
  st = check_launch("imbalance_batches_kernel");
  return st == MOGE_OK ? ok() : st;
}

extern "C" moge_status_t moge_imbalance(const moge_shape_t* shape, const int32_t* counts, int32_t* group_load,
                                        int32_t* is_raw, double* is_norm, hipStream_t stream) {
  moge_status_t st = validate_shape(shape);
  if (st != MOGE_OK) return st;
  if (!counts || !group_load || !is_raw || !is_norm)
    return fail(MOGE_ERR_NULL, "counts, group_load, is_raw and is_norm are required");
  hipLaunchKernelGGL(imbalance_kernel, dim3(1), dim3(256), 0, stream, shape->N, shape->M, (int64_t)shape->T, counts,
                     group_load, is_raw, is_norm);
  st = check_launch("imbalance_kernel");
  return st == MOGE_OK ? ok() : st;
}
