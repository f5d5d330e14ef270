// moge_imbalance: load per device (= per expert group) and the imbalance score,
// the gap in workload between the busiest and the idlest device in the batch
// (Pangu Pro MoE, lsdiaocha.cn summary, section 1).  Workload counts the
// (token, expert) assignments that land in the group.  One small workgroup.
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

}  // namespace moge

using namespace moge;

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
