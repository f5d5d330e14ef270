// moge_check_finite: counts the NaNs and infinities of an array and reports the
// first one, synchronously.  The pages (Pangu Pro MoE, lsdiaocha.cn summary,
// section 1) define the choice on the softmax of finite router scores and say
// nothing of non-finite ones, so the layer's own calls do not spend a pass on
// them; this call is for callers that want the scores (or an input) checked.
//
// Two launches, no atomics: each workgroup of the first writes its count and its
// first non-finite index to the workspace, one workgroup of the second folds
// those partials in a fixed order; the host then reads the 16-byte result.
#include <limits.h>

#include "moge_internal.hpp"

namespace moge {

constexpr int kCheckThreads = 256;

// count and first index of the block, reduced in LDS (all threads call it)
__device__ __forceinline__ void block_fold(int64_t cnt, int64_t first, int64_t* s_cnt, int64_t* s_first) {
  const int tid = threadIdx.x;
  s_cnt[tid] = cnt;
  s_first[tid] = first;
  __syncthreads();
  for (int w = kCheckThreads / 2; w > 0; w >>= 1) {
    if (tid < w) {
      s_cnt[tid] += s_cnt[tid + w];
      s_first[tid] = s_first[tid] < s_first[tid + w] ? s_first[tid] : s_first[tid + w];
    }
    __syncthreads();
  }
}

template <typename T>
__global__ __launch_bounds__(kCheckThreads) void check_partial_kernel(const T* __restrict__ a, int64_t n,
                                                                      int64_t* __restrict__ part) {
  __shared__ int64_t s_cnt[kCheckThreads], s_first[kCheckThreads];
  int64_t cnt = 0, first = LLONG_MAX;
  const int64_t stride = (int64_t)gridDim.x * kCheckThreads;
  for (int64_t i = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x; i < n; i += stride) {
    bool bad;
    if constexpr (sizeof(T) == 4) bad = (a[i] & 0x7F800000u) == 0x7F800000u;  // exponent all ones
    else bad = (a[i] & 0x7F80u) == 0x7F80u;
    if (bad) {
      ++cnt;
      if (i < first) first = i;
    }
  }
  block_fold(cnt, first, s_cnt, s_first);
  if (threadIdx.x == 0) {
    part[2 * blockIdx.x] = s_cnt[0];
    part[2 * blockIdx.x + 1] = s_first[0];
  }
}

__global__ __launch_bounds__(kCheckThreads) void check_fold_kernel(int nparts, const int64_t* __restrict__ part,
                                                                   int64_t* __restrict__ out) {
  __shared__ int64_t s_cnt[kCheckThreads], s_first[kCheckThreads];
  int64_t cnt = 0, first = LLONG_MAX;
  for (int b = threadIdx.x; b < nparts; b += kCheckThreads) {
    cnt += part[2 * b];
    first = part[2 * b + 1] < first ? part[2 * b + 1] : first;
  }
  block_fold(cnt, first, s_cnt, s_first);
  if (threadIdx.x == 0) {
    out[0] = s_cnt[0];
    out[1] = s_first[0];
  }
}

}  // namespace moge

using namespace moge;

extern "C" moge_status_t moge_check_finite(int32_t dtype, const void* a, int64_t n, void* ws, size_t ws_bytes,
                                           hipStream_t stream) {
  if (dtype != MOGE_BF16 && dtype != MOGE_F32) return fail(MOGE_ERR_DTYPE, "dtype must be MOGE_BF16 or MOGE_F32");
  if (n < 0) return fail(MOGE_ERR_SHAPE, "n must be >= 0");
  if (n == 0) return ok();
  if (!a) return fail(MOGE_ERR_NULL, "a is required");
  if (!ws || ws_bytes < check_workspace_bytes()) return fail(MOGE_ERR_WORKSPACE, "check workspace missing or too small");
  int64_t* part = static_cast<int64_t*>(ws);
  int64_t* res = part + 2 * kCheckBlocks;
  int64_t blocks = (n + kCheckThreads * 8 - 1) / (kCheckThreads * 8);
  if (blocks > kCheckBlocks) blocks = kCheckBlocks;
  if (dtype == MOGE_F32)
    hipLaunchKernelGGL(check_partial_kernel<uint32_t>, dim3((unsigned)blocks), dim3(kCheckThreads), 0, stream,
                       static_cast<const uint32_t*>(a), n, part);
  else
    hipLaunchKernelGGL(check_partial_kernel<uint16_t>, dim3((unsigned)blocks), dim3(kCheckThreads), 0, stream,
                       static_cast<const uint16_t*>(a), n, part);
  moge_status_t st = check_launch("check_partial_kernel");
  if (st != MOGE_OK) return st;
  hipLaunchKernelGGL(check_fold_kernel, dim3(1), dim3(kCheckThreads), 0, stream, (int)blocks, part, res);
  if ((st = check_launch("check_fold_kernel")) != MOGE_OK) return st;
  int64_t host[2] = {0, 0};
  hipError_t e = hipMemcpyAsync(host, res, sizeof(host), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(MOGE_ERR_HIP, std::string("moge_check_finite: ") + hipGetErrorString(e));
  if (host[0] > 0)
    return fail(MOGE_ERR_NONFINITE, std::to_string(host[0]) + " of " + std::to_string(n) +
                                        " values are NaN or infinite; the first at index " + std::to_string(host[1]));
  return ok();
}
