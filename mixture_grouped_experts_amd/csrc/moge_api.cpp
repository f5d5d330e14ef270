// Host-side part of the libmoge C ABI: shape validation, row bounds,
// workspace sizes, version and per-thread error messages (all usable without
// a GPU), plus the one-time dynamic-LDS attribute setup of large kernels.
#include <stdio.h>

#include <map>
#include <utility>
#include <mutex>
#include <string>

#include "moge_internal.hpp"

namespace moge {

static thread_local std::string g_last_error;

moge_status_t fail(moge_status_t st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

moge_status_t ok() {
  g_last_error.clear();
  return MOGE_OK;
}

moge_status_t check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MOGE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return MOGE_OK;
}

moge_status_t validate_shape(const moge_shape_t* s) {
  if (!s) return fail(MOGE_ERR_NULL, "shape is NULL");
  if (s->dtype != MOGE_BF16 && s->dtype != MOGE_F32) return fail(MOGE_ERR_DTYPE, "dtype must be MOGE_BF16 or MOGE_F32");
  if (s->T < 1) return fail(MOGE_ERR_SHAPE, "T must be >= 1");
  if (s->d < 8 || s->d % 8 != 0) return fail(MOGE_ERR_SHAPE, "d must be a positive multiple of 8");
  if (s->N < 1 || s->M < 1 || s->M > s->N) return fail(MOGE_ERR_SHAPE, "need 1 <= M <= N");
  if (s->N > kMaxExperts) return fail(MOGE_ERR_SHAPE, "N must be <= 256");
  if (s->N % s->M != 0) return fail(MOGE_ERR_SHAPE, "N must be a multiple of M (groups of equal size)");
  if (s->k_per_group < 1 || s->k_per_group > s->N / s->M)
    return fail(MOGE_ERR_SHAPE, "need 1 <= k_per_group <= N/M");
  if (s->F < 0 || (s->F > 0 && (s->F < 8 || s->F % 8 != 0)))
    return fail(MOGE_ERR_SHAPE, "F must be 0 (routing only) or a positive multiple of 8");
  const int64_t K = (int64_t)s->M * s->k_per_group;
  if ((int64_t)s->T * K >= (int64_t(1) << 31)) return fail(MOGE_ERR_SHAPE, "T*K must be < 2^31");
  if (s->tiles != MOGE_TILES_AUTO && s->tiles != MOGE_TILES_TALL && s->tiles != MOGE_TILES_WIDE &&
      s->tiles != MOGE_TILES_BALANCED)
    return fail(MOGE_ERR_ARG, "tiles must be MOGE_TILES_AUTO, _TALL, _WIDE or _BALANCED");
  return MOGE_OK;
}

moge_status_t raise_dynamic_lds(const void* kernel, size_t bytes, const char* what) {
  // the attribute is set once per (device, kernel): a process may drive several GPUs
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, size_t> done;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MOGE_ERR_HIP, std::string(what) + ": no current device");
  std::lock_guard<std::mutex> lock(mu);
  size_t& have = done[{dev, kernel}];
  if (bytes <= have) return MOGE_OK;
  const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess)
    return fail(MOGE_ERR_HIP, std::string(what) + ": cannot raise dynamic LDS: " + hipGetErrorString(e));
  have = bytes;
  return MOGE_OK;
}

int64_t rows_bound(const moge_shape_t& s, int32_t mode, int32_t e_lo, int32_t e_hi) {
  const int64_t G = s.N / s.M;
  const int64_t K = (int64_t)s.M * s.k_per_group;
  const int64_t pad = (int64_t)(kSegAlign - 1) * (e_hi - e_lo);  // each segment starts on a 16-row boundary
  if (mode == MOGE_ROUTE_GLOBAL) {
    const int64_t span = e_hi - e_lo;
    return (int64_t)s.T * (span < K ? span : K) + pad;
  }
  int64_t per_token = 0;
  for (int64_t g = 0; g < s.M; ++g) {
    const int64_t lo = e_lo > g * G ? e_lo : g * G;
    const int64_t hi = e_hi < (g + 1) * G ? e_hi : (g + 1) * G;
    if (hi > lo) per_token += (hi - lo) < s.k_per_group ? (hi - lo) : s.k_per_group;
  }
  return (int64_t)s.T * per_token + pad;
}

}  // namespace moge

using namespace moge;

extern "C" moge_status_t moge_validate(const moge_shape_t* shape) {
  const moge_status_t st = validate_shape(shape);
  return st == MOGE_OK ? ok() : st;
}

extern "C" int64_t moge_rows_bound(const moge_shape_t* shape, int32_t mode, int32_t e_lo, int32_t e_hi) {
  if (validate_shape(shape) != MOGE_OK) return -1;
  if (mode != MOGE_ROUTE_GROUPED && mode != MOGE_ROUTE_GLOBAL) return -1;
  if (e_lo < 0 || e_hi > shape->N || e_lo >= e_hi) return -1;
  return rows_bound(*shape, mode, e_lo, e_hi);
}

extern "C" int64_t moge_tiled_elems(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return -1;
  return round_up(rows, kTileRows) * round_up(cols, kTileCols);
}

extern "C" int64_t moge_packed_weight_elems(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return -1;
  return round_up(rows, kWeightRowAlign) * round_up(cols, kTileCols);
}

extern "C" size_t moge_workspace_size(const moge_shape_t* shape, int32_t stage) {
  if (validate_shape(shape) != MOGE_OK) return (size_t)-1;
  if (stage == MOGE_STAGE_DISPATCH) {
    // per (expert, token block) counts, then their exclusive prefix over blocks
    const int64_t nb = dispatch_blocks(shape->T);
    return (size_t)(2 * (int64_t)shape->N * nb) * sizeof(int32_t);
  }
  if (stage == MOGE_STAGE_CHECK) return check_workspace_bytes();
  if (stage == MOGE_STAGE_ROUTE) return route_workspace_bytes(*shape);
  return (size_t)-1;
}

extern "C" const char* moge_version(void) { return "libmoge 0.1.0 (gfx950)"; }

extern "C" const char* moge_last_error(void) { return g_last_error.c_str(); }
