// moge_pack_weights: expert weight matrices from the row-major layout of a linear
// layer into the tiled layout the expert GEMMs read (tiles of 16 rows x 32
// columns, 1 KiB each in bf16; rows padded with zeros to a multiple of 32 and
// columns to a multiple of 32).  Run once when the weights are loaded.
//
// One thread per 16-byte piece of the destination: destination writes are fully
// coalesced; each piece comes from 16 consecutive bytes of one source row.
#include "moge_internal.hpp"

namespace moge {

__global__ __launch_bounds__(256) void pack_weights_kernel(const char* __restrict__ src, char* __restrict__ dst,
                                                           int64_t E, int64_t rows, int64_t cols, int esz) {
  const int64_t rp = round_up(rows, kWeightRowAlign), cp = round_up(cols, kTileCols);
  const int epc = 16 / esz;                       // elements per 16-byte piece
  const int64_t per = rp * cp / epc;              // pieces per expert
  const int64_t n = E * per;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n; q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = q / per;
    const int64_t i = (q - e * per) * epc;        // element index inside the expert's tiled matrix
    const int64_t tile = i / kTileElems, in = i - tile * kTileElems;
    const int64_t tr = tile / (cp / kTileCols), tc = tile - tr * (cp / kTileCols);
    const int64_t r = tr * kTileRows + in / kTileCols, c = tc * kTileCols + (in % kTileCols);
    u32x4_t v = zero;
    if (r < rows && c < cols)
      v = *reinterpret_cast<const u32x4_t*>(src + ((e * rows + r) * cols + c) * esz);
    *reinterpret_cast<u32x4_t*>(dst + (e * rp * cp + i) * esz) = v;
  }
}

}  // namespace moge

using namespace moge;

extern "C" moge_status_t moge_pack_weights(int32_t dtype, int64_t E, int64_t rows, int64_t cols, const void* src,
                                           void* dst, hipStream_t stream) {
  if (dtype != MOGE_BF16 && dtype != MOGE_F32) return fail(MOGE_ERR_DTYPE, "dtype must be MOGE_BF16 or MOGE_F32");
  if (E < 1 || rows < 1 || cols < 8 || cols % 8 != 0)
    return fail(MOGE_ERR_SHAPE, "need E >= 1, rows >= 1 and cols a positive multiple of 8");
  if (!src || !dst) return fail(MOGE_ERR_NULL, "src and dst are required");
  const int esz = dtype == MOGE_BF16 ? 2 : 4;
  const int64_t pieces = E * round_up(rows, kWeightRowAlign) * round_up(cols, kTileCols) / (16 / esz);
  int64_t grid = (pieces + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)grid), dim3(256), 0, stream, static_cast<const char*>(src),
                     static_cast<char*>(dst), E, rows, cols, esz);
  const moge_status_t st = check_launch("pack_weights_kernel");
  return st == MOGE_OK ? ok() : st;
}

namespace moge {

// float32 -> bf16 with the rounding of the expert GEMMs' outputs (f32_to_bf16).
__global__ __launch_bounds__(256) void round_bf16_kernel(const float* __restrict__ x, uint16_t* __restrict__ y,
                                                         int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) y[i] = f32_to_bf16(x[i]);
}

}  // namespace moge

extern "C" moge_status_t moge_round_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t stream) {
  if (n < 0) return fail(MOGE_ERR_SHAPE, "n must be >= 0");
  if (n == 0) return ok();
  if (!x || !y) return fail(MOGE_ERR_NULL, "x and y are required");
  int64_t grid = (n + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(round_bf16_kernel, dim3((unsigned)grid), dim3(256), 0, stream, x, y, n);
  const moge_status_t st = check_launch("round_bf16_kernel");
  return st == MOGE_OK ? ok() : st;
}
