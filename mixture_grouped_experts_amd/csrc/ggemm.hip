// moge_grouped_ffn: the SwiGLU expert on every expert's row segment, as two
// grouped GEMMs over the expert-ordered rows.
//
//   GEMM 1 (gate/up + SwiGLU):  h[r][f] = silu(x_perm[r] . Wg[e][f]) * (x_perm[r] . Wu[e][f])
//   GEMM 2 (down):              out[r][j] = h[r] . Wd[e][j]
//
// The pages name a grouped matmul (SwiftGMM) as the dominant inference kernel
// (Pangu Pro MoE, lsdiaocha.cn summary, section 3): it is bound by weight
// traffic at high concurrency and double-buffers its loads.  That kernel was
// written for Ascend; on gfx950 the same ideas become:
//   * bf16 v_mfma_f32_32x32x16_bf16 with float32 accumulators; a 256-thread
//     workgroup owns a 128-row x 256-weight-row tile (GEMM 1: 128 gate + 128 up
//     rows of the same 128 h columns, so the SwiGLU is fused into the epilogue;
//     GEMM 2: 256 output columns) and each wave a 64 x 128 quarter of it;
//   * A and B panels staged in LDS in BK = 64 steps, double buffered: the next
//     step's global loads are in flight while the current step's MFMAs run; rows
//     padded by 16 B so the 16-byte operand reads are bank-conflict free;
//   * a persistent grid walks a device-built tile list (no host sync on the
//     expert counts): every workgroup derives the per-expert tile counts from
//     `offsets` in LDS.  Tiles of one expert are ordered in groups of 8 m-tiles,
//     n-tiles outer, so tiles that share a weight panel or an activation panel
//     run at the same time; consecutive tiles go to one XCD (workgroup b runs on
//     XCD b % 8), so that sharing happens in that XCD's L2;
//   * epilogue through LDS so each lane stores 16 contiguous bytes.
// float32 shapes use a plain vector-ALU kernel pair (small shapes only).
#include <math.h>

#include "moge_internal.hpp"

namespace moge {

constexpr int kBM = 128;      // rows per tile
constexpr int kBW = 256;      // weight rows per tile
constexpr int kBK = 64;       // reduction step
constexpr int kLD = kBK + 8;  // padded LDS row (bf16 elements)
constexpr int kGroupM = 8;    // m-tiles per scheduling group
constexpr int kStageElems = (kBM + kBW) * kLD;
constexpr size_t kGemmLds = 2 * (size_t)kStageElems * 2;

template <bool SWIGLU>
__global__ __launch_bounds__(256) void ggemm_bf16_kernel(const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets,
                                                         int e_lo, int E, int64_t rows_cap, const uint16_t* __restrict__ B0,
                                                         const uint16_t* __restrict__ B1, int NOUT, int KD,
                                                         uint16_t* __restrict__ C) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  __shared__ int tp[kMaxExperts];  // inclusive prefix of tiles per expert
  __shared__ int erow[kMaxExperts];  // rows per expert, clipped to [0, rows_cap)
  __shared__ int scratch[4];
  constexpr int BNO = SWIGLU ? kBW / 2 : kBW;  // output columns per tile
  const int NT = (NOUT + BNO - 1) / BNO;
  const int64_t wrows = NOUT;  // weight rows per expert in B0/B1
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // per-expert tile counts -> inclusive prefix (E <= 256)
  {
    int tiles = 0;
    if (tid < E) {
      const int64_t seg0 = (int64_t)offsets[e_lo + tid] - offsets[e_lo];
      int64_t rows = (int64_t)offsets[e_lo + tid + 1] - offsets[e_lo + tid];
      if (seg0 < 0 || rows < 0) rows = 0;
      if (seg0 + rows > rows_cap) rows = rows_cap > seg0 ? rows_cap - seg0 : 0;
      erow[tid] = (int)rows;
      tiles = (int)((rows + kBM - 1) / kBM) * NT;
    }
    int tot;
    const int ex = block_exclusive_scan(tiles, scratch, &tot);
    if (tid < E) tp[tid] = ex + tiles;
    __syncthreads();
  }
  const int total = E > 0 ? tp[E - 1] : 0;
  const int base0 = offsets[e_lo];

  const int P = gridDim.x;  // multiple of 8
  const int per_xcd = P >> 3;
  const int slot = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);

  for (int tile = slot; tile < total; tile += P) {
    // expert of this tile: first i with tp[i] > tile
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (tp[mid] > tile) hi = mid; else lo = mid + 1;
    }
    const int ei = lo;
    const int q = tile - (ei > 0 ? tp[ei - 1] : 0);
    const int seg0 = offsets[e_lo + ei] - base0;
    const int erows = erow[ei];
    const int MT = (erows + kBM - 1) / kBM;
    // grouped order: groups of kGroupM m-tiles; inside a group n outer, m inner
    const int gsz = kGroupM * NT;
    const int g = q / gsz, qi = q - g * gsz;
    const int gm0 = g * kGroupM;
    const int gm = (MT - gm0) < kGroupM ? (MT - gm0) : kGroupM;
    const int mt = gm0 + qi % gm, nt = qi / gm;
    const int m0 = seg0 + mt * kBM;
    const int mrows = (erows - mt * kBM) < kBM ? (erows - mt * kBM) : kBM;
    const int n0 = nt * BNO;

    // this thread's global sources: A rows tid/8 + 32i (i<4), B rows tid/8 + 32i (i<8)
    const int cc = (tid & 7) * 8;
    const uint16_t* asrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int r = (tid >> 3) + 32 * i;
      if (r > mrows - 1) r = mrows - 1;
      asrc[i] = A + (int64_t)(m0 + r) * KD + cc;
    }
    const uint16_t* bsrc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (tid >> 3) + 32 * i;
      if (SWIGLU) {
        int f = n0 + (r & 127);
        if (f > NOUT - 1) f = NOUT - 1;
        const uint16_t* W = r < 128 ? B0 : B1;
        bsrc[i] = W + ((int64_t)ei * wrows + f) * KD + cc;
      } else {
        int j = n0 + r;
        if (j > NOUT - 1) j = NOUT - 1;
        bsrc[i] = B0 + ((int64_t)ei * wrows + j) * KD + cc;
      }
    }
    auto gload = [&](int ks, u32x4_t* ar, u32x4_t* br) {
      const int k = ks * kBK;
      const bool in = k + cc < KD;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (in) v = *reinterpret_cast<const u32x4_t*>(asrc[i] + k);
        ar[i] = v;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (in) v = *reinterpret_cast<const u32x4_t*>(bsrc[i] + k);
        br[i] = v;
      }
    };
    auto lstore = [&](int buf, const u32x4_t* ar, const u32x4_t* br) {
      uint16_t* st = lds + buf * kStageElems;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4_t*>(st + ((tid >> 3) + 32 * i) * kLD + cc) = ar[i];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x4_t*>(st + (kBM + (tid >> 3) + 32 * i) * kLD + cc) = br[i];
    };

    f32x16_t acc[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.f;

    // B rows of this wave's four 32-column blocks
    int brow[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      if (SWIGLU)
        brow[cb] = (cb < 2 ? wn * 64 + cb * 32 : 128 + wn * 64 + (cb - 2) * 32) + (lane & 31);
      else
        brow[cb] = wn * 128 + cb * 32 + (lane & 31);
    }
    const int arow0 = wm * 64 + (lane & 31);
    const int kofs = (lane >> 5) * 8;

    const int nk = (KD + kBK - 1) / kBK;
    u32x4_t ar[4], br[8];
    gload(0, ar, br);
    lstore(0, ar, br);
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
      const int buf = ks & 1;
      const bool more = ks + 1 < nk;
      if (more) gload(ks + 1, ar, br);
      const uint16_t* sa = lds + buf * kStageElems;
      const uint16_t* sb = sa + kBM * kLD;
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        bf16x8_t a[2], b[4];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          a[rb] = __builtin_bit_cast(bf16x8_t,
                                     *reinterpret_cast<const u32x4_t*>(sa + (arow0 + rb * 32) * kLD + kk * 16 + kofs));
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          b[cb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(sb + brow[cb] * kLD + kk * 16 + kofs));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[rb], b[cb], acc[rb][cb], 0, 0, 0);
      }
      if (more) lstore(buf ^ 1, ar, br);
      __syncthreads();
    }

    // epilogue: tile -> LDS (bf16, [kBM][BNO + 8]) -> 16-byte coalesced stores
    constexpr int LDO = BNO + 8;
    uint16_t* ot = lds;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + rb * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (SWIGLU) {
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            const float gv = acc[rb][cb][r], uv = acc[rb][cb + 2][r];
            const float hv = gv / (1.f + expf(-gv)) * uv;
            ot[row * LDO + wn * 64 + cb * 32 + (lane & 31)] = f32_to_bf16(hv);
          }
        } else {
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
            ot[row * LDO + wn * 128 + cb * 32 + (lane & 31)] = f32_to_bf16(acc[rb][cb][r]);
        }
      }
    }
    __syncthreads();
    constexpr int CPR = BNO / 8;  // 16-byte chunks per tile row
    for (int i = tid; i < kBM * CPR; i += 256) {
      const int row = i / CPR, ch = i - row * CPR;
      const int col = n0 + ch * 8;
      if (row < mrows && col < NOUT)
        *reinterpret_cast<u32x4_t*>(C + (int64_t)(m0 + row) * NOUT + col) =
            *reinterpret_cast<const u32x4_t*>(ot + row * LDO + ch * 8);
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------
// float32 vector-ALU pair (small shapes): one thread per output element.
__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ offsets, int e_lo, int e_hi, int grow) {
  int lo = e_lo, hi = e_hi - 1;  // last e with offsets[e] <= grow
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= grow) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void ffn_f32_gateup_kernel(const float* __restrict__ X, const int32_t* __restrict__ offsets,
                                                             int e_lo, int e_hi, int64_t rows_cap, const float* __restrict__ Wg,
                                                             const float* __restrict__ Wu, int d, int F, float* __restrict__ H) {
  const int64_t live = offsets[e_hi] - offsets[e_lo];
  const int64_t n = (live < rows_cap ? live : rows_cap) * F;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / F;
    const int f = (int)(i - r * F);
    const int e = expert_of_row(offsets, e_lo, e_hi, (int)(r + offsets[e_lo]));
    const float* xr = X + r * d;
    const float* wg = Wg + ((int64_t)(e - e_lo) * F + f) * d;
    const float* wu = Wu + ((int64_t)(e - e_lo) * F + f) * d;
    float a = 0.f, b = 0.f;
    for (int c = 0; c < d; ++c) {
      a = fmaf(xr[c], wg[c], a);
      b = fmaf(xr[c], wu[c], b);
    }
    H[r * F + f] = a / (1.f + expf(-a)) * b;
  }
}

__global__ __launch_bounds__(256) void ffn_f32_down_kernel(const float* __restrict__ H, const int32_t* __restrict__ offsets,
                                                           int e_lo, int e_hi, int64_t rows_cap, const float* __restrict__ Wd,
                                                           int d, int F, float* __restrict__ O) {
  const int64_t live = offsets[e_hi] - offsets[e_lo];
  const int64_t n = (live < rows_cap ? live : rows_cap) * d;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / d;
    const int j = (int)(i - r * d);
    const int e = expert_of_row(offsets, e_lo, e_hi, (int)(r + offsets[e_lo]));
    const float* hr = H + r * F;
    const float* wd = Wd + ((int64_t)(e - e_lo) * d + j) * F;
    float acc = 0.f;
    for (int f = 0; f < F; ++f) acc = fmaf(hr[f], wd[f], acc);
    O[r * d + j] = acc;
  }
}

static int device_cus() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  }
  return cus;
}

template <bool SWIGLU>
static moge_status_t launch_ggemm(const uint16_t* A, const int32_t* offsets, int e_lo, int E, int64_t rows_cap,
                                  const uint16_t* B0, const uint16_t* B1, int NOUT, int KD, uint16_t* C,
                                  hipStream_t stream) {
  moge_status_t st = raise_dynamic_lds(reinterpret_cast<const void*>(ggemm_bf16_kernel<SWIGLU>), kGemmLds,
                                       "ggemm_bf16_kernel");
  if (st != MOGE_OK) return st;
  constexpr int BNO = SWIGLU ? kBW / 2 : kBW;
  const int64_t NT = (NOUT + BNO - 1) / BNO;
  const int64_t upper = ((rows_cap + kBM - 1) / kBM + E) * NT;  // >= live tiles
  int64_t grid = device_cus();                                   // one 108 KiB-LDS workgroup per CU
  if (upper < grid) grid = upper;
  grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL(ggemm_bf16_kernel<SWIGLU>, dim3((unsigned)grid), dim3(256), kGemmLds, stream, A, offsets, e_lo,
                     E, rows_cap, B0, B1, NOUT, KD, C);
  return check_launch(SWIGLU ? "ggemm_bf16_kernel<gate_up>" : "ggemm_bf16_kernel<down>");
}

}  // namespace moge

using namespace moge;

static moge_status_t ffn_common_checks(const moge_shape_t* shape, int32_t e_lo, int32_t e_hi, int64_t rows_cap) {
  moge_status_t st = validate_shape(shape);
  if (st != MOGE_OK) return st;
  if (shape->F <= 0) return fail(MOGE_ERR_SHAPE, "the expert FFN needs F > 0");
  if (e_lo < 0 || e_hi > shape->N || e_lo >= e_hi) return fail(MOGE_ERR_ARG, "need 0 <= e_lo < e_hi <= N");
  if (rows_cap < 1) return fail(MOGE_ERR_CAPACITY, "rows_cap must be >= 1");
  return MOGE_OK;
}

static int64_t grid_1d(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return g < 65536 ? (g > 0 ? g : 1) : 65536;
}

extern "C" moge_status_t moge_expert_gate_up(const moge_shape_t* shape, const void* x_perm, const int32_t* offsets,
                                             int32_t e_lo, int32_t e_hi, int64_t rows_cap, const void* w_gate,
                                             const void* w_up, void* h, hipStream_t stream) {
  moge_status_t st = ffn_common_checks(shape, e_lo, e_hi, rows_cap);
  if (st != MOGE_OK) return st;
  if (!x_perm || !offsets || !w_gate || !w_up || !h)
    return fail(MOGE_ERR_NULL, "x_perm, offsets, w_gate, w_up and h are required");
  const moge_shape_t& s = *shape;
  if (s.dtype == MOGE_BF16) {
    st = launch_ggemm<true>(static_cast<const uint16_t*>(x_perm), offsets, e_lo, e_hi - e_lo, rows_cap,
                            static_cast<const uint16_t*>(w_gate), static_cast<const uint16_t*>(w_up), s.F, s.d,
                            static_cast<uint16_t*>(h), stream);
  } else {
    hipLaunchKernelGGL(ffn_f32_gateup_kernel, dim3((unsigned)grid_1d(rows_cap * s.F)), dim3(256), 0, stream,
                       static_cast<const float*>(x_perm), offsets, e_lo, e_hi, rows_cap,
                       static_cast<const float*>(w_gate), static_cast<const float*>(w_up), s.d, s.F,
                       static_cast<float*>(h));
    st = check_launch("ffn_f32_gateup_kernel");
  }
  return st == MOGE_OK ? ok() : st;
}

extern "C" moge_status_t moge_expert_down(const moge_shape_t* shape, const void* h, const int32_t* offsets,
                                          int32_t e_lo, int32_t e_hi, int64_t rows_cap, const void* w_down, void* out,
                                          hipStream_t stream) {
  moge_status_t st = ffn_common_checks(shape, e_lo, e_hi, rows_cap);
  if (st != MOGE_OK) return st;
  if (!h || !offsets || !w_down || !out) return fail(MOGE_ERR_NULL, "h, offsets, w_down and out are required");
  const moge_shape_t& s = *shape;
  if (s.dtype == MOGE_BF16) {
    st = launch_ggemm<false>(static_cast<const uint16_t*>(h), offsets, e_lo, e_hi - e_lo, rows_cap,
                             static_cast<const uint16_t*>(w_down), nullptr, s.d, s.F, static_cast<uint16_t*>(out),
                             stream);
  } else {
    hipLaunchKernelGGL(ffn_f32_down_kernel, dim3((unsigned)grid_1d(rows_cap * s.d)), dim3(256), 0, stream,
                       static_cast<const float*>(h), offsets, e_lo, e_hi, rows_cap, static_cast<const float*>(w_down),
                       s.d, s.F, static_cast<float*>(out));
    st = check_launch("ffn_f32_down_kernel");
  }
  return st == MOGE_OK ? ok() : st;
}

extern "C" moge_status_t moge_grouped_ffn(const moge_shape_t* shape, const void* x_perm, const int32_t* offsets,
                                          int32_t e_lo, int32_t e_hi, int64_t rows_cap, const void* w_gate,
                                          const void* w_up, const void* w_down, void* h, void* out,
                                          hipStream_t stream) {
  moge_status_t st = moge_expert_gate_up(shape, x_perm, offsets, e_lo, e_hi, rows_cap, w_gate, w_up, h, stream);
  if (st != MOGE_OK) return st;
  return moge_expert_down(shape, h, offsets, e_lo, e_hi, rows_cap, w_down, out, stream);
}
