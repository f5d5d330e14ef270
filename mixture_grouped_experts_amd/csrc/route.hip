// moge_route: router scores -> softmax over all N experts -> top-K' inside each
// of the M expert groups (MoGE), or top-K over all experts (conventional router).
//
// Method: Pangu Pro MoE, lsdiaocha.cn summary, section 1 (architecture): the N
// experts are split evenly into M groups, one per device; a token's scores go
// through a softmax over all experts and then the K' = K/M best experts of every
// group are kept, which puts exactly K' of the token's assignments on each device.
//
// gfx950 design
//   * bf16 scores: x [T][d] is streamed from HBM exactly once.  A workgroup of 4
//     waves owns TM tokens x NP (N rounded up to 64) experts; each wave owns a
//     32-token x 64-expert block and accumulates it with v_mfma_f32_32x32x16_bf16
//     (float32 accumulate).  x goes straight from HBM into MFMA operand registers:
//     the reduction over d is order-free, so every lane reads a contiguous
//     BK/2-element run of its token row (lane half h owns k in [h*BK/2, (h+1)*BK/2)
//     of each BK step) and the router weights are read from LDS with the same k
//     assignment.  The router weight slab of each BK step is staged once per
//     workgroup in LDS (rows padded by 16 B, so the 16-byte operand reads are
//     bank-conflict free) and double buffered; the next step's x and weights are
//     in flight while the current step's MFMAs run.
//   * Epilogue in the same kernel: the TM x N score tile goes to LDS, the optional
//     score store is coalesced, and one wave per token does the softmax (wave-wide
//     max and sum) and the per-group rank count that picks the top-K'.
//   * float32 shapes and caller-supplied scores use the same epilogue.
#include <math.h>

#include "moge_internal.hpp"

namespace moge {

// Softmax over the token's N scores (LDS row `l`) and the per-group choice.
// One full wave per token; lane owns experts lane, lane+64, lane+128, lane+192.
// Narrow groups (G <= 64): rank(e) = #{e' in group(e) : l[e'] > l[e] or
// (l[e'] == l[e] and e' < e)}; experts with rank < k go to slot g*k + rank.
// Wide groups (G > 64, e.g. the global top-K over 256 experts): k rounds of a
// wave-wide argmax with the same order (higher score, then lower id) per group;
// round r fills slot g*k + r, which is the same slot the rank rule gives.
__device__ __forceinline__ void select_token(const float* __restrict__ l, int N, int n_groups, int k, int64_t t,
                                             int32_t* __restrict__ idx, float* __restrict__ gate) {
  const int lane = threadIdx.x & 63;
  const int G = N / n_groups;
  const int K = n_groups * k;
  float v[4], ex[4];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < N ? l[e] : -INFINITY;
    m = fmaxf(m, v[j]);
  }
  m = wave_max(m);
  float z = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    ex[j] = e < N ? expf(v[j] - m) : 0.f;
    z += ex[j];
  }
  z = wave_sum(z);
  if (G <= 64) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (e < N) {
        const int g = e / G;
        const int base = g * G;
        int rank = 0;
        for (int e2 = base; e2 < base + G; ++e2) {
          const float w = l[e2];
          rank += (w > v[j]) || (w == v[j] && e2 < e);
        }
        if (rank < k) {
          idx[t * K + g * k + rank] = e;
          gate[t * K + g * k + rank] = ex[j] / z;
        }
      }
    }
    return;
  }
  unsigned taken = 0u;  // bit j: expert lane + 64j already chosen
  for (int g = 0; g < n_groups; ++g) {
    for (int r = 0; r < k; ++r) {
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        if (e < N && e / G == g && !((taken >> j) & 1u) && (v[j] > bv || (v[j] == bv && e < bi))) {
          bv = v[j];
          bi = e;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      // the owner of expert bi records it
      if ((bi & 63) == lane) {
        const int j = bi >> 6;
        taken |= 1u << j;
        idx[t * K + g * k + r] = bi;
        gate[t * K + g * k + r] = ex[j] / z;
      }
    }
  }
}

// Writes the LDS score tile [rows][ld] to logits_out (if any) and runs the choice.
__device__ __forceinline__ void tile_epilogue(const float* __restrict__ lt, int ld, int rows, int64_t t0, int64_t T,
                                              int N, int n_groups, int k, float* __restrict__ logits_out,
                                              int32_t* __restrict__ idx, float* __restrict__ gate) {
  if (logits_out) {
    for (int i = threadIdx.x; i < rows * N; i += blockDim.x) {
      const int r = i / N, c = i - r * N;
      if (t0 + r < T) logits_out[(t0 + r) * N + c] = lt[r * ld + c];
    }
  }
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  for (int r = wave; r < rows; r += nwaves) {
    if (t0 + r < T) select_token(lt + r * ld, N, n_groups, k, t0 + r, idx, gate);
  }
}

// ----------------------------------------------------------------------------
// bf16 scores with MFMA.  WC waves across experts (NP = 64*WC), 4/WC across tokens.
template <int WC, int BK>
__global__ __launch_bounds__(256) void route_mfma_kernel(int64_t T, int d, int N, int n_groups, int k,
                                                         const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ w,
                                                         const float* __restrict__ bias,
                                                         float* __restrict__ logits_out, int32_t* __restrict__ idx,
                                                         float* __restrict__ gate) {
  constexpr int WR = 4 / WC;
  constexpr int TM = 32 * WR;
  constexpr int NP = 64 * WC;
  constexpr int LDW = BK + 8;          // padded LDS row, bf16 elements
  constexpr int HALF = BK / 2;         // k run per lane half
  constexpr int NCH = HALF / 8;        // 16-byte chunks per lane per step (= MFMAs per col block)
  constexpr int WCH = NP * (BK / 8) / 256;  // weight chunks per thread per step
  constexpr int WBUF = NP * LDW;       // bf16 elements per weight buffer
  constexpr int SMEM_W = 2 * WBUF * 2;
  constexpr int SMEM_L = TM * NP * 4;
  constexpr int SMEM = SMEM_W > SMEM_L ? SMEM_W : SMEM_L;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  uint16_t* wl = reinterpret_cast<uint16_t*>(smem);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wr = wave / WC, wc = wave % WC;
  const int64_t t0 = (int64_t)blockIdx.x * TM;
  int64_t arow = t0 + wr * 32 + (lane & 31);
  if (arow > T - 1) arow = T - 1;
  const uint16_t* aptr = x + arow * d + (lane >> 5) * HALF;
  const int nk = (d + BK - 1) / BK;

  // weight chunk c of a step: row c / (BK/8), 16-byte column c % (BK/8)
  auto load_w = [&](int ks, u32x4_t* reg) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int row = c / (BK / 8), col = (c % (BK / 8)) * 8;
      const int kk = ks * BK + col;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (row < N && kk < d) v = *reinterpret_cast<const u32x4_t*>(w + (int64_t)row * d + kk);
      reg[i] = v;
    }
  };
  auto store_w = [&](int buf, const u32x4_t* reg) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int row = c / (BK / 8), col = (c % (BK / 8)) * 8;
      *reinterpret_cast<u32x4_t*>(wl + buf * WBUF + row * LDW + col) = reg[i];
    }
  };
  auto load_a = [&](int ks, u32x4_t* reg) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int kk = ks * BK + (lane >> 5) * HALF + j * 8;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (kk < d) v = *reinterpret_cast<const u32x4_t*>(aptr + (int64_t)ks * BK + j * 8);
      reg[j] = v;
    }
  };

  f32x16_t acc[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;

  u32x4_t wreg[WCH], areg[NCH], anext[NCH];
  load_w(0, wreg);
  load_a(0, areg);
  store_w(0, wreg);
  __syncthreads();

  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    const bool more = ks + 1 < nk;
    if (more) {
      load_w(ks + 1, wreg);
      load_a(ks + 1, anext);
    }
    const uint16_t* wb = wl + buf * WBUF;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, areg[j]);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int col = wc * 64 + cb * 32 + (lane & 31);
        const u32x4_t braw = *reinterpret_cast<const u32x4_t*>(wb + col * LDW + (lane >> 5) * HALF + j * 8);
        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, braw), acc[cb], 0, 0, 0);
      }
    }
    if (more) {
      store_w(buf ^ 1, wreg);
#pragma unroll
      for (int j = 0; j < NCH; ++j) areg[j] = anext[j];
    }
    __syncthreads();
  }

  // scores -> LDS tile [TM][NP]; padded experts get -inf (never chosen, exp = 0)
  float* lt = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int col = wc * 64 + cb * 32 + (lane & 31);
    const float b = (bias && col < N) ? bias[col] : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wr * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      lt[row * NP + col] = col < N ? acc[cb][r] + b : -INFINITY;
    }
  }
  __syncthreads();
  tile_epilogue(lt, NP, TM, t0, T, N, n_groups, k, logits_out, idx, gate);
}

// ----------------------------------------------------------------------------
// bf16 scores for few tokens: 32 tokens per workgroup; the 4 waves split the
// experts (WC column groups of 64) and the hidden dimension (4/WC parts), so a
// small batch still spreads over many waves.  Operands are read straight from
// global memory in MFMA layout; the partial sums meet in LDS and are added in a
// fixed order (deterministic).
template <int WC>
__global__ __launch_bounds__(256) void route_mfma_splitk_kernel(int64_t T, int d, int N, int n_groups, int k,
                                                                const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ w,
                                                                const float* __restrict__ bias,
                                                                float* __restrict__ logits_out,
                                                                int32_t* __restrict__ idx, float* __restrict__ gate) {
  constexpr int KS = 4 / WC;
  constexpr int NP = 64 * WC;
  constexpr int TM = 32;
  __shared__ __attribute__((aligned(16))) float part[KS * TM * NP];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wc = wave % WC, q = wave / WC;
  const int64_t t0 = (int64_t)blockIdx.x * TM;
  int64_t arow = t0 + (lane & 31);
  if (arow > T - 1) arow = T - 1;
  const uint16_t* ap = x + arow * d + (lane >> 5) * 8;
  const uint16_t* bp[2];
  bool bval[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int col = wc * 64 + cb * 32 + (lane & 31);
    bval[cb] = col < N;
    bp[cb] = w + (int64_t)(col < N ? col : 0) * d + (lane >> 5) * 8;
  }
  f32x16_t acc[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
  const int nk = (d + 63) / 64;
  for (int ks = q; ks < nk; ks += KS) {
    u32x4_t a[4], b[2][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = ks * 64 + j * 16 + (lane >> 5) * 8;
      const u32x4_t zero = {0u, 0u, 0u, 0u};
      a[j] = kk < d ? *reinterpret_cast<const u32x4_t*>(ap + ks * 64 + j * 16) : zero;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        b[cb][j] = (kk < d && bval[cb]) ? *reinterpret_cast<const u32x4_t*>(bp[cb] + ks * 64 + j * 16) : zero;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[j]),
                                                          __builtin_bit_cast(bf16x8_t, b[cb][j]), acc[cb], 0, 0, 0);
  }
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int col = wc * 64 + cb * 32 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      part[(q * TM + row) * NP + col] = acc[cb][r];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < TM * NP; i += 256) {
    const int col = i % NP;
    float v = part[i];
#pragma unroll
    for (int p = 1; p < KS; ++p) v += part[p * TM * NP + i];
    part[i] = col < N ? v + (bias ? bias[col] : 0.f) : -INFINITY;
  }
  __syncthreads();
  tile_epilogue(part, NP, TM, t0, T, N, n_groups, k, logits_out, idx, gate);
}

// ----------------------------------------------------------------------------
// float32 scores on the vector ALUs (small shapes).  16 tokens per workgroup.
constexpr int kF32Tokens = 16;
__global__ __launch_bounds__(256) void route_f32_kernel(int64_t T, int d, int N, int n_groups, int k,
                                                        const float* __restrict__ x, const float* __restrict__ w,
                                                        const float* __restrict__ bias,
                                                        float* __restrict__ logits_out, int32_t* __restrict__ idx,
                                                        float* __restrict__ gate) {
  __shared__ float lt[kF32Tokens * kMaxExperts];
  const int64_t t0 = (int64_t)blockIdx.x * kF32Tokens;
  for (int i = threadIdx.x; i < kF32Tokens * N; i += blockDim.x) {
    const int r = i / N, e = i - r * N;
    int64_t t = t0 + r;
    if (t > T - 1) t = T - 1;
    const float* xr = x + t * d;
    const float* wr = w + (int64_t)e * d;
    float acc = 0.f;
    for (int c = 0; c < d; ++c) acc = fmaf(xr[c], wr[c], acc);
    if (bias) acc += bias[e];
    lt[r * N + e] = acc;
  }
  __syncthreads();
  tile_epilogue(lt, N, kF32Tokens, t0, T, N, n_groups, k, logits_out, idx, gate);
}

// ----------------------------------------------------------------------------
// Caller-supplied scores.  32 tokens per workgroup.
constexpr int kSelTokens = 32;
__global__ __launch_bounds__(256) void route_select_kernel(int64_t T, int N, int n_groups, int k,
                                                           const float* __restrict__ logits,
                                                           int32_t* __restrict__ idx, float* __restrict__ gate) {
  __shared__ float lt[kSelTokens * kMaxExperts];
  const int64_t t0 = (int64_t)blockIdx.x * kSelTokens;
  for (int i = threadIdx.x; i < kSelTokens * N; i += blockDim.x) {
    const int r = i / N, c = i - r * N;
    lt[r * N + c] = (t0 + r < T) ? logits[(t0 + r) * N + c] : 0.f;
  }
  __syncthreads();
  tile_epilogue(lt, N, kSelTokens, t0, T, N, n_groups, k, nullptr, idx, gate);
}

template <int WC, int BK>
static void launch_route_mfma(const moge_shape_t& s, int n_groups, int k, const void* x, const void* w,
                              const float* bias, float* logits, int32_t* idx, float* gate, hipStream_t stream) {
  constexpr int TM = 32 * (4 / WC);
  const int64_t grid = ((int64_t)s.T + TM - 1) / TM;
  hipLaunchKernelGGL((route_mfma_kernel<WC, BK>), dim3((unsigned)grid), dim3(256), 0, stream, (int64_t)s.T, s.d,
                     s.N, n_groups, k, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), bias,
                     logits, idx, gate);
}

}  // namespace moge

using namespace moge;

extern "C" moge_status_t moge_route(const moge_shape_t* shape, int32_t mode, const void* x, const void* w_router,
                                    const float* bias, float* logits, int32_t* idx, float* gate,
                                    hipStream_t stream) {
  moge_status_t st = validate_shape(shape);
  if (st != MOGE_OK) return st;
  const moge_shape_t& s = *shape;
  if (mode != MOGE_ROUTE_GROUPED && mode != MOGE_ROUTE_GLOBAL) return fail(MOGE_ERR_ARG, "unknown route mode");
  if (!idx || !gate) return fail(MOGE_ERR_NULL, "idx and gate are required");
  if (!x && !logits) return fail(MOGE_ERR_NULL, "either x (with w_router) or input logits is required");
  if (x && !w_router) return fail(MOGE_ERR_NULL, "w_router is required when x is given");
  if (!x && bias) return fail(MOGE_ERR_ARG, "bias must be NULL when logits are supplied (they include it)");
  const int n_groups = mode == MOGE_ROUTE_GROUPED ? s.M : 1;
  const int k = mode == MOGE_ROUTE_GROUPED ? s.k_per_group : s.M * s.k_per_group;

  if (!x) {
    const int64_t grid = ((int64_t)s.T + kSelTokens - 1) / kSelTokens;
    hipLaunchKernelGGL(route_select_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (int64_t)s.T, s.N,
                       n_groups, k, logits, idx, gate);
    st = check_launch("route_select_kernel");
  } else if (s.dtype == MOGE_F32) {
    const int64_t grid = ((int64_t)s.T + kF32Tokens - 1) / kF32Tokens;
    hipLaunchKernelGGL(route_f32_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (int64_t)s.T, s.d, s.N,
                       n_groups, k, static_cast<const float*>(x), static_cast<const float*>(w_router), bias, logits,
                       idx, gate);
    st = check_launch("route_f32_kernel");
  } else {
    // few tokens (fewer 128-token tiles than CUs) and N <= 128: the split-K kernel
    const bool few = ((int64_t)s.T + 127) / 128 < 256;
    if (few && s.N <= 64) {
      hipLaunchKernelGGL(route_mfma_splitk_kernel<1>, dim3((unsigned)(((int64_t)s.T + 31) / 32)), dim3(256), 0,
                         stream, (int64_t)s.T, s.d, s.N, n_groups, k, static_cast<const uint16_t*>(x),
                         static_cast<const uint16_t*>(w_router), bias, logits, idx, gate);
    } else if (few && s.N <= 128) {
      hipLaunchKernelGGL(route_mfma_splitk_kernel<2>, dim3((unsigned)(((int64_t)s.T + 31) / 32)), dim3(256), 0,
                         stream, (int64_t)s.T, s.d, s.N, n_groups, k, static_cast<const uint16_t*>(x),
                         static_cast<const uint16_t*>(w_router), bias, logits, idx, gate);
    } else if (s.N <= 64) {
      launch_route_mfma<1, 128>(s, n_groups, k, x, w_router, bias, logits, idx, gate, stream);
    } else if (s.N <= 128) {
      launch_route_mfma<2, 128>(s, n_groups, k, x, w_router, bias, logits, idx, gate, stream);
    } else {
      launch_route_mfma<4, 64>(s, n_groups, k, x, w_router, bias, logits, idx, gate, stream);
    }
    st = check_launch("route_mfma_kernel");
  }
  return st == MOGE_OK ? ok() : st;
}
