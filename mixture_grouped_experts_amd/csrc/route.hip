// moge_route: router scores -> softmax over all N experts -> top-K' inside each
// of the M expert groups (MoGE), or top-K over all experts (conventional router).
//
// Method: Pangu Pro MoE, lsdiaocha.cn summary, section 1 (architecture): the N
// experts are split evenly into M groups, one per device; a token's scores go
// through a softmax over all experts and then the K' = K/M best experts of every
// group are kept, which puts exactly K' of the token's assignments on each device.
//
// gfx950 design
//   * bf16 scores: x [T][d] is streamed from HBM once.  A workgroup of 4 waves owns
//     TM tokens x NP experts (128 x 64, 64 x 128 or 32 x 256 by N), TM*NP = 8192;
//     each wave owns a 32-token x 64-expert block and accumulates it with
//     v_mfma_f32_32x32x16_bf16 (float32 accumulate).  Token rows and router rows go
//     from global memory straight into a 6- to 8-stage LDS ring with direct-to-LDS
//     loads, several 32-element steps ahead, so each workgroup keeps tens of KiB of
//     x in flight without staging registers; the router slab of a step is shared by
//     the workgroup's waves.  Few tokens (fewer 128-token tiles than CUs, N <= 128):
//     a split-K kernel whose operands go straight from global memory into MFMA
//     registers.
//   * Epilogue in the same kernel: the TM x N score tile goes to LDS, the optional
//     score store is coalesced, and the choice runs lane-parallel (one lane per
//     token and group) or, for wide groups, one wave per token.
//   * N > 128 with the scores stored: the experts are split in two halves over the
//     XCDs (each XCD's L2 keeps its half of the router matrix), the kernel only
//     writes scores, and the choice is a second pass.
//   * The choice from stored scores (that pass, the global comparator, caller
//     scores) runs one lane per token with a sorted register list per group.
//   * float32 shapes use a vector-ALU scores kernel with the same epilogue.
#include <math.h>

#include "moge_internal.hpp"

namespace moge {

// The order the choice sorts by: the score itself, except that a NaN ranks as -inf
// (ties, -inf ones included, go to the lower expert id).  The pages define the choice
// on finite scores only; with this key every group still yields exactly k distinct
// experts of its own, whatever the scores (moge_check_finite reports non-finite ones).
__device__ __forceinline__ float order_key(float v) { return v == v ? v : -INFINITY; }

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
  float v[4], ex[4], kv[4];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < N ? l[e] : -INFINITY;
    kv[j] = order_key(v[j]);
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
          const float w = order_key(l[e2]);
          rank += (w > kv[j]) || (w == kv[j] && e2 < e);
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
        if (e < N && e / G == g && !((taken >> j) & 1u) && (kv[j] > bv || (kv[j] == bv && e < bi))) {
          bv = kv[j];
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

// Lane-parallel choice for up to 64 groups: in one wave pass, lane (tl, g) handles
// group g of token tl; a token's Mp lanes (n_groups rounded up to a power of two)
// are adjacent, so the softmax max and sum over its N scores are butterflies over
// Mp lanes, and a pass covers 64 / Mp tokens at once.  Inside the group, k rounds
// each take the best score that comes after the previous pick in the order
// (score descending, expert id ascending): round r finds the expert of rank r.
// Score rows are `ld` floats apart (ld odd keeps the lanes' reads on distinct banks).
__device__ __forceinline__ void select_tile(const float* __restrict__ lt, int ld, int rows, int64_t t0, int64_t T,
                                            int N, int n_groups, int k, int32_t* __restrict__ idx,
                                            float* __restrict__ gate) {
  const int G = N / n_groups, K = n_groups * k;
  int Mp = 1;
  while (Mp < n_groups) Mp <<= 1;
  const int tpp = 64 / Mp;  // tokens per wave pass
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int g = lane & (Mp - 1), tl = lane / Mp;
  for (int r0 = wave * tpp; r0 < rows; r0 += nw * tpp) {  // wave-uniform
    const int r = r0 + tl;
    const bool own = r < rows && t0 + r < T && g < n_groups;
    const float* v = lt + (int64_t)(own ? r : 0) * ld + (own ? g * G : 0);
    const int n = own ? G : 0;
    float m = -INFINITY;
    for (int i = 0; i < n; ++i) m = fmaxf(m, v[i]);
    for (int off = 1; off < Mp; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    float z = 0.f;
    for (int i = 0; i < n; ++i) z += expf(v[i] - m);
    for (int off = 1; off < Mp; off <<= 1) z += __shfl_xor(z, off, 64);
    if (own) {
      const int64_t t = t0 + r;
      float pv = INFINITY;
      int pi = -1;
      for (int rk = 0; rk < k; ++rk) {
        float bv = -INFINITY;
        int bi = -1;
        for (int i = 0; i < n; ++i) {
          const float x = order_key(v[i]);
          const bool after = x < pv || (x == pv && i > pi);  // not yet taken
          if (after && (bi < 0 || x > bv)) {
            bv = x;
            bi = i;
          }
        }
        pv = bv;
        pi = bi;
        idx[t * K + g * k + rk] = g * G + bi;
        gate[t * K + g * k + rk] = expf(bv - m) / z;
      }
    }
  }
}

// The same choice for a group size G known at compile time: each lane reads its G
// scores from LDS once into registers and the three scans are unrolled (the same
// operations in the same order, so the same results as select_tile).
template <int G>
__device__ __forceinline__ void select_tile_g(const float* __restrict__ lt, int ld, int rows, int64_t t0, int64_t T,
                                              int n_groups, int k, int32_t* __restrict__ idx,
                                              float* __restrict__ gate) {
  const int K = n_groups * k;
  int Mp = 1;
  while (Mp < n_groups) Mp <<= 1;
  const int tpp = 64 / Mp;  // tokens per wave pass
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int g = lane & (Mp - 1), tl = lane / Mp;
  for (int r0 = wave * tpp; r0 < rows; r0 += nw * tpp) {  // wave-uniform
    const int r = r0 + tl;
    const bool own = r < rows && t0 + r < T && g < n_groups;
    const float* v = lt + (int64_t)(own ? r : 0) * ld + (own ? g * G : 0);
    float s[G];
#pragma unroll
    for (int i = 0; i < G; ++i) s[i] = v[i];
    float m = -INFINITY;
    if (own) {
#pragma unroll
      for (int i = 0; i < G; ++i) m = fmaxf(m, s[i]);
    }
    for (int off = 1; off < Mp; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    float z = 0.f;
    if (own) {
#pragma unroll
      for (int i = 0; i < G; ++i) z += expf(s[i] - m);
    }
    for (int off = 1; off < Mp; off <<= 1) z += __shfl_xor(z, off, 64);
    if (own) {
      const int64_t t = t0 + r;
      float pv = INFINITY;
      int pi = -1;
      for (int rk = 0; rk < k; ++rk) {
        float bv = -INFINITY;
        int bi = -1;
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const float x = order_key(s[i]);
          const bool after = x < pv || (x == pv && i > pi);  // not yet taken
          if (after && (bi < 0 || x > bv)) {
            bv = x;
            bi = i;
          }
        }
        pv = bv;
        pi = bi;
        idx[t * K + g * k + rk] = g * G + bi;
        gate[t * K + g * k + rk] = expf(bv - m) / z;
      }
    }
  }
}

// The lane-parallel choice scans (k + 2) * G scores per lane; past a small budget
// (wide groups such as the global top-K over all experts) one wave per token with
// wave-wide reductions is faster.
__host__ __device__ __forceinline__ bool lane_parallel_choice(int N, int n_groups, int k) {
  return n_groups <= 64 && (k + 2) * (N / n_groups) <= 256;
}

// Writes the LDS score tile [rows][ld] to logits_out (if any) and runs the choice.
// (all threads of the block call it)
__device__ __forceinline__ void tile_epilogue(const float* __restrict__ lt, int ld, int rows, int64_t t0, int64_t T,
                                              int N, int n_groups, int k, float* __restrict__ logits_out,
                                              int32_t* __restrict__ idx, float* __restrict__ gate) {
  // The scores go out with the non-temporal hint: every tile writes them at the same
  // time at the end of the kernel, and streamed past the L2 they no longer wait there
  // for the kernel's final write-back (the route kernel at 65536 tokens x 4096 x 64
  // experts was 4% faster).
  if (logits_out) {
    for (int i = threadIdx.x; i < rows * N; i += blockDim.x) {
      const int r = i / N, c = i - r * N;
      if (t0 + r < T) __builtin_nontemporal_store(lt[r * ld + c], logits_out + (t0 + r) * N + c);
    }
  }
  if (lane_parallel_choice(N, n_groups, k)) {
    if (N == 8 * n_groups) select_tile_g<8>(lt, ld, rows, t0, T, n_groups, k, idx, gate);
    else select_tile(lt, ld, rows, t0, T, N, n_groups, k, idx, gate);
    return;
  }
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  for (int r = wave; r < rows; r += nwaves) {
    if (t0 + r < T) select_token(lt + r * ld, N, n_groups, k, t0 + r, idx, gate);
  }
}

// ----------------------------------------------------------------------------
// bf16 scores, many tokens.  A workgroup of 4 waves owns TM tokens x NP experts
// (NP = N rounded up to 64, 128 or 256 and TM = 8192 / NP, so every wave owns one
// 32-token x 64-expert block: two 32x32 accumulators).  The token rows and the
// router rows of each 32-element step go from global memory straight into an
// S-stage LDS ring (global_load_lds_dwordx4, 16 rows of 64 bytes per instruction,
// XOR-swizzled rows), S - 1 steps ahead, so x streams from HBM with several steps
// of loads in flight per workgroup and no staging registers; x is read exactly
// once.  One barrier per step.  The epilogue keeps the TM x NP score tile in LDS
// for the softmax and the per-group choice.
//
// PARTS > 1 (N > 128, scores stored): the experts are split in PARTS slices of NP;
// workgroup b computes slice b % PARTS of token tile b / PARTS and only writes its
// scores, and a second pass (route_select_kernel) makes the choice.  Workgroup b
// runs on XCD b % 8, so each XCD needs only its slice of the router matrix (1-2 MB
// at N = 256, d = 7680), which then stays in that XCD's 4 MB L2 instead of being
// fetched from the last-level cache by every workgroup, and the tile can take more
// tokens, so more of each step's loads are token rows streaming from HBM.
template <int TM, int NP, int S, int WV, int PARTS>
__global__ __launch_bounds__(64 * WV) void route_dma_kernel(int64_t T, int d, int N, int n_groups, int k,
                                                        const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ w,
                                                        const float* __restrict__ bias,
                                                        float* __restrict__ logits_out, int32_t* __restrict__ idx,
                                                        float* __restrict__ gate) {
  constexpr int ROWS = TM + NP;      // stage rows of 64 bytes: tokens, then experts
  constexpr int NI = ROWS / 16;      // load instructions per step
  constexpr int NJ = (NI + WV - 1) / WV;  // per wave, at most
  constexpr int CH = NJ;                  // loads per step of waves 0 .. NI%WV - 1 (all when NI%WV == 0)
  constexpr int CL = NI / WV;             // loads per step of the other waves
  constexpr int STAGE = ROWS * 64;
  constexpr int TB = TM / 32;        // token blocks; wave = token block + TB * expert slice
  static_assert(TM * NP == 2048 * WV && S >= 4, "route tile: one 32 x 64 block per wave");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tb = wave % TB, es = wave / TB;
  const int64_t t0 = (int64_t)(blockIdx.x / PARTS) * TM;
  const int e0 = (int)(blockIdx.x % PARTS) * NP;  // first expert of this workgroup
  const int nkf = d / 32;                        // full steps; a ragged tail follows the loop
  // token tiles start at different steps (and wrap around), so the workgroups do not all
  // read the same column range of their rows at once: each tile walks 64-byte pieces of
  // rows 8 KiB apart, and in a plain streaming probe of that pattern the staggered start
  // reads 9% faster (router -11% on 65536 tokens x 4096).  The order of the float32
  // accumulation over k then depends on the tile; scores stay within the tolerance.
  const int krot = nkf > 0 ? (int)(((t0 / TM) * 37) % nkf) : 0;
  const bool many = (NI % WV == 0) || wave < (NI % WV);  // this wave issues CH loads per step, else CL

  // load j of this wave moves stage rows 16 i .. 16 i + 15 with i = wave + WV j
  const uint16_t* src[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int srow = 16 * (wave + WV * j) + (lane >> 2);
    const int c = (lane & 3) ^ lds_swz(srow);
    if (srow < TM) {
      int64_t t = t0 + srow;
      if (t > T - 1) t = T - 1;
      src[j] = x + t * d + c * 8;
    } else {
      int e = e0 + srow - TM;
      if (e > N - 1) e = N - 1;
      src[j] = w + (int64_t)e * d + c * 8;
    }
  }
  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int ks) {
    if (ks >= nkf) return;
    const uint32_t st = lds0 + (uint32_t)((ks % S) * STAGE);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (wave + WV * j < NI) {
        const int kk = ks + krot < nkf ? ks + krot : ks + krot - nkf;
        dma_16x64(src[j] + kk * 32, st + (uint32_t)(16 * (wave + WV * j) * 64));
      }
  };
  // at most `steps` steps of this wave's loads still in flight (and, with lgkm, no LDS reads)
  auto wait_steps = [&](int steps_left_ok, bool lgkm) {
    // steps_left_ok is S - 3 (steady state) or 0 (prologue / tail); both branches are immediates
    if (steps_left_ok == 0) {
      if (lgkm) __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(0));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    } else if (many) {
      if (lgkm) __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm((S - 3) * CH));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 3) * CH));
    } else {
      if (lgkm) __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm((S - 3) * CL));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 3) * CL));
    }
  };

  const int kc = lane >> 5;
  const int arow = tb * 32 + (lane & 31);
  int brow[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) brow[cb] = TM + es * 64 + cb * 32 + (lane & 31);
  auto frag = [&](int stage, int kk, bf16x8_t& a, bf16x8_t (&b)[2]) {
    const char* st = lds + stage * STAGE;
    const int c = kk * 2 + kc;
    a = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(st + arow * 64 + ((c ^ lds_swz(arow)) << 4)));
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
      b[cb] = __builtin_bit_cast(bf16x8_t,
                                 *reinterpret_cast<const u32x4_t*>(st + brow[cb] * 64 + ((c ^ lds_swz(brow[cb])) << 4)));
  };
  f32x16_t acc[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
  auto mfma = [&](const bf16x8_t& a, const bf16x8_t (&b)[2]) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[cb], acc[cb], 0, 0, 0);
  };

  // prologue: steps 0 .. S-2 in flight; steps 0 and 1 landed
#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s);
  wait_steps(nkf >= S - 1 ? S - 3 : 0, false);
  __syncthreads();
  bf16x8_t a0, b0[2], a1, b1[2];
  frag(0, 0, a0, b0);
  for (int ks = 0; ks < nkf; ++ks) {
    issue(ks + S - 1);  // into stage (ks - 1) % S, last read before the previous barrier
    frag(ks % S, 1, a1, b1);
    mfma(a0, b0);
    frag((ks + 1) % S, 0, a0, b0);  // read-ahead (unused after the last step)
    mfma(a1, b1);
    // step ks + 2 landed (every step is waited for once the tail issues no more)
    wait_steps(ks + S - 1 < nkf ? S - 3 : 0, true);
    __syncthreads();
  }
  if (d % 32) {
    // ragged tail: one step through registers, columns at or past d are zero
    const int kt = nkf * 32;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (wave + WV * j < NI) {
        const int srow = 16 * (wave + WV * j) + (lane >> 2);
        const int c = (lane & 3) ^ lds_swz(srow);
        const u32x4_t v = (kt + c * 8 < d) ? *reinterpret_cast<const u32x4_t*>(src[j] + kt) : zero;
        *reinterpret_cast<u32x4_t*>(lds + 16 * (wave + WV * j) * 64 + lane * 16) = v;
      }
    }
    __syncthreads();
    frag(0, 0, a0, b0);
    frag(0, 1, a1, b1);
    mfma(a0, b0);
    mfma(a1, b1);
    __syncthreads();
  }

  if (PARTS > 1) {  // scores of this slice only, straight to logits (the choice is a second pass)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int col = e0 + es * 64 + cb * 32 + (lane & 31);
      const float b = (bias && col < N) ? bias[col] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = t0 + tb * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (col < N && row < T) logits_out[row * N + col] = acc[cb][r] + b;
      }
    }
    return;
  }
  // scores -> LDS tile [TM][NP + 1] (odd row stride); padded experts get -inf
  constexpr int LD = NP + 1;
  float* lt = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int col = es * 64 + cb * 32 + (lane & 31);
    const float b = (bias && col < N) ? bias[col] : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = tb * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      lt[row * LD + col] = col < N ? acc[cb][r] + b : -INFINITY;
    }
  }
  __syncthreads();
  tile_epilogue(lt, LD, TM, t0, T, N, n_groups, k, logits_out, idx, gate);
}

template <int TM, int NP, int S, int WV, int PARTS = 1>
static moge_status_t launch_route_dma(const moge_shape_t& s, int n_groups, int k, const void* x, const void* w,
                                      const float* bias, float* logits, int32_t* idx, float* gate,
                                      hipStream_t stream) {
  constexpr size_t ring = (size_t)S * (TM + NP) * 64;
  constexpr size_t tile = (size_t)TM * (NP + 1) * 4;
  constexpr size_t lds = ring > tile ? ring : tile;
  const void* kern = reinterpret_cast<const void*>(route_dma_kernel<TM, NP, S, WV, PARTS>);
  moge_status_t st = raise_dynamic_lds(kern, lds, "route_dma_kernel");
  if (st != MOGE_OK) return st;
  const int64_t grid = ((int64_t)s.T + TM - 1) / TM * PARTS;
  hipLaunchKernelGGL((route_dma_kernel<TM, NP, S, WV, PARTS>), dim3((unsigned)grid), dim3(64 * WV), lds, stream,
                     (int64_t)s.T, s.d, s.N, n_groups, k, static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(w), bias, logits, idx, gate);
  return check_launch("route_dma_kernel");
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
// Caller-supplied scores.  Lane-parallel choice: 64 tokens per workgroup, staged in
// LDS with an odd row stride.  Wide groups: one token per wave, 4 per workgroup
// (the choice is a chain of wave-wide reductions; many resident waves hide it).
constexpr int kSelTokens = 64;
constexpr int kSelTokensWide = 4;
template <bool LANES>
__global__ __launch_bounds__(256) void route_select_kernel(int64_t T, int N, int n_groups, int k,
                                                           const float* __restrict__ logits,
                                                           int32_t* __restrict__ idx, float* __restrict__ gate) {
  extern __shared__ float lt[];
  if (LANES) {  // [kSelTokens][N + 1]
    const int ld = N + 1;
    const int64_t t0 = (int64_t)blockIdx.x * kSelTokens;
    for (int i = threadIdx.x; i < kSelTokens * N; i += blockDim.x) {
      const int r = i / N, c = i - r * N;
      lt[r * ld + c] = (t0 + r < T) ? logits[(t0 + r) * N + c] : 0.f;
    }
    __syncthreads();
    select_tile(lt, ld, kSelTokens, t0, T, N, n_groups, k, idx, gate);
  } else {      // [kSelTokensWide][N]
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kSelTokensWide + wave;
    if (t >= T) return;  // wave-uniform; no barrier below
    float* row = lt + wave * N;
    for (int e = lane; e < N; e += 64) row[e] = logits[t * N + e];
    __builtin_amdgcn_wave_barrier();  // the row is written and read by this wave only (LDS is in order per wave)
    select_token(row, N, n_groups, k, t, idx, gate);
  }
}

// ----------------------------------------------------------------------------
// Caller-supplied scores, k <= 32 per group: one lane per token, 64 tokens per
// workgroup.  All four waves stage the 64 score rows in LDS (16-byte loads; odd row
// stride, so the row reads are conflict-free); then wave 0 chooses, each lane
// walking its own row: the maximum, the
// softmax denominator, and for every group a sorted register list of the KMAX best
// of that group (score desc, expert asc: a later equal score never displaces an
// earlier one), kept by a branch-free insertion network.  No cross-lane reduction
// at all, so a wave chooses for 64 tokens at once.
constexpr int kLaneTokens = 64;
template <int KMAX>
__global__ __launch_bounds__(256) void route_select_lane_kernel(int64_t T, int N, int n_groups, int k,
                                                               const float* __restrict__ logits,
                                                               int32_t* __restrict__ idx, float* __restrict__ gate) {
  extern __shared__ float lt[];  // [kLaneTokens][N + 1]
  const int ld = N + 1;
  const int64_t t0 = (int64_t)blockIdx.x * kLaneTokens;
  const int64_t nrows = (T - t0) < kLaneTokens ? (T - t0) : kLaneTokens;
  const float* src = logits + t0 * N;  // the tile's rows are contiguous
  const int total = (int)nrows * N;
  if ((N & 3) == 0) {  // 16-byte loads (rows start on 16-byte boundaries)
#pragma unroll 4
    for (int i = threadIdx.x * 4; i < total; i += 1024) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(src + i);
      const int r = i / N, c = i - r * N;  // c % 4 == 0 and c + 3 < N: the 4 values share a row
#pragma unroll
      for (int j = 0; j < 4; ++j) lt[r * ld + c + j] = v[j];
    }
  } else {
#pragma unroll 4
    for (int i = threadIdx.x; i < total; i += 256) {
      const int r = i / N;
      lt[r * ld + (i - r * N)] = src[i];
    }
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;  // wave 0 chooses
  const int lane = threadIdx.x;
  const int64_t t = t0 + lane;
  if (t >= T) return;
  const float* row = lt + lane * ld;
  // pass 1: the maximum; pass 2: the denominator (8 interleaved partial sums, then a tree)
  float mp[8] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY, -INFINITY, -INFINITY, -INFINITY, -INFINITY};
  int e8 = 0;
  for (; e8 + 8 <= N; e8 += 8)
#pragma unroll
    for (int j = 0; j < 8; ++j) mp[j] = fmaxf(mp[j], row[e8 + j]);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (e8 + j < N) mp[j] = fmaxf(mp[j], row[e8 + j]);
  const float m = fmaxf(fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3])), fmaxf(fmaxf(mp[4], mp[5]), fmaxf(mp[6], mp[7])));
  float zp[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (e8 = 0; e8 + 8 <= N; e8 += 8)
#pragma unroll
    for (int j = 0; j < 8; ++j) zp[j] += expf(row[e8 + j] - m);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (e8 + j < N) zp[j] += expf(row[e8 + j] - m);
  const float z = ((zp[0] + zp[1]) + (zp[2] + zp[3])) + ((zp[4] + zp[5]) + (zp[6] + zp[7]));
  // pass 3, per group: its KMAX best, in expert order (8 scores read ahead at a time)
  const int G = N / n_groups, K = n_groups * k;
  float bv[KMAX];
  int bi[KMAX];
  // Entries start as empty places (bi = -1) that any expert fills; experts arrive in
  // increasing id order, so a later equal key never displaces an earlier expert.
  auto insert = [&](float v, int e) {
    // position of v: below every entry >= v; entries below it move down one place
#pragma unroll
    for (int j = KMAX - 1; j > 0; --j) {
      const bool up = v > bv[j - 1] || bi[j - 1] < 0;  // v lands above j - 1: entry j - 1 moves to j
      const bool here = v > bv[j] || bi[j] < 0;
      bv[j] = up ? bv[j - 1] : (here ? v : bv[j]);
      bi[j] = up ? bi[j - 1] : (here ? e : bi[j]);
    }
    if (v > bv[0] || bi[0] < 0) {
      bv[0] = v;
      bi[0] = e;
    }
  };
  for (int g = 0; g < n_groups; ++g) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      bv[j] = -INFINITY;
      bi[j] = -1;
    }
    const int ge = (g + 1) * G;
    for (e8 = g * G; e8 + 8 <= ge; e8 += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = order_key(row[e8 + j]);
#pragma unroll
      for (int j = 0; j < 8; ++j) insert(v[j], e8 + j);
    }
    for (; e8 < ge; ++e8) insert(order_key(row[e8]), e8);
#pragma unroll
    for (int r = 0; r < KMAX; ++r) {
      if (r < k) {
        idx[t * K + g * k + r] = bi[r];
        gate[t * K + g * k + r] = expf(bv[r] - m) / z;
      }
    }
  }
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

  // the choice from stored scores (caller scores, or the split scores pass below)
  auto select = [&]() -> moge_status_t {
    if (k <= 32) {  // one lane per token
      const int64_t grid = ((int64_t)s.T + kLaneTokens - 1) / kLaneTokens;
      const size_t lds = sizeof(float) * kLaneTokens * (size_t)(s.N + 1);
#define MOGE_SEL(KM)                                                                                              \
  do {                                                                                                            \
    if (lds > 64 * 1024) {                                                                                        \
      st = raise_dynamic_lds(reinterpret_cast<const void*>(route_select_lane_kernel<KM>), lds,                     \
                             "route_select_lane_kernel");                                                         \
      if (st != MOGE_OK) return st;                                                                               \
    }                                                                                                             \
    hipLaunchKernelGGL(route_select_lane_kernel<KM>, dim3((unsigned)grid), dim3(256), lds, stream, (int64_t)s.T, \
                       s.N, n_groups, k, logits, idx, gate);                                                      \
  } while (0)
      if (k <= 1) MOGE_SEL(1);
      else if (k <= 2) MOGE_SEL(2);
      else if (k <= 4) MOGE_SEL(4);
      else if (k <= 8) MOGE_SEL(8);
      else if (k <= 16) MOGE_SEL(16);
      else MOGE_SEL(32);
#undef MOGE_SEL
      return check_launch("route_select_lane_kernel");
    }
    if (lane_parallel_choice(s.N, n_groups, k)) {
      const int64_t grid = ((int64_t)s.T + kSelTokens - 1) / kSelTokens;
      const size_t lds = sizeof(float) * kSelTokens * (size_t)(s.N + 1);
      if (lds > 64 * 1024) {
        st = raise_dynamic_lds(reinterpret_cast<const void*>(route_select_kernel<true>), lds, "route_select_kernel");
        if (st != MOGE_OK) return st;
      }
      hipLaunchKernelGGL(route_select_kernel<true>, dim3((unsigned)grid), dim3(256), lds, stream, (int64_t)s.T, s.N,
                         n_groups, k, logits, idx, gate);
    } else {
      const int64_t grid = ((int64_t)s.T + kSelTokensWide - 1) / kSelTokensWide;
      hipLaunchKernelGGL(route_select_kernel<false>, dim3((unsigned)grid), dim3(256),
                         sizeof(float) * kSelTokensWide * (size_t)s.N, stream, (int64_t)s.T, s.N, n_groups, k, logits,
                         idx, gate);
    }
    return check_launch("route_select_kernel");
  };

  if (!x) {
    st = select();
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
      st = check_launch("route_mfma_splitk_kernel");
    } else if (few && s.N <= 128) {
      hipLaunchKernelGGL(route_mfma_splitk_kernel<2>, dim3((unsigned)(((int64_t)s.T + 31) / 32)), dim3(256), 0,
                         stream, (int64_t)s.T, s.d, s.N, n_groups, k, static_cast<const uint16_t*>(x),
                         static_cast<const uint16_t*>(w_router), bias, logits, idx, gate);
      st = check_launch("route_mfma_splitk_kernel");
    } else if (s.N <= 64) {
      st = launch_route_dma<128, 64, 6, 4>(s, n_groups, k, x, w_router, bias, logits, idx, gate, stream);
    } else if (s.N <= 128) {
      st = launch_route_dma<64, 128, 6, 4>(s, n_groups, k, x, w_router, bias, logits, idx, gate, stream);
    } else if (logits) {  // N > 128 with the scores stored: the sliced scores pass, then the choice
      st = launch_route_dma<64, 128, 8, 4, 2>(s, n_groups, k, x, w_router, bias, logits, idx, gate, stream);
      if (st == MOGE_OK) st = select();
    } else {
      st = launch_route_dma<32, 256, 7, 4>(s, n_groups, k, x, w_router, bias, logits, idx, gate, stream);
    }
  }
  return st == MOGE_OK ? ok() : st;
}
