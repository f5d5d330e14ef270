// moge_route / moge_route_pair: router scores -> softmax over all N experts -> top-K'
// inside each of the M expert groups (MoGE), and/or top-K over all experts (the
// conventional router the pages compare MoGE with), from one pass over x.
//
// Method: Pangu Pro MoE, lsdiaocha.cn summary, section 1 (architecture): the N
// experts are split evenly into M groups, one per device; a token's scores go
// through a softmax over all experts and then the K' = K/M best experts of every
// group are kept, which puts exactly K' of the token's assignments on each device.
//
// gfx950 design
//   * bf16 scores, N <= 128: x [T][d] is streamed from HBM once.  A workgroup owns TM
//     tokens x NP experts (128 x 64 with 8 waves of one 32 x 32 block each, or 64 x 128
//     with 4 waves of 32 x 64), accumulated with v_mfma_f32_32x32x16_bf16 (float32).  Token rows
//     and router rows go from global memory straight into a 3-stage LDS ring with
//     direct-to-LDS loads of whole 128-byte lines, two 64-element steps ahead.  With fewer token tiles than
//     CUs the same kernel runs in slices of the hidden dimension (workgroup b: slice
//     b % S of token tile b / S) and writes partial sums instead of choosing.
//   * bf16 scores, 128 < N <= 256: split over the hidden dimension too, with a
//     128-token x 256-expert tile (S up to 4 for many tokens, up to 32 for few);
//     workgroup b runs on XCD b % 8, so an XCD only ever reads its slices of the router
//     matrix, which stay in its L2, and x is read from HBM exactly once.
//   * Slice partial sums go to the workspace; a second kernel adds them in slice order
//     (deterministic), adds the bias and chooses.
//   * The choice (one epilogue for every kernel): the score tile sits in LDS; lane
//     (token, group) keeps its group's best experts in a sorted register list; the
//     token's softmax max and sum are butterflies over its lanes; MoGE takes the first
//     K' of every list, the global top-K merges the lists head by head -- both routers
//     from the same tile, so the comparator needs no stored scores.  Shapes past the
//     lists' limits use one lane per (token, group) rank rounds or one wave per token.
//   * float32 shapes use a vector-ALU scores kernel with the same epilogue.
#include <math.h>

#include <type_traits>

#include "moge_internal.hpp"

namespace moge {

// The order the choice sorts by: the score itself, except that a NaN ranks as -inf
// (ties, -inf ones included, go to the lower expert id).  The pages define the choice
// on finite scores only; with this key every group still yields exactly k distinct
// experts of its own, whatever the scores (moge_check_finite reports non-finite ones).
__device__ __forceinline__ float order_key(float v) { return v == v ? v : -INFINITY; }

// The bf16 routers stage 64-element steps of every token row and router row: 128-byte LDS
// rows, whose 16-byte chunk c lives in slot c ^ route_swz(row).  Rows r and r + 2 share a
// bank line, so this swizzle puts the 16 rows that one 16-byte fragment read touches per
// clock on all 64 banks.
constexpr int kRouteBK = 64;
constexpr int kRouteRowB = kRouteBK * 2;
__device__ __forceinline__ int route_swz(int r) { return (r >> 1) & 7; }

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


// Butterfly partner of a lane at distance `off` (1, 2, 4, ...) inside its group of 2 off lanes,
// for the lane-parallel choices' reductions over a token's lanes.  Up to 16 lanes the partner
// comes through DPP (quad permutations, then the half-row and row mirrors: the pairing differs
// from lane ^ off but, applied in this order, every lane ends with its group's result), beyond
// that through the cross-lane permute.
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int partner_i(int v, int off) {
  switch (off) {
    case 1: return dpp_mov<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    case 2: return dpp_mov<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    case 4: return dpp_mov<0x141>(v);  // row_half_mirror
    case 8: return dpp_mov<0x140>(v);  // row_mirror
    default: return __shfl_xor(v, off, 64);
  }
}
__device__ __forceinline__ float partner_f(float v, int off) {
  return __builtin_bit_cast(float, partner_i(__builtin_bit_cast(int, v), off));
}

// Length of the sorted per-group list that choose_lanes keeps (a power of two <= 32), or 0
// when the lanes cannot take the shape: the MoGE choice needs the k best of a group, the
// global top-K (K = M k) at most min(G, K) of one group.
__host__ __device__ __forceinline__ int lane_list_len(int N, int M, int k, bool global) {
  const int G = N / M;
  const int need = global ? (G < M * k ? G : M * k) : k;
  if (M > 64 || need > 32 || G * need > 8192) return 0;
  int L = 1;
  while (L < need) L <<= 1;
  return L;
}

// Both routers from one LDS score tile [rows][ld].  Lane (tl, g) of a wave owns group g
// of token tl: a token's Mp lanes (M rounded up to a power of two) are adjacent, so a
// wave pass covers 64 / Mp tokens.  The lane keeps the KMAX best experts of its group,
// best first (score descending, expert id ascending; a branch-free insertion network
// over the scores in id order: a later equal score never displaces an earlier one, and
// empty places take any expert).  The token's softmax maximum and denominator over all
// N scores are butterflies over its lanes.
//   MoGE  (idx != NULL):  slot g*k + r <- the group's r-th best, r < k;
//   global (gidx != NULL): K = M*k rounds; each takes the best head among the token's
//         lists (higher score, then lower id: ids grow with the group) and pops it, so
//         slot r gets the expert of global rank r.  Round r's result is kept by lane
//         r mod Mp, so the gates are computed once per slot and a token's slots leave
//         as one contiguous store.
// Gates are the softmax probabilities over all N experts, e^(l - max) / sum, with the
// hardware exp2 and reciprocal (a few float32 ulps).
template <int KMAX, int MPC>  // MPC: the lanes per token when known at compile time, else 0
__device__ __forceinline__ void choose_lanes(const float* __restrict__ lt, int ld, int rows, int64_t t0, int64_t T,
                                             int N, int M, int k, int32_t* __restrict__ idx,
                                             float* __restrict__ gate, int32_t* __restrict__ gidx,
                                             float* __restrict__ ggate) {
  constexpr float kLog2e = 1.4426950408889634f;
  const int G = N / M, K = M * k;
  int Mp = 1;
  while (Mp < M) Mp <<= 1;
  if constexpr (MPC > 0) Mp = MPC;
  const int tpp = 64 / Mp;  // tokens per wave pass
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int g = lane & (Mp - 1), tl = lane / Mp;
  for (int r0 = wave * tpp; r0 < rows; r0 += nw * tpp) {  // wave-uniform
    const int r = r0 + tl;
    const bool tok = r < rows && t0 + r < T;
    const bool own = tok && g < M;
    const float* v = lt + (int64_t)(own ? r : 0) * ld + (own ? g * G : 0);
    const int n = own ? G : 0;
    float m = -INFINITY;
    for (int i = 0; i < n; ++i) m = fmaxf(m, v[i]);
    for (int off = 1; off < Mp; off <<= 1) m = fmaxf(m, partner_f(m, off));
    const float ml = m * kLog2e;
    float z = 0.f;
    for (int i = 0; i < n; ++i) z += __builtin_amdgcn_exp2f(__builtin_fmaf(v[i], kLog2e, -ml));
    for (int off = 1; off < Mp; off <<= 1) z += partner_f(z, off);
    const float rz = __builtin_amdgcn_rcpf(z);
    auto prob = [&](float l) { return __builtin_amdgcn_exp2f(__builtin_fmaf(l, kLog2e, -ml)) * rz; };
    float bv[KMAX];
    int bi[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      bv[j] = -INFINITY;
      bi[j] = -1;
    }
    for (int i = 0; i < n; ++i) {
      const float x = order_key(v[i]);
      const int e = g * G + i;
#pragma unroll
      for (int j = KMAX - 1; j > 0; --j) {
        const bool up = x > bv[j - 1] || bi[j - 1] < 0;  // x lands above j - 1: entry j - 1 moves to j
        const bool here = x > bv[j] || bi[j] < 0;
        bv[j] = up ? bv[j - 1] : (here ? x : bv[j]);
        bi[j] = up ? bi[j - 1] : (here ? e : bi[j]);
      }
      if (x > bv[0] || bi[0] < 0) {
        bv[0] = x;
        bi[0] = e;
      }
    }
    const int64_t t = t0 + r;
    if (idx && own) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j < k) {
          idx[t * K + g * k + j] = bi[j];
          gate[t * K + g * k + j] = prob(bv[j]);
        }
      }
    }
    if (gidx) {
      // round rk = j * Mp + q takes the best head among the token's lists (a lane whose head is
      // taken shifts its list up) and lane q keeps the result
      float rv[KMAX];  // K / Mp <= k <= KMAX rounds per lane
      int ri[KMAX];
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        rv[j] = -INFINITY;
        ri[j] = 0;
      }
      auto round = [&](float& wv, int& wi) {
        wv = bv[0];
        wi = own && bi[0] >= 0 ? bi[0] : 0x7FFFFFFF;  // no entry: loses every tie against a real one
        if (!own) wv = -INFINITY;
        for (int off = 1; off < Mp; off <<= 1) {
          const float ov = partner_f(wv, off);
          const int oi = partner_i(wi, off);
          const bool take = ov > wv || (ov == wv && oi < wi);
          wv = take ? ov : wv;
          wi = take ? oi : wi;
        }
        const bool pop = own && bi[0] == wi;
#pragma unroll
        for (int j = 0; j < KMAX - 1; ++j) {
          bv[j] = pop ? bv[j + 1] : bv[j];
          bi[j] = pop ? bi[j + 1] : bi[j];
        }
        bv[KMAX - 1] = pop ? -INFINITY : bv[KMAX - 1];
        bi[KMAX - 1] = pop ? -1 : bi[KMAX - 1];
      };
      if constexpr (MPC > 0) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
#pragma unroll
          for (int q = 0; q < MPC; ++q) {
            if (j * MPC + q < K) {
              float wv;
              int wi;
              round(wv, wi);
              if (g == q) {
                rv[j] = wv;
                ri[j] = wi;
              }
            }
          }
        }
      } else {
        for (int rk = 0; rk < K; ++rk) {  // K is the same for the whole wave
          float wv;
          int wi;
          round(wv, wi);
          const int slot = rk / Mp;
          if (g == (rk & (Mp - 1))) {
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
              if (j == slot) {
                rv[j] = wv;
                ri[j] = wi;
              }
            }
          }
        }
      }
      if (tok) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          const int rk = j * Mp + g;
          if (rk < K) {
            gidx[t * K + rk] = ri[j];
            ggate[t * K + rk] = prob(rv[j]);
          }
        }
      }
    }
  }
}

// Groups of exactly 8 experts, at most 8 groups (64 experts in 8 groups: the Pangu Pro shape).  Lane (tl, g)
// holds its group's 8 scores in registers and sorts them completely with a 19-comparator
// network (Knuth's for 8 inputs), comparing (score descending, expert id ascending): ids are
// distinct, so the order is total and the sorted list unique.  The MoGE choice is its first
// k entries; the global top-K merges the token's sorted lists head by head as choose_lanes
// does, a lane shifting its list up when its head is taken.  Same results as choose_lanes.
constexpr int kListG8 = 64;  // the host's code for this form
template <int MP>  // lanes per token: M rounded up to a power of two
__device__ __forceinline__ void choose_g8(const float* __restrict__ lt, int ld, int rows, int64_t t0, int64_t T,
                                          int M, int k, int32_t* __restrict__ idx, float* __restrict__ gate,
                                          int32_t* __restrict__ gidx, float* __restrict__ ggate) {
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr int tpp = 64 / MP;  // tokens per wave pass
  const int K = M * k;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int g = lane & (MP - 1), tl = lane / MP;
  for (int r0 = wave * tpp; r0 < rows; r0 += nw * tpp) {  // wave-uniform
    const int r = r0 + tl;
    const bool tok = r < rows && t0 + r < T;
    const bool own = tok && g < M;
    const float* v = lt + (int64_t)(own ? r : 0) * ld + (own ? g * 8 : 0);
    float key[8];
    int id[8];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = own ? v[i] : -INFINITY;
      m = fmaxf(m, x);
      key[i] = x;
    }
#pragma unroll
    for (int off = 1; off < MP; off <<= 1) m = fmaxf(m, partner_f(m, off));
    const float ml = m * kLog2e;
    float z = 0.f;
    if (own) {
#pragma unroll
      for (int i = 0; i < 8; ++i) z += __builtin_amdgcn_exp2f(__builtin_fmaf(key[i], kLog2e, -ml));
    }
#pragma unroll
    for (int off = 1; off < MP; off <<= 1) z += partner_f(z, off);
    const float rz = __builtin_amdgcn_rcpf(z);
    auto prob = [&](float l) { return __builtin_amdgcn_exp2f(__builtin_fmaf(l, kLog2e, -ml)) * rz; };
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      key[i] = order_key(key[i]);
      id[i] = own ? g * 8 + i : 0x7FFFFFFF;
    }
    const int64_t t = t0 + r;
    if (!gidx && k == 1) {  // MoGE alone with one expert per group: the group's best, no sort
      float bk = key[0];
      int bid = id[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) {  // ids ascend, so a later equal score never wins
        const bool take = key[i] > bk;
        bk = take ? key[i] : bk;
        bid = take ? id[i] : bid;
      }
      if (own) {
        idx[t * K + g] = bid;
        gate[t * K + g] = prob(bk);
      }
      continue;
    }
    auto ce = [&](int a, int b) {  // a before b: higher score, then lower id
      const bool keep = key[a] > key[b] || (key[a] == key[b] && id[a] < id[b]);
      const float ka = key[a], kb = key[b];
      const int ia = id[a], ib = id[b];
      key[a] = keep ? ka : kb;
      key[b] = keep ? kb : ka;
      id[a] = keep ? ia : ib;
      id[b] = keep ? ib : ia;
    };
    ce(0, 2); ce(1, 3); ce(4, 6); ce(5, 7);
    ce(0, 4); ce(1, 5); ce(2, 6); ce(3, 7);
    ce(0, 1); ce(2, 3); ce(4, 5); ce(6, 7);
    ce(2, 4); ce(3, 5);
    ce(1, 4); ce(3, 6);
    ce(1, 2); ce(3, 4); ce(5, 6);
    if (idx && own) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < k) {
          idx[t * K + g * k + j] = id[j];
          gate[t * K + g * k + j] = prob(key[j]);
        }
      }
    }
    if (gidx) {
      // round rk = j * MP + q takes the best head among the token's lists; lane q keeps it
      float rv[8];
      int ri[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        rv[j] = -INFINITY;
        ri[j] = 0;
#pragma unroll
        for (int q = 0; q < MP; ++q) {
          if (j * MP + q < K) {  // K = M k <= 8 MP: at most 8 rounds per lane
            float wv = key[0];
            int wi = id[0];  // an exhausted or foreign lane offers (-inf, INT_MAX): it loses every tie
#pragma unroll
            for (int off = 1; off < MP; off <<= 1) {
              const float ov = partner_f(wv, off);
              const int oi = partner_i(wi, off);
              const bool take = ov > wv || (ov == wv && oi < wi);
              wv = take ? ov : wv;
              wi = take ? oi : wi;
            }
            const bool pop = id[0] == wi;  // this lane's head was taken: the list moves up
#pragma unroll
            for (int i = 0; i < 7; ++i) {
              key[i] = pop ? key[i + 1] : key[i];
              id[i] = pop ? id[i + 1] : id[i];
            }
            key[7] = pop ? -INFINITY : key[7];
            id[7] = pop ? 0x7FFFFFFF : id[7];
            if (g == q) {
              rv[j] = wv;
              ri[j] = wi;
            }
          }
        }
      }
      if (tok) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int rk = j * MP + g;
          if (rk < K) {
            gidx[t * K + rk] = ri[j];
            ggate[t * K + rk] = prob(rv[j]);
          }
        }
      }
    }
  }
}

// At most 64 experts, one wave per token, lane e owning expert e: every choice is the rank
// definition itself, counted.  rank_key packs (score, id) into one 64-bit integer ordered as
// the choice orders experts -- higher score first, then lower id; NaN ranks as -inf, -0
// equals +0 -- so rank(e) = #{e' : key(e') > key(e)}, over the token for the global top-K
// (slot rank) and over e's group for MoGE (slot g*k + rank).  The keys go through a
// 64-entry LDS row per wave.  Unique ranks, so the same choices as the lists, and the
// gates in the lists' arithmetic: the softmax denominator sums each group's exponentials
// in id order, then the groups' sums pairwise (g with g ^ 1, then g ^ 2, ...), so a gate
// is bit-identical to the one the lists give from the same scores.  For few tokens per
// workgroup (the reduction after a split), where the lists' serial rounds would keep all
// but one wave of the workgroup idle.
constexpr int kListRank = 65;  // the host's code for this form
__device__ __forceinline__ uint64_t rank_key(float v, int e) {
  uint32_t u = __builtin_bit_cast(uint32_t, order_key(v));
  if (u == 0x80000000u) u = 0u;                    // -0 -> +0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // float order -> unsigned order
  return ((uint64_t)u << 32) | (uint32_t)(63 - e); // equal scores: the lower id is the larger key
}
__device__ __forceinline__ void choose_rank64(const float* __restrict__ lt, int ld, int rows, int64_t t0, int64_t T,
                                              int N, int M, int k, int32_t* __restrict__ idx,
                                              float* __restrict__ gate, int32_t* __restrict__ gidx,
                                              float* __restrict__ ggate, uint64_t* __restrict__ keys) {
  constexpr float kLog2e = 1.4426950408889634f;
  const int G = N / M, K = M * k;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const bool own = lane < N;
  const int g = own ? lane / G : 0;
  const int j = lane - g * G;  // the lane's place in its group (own lanes)
  int Mp = 1;
  while (Mp < M) Mp <<= 1;
  uint64_t* kw = keys + wave * 64;
  for (int r = wave; r < rows; r += nw) {  // wave-uniform
    const int64_t t = t0 + r;
    if (t >= T) break;
    const float* row = lt + r * ld;
    const float v = own ? row[lane] : -INFINITY;
    float m = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, partner_f(m, off));
    const float ml = m * kLog2e;
    float z = 0.f;
    if (own) {
      for (int i = 0; i < G; ++i) z += __builtin_amdgcn_exp2f(__builtin_fmaf(row[g * G + i], kLog2e, -ml));
    }
    for (int off = 1; off < Mp; off <<= 1) {  // every lane takes part in the exchange
      const int pg = g ^ off;
      const float o = __shfl(z, (pg < M ? pg : g) * G + j, 64);
      z += pg < M ? o : 0.f;  // a group past M adds nothing, as its empty lane does in the lists
    }
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(order_key(v), kLog2e, -ml)) * __builtin_amdgcn_rcpf(z);
    const uint64_t key = rank_key(v, lane);
    kw[lane] = key;
    // the row's keys are read by every lane of this wave only: LDS runs one wave's
    // accesses in order, the fences keep the compiler from moving them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (idx) {
      const int base = g * G;
      int rank = 0;
      for (int i = 0; i < G; ++i) rank += kw[base + i] > key ? 1 : 0;
      if (own && rank < k) {
        idx[t * K + g * k + rank] = lane;
        gate[t * K + g * k + rank] = p;
      }
    }
    if (gidx) {
      int rank = 0;
#pragma unroll 8
      for (int e = 0; e < N; ++e) rank += kw[e] > key ? 1 : 0;
      if (own && rank < K) {
        gidx[t * K + rank] = lane;
        ggate[t * K + rank] = p;
      }
    }
    // every lane's reads of this row come before the next row's writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// The choices of the older per-mode forms, for shapes past the lists' limits: lane-parallel
// rank rounds per (token, group) or one wave per token.
__device__ __forceinline__ void choose_fallback(const float* __restrict__ lt, int ld, int rows, int64_t t0, int64_t T,
                                                int N, int n_groups, int k, int32_t* __restrict__ idx,
                                                float* __restrict__ gate) {
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

// Writes the LDS score tile [rows][ld] to logits_out (if any) and makes the choices: MoGE
// into idx/gate when idx is set, the global top-K into gidx/ggate when gidx is set.  KL is
// lane_list_len of the call (the host picks the kernel instance): the lists' length, or 0
// for the fallback forms.  (all threads of the block call it)
// The scores go out with the non-temporal hint: every tile writes them at the same time
// at the end of the kernel, and streamed past the L2 they no longer wait there for the
// kernel's final write-back (the route kernel at 65536 tokens x 4096 x 64 experts was 4%
// faster).
__device__ __forceinline__ void store_scores(const float* __restrict__ lt, int ld, int rows, int64_t t0, int64_t T,
                                             int N, float* __restrict__ logits_out) {
  if (!logits_out) return;
  for (int i = threadIdx.x; i < rows * N; i += blockDim.x) {
    const int r = i / N, c = i - r * N;
    if (t0 + r < T) __builtin_nontemporal_store(lt[r * ld + c], logits_out + (t0 + r) * N + c);
  }
}

template <int KL>
__device__ __forceinline__ void tile_epilogue(const float* __restrict__ lt, int ld, int rows, int64_t t0, int64_t T,
                                              int N, int M, int k, float* __restrict__ logits_out,
                                              int32_t* __restrict__ idx, float* __restrict__ gate,
                                              int32_t* __restrict__ gidx, float* __restrict__ ggate) {
  store_scores(lt, ld, rows, t0, T, N, logits_out);
  if constexpr (KL == kListG8) {
    if (M <= 1) choose_g8<1>(lt, ld, rows, t0, T, M, k, idx, gate, gidx, ggate);
    else if (M <= 2) choose_g8<2>(lt, ld, rows, t0, T, M, k, idx, gate, gidx, ggate);
    else if (M <= 4) choose_g8<4>(lt, ld, rows, t0, T, M, k, idx, gate, gidx, ggate);
    else choose_g8<8>(lt, ld, rows, t0, T, M, k, idx, gate, gidx, ggate);
  } else if constexpr (KL > 0) {
    if (M == 8) choose_lanes<KL, 8>(lt, ld, rows, t0, T, N, M, k, idx, gate, gidx, ggate);
    else choose_lanes<KL, 0>(lt, ld, rows, t0, T, N, M, k, idx, gate, gidx, ggate);
  } else {
    if (idx) choose_fallback(lt, ld, rows, t0, T, N, M, k, idx, gate);
    if (gidx) choose_fallback(lt, ld, rows, t0, T, N, 1, M * k, gidx, ggate);
  }
}

// Calls f(std::integral_constant<int, KL>{}) with KL = the list length the host picked
// (one kernel instance per length).
template <typename Fn>
static moge_status_t with_list_len(int kl, Fn&& f) {
  switch (kl) {
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 4: return f(std::integral_constant<int, 4>{});
    case 8: return f(std::integral_constant<int, 8>{});
    case 16: return f(std::integral_constant<int, 16>{});
    case 32: return f(std::integral_constant<int, 32>{});
    case kListG8: return f(std::integral_constant<int, kListG8>{});
    default: return f(std::integral_constant<int, 0>{});
  }
}

// ----------------------------------------------------------------------------
// bf16 scores, many tokens, N <= 128.  A workgroup of WV waves owns TM tokens x NP experts
// (NP = N rounded up to 64 or 128, TM = 8192 / NP), every wave one 32-token x 32 CB-expert
// block of CB 32x32 accumulators: 8 waves of one block for 64 experts (twice the waves
// to interleave the choice epilogue), 4 waves of two blocks for 128.  A step is 64
// elements: every token row and router row contributes 128 bytes, one whole cache line
// (the L2 delivers whole lines at about 1.4 times the rate of half lines), moved from
// global memory straight into an S-stage LDS ring (global_load_lds_dwordx4, 8 rows of
// 128 bytes per instruction, chunks XOR-swizzled by (row / 2) % 8), S - 1 steps ahead, so
// x streams from HBM with two steps of loads in flight per workgroup and no staging
// registers; x is read exactly once.  One barrier per step.  The epilogue keeps the
// TM x NP score tile in LDS for the softmax and the choices.
template <int TM, int NP, int S, int WV, int CB, int KL>
__global__ __launch_bounds__(64 * WV) void route_dma_kernel(int64_t T, int d, int N, int n_groups, int k,
                                                        const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ w,
                                                        const float* __restrict__ bias,
                                                        float* __restrict__ logits_out, int32_t* __restrict__ idx,
                                                        float* __restrict__ gate, int32_t* __restrict__ gidx,
                                                        float* __restrict__ ggate, int nsl, float* __restrict__ part) {
  constexpr int RB = kRouteRowB;
  constexpr int ROWS = TM + NP;      // stage rows of 128 bytes: tokens, then experts
  constexpr int NI = ROWS / 8;       // load instructions per step (8 rows each)
  constexpr int NJ = (NI + WV - 1) / WV;  // per wave, at most
  constexpr int CH = NJ;                  // loads per step of waves 0 .. NI%WV - 1 (all when NI%WV == 0)
  constexpr int CL = NI / WV;             // loads per step of the other waves
  constexpr int STAGE = ROWS * RB;
  constexpr int TB = TM / 32;        // token blocks; wave = token block + TB * expert slice
  static_assert(TM * NP == 1024 * CB * WV && S >= 3 && ROWS % 8 == 0, "route tile: one 32 x (32 CB) block per wave");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tb = wave % TB, es = wave / TB;
  // nsl > 1: the slice mode -- workgroup b computes slice b % nsl of the reduction (steps
  // k0 .. k1 - 1 of d / 64) for token tile b / nsl and writes the float32 partial sums to
  // part[slice][t][e] (the reduction kernel adds them and chooses); nsl == 1: one pass
  const int slice = (int)(blockIdx.x % nsl);
  const int64_t t0 = (int64_t)(blockIdx.x / nsl) * TM;
  const int nkf = d / kRouteBK;                  // full steps; a ragged tail follows the loop
  const int k0 = (int)((int64_t)nkf * slice / nsl);
  const int nks = (int)((int64_t)nkf * (slice + 1) / nsl) - k0;  // this workgroup's steps
  // token tiles start at different steps (and wrap around), so the workgroups do not all
  // read the same column range of their rows at once (router -11% on 65536 tokens x 4096
  // when it was measured).  The order of the float32 accumulation over k then depends on
  // the tile; scores stay within the tolerance.
  const int krot = nks > 0 ? (int)(((t0 / TM) * 37) % nks) : 0;
  const bool many = (NI % WV == 0) || wave < (NI % WV);  // this wave issues CH loads per step, else CL

  // load j of this wave moves stage rows 8 i .. 8 i + 7 with i = wave + WV j; lane l brings
  // physical chunk l % 8 of row 8 i + l / 8
  const uint16_t* src[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int srow = 8 * (wave + WV * j) + (lane >> 3);
    const int c = (lane & 7) ^ route_swz(srow);
    if (srow < TM) {
      int64_t t = t0 + srow;
      if (t > T - 1) t = T - 1;
      src[j] = x + t * d + c * 8;
    } else {
      int e = srow - TM;
      if (e > N - 1) e = N - 1;
      src[j] = w + (int64_t)e * d + c * 8;
    }
  }
  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int ks) {
    if (ks >= nks) return;
    const uint32_t st = lds0 + (uint32_t)((ks % S) * STAGE);
    const int kk = k0 + (ks + krot < nks ? ks + krot : ks + krot - nks);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (wave + WV * j < NI) dma_16x64(src[j] + kk * kRouteBK, st + (uint32_t)((wave + WV * j) * 1024));
  };

  const int kc = lane >> 5;
  const int arow = tb * 32 + (lane & 31);
  int brow[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) brow[cb] = TM + es * 32 * CB + cb * 32 + (lane & 31);
  // fragments of 16-element sub-step kk (0 .. 3) of the step in `stage`
  auto frag = [&](int stage, int kk, bf16x8_t& a, bf16x8_t (&b)[CB]) {
    const char* st = lds + stage * STAGE;
    const int c = kk * 2 + kc;
    a = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(st + arow * RB + ((c ^ route_swz(arow)) << 4)));
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      b[cb] = __builtin_bit_cast(bf16x8_t,
                                 *reinterpret_cast<const u32x4_t*>(st + brow[cb] * RB + ((c ^ route_swz(brow[cb])) << 4)));
  };
  f32x16_t acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
  auto mfma = [&](const bf16x8_t& a, const bf16x8_t (&b)[CB]) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[cb], acc[cb], 0, 0, 0);
  };
  auto step = [&](int stage) {
    bf16x8_t a0, b0[CB], a1, b1[CB];
    frag(stage, 0, a0, b0);
    frag(stage, 1, a1, b1);
    mfma(a0, b0);
    frag(stage, 2, a0, b0);
    mfma(a1, b1);
    frag(stage, 3, a1, b1);
    mfma(a0, b0);
    mfma(a1, b1);
  };

#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s);
  for (int ks = 0; ks < nks; ++ks) {
    // step ks landed for every wave (this wave's later steps, S - 2 of them, may be in flight)
    if (ks + S - 2 < nks) {
      if (many) __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 2) * CH));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 2) * CL));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    __syncthreads();
    issue(ks + S - 1);  // into stage (ks - 1) % S, whose reads all finished before the barrier
    step(ks % S);
  }
  __syncthreads();  // every wave is done with the ring (the tail and the score tile reuse it)
  if ((d % kRouteBK) && slice == nsl - 1) {
    // ragged tail: one step through registers into stage 0, columns at or past d are zero
    const int kt = nkf * kRouteBK;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (wave + WV * j < NI) {
        const int srow = 8 * (wave + WV * j) + (lane >> 3);
        const int c = (lane & 7) ^ route_swz(srow);
        const u32x4_t v = (kt + c * 8 < d) ? *reinterpret_cast<const u32x4_t*>(src[j] + kt) : zero;
        *reinterpret_cast<u32x4_t*>(lds + (wave + WV * j) * 1024 + lane * 16) = v;
      }
    }
    __syncthreads();
    step(0);
    __syncthreads();
  }

  if (nsl > 1) {  // partial sums of this slice (no bias: the reduction adds it once)
    float* dst = part + (int64_t)slice * T * N;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int col = es * 32 * CB + cb * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = t0 + tb * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (col < N && row < T) dst[row * N + col] = acc[cb][r];
      }
    }
    return;
  }
  // scores -> LDS tile [TM][NP + 1] (odd row stride); padded experts get -inf
  constexpr int LD = NP + 1;
  float* lt = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int col = es * 32 * CB + cb * 32 + (lane & 31);
    const float b = (bias && col < N) ? bias[col] : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = tb * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      lt[row * LD + col] = col < N ? acc[cb][r] + b : -INFINITY;
    }
  }
  __syncthreads();
  tile_epilogue<KL>(lt, LD, TM, t0, T, N, n_groups, k, logits_out, idx, gate, gidx, ggate);
}

template <int TM, int NP, int S, int WV, int CB>
static moge_status_t launch_route_dma(const moge_shape_t& s, int kl, const void* x, const void* w, const float* bias,
                                      float* logits, int32_t* idx, float* gate, int32_t* gidx, float* ggate,
                                      int nsl, float* part, hipStream_t stream) {
  return with_list_len(kl, [&](auto klc) {
    constexpr int KL = decltype(klc)::value;
    constexpr size_t ring = (size_t)S * (TM + NP) * kRouteRowB;
    constexpr size_t tile = (size_t)TM * (NP + 1) * 4;
    constexpr size_t lds = ring > tile ? ring : tile;
    const void* kern = reinterpret_cast<const void*>(route_dma_kernel<TM, NP, S, WV, CB, KL>);
    moge_status_t st = raise_dynamic_lds(kern, lds, "route_dma_kernel");
    if (st != MOGE_OK) return st;
    const int64_t grid = ((int64_t)s.T + TM - 1) / TM * nsl;
    hipLaunchKernelGGL((route_dma_kernel<TM, NP, S, WV, CB, KL>), dim3((unsigned)grid), dim3(64 * WV), lds, stream,
                       (int64_t)s.T, s.d, s.N, s.M, s.k_per_group, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(w), bias, logits, idx, gate, gidx, ggate, nsl, part);
    return check_launch("route_dma_kernel");
  });
}

// ----------------------------------------------------------------------------
// bf16 scores split over the hidden dimension, 128 < N <= 256.
// Workgroup b computes slice b % S of the reduction (its steps k0 .. k1 - 1 of d / 64) for
// the 128-token x 256-expert tile b / S, and stores the float32 partial sums to
// part[slice][t][e].  8 waves; wave w owns tokens (w / 4) * 64 .. + 64 and experts
// (w % 4) * 64 .. + 64 as 2 x 2 accumulators of 32 x 32 (v_mfma_f32_32x32x16_bf16; experts
// past N repeat the last router row and are not stored).  A step is 64 elements: each of its
// 128 token rows and 256 router rows contributes 128 bytes, one whole cache line, which the
// L2 delivers at about 1.4 times the rate of the half lines a 32-element step takes (measured
// with the loads alone on this tile: 20.8 against 29.7 us at 8192 tokens x 7680).  The
// stage rows go straight into a 3-stage LDS ring (48 loads of 8 rows x 128 bytes per step,
// 6 per wave), two steps ahead, one barrier per step; the 16-byte chunks of a row are
// XOR-swizzled by (row / 2) % 8, so the 16 rows a fragment read touches per clock cover all
// 64 banks.  Workgroup b runs on XCD b % 8 and S is a power of two, so an XCD reads only
// its own slices of the router matrix (at most 983 KB of a 256 x 7680 matrix at S = 4),
// which stay in its L2, while x streams from HBM once.  The last slice also takes the
// ragged tail of d (d % 64 columns, a multiple of 8) through registers.
constexpr int kPartTM = 128, kPartNP = 256, kPartStages = 3;
__host__ __forceinline__ int route_slices(int64_t T, int d);
__global__ __launch_bounds__(512) void route_part_kernel(int64_t T, int d, int N, int S,
                                                         const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ w,
                                                         float* __restrict__ part) {
  constexpr int TM = kPartTM, NP = kPartNP, SG = kPartStages, RB = kRouteRowB;
  constexpr int ROWS = TM + NP;           // 384 stage rows of 128 bytes
  constexpr int STAGE = ROWS * RB;        // 48 KiB
  constexpr int PW = ROWS / 8 / 8;        // loads per wave per step (8 rows each): 6
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave >> 2, wc = wave & 3;
  const int slice = (int)(blockIdx.x % S);
  const int64_t t0 = (int64_t)(blockIdx.x / S) * TM;
  const int nkf = d / kRouteBK;
  const int k0 = (int)((int64_t)nkf * slice / S), k1 = (int)((int64_t)nkf * (slice + 1) / S);
  const int nks = k1 - k0;
  // token tiles start their slice at staggered steps (as the one-pass kernel does)
  const int krot = nks > 0 ? (int)(((t0 / TM) * 37) % nks) : 0;
  // load j of this wave moves stage rows 8 i .. 8 i + 7, i = wave + 8 j (j = 0, 1: token
  // rows; j = 2 .. 5: router rows); lane l brings physical chunk l % 8 of row 8 i + l / 8
  const uint16_t* src[PW];
#pragma unroll
  for (int j = 0; j < PW; ++j) {
    const int srow = 8 * (wave + 8 * j) + (lane >> 3);
    const int c = (lane & 7) ^ route_swz(srow);
    if (srow < TM) {
      int64_t t = t0 + srow;
      if (t > T - 1) t = T - 1;
      src[j] = x + t * d + c * 8;
    } else {
      int e = srow - TM;
      if (e > N - 1) e = N - 1;
      src[j] = w + (int64_t)e * d + c * 8;
    }
  }
  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int ks) {
    if (ks >= nks) return;
    const uint32_t st = lds0 + (uint32_t)((ks % SG) * STAGE);
    const int kr = ks + krot < nks ? ks + krot : ks + krot - nks;
    const int kk = k0 + kr;
#pragma unroll
    for (int j = 0; j < PW; ++j) dma_16x64(src[j] + kk * kRouteBK, st + (uint32_t)((wave + 8 * j) * 1024));
  };
  const int kc = lane >> 5;
  int arow[2], brow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    arow[i] = wr * 64 + i * 32 + (lane & 31);
    brow[i] = TM + wc * 64 + i * 32 + (lane & 31);
  }
  // fragments of 16-element sub-step kk (0 .. 3) of the step in `stage`
  auto frag = [&](int stage, int kk, bf16x8_t (&a)[2], bf16x8_t (&b)[2]) {
    const char* st = lds + stage * STAGE;
    const int c = kk * 2 + kc;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      a[i] = __builtin_bit_cast(bf16x8_t,
                                *reinterpret_cast<const u32x4_t*>(st + arow[i] * RB + ((c ^ route_swz(arow[i])) << 4)));
      b[i] = __builtin_bit_cast(bf16x8_t,
                                *reinterpret_cast<const u32x4_t*>(st + brow[i] * RB + ((c ^ route_swz(brow[i])) << 4)));
    }
  };
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  auto mfma = [&](const bf16x8_t (&a)[2], const bf16x8_t (&b)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  };
  auto step = [&](int stage) {
    bf16x8_t a0[2], b0[2], a1[2], b1[2];
    frag(stage, 0, a0, b0);
    frag(stage, 1, a1, b1);
    mfma(a0, b0);
    frag(stage, 2, a0, b0);
    mfma(a1, b1);
    frag(stage, 3, a1, b1);
    mfma(a0, b0);
    mfma(a1, b1);
  };
#pragma unroll
  for (int s = 0; s < SG - 1; ++s) issue(s);
  for (int ks = 0; ks < nks; ++ks) {
    // step ks landed (this wave's loads of step ks + 1 may still be in flight), for every wave
    if (ks + 1 < nks) __builtin_amdgcn_s_waitcnt(vmcnt_imm(PW));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    issue(ks + SG - 1);  // into stage (ks - 1) % SG, whose reads all finished before the barrier
    step(ks % SG);
  }
  if (slice == S - 1 && (d % kRouteBK)) {
    // ragged tail: one step through registers into stage 0, columns at or past d are zero
    __syncthreads();  // every wave's reads of the last step are done
    const int kt = nkf * kRouteBK;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < PW; ++j) {
      const int srow = 8 * (wave + 8 * j) + (lane >> 3);
      const int c = (lane & 7) ^ route_swz(srow);
      const u32x4_t v = (kt + c * 8 < d) ? *reinterpret_cast<const u32x4_t*>(src[j] + kt) : zero;
      *reinterpret_cast<u32x4_t*>(lds + (wave + 8 * j) * 1024 + lane * 16) = v;
    }
    __syncthreads();
    step(0);
  }
  float* dst = part + (int64_t)slice * T * N;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = wc * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = t0 + wr * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (col < N && row < T) dst[row * N + col] = acc[i][j][r];
      }
    }
}

// Slices per token tile for the split kernel: enough that the token tiles times the slices
// fill the 256 CUs, at most 4 for many tokens (each XCD then holds whole slices of the router
// matrix) and, for few tokens, up to 32 while every slice keeps at least 2 steps of 64.
__host__ __forceinline__ int route_slices(int64_t T, int d) {
  const int64_t tiles = (T + kPartTM - 1) / kPartTM;
  const int nkf = d / kRouteBK;
  const int cap = tiles >= 16 ? 4 : 32;
  int S = 1;
  while (S < cap && tiles * S < 256 && nkf / (2 * S) >= 1) S <<= 1;
  return S;
}

// How bf16 scores from x are computed: kind 0 one pass (the one-pass kernel, or its
// token tiles fill the CUs); kind 1 the one-pass kernel in slices of d plus the reduction
// (N <= 128 with fewer token tiles than CUs); kind 2 the 256-expert split kernel plus the
// reduction (N > 128).
struct RoutePlan {
  int kind;
  int S;  // slices of d (1 for one pass)
};
__host__ __forceinline__ int dma_tile_tokens(int N) { return N <= 64 ? 128 : 64; }
// Slices for the one-pass kernel's slice mode: until the token tiles times the slices give
// two 72 KiB workgroups per CU, at most 32, every slice keeping at least 2 steps of 64.
__host__ __forceinline__ int dma_slices(int64_t T, int d, int N) {
  const int64_t tiles = (T + dma_tile_tokens(N) - 1) / dma_tile_tokens(N);
  const int nkf = d / kRouteBK;
  int S = 1;
  while (S < 32 && tiles * S < 512 && nkf / (2 * S) >= 1) S <<= 1;
  return S;
}
__host__ __forceinline__ RoutePlan route_plan(const moge_shape_t& s) {
  if (s.dtype != MOGE_BF16) return RoutePlan{0, 1};
  if (s.N > 128) return RoutePlan{2, route_slices(s.T, s.d)};
  const int64_t tiles = ((int64_t)s.T + dma_tile_tokens(s.N) - 1) / dma_tile_tokens(s.N);
  if (tiles >= 256) return RoutePlan{0, 1};
  const int S = dma_slices(s.T, s.d, s.N);
  return S > 1 ? RoutePlan{1, S} : RoutePlan{0, 1};
}

// The split kernel's partial sums -> scores -> the choices.  TPW tokens per workgroup (many
// workgroups, so every CU has several tiles' loads in flight): the S slices of each score
// are added in slice order (bit-identical results run to run), plus the bias, into an LDS
// tile [TPW][N + 1]; then the choice: the rank count (KL = kListRank, at most 64 experts: the
// 4 waves take the tokens in turn) or the common epilogue.  TPW = 8, or 2 for the rank count
// on small batches, whose few workgroups otherwise wait on their loads one after another.
constexpr int kReduceTokens = 8;
constexpr int kReduceTokensSmall = 2;
constexpr int64_t kReduceSmallT = 2048;  // batches up to this many tokens take kReduceTokensSmall
template <int KL, int TPW>
__global__ __launch_bounds__(256) void route_reduce_kernel(int64_t T, int N, int M, int k, int S,
                                                           const float* __restrict__ part,
                                                           const float* __restrict__ bias,
                                                           float* __restrict__ logits_out, int32_t* __restrict__ idx,
                                                           float* __restrict__ gate, int32_t* __restrict__ gidx,
                                                           float* __restrict__ ggate) {
  constexpr int tpw = TPW;
  constexpr int PU = 16;  // slices of one chunk in flight together
  __shared__ float lt[tpw * (kMaxExperts + 1)];
  const int ld = N + 1;
  const int64_t t0 = (int64_t)blockIdx.x * tpw;
  const int64_t nrows = (T - t0) < tpw ? (T - t0) : tpw;
  const int total = (int)nrows * N;
  const int64_t plane = T * N;
  const float* src = part + t0 * N;  // the tile's rows are contiguous in every slice
  if ((N & 3) == 0) {
    // 16-byte chunks, one per thread at a time, with up to 16 of its slices loaded together
    for (int i = threadIdx.x * 4; i < total; i += 256 * 4) {
      f32x4_t a = {0.f, 0.f, 0.f, 0.f};
      for (int p0 = 0; p0 < S; p0 += PU) {
        f32x4_t v[PU];
#pragma unroll
        for (int p = 0; p < PU; ++p)
          v[p] = p0 + p < S ? *reinterpret_cast<const f32x4_t*>(src + (p0 + p) * plane + i) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < PU; ++p)
          if (p0 + p < S) a = p0 + p == 0 ? v[p] : a + v[p];
      }
      const int r = i / N, c = i - r * N;  // c % 4 == 0: the 4 values share a row
#pragma unroll
      for (int q = 0; q < 4; ++q) lt[r * ld + c + q] = a[q] + (bias ? bias[c + q] : 0.f);
    }
  } else {
    for (int i = threadIdx.x; i < total; i += 256) {
      float a = src[i];
      for (int p = 1; p < S; ++p) a += src[p * plane + i];
      const int r = i / N, c = i - r * N;
      lt[r * ld + c] = a + (bias ? bias[c] : 0.f);
    }
  }
  __syncthreads();
  if constexpr (KL == kListRank) {
    __shared__ uint64_t keys[4 * 64];  // one row per wave (256 threads)
    store_scores(lt, ld, (int)nrows, t0, T, N, logits_out);
    choose_rank64(lt, ld, (int)nrows, t0, T, N, M, k, idx, gate, gidx, ggate, keys);
  } else {
    tile_epilogue<KL>(lt, ld, (int)nrows, t0, T, N, M, k, logits_out, idx, gate, gidx, ggate);
  }
}


// ----------------------------------------------------------------------------
// float32 scores on the vector ALUs (small shapes).  16 tokens per workgroup.
constexpr int kF32Tokens = 16;
template <int KL>
__global__ __launch_bounds__(256) void route_f32_kernel(int64_t T, int d, int N, int n_groups, int k,
                                                        const float* __restrict__ x, const float* __restrict__ w,
                                                        const float* __restrict__ bias,
                                                        float* __restrict__ logits_out, int32_t* __restrict__ idx,
                                                        float* __restrict__ gate, int32_t* __restrict__ gidx,
                                                        float* __restrict__ ggate) {
  __shared__ float lt[kF32Tokens * (kMaxExperts + 1)];
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
    lt[r * (N + 1) + e] = acc;
  }
  __syncthreads();
  tile_epilogue<KL>(lt, N + 1, kF32Tokens, t0, T, N, n_groups, k, logits_out, idx, gate, gidx, ggate);
}

// ----------------------------------------------------------------------------
// Caller-supplied scores: 64 tokens per workgroup, their rows staged in LDS (16-byte
// loads when N % 4 == 0; odd row stride), then the common epilogue.
constexpr int kSelTokens = 64;
template <int KL>
__global__ __launch_bounds__(256) void route_select_kernel(int64_t T, int N, int M, int k,
                                                           const float* __restrict__ logits,
                                                           int32_t* __restrict__ idx, float* __restrict__ gate,
                                                           int32_t* __restrict__ gidx, float* __restrict__ ggate) {
  extern __shared__ float lt[];  // [kSelTokens][N + 1]
  const int ld = N + 1;
  const int64_t t0 = (int64_t)blockIdx.x * kSelTokens;
  const int64_t nrows = (T - t0) < kSelTokens ? (T - t0) : kSelTokens;
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
  tile_epilogue<KL>(lt, ld, (int)nrows, t0, T, N, M, k, nullptr, idx, gate, gidx, ggate);
}

}  // namespace moge

using namespace moge;

// Bytes of workspace the scores need: the partial sums of a reduction split over slices of d
// (bf16 scores from x, plan kinds 1 and 2), else none.
size_t moge::route_workspace_bytes(const moge_shape_t& s) {
  const RoutePlan pl = route_plan(s);
  if (pl.kind == 0) return 0;
  return (size_t)pl.S * (size_t)s.T * (size_t)s.N * sizeof(float);
}

// Scores (from x, or the caller's) and the choices: MoGE into idx/gate when idx is set, the
// global top-K into gidx/ggate when gidx is set.
static moge_status_t route_impl(const moge_shape_t* shape, const void* x, const void* w_router, const float* bias,
                                float* logits, int32_t* idx, float* gate, int32_t* gidx, float* ggate, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  moge_status_t st = validate_shape(shape);
  if (st != MOGE_OK) return st;
  const moge_shape_t& s = *shape;
  if (!x && !logits) return fail(MOGE_ERR_NULL, "either x (with w_router) or input logits is required");
  if (x && !w_router) return fail(MOGE_ERR_NULL, "w_router is required when x is given");
  if (!x && bias) return fail(MOGE_ERR_ARG, "bias must be NULL when logits are supplied (they include it)");
  const size_t need = x ? route_workspace_bytes(s) : 0;
  if (need && (!ws || ws_bytes < need)) return fail(MOGE_ERR_WORKSPACE, "route workspace missing or too small");

  const int kl = (s.N == 8 * s.M && s.M <= 8) ? kListG8 : lane_list_len(s.N, s.M, s.k_per_group, gidx != nullptr);
  if (!x) {
    st = with_list_len(kl, [&](auto klc) {
      constexpr int KL = decltype(klc)::value;
      const int64_t grid = ((int64_t)s.T + kSelTokens - 1) / kSelTokens;
      const size_t lds = sizeof(float) * kSelTokens * (size_t)(s.N + 1);
      if (lds > 64 * 1024) {
        moge_status_t r = raise_dynamic_lds(reinterpret_cast<const void*>(route_select_kernel<KL>), lds,
                                            "route_select_kernel");
        if (r != MOGE_OK) return r;
      }
      hipLaunchKernelGGL(route_select_kernel<KL>, dim3((unsigned)grid), dim3(256), lds, stream, (int64_t)s.T, s.N,
                         s.M, s.k_per_group, logits, idx, gate, gidx, ggate);
      return check_launch("route_select_kernel");
    });
  } else if (s.dtype == MOGE_F32) {
    st = with_list_len(kl, [&](auto klc) {
      constexpr int KL = decltype(klc)::value;
      const int64_t grid = ((int64_t)s.T + kF32Tokens - 1) / kF32Tokens;
      hipLaunchKernelGGL(route_f32_kernel<KL>, dim3((unsigned)grid), dim3(256), 0, stream, (int64_t)s.T, s.d, s.N,
                         s.M, s.k_per_group, static_cast<const float*>(x), static_cast<const float*>(w_router), bias,
                         logits, idx, gate, gidx, ggate);
      return check_launch("route_f32_kernel");
    });
  } else {
    const RoutePlan pl = route_plan(s);
    float* part = static_cast<float*>(ws);
    if (pl.kind == 2) {
      constexpr size_t lds = (size_t)kPartStages * (kPartTM + kPartNP) * kRouteRowB;
      st = raise_dynamic_lds(reinterpret_cast<const void*>(route_part_kernel), lds, "route_part_kernel");
      if (st != MOGE_OK) return st;
      const int64_t grid = ((int64_t)s.T + kPartTM - 1) / kPartTM * pl.S;
      hipLaunchKernelGGL(route_part_kernel, dim3((unsigned)grid), dim3(512), lds, stream, (int64_t)s.T, s.d, s.N,
                         pl.S, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router), part);
      st = check_launch("route_part_kernel");
    } else if (s.N <= 64) {
      st = launch_route_dma<128, 64, 3, 8, 1>(s, kl, x, w_router, bias, logits, idx, gate, gidx, ggate, pl.S, part,
                                              stream);
    } else {
      st = launch_route_dma<64, 128, 3, 4, 2>(s, kl, x, w_router, bias, logits, idx, gate, gidx, ggate, pl.S, part,
                                              stream);
    }
    if (st == MOGE_OK && pl.kind != 0 && s.N <= 64 && kl != 0) {  // the slices' sum, the rank-count choice
      if (s.T <= kReduceSmallT) {
        const int tpw = kReduceTokensSmall;
        hipLaunchKernelGGL((route_reduce_kernel<kListRank, kReduceTokensSmall>),
                           dim3((unsigned)(((int64_t)s.T + tpw - 1) / tpw)), dim3(256), 0, stream, (int64_t)s.T, s.N,
                           s.M, s.k_per_group, pl.S, part, bias, logits, idx, gate, gidx, ggate);
      } else {
        const int tpw = kReduceTokens;
        hipLaunchKernelGGL((route_reduce_kernel<kListRank, kReduceTokens>),
                           dim3((unsigned)(((int64_t)s.T + tpw - 1) / tpw)), dim3(256), 0, stream, (int64_t)s.T, s.N,
                           s.M, s.k_per_group, pl.S, part, bias, logits, idx, gate, gidx, ggate);
      }
      st = check_launch("route_reduce_kernel");
    } else if (st == MOGE_OK && pl.kind != 0) {  // the slices' partial sums -> scores -> the choices
      const int tpw = kReduceTokens;
      st = with_list_len(kl, [&](auto klc) {
        constexpr int KL = decltype(klc)::value;
        hipLaunchKernelGGL((route_reduce_kernel<KL, kReduceTokens>), dim3((unsigned)(((int64_t)s.T + tpw - 1) / tpw)),
                           dim3(256), 0,
                           stream, (int64_t)s.T, s.N, s.M, s.k_per_group, pl.S, part, bias, logits, idx, gate, gidx,
                           ggate);
        return check_launch("route_reduce_kernel");
      });
    }
  }
  return st == MOGE_OK ? ok() : st;
}

extern "C" moge_status_t moge_route(const moge_shape_t* shape, int32_t mode, const void* x, const void* w_router,
                                    const float* bias, float* logits, int32_t* idx, float* gate, void* ws,
                                    size_t ws_bytes, hipStream_t stream) {
  if (mode != MOGE_ROUTE_GROUPED && mode != MOGE_ROUTE_GLOBAL) {
    const moge_status_t st = validate_shape(shape);
    return st != MOGE_OK ? st : fail(MOGE_ERR_ARG, "unknown route mode");
  }
  if (!idx || !gate) {
    const moge_status_t st = validate_shape(shape);
    return st != MOGE_OK ? st : fail(MOGE_ERR_NULL, "idx and gate are required");
  }
  if (mode == MOGE_ROUTE_GROUPED)
    return route_impl(shape, x, w_router, bias, logits, idx, gate, nullptr, nullptr, ws, ws_bytes, stream);
  return route_impl(shape, x, w_router, bias, logits, nullptr, nullptr, idx, gate, ws, ws_bytes, stream);
}

extern "C" moge_status_t moge_route_pair(const moge_shape_t* shape, const void* x, const void* w_router,
                                         const float* bias, float* logits, int32_t* idx, float* gate, int32_t* gidx,
                                         float* ggate, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!idx || !gate || !gidx || !ggate) {
    const moge_status_t st = validate_shape(shape);
    return st != MOGE_OK ? st : fail(MOGE_ERR_NULL, "idx, gate, gidx and ggate are required");
  }
  return route_impl(shape, x, w_router, bias, logits, idx, gate, gidx, ggate, ws, ws_bytes, stream);
}
