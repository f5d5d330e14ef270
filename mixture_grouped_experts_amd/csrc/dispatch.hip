// moge_dispatch: per-expert counts and offsets, the stable token permutation and
// the gather of token rows into expert order (dropless: every (token, slot) pair
// gets a row; Pangu Ultra MoE digests on reportify.cn, dropless training).
//
// Up to four launches (two for T * K <= 8192: dispatch_small_kernel does 1-3 in
// one workgroup); the only atomics are a count and a bitwise OR, whose results do not
// depend on their order, so every output is deterministic:
//   1. dispatch_hist_kernel   one workgroup per block of 64 tokens counts its
//                             assignments per expert (LDS integer histogram).
//   2. dispatch_scan_kernel   one workgroup per expert scans that expert's block
//                             counts -> per-block starting rows and counts[e].
//   3. dispatch_permute_kernel one workgroup per token block: offsets from counts;
//                             each expert's 64-bit mask of the block's tokens that
//                             chose it (LDS OR); then every (token, slot) gets its
//                             row = segment start + rows of the expert in earlier
//                             blocks + popcount of the mask below the token, so rows
//                             of an expert stay in ascending token order -> inv, perm.
//   4. dispatch_copy_kernel   one wave per token reads its row from HBM once and
//                             writes it to all of its slots' rows (16-byte stores)
//                             in the tiled layout the expert GEMMs read, plus the
//                             token-order tiled copy the shared expert reads (only
//                             when the expert GEMMs cannot read the rows from x).
// Every expert's rows start on a 16-row boundary (P(e) in moge.h), so a 16-row
// tile of the GEMM operands never mixes experts.
#include <mutex>
#include <string>

#include "moge_internal.hpp"

namespace moge {

constexpr int kTB = kDispatchTokens;

__global__ __launch_bounds__(256) void dispatch_hist_kernel(int64_t T, int K, int N, int64_t nb,
                                                            const int32_t* __restrict__ idx,
                                                            int32_t* __restrict__ bcount) {
  __shared__ int hist[kMaxExperts];
  for (int e = threadIdx.x; e < N; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t b = blockIdx.x;
  const int64_t j0 = b * kTB * K;
  const int64_t t1 = (b + 1) * kTB < T ? (b + 1) * kTB : T;
  const int64_t j1 = t1 * K;
  for (int64_t j = j0 + threadIdx.x; j < j1; j += 256) {
    const int e = idx[j];
    if ((unsigned)e < (unsigned)N) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += 256) bcount[(int64_t)e * nb + b] = hist[e];
}

__global__ __launch_bounds__(256) void dispatch_scan_kernel(int64_t nb, const int32_t* __restrict__ bcount,
                                                            int32_t* __restrict__ bprefix,
                                                            int32_t* __restrict__ counts) {
  __shared__ int scratch[4];
  const int64_t e = blockIdx.x;
  const int32_t* src = bcount + e * nb;
  int32_t* dst = bprefix + e * nb;
  int running = 0;
  for (int64_t c = 0; c < nb; c += 256) {
    const int64_t i = c + threadIdx.x;
    const int v = i < nb ? src[i] : 0;
    int tot;
    const int ex = block_exclusive_scan(v, scratch, &tot);
    if (i < nb) dst[i] = running + ex;
    running += tot;
  }
  if (threadIdx.x == 0) counts[e] = running;
}

// Dynamic LDS: keys[kTB][KS] | offs[N+1] | base[N] | pbase[N+1]
__global__ __launch_bounds__(256) void dispatch_permute_kernel(
    int64_t T, int K, int N, int64_t nb, const int32_t* __restrict__ idx, int e_lo, int e_hi, int64_t rows_cap,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ bprefix, int32_t* __restrict__ offsets_out,
    int32_t* __restrict__ inv, int32_t* __restrict__ perm) {
  // inv == nullptr: offsets only (launched with one workgroup)
  extern __shared__ __attribute__((aligned(16))) int lds[];
  const int KS = K + 1;  // odd row stride: lanes of a wave hit distinct banks
  uint64_t* emask = reinterpret_cast<uint64_t*>(lds);  // per expert: the block's tokens that chose it
  int* keys = reinterpret_cast<int*>(emask + N);
  int* offs = keys + kTB * KS;
  int* base = offs + (N + 1);
  int* pbase = base + N;  // P(e): first local row of expert e (16-row aligned segments)
  __shared__ int scratch[4];

  const int64_t b = blockIdx.x;
  const int64_t t0 = b * kTB;

  // offsets = exclusive prefix of counts (N <= 256: one pass)
  {
    const int e = threadIdx.x;
    const int v = e < N ? counts[e] : 0;
    int tot;
    const int ex = block_exclusive_scan(v, scratch, &tot);
    if (e < N) offs[e] = ex;
    if (e == 0) offs[N] = tot;
    __syncthreads();
    if (b == 0) {
      if (e < N) offsets_out[e] = ex;
      if (e == 0) offsets_out[N] = tot;
    }
    if (e < N) base[e] = bprefix[(int64_t)e * nb + b];  // rows of e in earlier blocks
  }
  if (!inv) return;
  {
    // P(e) = sum over e_lo <= e' < e of counts[e'] rounded up to 16
    const int e = threadIdx.x;
    const int v = (e >= e_lo && e < e_hi) ? (counts[e] + kSegAlign - 1) / kSegAlign * kSegAlign : 0;
    int tot;
    const int ex = block_exclusive_scan(v, scratch, &tot);
    if (e < N) pbase[e] = ex;
    if (e == 0) pbase[N] = tot;
    // padding rows of a segment: perm = -1 (expert e handled by block e % nb)
    if (e >= e_lo && e < e_hi && (int64_t)(e % nb) == b) {
      for (int r = ex + counts[e]; r < ex + v; ++r)
        if ((int64_t)r < rows_cap) perm[r] = -1;
    }
  }
  for (int e = threadIdx.x; e < N; e += 256) emask[e] = 0;
  __syncthreads();
  // stage this block's expert ids (token tl = i / K); slots of other experts get inv = -1;
  // every in-range choice sets its token's bit in the expert's mask (OR: order-independent)
  for (int i = threadIdx.x; i < kTB * K; i += 256) {
    const int tl = i / K, s = i - tl * K;
    const int64_t t = t0 + tl;
    int e = -1;
    if (t < T) {
      e = idx[t * K + s];
      if ((unsigned)e >= (unsigned)N) e = -1;
      if (e < e_lo || e >= e_hi) inv[t * K + s] = -1;
      else atomicOr(reinterpret_cast<unsigned long long*>(&emask[e]), 1ull << tl);
    }
    keys[tl * KS + s] = e;
  }
  __syncthreads();

  // row of (token, slot) = P(e) + rows of e in earlier blocks + tokens of this block
  // before it that chose e (a token holds an expert at most once): stable token order
  for (int i = threadIdx.x; i < kTB * K; i += 256) {
    const int tl = i / K, s = i - tl * K;
    const int e = keys[tl * KS + s];
    if (e < e_lo || e >= e_hi) continue;  // (also e = -1: token past T or invalid id)
    const int64_t t = t0 + tl;
    int r = pbase[e] + base[e] + __popcll(emask[e] & ((1ull << tl) - 1ull));  // local row, padded numbering
    if ((int64_t)r >= rows_cap || r < 0) r = -1;
    inv[t * K + s] = r;
    if (r >= 0) perm[r] = (int32_t)t;
  }
}

// Small batches (T * K <= kSmallSlots): counts, offsets, inv and perm in one launch
// of one 1024-thread workgroup.  Every expert id is read once into LDS (with the
// counts, an LDS histogram); the permutation then takes the tokens in chunks of 64
// in order, each chunk ranking its tokens by the same per-expert masks and popcounts
// as dispatch_permute_kernel and then advancing each expert's running row count, so
// the rows are those of the multi-block path.
constexpr int kSmallSlots = 8192;
constexpr int kSmallThreads = 1024;
__global__ __launch_bounds__(kSmallThreads) void dispatch_small_kernel(int64_t T, int K, int N,
                                                                       const int32_t* __restrict__ idx, int e_lo,
                                                                       int e_hi, int64_t rows_cap,
                                                                       int32_t* __restrict__ counts_out,
                                                                       int32_t* __restrict__ offsets_out,
                                                                       int32_t* __restrict__ inv,
                                                                       int32_t* __restrict__ perm) {
  extern __shared__ __attribute__((aligned(16))) int lds[];
  const int KS = K + 1;                                 // odd row stride
  uint64_t* emask = reinterpret_cast<uint64_t*>(lds);  // per expert: the chunk's tokens that chose it
  int* keys = reinterpret_cast<int*>(emask + N);      // [T][K + 1]
  int* cnt = keys + T * KS;                            // [N]
  int* base = cnt + N;                                 // [N]: rows of e in earlier chunks
  int* pbase = base + N;                               // [N + 1]
  const int tid = threadIdx.x;
  for (int e = tid; e < N; e += kSmallThreads) {
    cnt[e] = 0;
    base[e] = 0;
  }
  __syncthreads();
  for (int j = tid; j < (int)T * K; j += kSmallThreads) {
    int e = idx[j];
    if ((unsigned)e >= (unsigned)N) e = -1;
    else atomicAdd(&cnt[e], 1);
    keys[(j / K) * KS + j % K] = e;
  }
  __syncthreads();
  if (tid < 64) {  // wave 0: offsets (all experts) and P(e) (16-row aligned segments of [e_lo, e_hi))
    const int lane = tid;
    int run = 0, prun = 0;
    for (int c = 0; c < N; c += 64) {
      const int e = c + lane;
      const int v = e < N ? cnt[e] : 0;
      const int vp = (e >= e_lo && e < e_hi) ? (v + kSegAlign - 1) / kSegAlign * kSegAlign : 0;
      int incl = v, pincl = vp;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(incl, off, 64), pu = __shfl_up(pincl, off, 64);
        if (lane >= off) {
          incl += u;
          pincl += pu;
        }
      }
      const int ex = run + incl - v, pex = prun + pincl - vp;
      if (e < N) {
        counts_out[e] = v;
        offsets_out[e] = ex;
        pbase[e] = pex;
      }
      if (inv && e >= e_lo && e < e_hi)  // padding rows of the segment
        for (int r = pex + v; r < pex + vp; ++r)
          if ((int64_t)r < rows_cap) perm[r] = -1;
      run += __shfl(incl, 63, 64);
      prun += __shfl(pincl, 63, 64);
    }
    if (lane == 0) {
      offsets_out[N] = run;
      pbase[N] = prun;
    }
  }
  if (!inv) return;
  __syncthreads();
  for (int t0 = 0; t0 < (int)T; t0 += kTB) {
    for (int e = tid; e < N; e += kSmallThreads) emask[e] = 0;
    __syncthreads();
    for (int i = tid; i < kTB * K; i += kSmallThreads) {
      const int tl = i / K, s = i - tl * K, t = t0 + tl;
      if (t >= (int)T) continue;
      const int e = keys[t * KS + s];
      if (e < e_lo || e >= e_hi) inv[(int64_t)t * K + s] = -1;
      else atomicOr(reinterpret_cast<unsigned long long*>(&emask[e]), 1ull << tl);
    }
    __syncthreads();
    for (int i = tid; i < kTB * K; i += kSmallThreads) {
      const int tl = i / K, s = i - tl * K, t = t0 + tl;
      if (t >= (int)T) continue;
      const int e = keys[t * KS + s];
      if (e < e_lo || e >= e_hi) continue;
      int r = pbase[e] + base[e] + __popcll(emask[e] & ((1ull << tl) - 1ull));  // local row, padded numbering
      if ((int64_t)r >= rows_cap || r < 0) r = -1;
      inv[(int64_t)t * K + s] = r;
      if (r >= 0) perm[r] = t;
    }
    __syncthreads();
    for (int e = tid; e < N; e += kSmallThreads) base[e] += __popcll(emask[e]);
    __syncthreads();
  }
}

// Row gather: one wave per token reads x[t] once (16-byte chunks, 8 in flight per
// lane) and writes it to every row that inv gives the token, in the tiled layout
// (a 16-byte chunk never straddles a tile; padding columns are written as zeros),
// and to row t of the token-order tiled copy when one is requested.
__global__ __launch_bounds__(256) void dispatch_copy_kernel(int64_t T, int K, const char* __restrict__ x, int esz,
                                                            int64_t d, int64_t rows_cap,
                                                            const int32_t* __restrict__ inv,
                                                            char* __restrict__ x_perm, char* __restrict__ x_tiled) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  const int64_t nch = (d * esz) >> 4;       // 16-byte chunks of a source row
  const int64_t dp = round_up(d, kTileCols);
  const int64_t ncp = (dp * esz) >> 4;      // chunks of a padded row
  const int epc = 16 / esz;                 // elements per chunk
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += nw) {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + t * d * esz);
    const int32_t* rr = inv + t * K;
    for (int64_t c0 = 0; c0 < ncp; c0 += 64 * 8) {
      u32x4_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t c = c0 + u * 64 + lane;
        v[u] = c < nch ? src[c] : zero;
      }
      auto put = [&](char* base, int64_t r) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t c = c0 + u * 64 + lane;
          if (c < ncp) *reinterpret_cast<u32x4_t*>(base + tiled_index(r, c * epc, dp) * esz) = v[u];
        }
      };
      if (x_tiled) put(x_tiled, t);
      for (int s = 0; s < K; ++s) {
        const int r = rr[s];
        if (r < 0 || (int64_t)r >= rows_cap) continue;
        put(x_perm, r);
      }
    }
  }
}

}  // namespace moge

using namespace moge;

// Multi-block path: histogram per 64-token block, scan per expert over blocks, permutation.
static moge_status_t dispatch_blocks_path(const moge_shape_t& s, int K, const int32_t* idx, int32_t e_lo,
                                          int32_t e_hi, int64_t rows_cap, int32_t* counts, int32_t* offsets,
                                          int32_t* inv, int32_t* perm, void* ws, hipStream_t stream) {
  moge_status_t st;
  const int64_t nb = dispatch_blocks(s.T);
  int32_t* bcount = static_cast<int32_t*>(ws);
  int32_t* bprefix = bcount + (int64_t)s.N * nb;

  hipLaunchKernelGGL(dispatch_hist_kernel, dim3((unsigned)nb), dim3(256), 0, stream, (int64_t)s.T, K, s.N, nb, idx,
                     bcount);
  if ((st = check_launch("dispatch_hist_kernel")) != MOGE_OK) return st;
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3((unsigned)s.N), dim3(256), 0, stream, nb, bcount, bprefix, counts);
  if ((st = check_launch("dispatch_scan_kernel")) != MOGE_OK) return st;

  const size_t lds = sizeof(uint64_t) * (size_t)s.N +
                     sizeof(int) * ((size_t)kTB * (K + 1) + (size_t)(s.N + 1) + (size_t)s.N + (size_t)(s.N + 1));
  if (lds > 64 * 1024) {
    st = raise_dynamic_lds(reinterpret_cast<const void*>(dispatch_permute_kernel), lds, "dispatch_permute_kernel");
    if (st != MOGE_OK) return st;
  }
  hipLaunchKernelGGL(dispatch_permute_kernel, dim3(inv ? (unsigned)nb : 1u), dim3(256), lds, stream, (int64_t)s.T, K, s.N, nb,
                     idx, e_lo, e_hi, rows_cap, counts, bprefix, offsets, inv, perm);
  st = check_launch("dispatch_permute_kernel");
  return st;
}

// Argument checks shared by both entry points (no workspace check).
static moge_status_t dispatch_checks(const moge_shape_t* shape, int32_t mode, const int32_t* idx, const void* x,
                                     int32_t e_lo, int32_t e_hi, int64_t rows_cap, int32_t* counts, int32_t* offsets,
                                     int32_t* inv, int32_t* perm, void* x_perm, void* x_tiled) {
  moge_status_t st = validate_shape(shape);
  if (st != MOGE_OK) return st;
  const moge_shape_t& s = *shape;
  if (mode != MOGE_ROUTE_GROUPED && mode != MOGE_ROUTE_GLOBAL) return fail(MOGE_ERR_ARG, "unknown route mode");
  if (!idx || !counts || !offsets) return fail(MOGE_ERR_NULL, "idx, counts and offsets are required");
  if ((x == nullptr) != (x_perm == nullptr)) return fail(MOGE_ERR_NULL, "x and x_perm must be given together");
  if ((inv == nullptr) != (perm == nullptr)) return fail(MOGE_ERR_NULL, "inv and perm must be given together");
  if (x && !inv) return fail(MOGE_ERR_NULL, "row copies need inv and perm");
  if (x_tiled && !x) return fail(MOGE_ERR_NULL, "x_tiled needs x");
  if (e_lo < 0 || e_hi > s.N || e_lo >= e_hi) return fail(MOGE_ERR_ARG, "need 0 <= e_lo < e_hi <= N");
  const int64_t bound = rows_bound(s, mode, e_lo, e_hi);
  if (inv && rows_cap < bound)
    return fail(MOGE_ERR_CAPACITY, "rows_cap is below moge_rows_bound() for this expert range");
  return MOGE_OK;
}

// The launches (arguments already checked; ws holds moge_workspace_size(MOGE_STAGE_DISPATCH) bytes).
static moge_status_t dispatch_launch(const moge_shape_t& s, const int32_t* idx, const void* x, int32_t e_lo,
                                     int32_t e_hi, int64_t rows_cap, int32_t* counts, int32_t* offsets, int32_t* inv,
                                     int32_t* perm, void* x_perm, void* x_tiled, void* ws, hipStream_t stream) {
  moge_status_t st;
  const int K = s.M * s.k_per_group;  // <= N <= 256 (moge_validate)
  if ((int64_t)s.T * K <= kSmallSlots) {  // one workgroup does counts, offsets and the permutation
    // 8 N + 4 (T (K + 1) + 3 N + 1) bytes: with T K <= 8192 and N <= 256 at most
    // 8 * 256 + 4 * (2 * 8192 + 769) = 70.7 KiB (T = 8192, K = 1), above the 64 KiB default
    const size_t slds = sizeof(uint64_t) * (size_t)s.N +
                        sizeof(int) * ((size_t)s.T * (K + 1) + (size_t)s.N * 3 + 1);
    if (slds > 64 * 1024) {
      st = raise_dynamic_lds(reinterpret_cast<const void*>(dispatch_small_kernel), slds, "dispatch_small_kernel");
      if (st != MOGE_OK) return st;
    }
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(kSmallThreads), slds, stream, (int64_t)s.T, K, s.N, idx,
                       e_lo, e_hi, rows_cap, counts, offsets, inv, perm);
    st = check_launch("dispatch_small_kernel");
  } else {
    st = dispatch_blocks_path(s, K, idx, e_lo, e_hi, rows_cap, counts, offsets, inv, perm, ws, stream);
  }
  const int esz = s.dtype == MOGE_BF16 ? 2 : 4;
  if (st == MOGE_OK && x) {
    int64_t grid = ((int64_t)s.T + 3) / 4;
    if (grid > 16384) grid = 16384;
    hipLaunchKernelGGL(dispatch_copy_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (int64_t)s.T, K,
                       static_cast<const char*>(x), esz, (int64_t)s.d, rows_cap, inv, static_cast<char*>(x_perm),
                       static_cast<char*>(x_tiled));
    st = check_launch("dispatch_copy_kernel");
  }
  return st;
}

extern "C" moge_status_t moge_dispatch(const moge_shape_t* shape, int32_t mode, const int32_t* idx, const void* x,
                                       int32_t e_lo, int32_t e_hi, int64_t rows_cap, int32_t* counts,
                                       int32_t* offsets, int32_t* inv, int32_t* perm, void* x_perm, void* x_tiled,
                                       void* ws, size_t ws_bytes, hipStream_t stream) {
  moge_status_t st = dispatch_checks(shape, mode, idx, x, e_lo, e_hi, rows_cap, counts, offsets, inv, perm, x_perm,
                                     x_tiled);
  if (st != MOGE_OK) return st;
  const size_t need = moge_workspace_size(shape, MOGE_STAGE_DISPATCH);
  if (!ws || ws_bytes < need) return fail(MOGE_ERR_WORKSPACE, "dispatch workspace missing or too small");
  st = dispatch_launch(*shape, idx, x, e_lo, e_hi, rows_cap, counts, offsets, inv, perm, x_perm, x_tiled, ws, stream);
  return st == MOGE_OK ? ok() : st;
}

// ---- moge_dispatch_noalloc: the same work with the workspace in a file-scope device array.
// Each GPU that runs the library holds its own copy of `scratch` until the process ends; host
// code never passes the array's name to a kernel (on the host it is only a stand-in for the
// symbol): it asks the runtime for the device address once per device, with that device
// current, and uses that address from then on.  Nothing in the array has to start at zero (the
// block counts and their prefixes are fully written before they are read), so no call clears it.
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;  // 4 MiB: N * ceil(T / 64) <= 524288
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// The device address of `scratch` on the device that runs `stream` (looked up once per device).
static moge_status_t scratch_address(hipStream_t stream, void** out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(MOGE_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  int dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return fail(MOGE_ERR_HIP, std::string("hipStreamGetDevice: ") + hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(MOGE_ERR_HIP, "device id out of the supported range");
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(MOGE_ERR_HIP, std::string("hipSetDevice: ") + hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) hipSetDevice(cur);
    if (e != hipSuccess || !p)
      return fail(MOGE_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    addr[dev] = p;
  }
  *out = addr[dev];
  return MOGE_OK;
}

extern "C" moge_status_t moge_dispatch_noalloc(const moge_shape_t* shape, int32_t mode, const int32_t* idx,
                                               const void* x, int32_t e_lo, int32_t e_hi, int64_t rows_cap,
                                               int32_t* counts, int32_t* offsets, int32_t* inv, int32_t* perm,
                                               void* x_perm, void* x_tiled, hipStream_t stream) {
  moge_status_t st = dispatch_checks(shape, mode, idx, x, e_lo, e_hi, rows_cap, counts, offsets, inv, perm, x_perm,
                                     x_tiled);
  if (st != MOGE_OK) return st;
  const size_t need = moge_workspace_size(shape, MOGE_STAGE_DISPATCH);
  if (need > kNoAllocScratchBytes)
    return fail(MOGE_ERR_WORKSPACE, "moge_dispatch_noalloc: the shape needs " + std::to_string(need) +
                                        " bytes of workspace, above its fixed " +
                                        std::to_string(kNoAllocScratchBytes) + " (N * ceil(T / 64) <= 524288)");
  void* ws = nullptr;
  if ((st = scratch_address(stream, &ws)) != MOGE_OK) return st;
  st = dispatch_launch(*shape, idx, x, e_lo, e_hi, rows_cap, counts, offsets, inv, perm, x_perm, x_tiled, ws, stream);
  return st == MOGE_OK ? ok() : st;
}
