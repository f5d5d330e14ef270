// Internal helpers shared by the libmoge translation units (host validation,
// error reporting and small device utilities for gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "moge.h"

namespace moge {

// ---------------------------------------------------------------- host side
moge_status_t fail(moge_status_t st, const std::string& msg);
moge_status_t ok();
moge_status_t check_launch(const char* what);
moge_status_t validate_shape(const moge_shape_t* s);
int64_t rows_bound(const moge_shape_t& s, int32_t mode, int32_t e_lo, int32_t e_hi);
// Lets `kernel` use `bytes` of dynamic LDS (above the 64 KiB default).  Thread-safe;
// remembers the largest size set per kernel.
moge_status_t raise_dynamic_lds(const void* kernel, size_t bytes, const char* what);

constexpr int kMaxExperts = 256;

// Tiled operand layout: tiles of 16 rows x 32 columns (512 elements), tiles of a
// 16-row band consecutive; element (r, c) of a matrix with cp (a multiple of 32)
// padded columns is at tiled_index(r, c, cp).
constexpr int kTileRows = 16;
constexpr int kTileCols = 32;
constexpr int kTileElems = kTileRows * kTileCols;
constexpr int kSegAlign = 16;        // expert row segments start on a 16-row boundary
constexpr int kWeightRowAlign = 32;  // packed weights: rows padded with zeros to a multiple of 32
__host__ __device__ __forceinline__ int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }
__host__ __device__ __forceinline__ int64_t tiled_index(int64_t r, int64_t c, int64_t cp) {
  return ((r >> 4) * (cp >> 5) + (c >> 5)) * kTileElems + (r & 15) * kTileCols + (c & 31);
}

// moge_check_finite: partial results per workgroup (count, first index) in its workspace.
constexpr int kCheckBlocks = 1024;
inline size_t check_workspace_bytes() { return (size_t)kCheckBlocks * 2 * sizeof(int64_t) + 2 * sizeof(int64_t); }

// Bytes of workspace moge_route needs for the shape when it computes the scores from x.
size_t route_workspace_bytes(const moge_shape_t& s);

// Dispatch geometry (shared by moge_workspace_size and the dispatch kernels).
constexpr int kDispatchTokens = 64;   // tokens per dispatch workgroup (one per lane)
inline int64_t dispatch_blocks(int64_t T) { return (T + kDispatchTokens - 1) / kDispatchTokens; }

// ---------------------------------------------------------------- device side
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// binary32 -> bf16, round to nearest even (finite inputs; NaN stays NaN).
// float -> bf16, round to nearest even: gfx950's v_cvt_pk_bf16_f32 (two values per
// instruction where two conversions meet).  It equals the plain integer rounding (add
// 0x7FFF plus the kept lsb, keep the top half) for every finite value and infinity;
// NaNs come out quiet (moge_round_bf16 exposes it; its test checks every exponent's
// ties and neighbours, denormals, overflow and a million random patterns).  In the
// GEMM epilogues the integer form cost 7-8 vector instructions per value.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ---- direct-to-LDS staging of 64-byte rows (the expert GEMMs and the router)
// 16-byte chunk c of 64-byte LDS row r lives in slot c ^ lds_swz(r).  Four such rows
// share a 256-byte bank line; with this swizzle the 16 rows that one 16-byte
// fragment read touches per clock cover all 64 banks (measured conflict-free on
// gfx950).
__device__ __forceinline__ int lds_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// s_waitcnt immediates (gfx9 encoding): at most n vector memory operations of this
// wave outstanding; the second form also waits for all of the wave's LDS reads.
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int vmcnt_lgkm0_imm(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }
constexpr int lgkm0_imm() { return 15 | (7 << 4) | (3 << 14); }  // all of the wave's LDS operations done

// LDS byte address of a __shared__ pointer (what M0 takes for a direct load).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One wave moves 64 x 16 bytes from global memory straight into LDS: lane l's 16
// bytes at `src` land at LDS byte m0 + 16 l (m0 wave-uniform).  Issued from inline
// assembly so the compiler does not turn the LDS side effect into a full vmcnt wait
// before every LDS read; callers wait with vmcnt_imm and a barrier before reading.
// The instruction has no register result, only an address operand read at issue.
__device__ __forceinline__ void dma_16x64(const void* src, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(m0))
               : "memory", "m0");
}

// The same with the non-temporal hint, for data read once (expert weights): it
// streams through the caches instead of displacing data that is read again.
__device__ __forceinline__ void dma_16x64_stream(const void* src, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(m0))
               : "memory", "m0");
}

// Number of lanes below the calling lane whose bit is set in `mask`.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Exclusive scan of a 256-wide block; returns this thread's prefix, *total = block sum.
// (256 threads; all threads of the block must call it)
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch /* >= 4 ints */, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(incl, off, 64);
    if (lane >= off) incl += u;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int wbase = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int s = scratch[w];
    if (w < wave) wbase += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return wbase + incl - v;
}

}  // namespace moge
