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
//   * bf16 v_mfma_f32_16x16x32_bf16 with float32 accumulators; a 512-thread
//     workgroup (two waves per SIMD) owns a 320-row x 256-weight-row tile (GEMM 1:
//     128 gate + 128 up rows of the same 128 h columns, so the SwiGLU is fused into
//     the epilogue; GEMM 2: 256 output columns), each wave a 160 x 64 part of it;
//     when the experts average at most 64 rows (decode) a 96 x 512 tile instead,
//     which streams twice the weight bytes per step -- SwiftGMM's switch of mode by
//     workload;
//   * the weights are packed once at load time into the tiled layout (16 x 32
//     tiles of 1 KiB, see moge.h), so every weight load instruction moves one
//     contiguous 1 KiB tile (one burst per 16 rows, one address-translation page
//     per instruction) instead of 16 half cache lines of 16 long rows; K is padded
//     with zeros to a multiple of 32, so there is no ragged reduction step;
//   * GEMM 1 takes its token rows straight from the row-major x, each lane's
//     address from perm (moge_expert_gate_up_gather), so dispatch never writes an
//     x_perm (R x d, 1 GB for 8192 tokens x 8 slots x 7680); or from a tiled x_perm
//     where that cannot apply (float32, d % 32 != 0).  GEMM 2 reads the tiled h;
//   * both panels go straight from global memory to a 4-stage LDS ring
//     (global_load_lds_dwordx4, BK = 32), so every load has three steps of MFMA
//     work to arrive and no registers stage it; 64-byte LDS rows with an XOR
//     swizzle keep the 16-byte fragment reads bank-conflict free at the LDS's full
//     rate, which takes at least two waves per SIMD to reach;
//   * a tile with few live rows (the last tile of an expert) skips the MFMAs of
//     its empty 16-row blocks, so an expert's tail costs at most 15 rows of padding
//     work (a 32-row MFMA block wasted about 6% of the work at 256 rows per
//     expert); the row blocks are interleaved over the waves;
//   * a persistent grid walks a device-built tile list (no host sync on the
//     expert counts): every workgroup derives the per-expert tile counts from
//     `offsets` in LDS.  Tiles of one expert are ordered in groups of 4 m-tiles,
//     n-tiles outer, so tiles that share a weight panel or an activation panel
//     run at the same time; consecutive tiles go to one XCD (workgroup b runs on
//     XCD b % 8), so that sharing happens in that XCD's L2;
//   * the weight fragment is the MFMA's first operand, so each lane ends with 4
//     consecutive output columns of one token row: the epilogue (SwiGLU for
//     GEMM 1, into the tiled h; GEMM 2 into the row-major expert output, or
//     straight into y for one-group shares) packs them into 8- or 16-byte stores.
// float32 shapes use a plain vector-ALU kernel pair on the same layouts (small
// shapes only).
#include <math.h>

#include <algorithm>
#include <vector>

#include "moge_internal.hpp"

namespace moge {

// silu(g) * u = g / (1 + e^-g) * u with the hardware exp2 and reciprocal (v_exp_f32,
// v_rcp_f32): a few float32 ulps, four orders of magnitude below the bf16 rounding
// that h gets next; the IEEE expf and division cost 1-6% of the gate/up GEMM in its
// epilogue.  Large -g gives e^-g = inf and a result of -0 * u, as silu's limit.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-g * 1.44269504f)) * u;
}

constexpr int kBK = 32;                     // reduction step (elements)
constexpr int kRowB = kBK * 2;              // 64-byte LDS rows (unpadded; chunks are XOR-swizzled)
constexpr int kStages = 4;
constexpr int kThreads = 512;               // 8 waves: two per SIMD
constexpr int kMaxBM = 320;                 // largest token-row tile

// Two tile shapes; every wave owns 64 weight rows and the 16-row token blocks
// wm, wm + WMG, wm + 2 WMG, ... of the tile (WMG wave rows x 8 / WMG wave columns):
//   WMG = 2: 320 token rows x 256 weight rows (10 token blocks per wave) -- the
//            general case, where an expert's rows fill a 320-row tile;
//   WMG = 1: 96 token rows x 512 weight rows (6 token blocks per wave) -- few rows
//            per expert (decode): twice the weight bytes per step, so each CU keeps
//            twice as many weight bytes in flight and the weight stream runs nearer
//            the HBM rate.
// Both stage 64-byte rows of BM + BW rows per step in a 4-stage ring.
template <int WMG>
struct TileShape;
template <>
struct TileShape<2> {
  static constexpr int kBlocks = 10, BM = 320, BW = 256;  // kBlocks: 16-row token blocks per wave
};
template <>
struct TileShape<1> {
  static constexpr int kBlocks = 6, BM = 96, BW = 512;
};
template <int WMG>
constexpr int stage_bytes() { return (TileShape<WMG>::BM + TileShape<WMG>::BW) * kRowB; }  // 36 / 38 KiB
template <int WMG>
constexpr size_t gemm_lds() { return (size_t)kStages * stage_bytes<WMG>(); }  // 144 / 152 KiB
constexpr int kGroupM = 4;                  // m-tiles per scheduling group
constexpr int kAhead = 3;                   // token-block fragment reads issued ahead of the MFMAs

__device__ __forceinline__ int swz(int r) { return lds_swz(r); }

// How the token-row operand A is addressed.
constexpr int kATiled = 0;   // tiled [rows][KP] (x_perm from dispatch, or h)
constexpr int kAGather = 1;  // row-major x [arows][KP]; local row r is token perm[r] (-1: padding row)
constexpr int kARows = 2;    // row-major x [arows][KP]; local row r is token r

// Operands of one grouped GEMM problem.
//   GEMM 1 (SWIGLU):  A = token rows (tiled x_perm, or x itself read through perm),
//                     B0/B1 = packed gate/up [E][NOUT][KP], C = h tiled [rows][NPAD],
//                     NPAD = NOUT rounded up to 32.
//   GEMM 2:           A = h tiled [rows][KP], B0 = packed down [E][NOUT][KP], C = out [rows][NOUT].
// KP = the reduction length rounded up to 32 (zero padded in tiled A and in B; a
// row-major A needs KP == its row length, i.e. d % 32 == 0).
struct GemmOperands {
  const uint16_t* A;
  const uint16_t* B0;
  const uint16_t* B1;
  uint16_t* C;
  int NOUT;
  int KP;
  int amode;            // kATiled, kAGather or kARows
  const int32_t* perm;  // kAGather: token of each local row; combine epilogue: the same for C's rows
  int64_t arows;        // kAGather, kARows: rows of x (out-of-range tokens read row 0)
  int64_t prows;        // kAGather: entries of perm (rows past them read token 0)
  // GEMM 2 only, when Y is set: instead of storing row r of C, the epilogue writes the
  // combined output y[t] = gate[t][gslot] * C[r] (float32, row-major [T][NOUT]) for the token
  // t = perm[r] that owns the row (each token owns exactly one row of the problem).
  float* Y;
  const float* gate;
  int gstride, gslot;
};

// One tile: reduction loop and epilogue, 8 waves.  Wave (wm, wn), wm in {0,1},
// wn in {0..3} (320 x 256 tiles; wm = wave / 4, so each SIMD runs one wave of each
// half), owns the token row blocks wm, wm+2, ..., wm+18 (16 rows each,
// interleaved so a partly filled tile keeps the waves balanced) and 4 weight
// quarters of 16 rows (GEMM 1: the gate and the up rows of the same 32 h columns;
// GEMM 2: 64 output columns).  NL of its row blocks hold live rows; the others
// skip their MFMAs.  A tile spans 320 token rows so that an expert whose row
// count is a little above 256 (the common case when the rows spread evenly over
// hundreds of experts) still reads each weight panel once.  The MFMA takes the
// weight fragment as its first operand, so each lane ends with 4 consecutive
// output columns of one token row, which the epilogue packs into 8-byte stores.
//
// Pipeline: global -> LDS directly (global_load_lds_dwordx4, no staging registers)
// into a 4-stage ring.  Per step waves 0-3 move token rows wave*64 .. +64 and
// waves 4-7 weight rows (wave-4)*64 .. +64 plus token rows 256 + (wave-4)*16 .. +16,
// 64 B per row.  Step s is issued at step s-3 and read at step s only (no fragment
// is read ahead across the barrier), so every load has three steps of MFMA work to
// land; the end of each step waits (vmcnt) for its own loads of step s+1, then one
// barrier.  Two waves per SIMD keep the MFMA pipe fed across the barriers and give
// the LDS enough concurrent readers to reach its full rate.  Token rows come from
// the tiled x_perm / h (one contiguous 1 KiB tile per instruction) or straight from
// the row-major x through perm (16 rows x 64 B per instruction), which saves
// materialising x_perm at all.

// First stage row of DMA instruction j of this wave (wave-uniform):
//   320 x 256: waves 0-3 move token rows wave*64 .. +64 (4 instructions); waves
//              4-7 weight rows (wave-4)*64 .. +64 and token rows 256 + (wave-4)*16;
//   96 x 512:  every wave moves weight rows wave*64 .. +64; waves 0-5 also token
//              rows wave*16 .. +16.
// Each instruction moves one tile of 16 rows x 32 columns; lane l brings 16 bytes of
// row lrow + l/4.
template <int WMG>
__device__ __forceinline__ int dma_stage_row(int wave, int j) {
  constexpr int BM = TileShape<WMG>::BM;
  const bool wtok = WMG == 2 && wave < 4;
  const bool five = WMG == 2 ? wave >= 4 : wave < BM / kTileRows;
  if (WMG == 2) return wtok ? wave * 64 + j * 16 : (j < 4 ? BM + (wave - 4) * 64 + j * 16 : 256 + (wave - 4) * 16);
  return j < 4 ? BM + wave * 64 + j * 16 : (five ? wave * 16 : 0);
}

// The token row read by this lane in each of its DMA instructions: the local row for
// the tiled A (bands past the live rows re-read the last live band, never stored), the
// token itself for the gathered A (loaded from perm, all five loads together, indices
// kept inside perm; -1 past it), the row for row-major A.
template <int WMG>
__device__ __forceinline__ void token_rows(const GemmOperands& op, int64_t mband0, int mrows, int32_t (&tok)[5]) {
  constexpr int BM = TileShape<WMG>::BM;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int live_bands = (mrows + kTileRows - 1) / kTileRows;
  int64_t trow[5];
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int lrow = dma_stage_row<WMG>(wave, j);
    int band = lrow < BM ? lrow / kTileRows : 0;
    if (band >= live_bands) band = live_bands - 1;
    trow[j] = (mband0 + band) * kTileRows + (lane >> 2);
  }
  if (op.amode == kAGather) {
    int32_t t32[5];
#pragma unroll
    for (int j = 0; j < 5; ++j) t32[j] = op.perm[trow[j] < op.prows ? trow[j] : op.prows - 1];
#pragma unroll
    for (int j = 0; j < 5; ++j) tok[j] = trow[j] < op.prows ? t32[j] : -1;
  } else {
#pragma unroll
    for (int j = 0; j < 5; ++j) tok[j] = (int32_t)trow[j];
  }
}

// Per-lane global sources of this wave's DMA instructions for step 0 of a tile.
template <bool SWIGLU, int WMG>
__device__ __forceinline__ void dma_sources(const GemmOperands& op, const uint16_t* __restrict__ wbase0,
                                            const uint16_t* __restrict__ wbase1, int wbands, int nkf, int n0,
                                            const int32_t (&tok)[5], const uint16_t* (&dsrc)[5]) {
  constexpr int BM = TileShape<WMG>::BM, BW = TileShape<WMG>::BW;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int lrow = dma_stage_row<WMG>(wave, j);
    const int srow = lrow + (lane >> 2);                 // stage row (token rows 0..BM-1, then weight rows)
    const int chunk = (lane & 3) ^ swz(srow);            // 16-byte chunk of the tile row fetched by this lane
    const int inner = (lane >> 2) * kTileCols + chunk * 8;
    if (lrow < BM) {
      if (op.amode == kATiled) {
        dsrc[j] = op.A + (int64_t)(tok[j] >> 4) * nkf * kTileElems + inner;
      } else {  // row-major x: this lane's row is one token's row, 64 bytes of it per step
        const int64_t t = tok[j] < 0 || tok[j] >= op.arows ? 0 : tok[j];  // padding rows read token 0 (never stored)
        dsrc[j] = op.A + t * op.KP + chunk * 8;
      }
    } else {
      const int r = lrow - BM;  // GEMM 1: rows < BW/2 are gate rows, the rest the up rows of the same columns
      int band = (SWIGLU ? n0 + (r & (BW / 2 - 1)) : n0 + r) / kTileRows;
      if (band >= wbands) band = wbands - 1;
      dsrc[j] = (SWIGLU && r >= BW / 2 ? wbase1 : wbase0) + (int64_t)band * nkf * kTileElems + inner;
    }
  }
}

// Where a tile's first three steps come from and where the next tile's go: with pre,
// steps 0-2 were issued by the previous tile into stages 1-3 (step s in stage
// (1 + s) % 4); with chain, this tile issues the next one's steps 0-2 into stages 1-3
// right after its reduction loop, so they land during this tile's epilogue, which
// then stages its output in stage 0 only.
struct NextTile {
  const uint16_t* wb0;
  const uint16_t* wb1;
  int64_t mband0;
  int wbands, nkf, n0, mrows, krot, unused1;  // (no padding bytes: copies stay in registers)
};

template <bool SWIGLU, int NL, int WMG>
__device__ __forceinline__ void tile_compute(const GemmOperands& op, char* __restrict__ lds,
                                             const uint16_t* __restrict__ wbase0, const uint16_t* __restrict__ wbase1,
                                             int wbands, int nkf, int mrows, int64_t row0, int n0, int NOUT, int NPAD,
                                             uint16_t* __restrict__ C, const int32_t (&tokc)[5], bool pre, bool chain,
                                             const GemmOperands& nop, const NextTile& nx, int32_t (&tokn)[5],
                                             int krot) {
  constexpr int BM = TileShape<WMG>::BM, BW = TileShape<WMG>::BW, NB = TileShape<WMG>::kBlocks;
  constexpr int kStageB = stage_bytes<WMG>();
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in a scalar register
  // the two waves on a SIMD (w and w + 4) take different token-row halves, so an odd
  // number of live row blocks still gives every SIMD the same MFMA count
  const int wm = WMG == 2 ? wave >> 2 : 0, wn = WMG == 2 ? wave & 3 : wave;
  const bool wtok = WMG == 2 && wave < 4;
  const bool five = WMG == 2 ? wave >= 4 : wave < BM / kTileRows;
  int lrow[5];
#pragma unroll
  for (int j = 0; j < 5; ++j) lrow[j] = dma_stage_row<WMG>(wave, j);
  const uint16_t* dsrc[5];
  dma_sources<SWIGLU, WMG>(op, wbase0, wbase1, wbands, nkf, n0, tokc, dsrc);
  const int astep = op.amode == kATiled ? kTileElems : kTileCols;  // token-row elements per step
  const int sbase = pre ? 1 : 0;
  // Step ks into stage (sbase + ks) % 4 (steps past the last full step reload step 0);
  // the waits are explicit (vmcnt_imm) and each is followed by a barrier before the
  // stage is read.
  const uint32_t lds0 = lds_addr(lds);
  auto issue_from = [&](const uint16_t* const (&src)[5], int offa, int offb, uint32_t st) {
    if (wtok) {  // four token-row instructions
#pragma unroll
      for (int j = 0; j < 4; ++j) dma_16x64(src[j] + offa, st + (uint32_t)(lrow[j] * kRowB));
    } else {     // four weight-row instructions and (five) one token-row instruction
#pragma unroll
      for (int j = 0; j < 4; ++j) dma_16x64_stream(src[j] + offb, st + (uint32_t)(lrow[j] * kRowB));
      if (WMG == 2 || five) dma_16x64(src[4] + offa, st + (uint32_t)(lrow[4] * kRowB));
    }
  };
  auto issue = [&](int ks) {
    const int kr = (ks < nkf ? ks : 0) + krot;
    const int kq = kr < nkf ? kr : kr - nkf;
    issue_from(dsrc, kq * astep, kq * kTileElems, lds0 + (uint32_t)(((sbase + ks) & (kStages - 1)) * kStageB));
  };
  // Fragments of one 32-column step for v_mfma_f32_16x16x32_bf16: lane l holds 8
  // consecutive columns (16-byte chunk l/16) of row l%16 of a 16-row block, for the
  // weight operand (the MFMA's first) and the token operand alike; the product block
  // gives lane l 4 consecutive weight rows 4(l/16) .. +3 (output columns) of token row
  // l%16.  Token blocks of 16 rows keep a partly filled expert tail to at most 15
  // padding rows of MFMA work.  Weight quarters q of 16 rows: GEMM 1: q = 0, 1 the gate
  // rows of the wave's 32 columns, q = 2, 3 the up rows of the same columns; GEMM 2:
  // q = 0..3 the wave's 64 output columns.
  const int kq = lane >> 4;
  int arow[NB], brow[4];
#pragma unroll
  for (int t = 0; t < NB; ++t) arow[t] = (wm + WMG * t) * 16 + (lane & 15);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    brow[q] = BM + (SWIGLU ? (q >> 1) * (BW / 2) + wn * 32 + (q & 1) * 16 : wn * 64 + q * 16) + (lane & 15);
  auto rd = [&](const char* st, int row) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(st + row * kRowB + ((kq ^ swz(row)) << 4)));
  };
  f32x4_t acc[NL > 0 ? NL : 1][4];
  static_assert(NL <= NB, "row blocks per wave");
#pragma unroll
  for (int t = 0; t < (NL > 0 ? NL : 1); ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][q][r] = 0.f;

  // (the previous tile's epilogue stores may still be in flight: the loads do not
  // depend on them, and loads complete in order among themselves, so each wait
  // below still guarantees its step; older stores only make it stricter)
  if (!pre) {
    issue(0);
    issue(1);
    issue(2);
  }
  // step 0 landed (this wave issues 4 or 5 loads per step; with pre, steps 0-2 and
  // then the previous epilogue's stores are the operations in flight)
  if (five) __builtin_amdgcn_s_waitcnt(vmcnt_imm(10));
  else __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));
  __syncthreads();
  for (int ks = 0; ks < nkf; ++ks) {
    issue(ks + 3);
    if (NL) {
      const char* st = lds + ((sbase + ks) & (kStages - 1)) * kStageB;
      bf16x8_t bq[4], at[NB];
#pragma unroll
      for (int q = 0; q < 4; ++q) bq[q] = rd(st, brow[q]);
#pragma unroll
      for (int t = 0; t < NL; ++t) at[t] = rd(st, arow[t]);
#pragma unroll
      for (int t = 0; t < NL; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[t][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bq[q], at[t], acc[t][q], 0, 0, 0);
      // the weight quarters and the first three token blocks, then each block's four
      // MFMAs with the read of the block three ahead in their shadow (one or two ahead,
      // no hints, or all reads first were measured 1-7% slower)
      __builtin_amdgcn_sched_group_barrier(0x100, 4 + (NL < kAhead ? NL : kAhead), 0);
#pragma unroll
      for (int t = 0; t < NL; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        if (t + kAhead < NL) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    // step ks+1 landed (this wave) and this step's LDS reads are done, so the DMA
    // issued after the barrier may overwrite stage ks % 4
    if (five) __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(10));
    else __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(8));
    __syncthreads();
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // drain the trailing reloads before LDS is reused
  __syncthreads();
  if (chain) {  // the next tile's steps 0-2 into stages 1-3, in flight during this epilogue
    const uint16_t* ndsrc[5];
    // GEMM 2's token rows are plain arithmetic, done here (its registers are at their
    // limit in the loop); GEMM 1's were loaded by the caller a tile ahead
    if constexpr (!SWIGLU) token_rows<WMG>(nop, nx.mband0, nx.mrows, tokn);
    dma_sources<SWIGLU, WMG>(nop, nx.wb0, nx.wb1, nx.wbands, nx.nkf, nx.n0, tokn, ndsrc);
    const int nastep = nop.amode == kATiled ? kTileElems : kTileCols;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int kr = j + nx.krot;
      const int kq = kr < nx.nkf ? kr : kr - nx.nkf;
      issue_from(ndsrc, kq * nastep, kq * kTileElems, lds0 + (uint32_t)((1 + j) * kStageB));
    }
  }
  // epilogue (rows of dead blocks are never stored).  GEMM 1 writes the tiled h
  // (NPAD = F rounded up to 32 columns; its padding columns come out as zeros from
  // the zero rows of the packed weights); GEMM 2 writes row-major [row][NOUT].
  // h leaves with the non-temporal hint: its writes, spread over the kernel, otherwise
  // break up the weight read stream (measured, same box: 256-token decode gate/up 279 ->
  // 257 us, 8192-token Ultra 4.47 -> 4.36 ms; h stores aimed at one L2-resident block
  // gave the same time as the hinted ones, so the cost was the DRAM writes, not the
  // instructions).  GEMM 2's expert outputs take the hint only in the wide shape (few
  // rows per expert, a weight stream, decode down 148 -> 134 us): with the tall shape
  // the combine that reads them slowed (Ultra 244 -> 266 us) more than the GEMM gained.
  if (!SWIGLU && !op.Y && (NOUT & 7) == 0) {
    // GEMM 2 through LDS (the ring is idle now): each wave writes its 64 columns of up
    // to kPassBlocks row blocks into its own 10 KiB of LDS as 128-byte rows (16-byte
    // chunks XOR-swizzled by row), then reads back 16 bytes per lane, so each row's
    // 128 bytes leave as whole cache lines instead of four 32-byte pieces.  Only this
    // wave touches its region, so the ordering needed is the wave's own (its LDS
    // operations complete in order; the waits keep the compiler from reordering).
    constexpr int kPassBlocks = 5;  // 10 KiB per wave (GEMM 2 does not chain: the ring is free)
    char* wl = lds + wave * (kPassBlocks * 16 * 128);
#pragma unroll
    for (int p0 = 0; p0 < NL; p0 += kPassBlocks) {
      const int p1 = p0 + kPassBlocks < NL ? p0 + kPassBlocks : NL;
#pragma unroll
      for (int t = p0; t < p1; ++t) {
        const int r = (t - p0) * 16 + (lane & 15);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint2 pk;
          pk.x = (uint32_t)f32_to_bf16(acc[t][q][0]) | ((uint32_t)f32_to_bf16(acc[t][q][1]) << 16);
          pk.y = (uint32_t)f32_to_bf16(acc[t][q][2]) | ((uint32_t)f32_to_bf16(acc[t][q][3]) << 16);
          const int ch = 2 * q + (kq >> 1);
          *reinterpret_cast<uint2*>(wl + r * 128 + ((ch ^ (r & 7)) << 4) + (kq & 1) * 8) = pk;
        }
      }
      __builtin_amdgcn_s_waitcnt(lgkm0_imm());
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < (p1 - p0) * 2; ++i) {
        const int r = i * 8 + (lane >> 3), c8 = lane & 7;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(wl + r * 128 + ((c8 ^ (r & 7)) << 4));
        const int trow = (wm + WMG * (p0 + (r >> 4))) * 16 + (r & 15);
        const int col = n0 + wn * 64 + c8 * 8;
        if (trow < mrows && col < NOUT) {
          u32x4_t* dst = reinterpret_cast<u32x4_t*>(C + (row0 + trow) * NOUT + col);
          if (WMG == 1) __builtin_nontemporal_store(v, dst);  // the wide shape: a weight stream (note above)
          else *dst = v;
        }
      }
      __builtin_amdgcn_s_waitcnt(lgkm0_imm());
      __builtin_amdgcn_wave_barrier();
    }
    return;
  }
  if (SWIGLU) {
    // GEMM 1: a wave's 16 rows x 32 h columns of one row block are exactly one 1 KiB
    // tile of the tiled layout.  Each lane puts its SwiGLU values into the wave's own
    // LDS (16-byte chunks XOR-swizzled by row / 4) and reads back the 16 bytes at its
    // position in the tile, so the block leaves as one contiguous 1 KiB store (rows
    // past mrows masked) instead of two stores of 32-byte pieces.
    constexpr int kPassBlocks = 4;  // 4 KiB per wave: the 8 waves stay inside stage 0
    char* wl = lds + wave * (kPassBlocks * 1024);
    const int col0 = n0 + wn * 32;
    if (col0 < NPAD) {
#pragma unroll
      for (int p0 = 0; p0 < NL; p0 += kPassBlocks) {
        const int p1 = p0 + kPassBlocks < NL ? p0 + kPassBlocks : NL;
#pragma unroll
        for (int t = p0; t < p1; ++t) {
          const int r = lane & 15;
#pragma unroll
          for (int qo = 0; qo < 2; ++qo) {
            uint16_t hv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float gv = acc[t][qo][i], uv = acc[t][2 + qo][i];
              hv[i] = f32_to_bf16(silu_mul(gv, uv));
            }
            uint2 pk;
            pk.x = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
            pk.y = (uint32_t)hv[2] | ((uint32_t)hv[3] << 16);
            const int ch = 2 * qo + (kq >> 1);
            *reinterpret_cast<uint2*>(wl + (t - p0) * 1024 + r * 64 + ((ch ^ ((r >> 2) & 3)) << 4) + (kq & 1) * 8) = pk;
          }
        }
        __builtin_amdgcn_s_waitcnt(lgkm0_imm());
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int t = p0; t < p1; ++t) {
          const int r = lane >> 2, c = lane & 3;
          const u32x4_t v =
              *reinterpret_cast<const u32x4_t*>(wl + (t - p0) * 1024 + r * 64 + ((c ^ ((r >> 2) & 3)) << 4));
          const int trow = (wm + WMG * t) * 16 + r;
          if (trow < mrows)
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(C + tiled_index(row0 + trow, col0 + c * 8, NPAD)));
        }
        __builtin_amdgcn_s_waitcnt(lgkm0_imm());
        __builtin_amdgcn_wave_barrier();
      }
    }
    return;
  }
  // combine epilogue: the token and gate of each of this lane's rows.  The loads are
  // unconditional (clamped indices) and their values used on every path, so none is
  // still outstanding when the next tile's reduction loop starts.
  int64_t ytoks[NL > 0 ? NL : 1];
  float ygs[NL > 0 ? NL : 1];
  if (!SWIGLU && op.Y) {
    int32_t pv[NL > 0 ? NL : 1];
#pragma unroll
    for (int t = 0; t < NL; ++t) {
      const int trow = (wm + WMG * t) * 16 + (lane & 15);
      pv[t] = op.perm[row0 + (trow < mrows ? trow : 0)];
    }
    float gv[NL > 0 ? NL : 1];
#pragma unroll
    for (int t = 0; t < NL; ++t) {
      const int trow = (wm + WMG * t) * 16 + (lane & 15);
      // (a live row always has a token; never store out of range)
      ytoks[t] = trow < mrows && pv[t] >= 0 && pv[t] < op.arows ? (int64_t)pv[t] : -1;
      gv[t] = op.gate[(ytoks[t] >= 0 ? ytoks[t] : 0) * op.gstride + op.gslot];
    }
#pragma unroll
    for (int t = 0; t < NL; ++t) ygs[t] = ytoks[t] >= 0 ? gv[t] : 0.f;
  }
#pragma unroll
  for (int t = 0; t < NL; ++t) {
    const int trow = (wm + WMG * t) * 16 + (lane & 15);
    if (trow < mrows) {
      const int64_t row = row0 + trow;
      const int64_t ytok = !SWIGLU && op.Y ? ytoks[t] : -1;
      const float yg = !SWIGLU && op.Y ? ygs[t] : 0.f;
#pragma unroll
      for (int qo = 0; qo < (SWIGLU ? 2 : 4); ++qo) {
        const int col = n0 + (SWIGLU ? wn * 32 : wn * 64) + qo * 16 + kq * 4;
        if (col < (SWIGLU ? NPAD : NOUT)) {
          uint16_t hv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v;
            if (SWIGLU) {
              const float gv = acc[t][qo][i], uv = acc[t][2 + qo][i];
              v = silu_mul(gv, uv);
            } else {
              v = acc[t][qo][i];
            }
            hv[i] = f32_to_bf16(v);
          }
          if (!SWIGLU && op.Y) {
            // y = gate * o with o rounded to bf16 first, exactly as the separate combine pass
            f32x4_t yv;
#pragma unroll
            for (int i = 0; i < 4; ++i) yv[i] = fmaf(yg, bf16_to_f32(hv[i]), 0.f);
            if (ytok >= 0) *reinterpret_cast<f32x4_t*>(op.Y + ytok * NOUT + col) = yv;
          } else {
            uint2 pk;
            pk.x = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
            pk.y = (uint32_t)hv[2] | ((uint32_t)hv[3] << 16);
            uint16_t* dst = SWIGLU ? C + tiled_index(row, col, NPAD) : C + row * NOUT + col;
            *reinterpret_cast<uint2*>(dst) = pk;
          }
        }
      }
    }
  }
}

// Per-expert rows (clipped to rows_cap) and first local rows P(e) (segments rounded
// up to 16 rows), for experts e_lo .. e_lo+E-1, by one wave; optionally also the
// inclusive prefix of tiles per expert (tiles of `bm` rows times nt column tiles).
__device__ __forceinline__ void expert_segments(const int32_t* __restrict__ offsets, int e_lo, int E, int64_t rows_cap,
                                                int bm, int nt, int* erow, int* pbase, int* tp) {
  const int lane = threadIdx.x & 63;
  int run_rows = 0, run_tiles = 0;
  for (int b = 0; b < E; b += 64) {
    const int i = b + lane;
    int rows = 0;
    if (i < E) {
      rows = offsets[e_lo + i + 1] - offsets[e_lo + i];
      if (rows < 0) rows = 0;
    }
    int prow = (rows + kSegAlign - 1) / kSegAlign * kSegAlign;
    int incl = prow;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(incl, off, 64);
      if (lane >= off) incl += u;
    }
    const int64_t p0 = (int64_t)run_rows + incl - prow;  // P(e)
    if (p0 + rows > rows_cap) rows = rows_cap > p0 ? (int)(rows_cap - p0) : 0;
    int tiles = ((rows + bm - 1) / bm) * nt;
    int tincl = tiles;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(tincl, off, 64);
      if (lane >= off) tincl += u;
    }
    if (i < E) {
      erow[i] = rows;
      pbase[i] = (int)p0;
      if (tp) tp[i] = run_tiles + tincl;
    }
    run_rows += __shfl(incl, 63, 64);
    run_tiles += __shfl(tincl, 63, 64);
  }
}



// One persistent launch runs the tiles of two problems: the routed experts (problem
// 0: segments from `offsets`) and, when rows1 > 0, one dense expert over rows1 rows
// (problem 1: the always-on shared expert), whose tiles follow the routed ones in the
// same list, so they fill the last, partly empty round of routed tiles instead of
// running as separate launches with half-empty rounds of their own.  (Spreading them
// evenly through the list was measured to cost 50% more HBM reads: tiles of unequal
// length let the workgroups drift apart, so the 16 column tiles of a routed expert no
// longer run together and its row panel leaves L2 between uses.)
//
// nts0 > 0 (GEMM 1 only): each routed expert's output columns go to nts0 column tiles of
// 32-column units as equal as the units allow -- the first U mod nts0 of them one unit
// wider, U = the columns in units -- instead of BNO-column tiles: for few rows per expert,
// where a tile is a weight stream, this makes the tiles fill whole rounds of the CUs (at
// 256 tokens x 64 experts x 1408 columns: 12 tiles of 128 and 96 columns per expert, every
// CU streams two of 128 and one of 96, instead of 11 of 128 in 2.75 rounds).  A wave whose
// 32 columns lie past its tile's runs no MFMAs and stores nothing, and the weight rows past
// the tile's load its last band again (a cache hit).  Every output is computed by one tile
// with the same reduction order as without the split: bit-identical.
template <bool SWIGLU, int WMG>
__global__ __launch_bounds__(kThreads) void ggemm_bf16_kernel(GemmOperands p0, const int32_t* __restrict__ offsets,
                                                              int e_lo, int E, int64_t rows_cap, GemmOperands p1,
                                                              int rows1, int nts0) {
  constexpr int kBM = TileShape<WMG>::BM, kBW = TileShape<WMG>::BW;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int tp[kMaxExperts];     // inclusive prefix of tiles per expert
  __shared__ int erow[kMaxExperts];   // rows per expert, clipped to rows_cap
  __shared__ int pbase[kMaxExperts];  // first local row of each expert (16-row aligned)
  __shared__ int ttab[kMaxExperts];   // token rows per m-tile of each expert (split_rows)
  constexpr int BNO = SWIGLU ? kBW / 2 : kBW;  // output columns per tile
  const bool split = SWIGLU && nts0 > 0;
  const int NT0 = split ? nts0 : (p0.NOUT + BNO - 1) / BNO;
  const int NT1 = (p1.NOUT + BNO - 1) / BNO;
  const int units0 = (p0.NOUT + 31) / 32;                             // 32-column units (split)
  const int ubase = split ? units0 / nts0 : 0, urem = split ? units0 % nts0 : 0;
  const int tid = threadIdx.x, wave = tid >> 6;

  if (wave == 0) expert_segments(offsets, e_lo, E, rows_cap, kBM, NT0, erow, pbase, tp);
  __syncthreads();
  // an expert's rows split evenly over its MT m-tiles (16-row multiples), so that 512
  // rows run as 2 x 256 rather than 320 + 192 and 1024 as 4 x 256 rather than three
  // full tiles and one of 64 rows: the tiles of a round stay of one length (Pro layer
  // 5.05 -> 4.69 ms, 16384-token Ultra layer -10%).  With MT <= kBM / 16 every tile
  // keeps live rows (the last one starts at (MT - 1) * rows < the expert's rows);
  // larger MT keep kBM-row tiles.  Computed once per expert here: the same division
  // in every tile's set-up slowed the down GEMM by 2%.
  auto split_rows = [](int rows) {
    const int mt = (rows + kBM - 1) / kBM;
    return mt >= 1 && mt <= kBM / 16 ? (int)round_up((rows + mt - 1) / mt, kTileRows) : kBM;
  };
  for (int i = tid; i < E; i += kThreads) ttab[i] = split_rows(erow[i]);
  const int trows1 = split_rows(rows1);
  __syncthreads();
  const int n0 = E > 0 ? tp[E - 1] : 0;
  const int n1 = rows1 > 0 ? ((rows1 + kBM - 1) / kBM) * NT1 : 0;
  const int total = n0 + n1;

  const int P = gridDim.x;  // multiple of 8
  const int per_xcd = P >> 3;
  const int slot = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);

  const int wm = WMG == 2 ? wave >> 2 : 0;
  const int wn = WMG == 2 ? wave & 3 : wave;  // this wave's 32 output columns of a GEMM 1 tile
  // a tile's wave-uniform description from its index in the list
  auto decode = [&](int tile, bool& dense, int& mrows, int64_t& row0, int& ncol0, int& nl, int& nkf,
                    const uint16_t*& wb0, const uint16_t*& wb1, int& wbands, int& krot) {
    dense = tile >= n0;
    const GemmOperands& op = dense ? p1 : p0;
    int ei = 0, q, erows, pb, trows;
    if (dense) {
      q = tile - n0;
      erows = rows1;
      pb = 0;
      trows = trows1;
    } else {
      q = tile;
      // expert of this tile: first i with tp[i] > q
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (tp[mid] > q) hi = mid; else lo = mid + 1;
      }
      ei = lo;
      q -= ei > 0 ? tp[ei - 1] : 0;
      erows = erow[ei];
      pb = pbase[ei];
      trows = ttab[ei];
    }
    const int NT = dense ? NT1 : NT0;
    const int MT = (erows + kBM - 1) / kBM;
    // grouped order: groups of kGroupM m-tiles; inside a group n outer, m inner
    const int gsz = kGroupM * NT;
    const int g = q / gsz, qi = q - g * gsz;
    const int gm0 = g * kGroupM;
    const int gm = (MT - gm0) < kGroupM ? (MT - gm0) : kGroupM;
    const int mt = gm0 + qi % gm, nt = qi / gm;
    row0 = (int64_t)pb + (int64_t)mt * trows;  // multiple of 16
    mrows = (erows - mt * trows) < trows ? (erows - mt * trows) : trows;
    const bool sp = split && !dense;
    const int width = sp ? 32 * (ubase + (nt < urem ? 1 : 0)) : BNO;  // this tile's output columns
    ncol0 = sp ? 32 * (nt * ubase + (nt < urem ? nt : urem)) : nt * BNO;
    const int wrows = (int)round_up(op.NOUT, kWeightRowAlign);  // packed weight rows per expert
    wb0 = op.B0 + (int64_t)ei * wrows * op.KP;
    wb1 = SWIGLU ? op.B1 + (int64_t)ei * wrows * op.KP : wb0;
    wbands = wrows / kTileRows;
    if (sp && (ncol0 + width) / kTileRows < wbands) wbands = (ncol0 + width) / kTileRows;  // the tile's last band
    nkf = op.KP / kTileCols;
    // GEMM 1's first reduction step is staggered by expert: the workgroups then do not all
    // stream the same column range of their weight bands at once (gate/up -2 to -3%), while
    // all tiles of one expert still start together and share its token rows in L2.  The
    // offset is keyed on the absolute expert id (and 0 for the dense shared-expert problem),
    // so the order of an output's float32 sums depends on that expert alone: the same under
    // both tile shapes, for any expert range of the call, and for the shared expert fused
    // into the routed launch or run on its own.  (GEMM 2 measured 0-2% slower with it.)
    krot = SWIGLU && !dense ? (int)(((int64_t)(e_lo + ei) * 37) % nkf) : 0;
    // live row blocks of this wave (wave-uniform): block wm + WMG t is live if it starts below mrows
    const int nrb = (mrows + 15) / 16;
    nl = nrb > wm ? (nrb - wm + WMG - 1) / WMG : 0;
    if (sp && wn * 32 >= width) nl = 0;  // columns past the tile: no MFMAs, no stores
  };

  if (slot >= total) return;
  bool c_dense;
  int c_mrows, c_ncol0, c_nl, c_nkf, c_wbands, c_krot;
  int64_t c_row0;
  const uint16_t *c_wb0, *c_wb1;
  decode(slot, c_dense, c_mrows, c_row0, c_ncol0, c_nl, c_nkf, c_wb0, c_wb1, c_wbands, c_krot);
  int32_t tokc[5], tokn[5];
  if constexpr (SWIGLU) token_rows<WMG>(c_dense ? p1 : p0, c_row0 / kTileRows, c_mrows, tokc);
  bool pre = false;  // this tile's steps 0-2 were issued by the previous one
  for (int tile = slot; tile < total; tile += P) {
    const bool more = tile + P < total;
    bool n_dense = false;
    int n_mrows = 1, n_ncol0 = 0, n_nl = 0, n_nkf = 0, n_wbands = 1, n_krot = 0;
    int64_t n_row0 = 0;
    const uint16_t *n_wb0 = c_wb0, *n_wb1 = c_wb1;
    if (more) decode(tile + P, n_dense, n_mrows, n_row0, n_ncol0, n_nl, n_nkf, n_wb0, n_wb1, n_wbands, n_krot);
    if constexpr (SWIGLU) {  // the next tile's gathered tokens, a whole tile ahead of their use
      if (more) token_rows<WMG>(n_dense ? p1 : p0, n_row0 / kTileRows, n_mrows, tokn);
      else {
#pragma unroll
        for (int j = 0; j < 5; ++j) tokn[j] = tokc[j];
      }
    } else {
      token_rows<WMG>(c_dense ? p1 : p0, c_row0 / kTileRows, c_mrows, tokc);
    }
    // GEMM 1 chains; GEMM 2 (64-step tiles at 2048 columns) keeps its epilogue in two
    // passes over the whole ring instead, which measured faster than five in one stage
    const bool chain = SWIGLU && more && c_nkf >= 3 && n_nkf >= 3;
    const GemmOperands& op = c_dense ? p1 : p0;
    const GemmOperands& nop = n_dense ? p1 : p0;
    const NextTile nx{n_wb0, n_wb1, n_row0 / kTileRows, n_wbands, n_nkf, n_ncol0, n_mrows, n_krot, 0};
    const int npad = (int)round_up(op.NOUT, kTileCols);
#define MOGE_TILE(NLV)                                                                                               \
  tile_compute<SWIGLU, NLV, WMG>(op, lds, c_wb0, c_wb1, c_wbands, c_nkf, c_mrows, c_row0, c_ncol0, op.NOUT, npad, op.C, \
                                 tokc, pre, chain, nop, nx, tokn, c_krot)
    switch (c_nl) {
      case 10: if constexpr (TileShape<WMG>::kBlocks >= 10) MOGE_TILE(10); break;
      case 9: if constexpr (TileShape<WMG>::kBlocks >= 9) MOGE_TILE(9); break;
      case 8: if constexpr (TileShape<WMG>::kBlocks >= 8) MOGE_TILE(8); break;
      case 7: if constexpr (TileShape<WMG>::kBlocks >= 7) MOGE_TILE(7); break;
      case 6: MOGE_TILE(6); break;
      case 5: MOGE_TILE(5); break;
      case 4: MOGE_TILE(4); break;
      case 3: MOGE_TILE(3); break;
      case 2: MOGE_TILE(2); break;
      case 1: MOGE_TILE(1); break;
      default: MOGE_TILE(0); break;
    }
#undef MOGE_TILE
    __syncthreads();  // LDS stages are reused by the next tile
    pre = chain;
    c_dense = n_dense; c_mrows = n_mrows; c_row0 = n_row0; c_ncol0 = n_ncol0; c_nl = n_nl; c_nkf = n_nkf;
    c_wb0 = n_wb0; c_wb1 = n_wb1; c_wbands = n_wbands; c_krot = n_krot;
    if constexpr (SWIGLU) {
#pragma unroll
      for (int j = 0; j < 5; ++j) tokc[j] = tokn[j];
    }
  }
}

// ----------------------------------------------------------------------------
// float32 vector-ALU pair (small shapes): one thread per output element, same
// layouts as the bf16 kernels (tiled x_perm and h, packed weights, row-major out).
// Each workgroup first derives the experts' segments.
__device__ __forceinline__ int segment_of_row(const int* __restrict__ pbase, int E, int64_t r) {
  int lo = 0, hi = E - 1;  // last i with pbase[i] <= r
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pbase[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void ffn_f32_gateup_kernel(const float* __restrict__ X, const int32_t* __restrict__ offsets,
                                                             int e_lo, int E, int64_t rows_cap, const float* __restrict__ Wg,
                                                             const float* __restrict__ Wu, int d, int F, float* __restrict__ H) {
  __shared__ int erow[kMaxExperts], pbase[kMaxExperts];
  if (threadIdx.x < 64) expert_segments(offsets, e_lo, E, rows_cap, 1, 1, erow, pbase, nullptr);
  __syncthreads();
  const int64_t dp = round_up(d, kTileCols), fp = round_up(F, kTileCols), wr = round_up(F, kWeightRowAlign);
  const int64_t rows = (int64_t)pbase[E - 1] + erow[E - 1];
  const int64_t n = rows * fp;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / fp;
    const int f = (int)(i - r * fp);
    const int e = segment_of_row(pbase, E, r);
    if (r - pbase[e] >= erow[e]) continue;  // padding row
    const float* wg = Wg + (int64_t)e * wr * dp;
    const float* wu = Wu + (int64_t)e * wr * dp;
    float a = 0.f, b = 0.f;
    for (int c = 0; c < d; ++c) {
      const float xv = X[tiled_index(r, c, dp)];
      a = fmaf(xv, wg[tiled_index(f, c, dp)], a);
      b = fmaf(xv, wu[tiled_index(f, c, dp)], b);
    }
    H[tiled_index(r, f, fp)] = a / (1.f + expf(-a)) * b;
  }
}

__global__ __launch_bounds__(256) void ffn_f32_down_kernel(const float* __restrict__ H, const int32_t* __restrict__ offsets,
                                                           int e_lo, int E, int64_t rows_cap, const float* __restrict__ Wd,
                                                           int d, int F, float* __restrict__ O) {
  __shared__ int erow[kMaxExperts], pbase[kMaxExperts];
  if (threadIdx.x < 64) expert_segments(offsets, e_lo, E, rows_cap, 1, 1, erow, pbase, nullptr);
  __syncthreads();
  const int64_t fp = round_up(F, kTileCols), wr = round_up(d, kWeightRowAlign);
  const int64_t rows = (int64_t)pbase[E - 1] + erow[E - 1];
  const int64_t n = rows * d;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / d;
    const int j = (int)(i - r * d);
    const int e = segment_of_row(pbase, E, r);
    if (r - pbase[e] >= erow[e]) continue;  // padding row
    const float* wd = Wd + (int64_t)e * wr * fp;
    float acc = 0.f;
    for (int f = 0; f < F; ++f) acc = fmaf(H[tiled_index(r, f, fp)], wd[tiled_index(j, f, fp)], acc);
    O[r * d + j] = acc;
  }
}

// CUs of the current device, queried once per process (thread-safe static init);
// the persistent grids are sized to it (any size is correct, this one fills the chip).
static int query_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}
static int device_cus() {
  static const int cus = query_cus();
  return cus;
}

// rows1 = 0: routed problem only.
template <bool SWIGLU, int WMG>
static moge_status_t launch_ggemm_shape(const GemmOperands& p0, const int32_t* offsets, int e_lo, int E,
                                        int64_t rows_cap, const GemmOperands& p1, int rows1, int nts0,
                                        hipStream_t stream) {
  constexpr int kBM = TileShape<WMG>::BM, kBW = TileShape<WMG>::BW;
  moge_status_t st = raise_dynamic_lds(reinterpret_cast<const void*>(ggemm_bf16_kernel<SWIGLU, WMG>), gemm_lds<WMG>(),
                                       "ggemm_bf16_kernel");
  if (st != MOGE_OK) return st;
  constexpr int BNO = SWIGLU ? kBW / 2 : kBW;
  const int64_t nt0 = SWIGLU && nts0 > 0 ? nts0 : (p0.NOUT + BNO - 1) / BNO;
  const int64_t upper = ((rows_cap + kBM - 1) / kBM + E) * nt0 +
                        ((int64_t)rows1 + kBM - 1) / kBM * ((p1.NOUT + BNO - 1) / BNO);  // >= live tiles
  int64_t grid = device_cus();  // one 144-152 KiB-LDS workgroup per CU
  if (upper < grid) grid = upper;
  grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL((ggemm_bf16_kernel<SWIGLU, WMG>), dim3((unsigned)grid), dim3(kThreads), gemm_lds<WMG>(), stream,
                     p0, offsets, e_lo, E, rows_cap, p1, rows1, SWIGLU ? nts0 : 0);
  return check_launch(SWIGLU ? "ggemm_bf16_kernel<gate_up>" : "ggemm_bf16_kernel<down>");
}

// The tile table ([P1] section 3: SwiftGMM picks its tiling from a cache keyed by the
// problem and switches to a matrix-vector-like mode when the rows are few).  Here the
// candidates are the two tile shapes and the key is the shape of the call: the rows per
// expert expected under MoGE routing (every group receives exactly T K' rows, so an expert
// averages T K' / (N / M)), the experts of the call, the output width and the CU count.
// Few rows per expert make a GEMM a weight stream whose time is set by the CU that streams
// the most weight rows: every tile streams its BW weight rows over the whole reduction, and
// the persistent grid hands tile i to workgroup i mod CUs, so that CU streams
// ceil(tiles / CUs) * BW rows.  The table takes the shape with the smaller figure, the wide
// one on a tie (twice the weight bytes in flight per step).  Measured at 64-512 tokens x
// 4096 x 64 experts over expert ranges of 16-64, this picks the faster shape of each GEMM
// (e.g. gate/up at 256 tokens: 704 tall tiles = 3 rounds x 256 rows against 384 wide tiles
// = 2 rounds x 512 rows, 289 against 300 us); many rows per expert give the tall shape
// anyway (a wide tile then splits an expert into several m-tiles).
static int64_t tile_rounds_rows(int bm, int bw, bool swiglu, int64_t rows_per_expert, int64_t E, int64_t nout,
                                int64_t rows1, int64_t nout1, int64_t cus) {
  const int64_t bno = swiglu ? bw / 2 : bw;
  auto tiles_of = [&](int64_t rows, int64_t n) { return ((rows + bm - 1) / bm) * ((n + bno - 1) / bno); };
  int64_t tiles = E * tiles_of(rows_per_expert > 0 ? rows_per_expert : 1, nout);
  if (rows1 > 0) tiles += tiles_of(rows1, nout1);
  return (tiles + cus - 1) / cus * bw;
}

static int64_t expected_rows_per_expert(const moge_shape_t& s) {
  const int64_t G = s.N / s.M;
  return ((int64_t)s.T * s.k_per_group + G - 1) / G;
}

static bool wide_tiles(const moge_shape_t& s, bool swiglu, int64_t E, int64_t nout, int64_t rows1, int64_t nout1) {
  if (s.tiles != MOGE_TILES_AUTO) return s.tiles == MOGE_TILES_WIDE;
  const int64_t rows_per_expert = expected_rows_per_expert(s);
  const int64_t cus = device_cus();
  const int64_t tall = tile_rounds_rows(TileShape<2>::BM, TileShape<2>::BW, swiglu, rows_per_expert, E, nout, rows1,
                                        nout1, cus);
  const int64_t wide = tile_rounds_rows(TileShape<1>::BM, TileShape<1>::BW, swiglu, rows_per_expert, E, nout, rows1,
                                        nout1, cus);
  return wide <= tall;
}

// Weight rows streamed by the busiest workgroup of a tall GEMM 1 launch whose routed experts
// (E of them, rows_per_expert rows each) have their F output columns in nts column tiles
// (nts = 0: the plain 128-column tiles), followed by the shared expert's tiles: the tiles in
// the kernel's list order (per expert: groups of 4 m-tiles, column tiles outer), tile i on
// workgroup slot i mod CUs, a tile of c columns streaming 2c weight rows.
static int64_t split_busiest_rows(int64_t rows_per_expert, int64_t E, int64_t nout, int nts, int64_t rows1,
                                  int64_t nout1, int64_t cus) {
  constexpr int BM = TileShape<2>::BM, BNO = TileShape<2>::BW / 2;
  const int64_t units = (nout + 31) / 32;
  const int64_t nt = nts > 0 ? nts : (nout + BNO - 1) / BNO;
  std::vector<int64_t> load((size_t)cus, 0);
  int64_t i = 0;
  auto add = [&](int64_t cols) { load[(size_t)(i++ % cus)] += 2 * cols; };
  const int64_t mt = (rows_per_expert > 0 ? rows_per_expert + BM - 1 : BM) / BM;
  for (int64_t e = 0; e < E; ++e)
    for (int64_t g0 = 0; g0 < mt; g0 += kGroupM)
      for (int64_t n = 0; n < nt; ++n)
        for (int64_t m = g0; m < mt && m < g0 + kGroupM; ++m) {
          if (nts > 0) add(32 * (units / nts + (n < units % nts ? 1 : 0)));
          else add(std::min<int64_t>(BNO, nout - n * BNO));
        }
  if (rows1 > 0) {
    const int64_t mt1 = (rows1 + BM - 1) / BM, nt1 = (nout1 + BNO - 1) / BNO;
    for (int64_t m = 0; m < mt1; ++m)
      for (int64_t n = 0; n < nt1; ++n) add(std::min<int64_t>(BNO, nout1 - n * BNO));
  }
  return *std::max_element(load.begin(), load.end());
}

// Column tiles per routed expert for a tall GEMM 1 (0: the plain 128-column tiles).  With few
// rows per expert (at most 64, where a tile is a weight stream) the table also weighs splits of
// an expert's columns into nts tiles of 4 and 3 units (128 and 96 columns; up to 8 more tiles
// than the plain ones), and takes the split whose busiest workgroup streams the fewest weight
// rows if it beats the plain tiles; MOGE_TILES_BALANCED takes the best split whenever one
// exists.  Measured (4096 hidden, 64 experts, 1408 columns, same box): 64 tokens 249 -> 239 us,
// 256 tokens within 1%, 512 tokens (128 rows per expert) 1% slower, hence the limit; the gain
// is smaller than the busiest workgroup's share suggests because the workgroups that finish
// first leave their HBM bandwidth to the others.
static int gate_up_split(const moge_shape_t& s, int64_t E, int64_t nout, int64_t rows1, int64_t nout1) {
  const bool forced = s.tiles == MOGE_TILES_BALANCED;
  if (!forced && (s.tiles != MOGE_TILES_AUTO || wide_tiles(s, true, E, nout, rows1, nout1))) return 0;
  const int64_t rows_per_expert = expected_rows_per_expert(s);
  if (!forced && rows_per_expert > 64) return 0;
  const int64_t cus = device_cus();
  const int64_t units = (nout + 31) / 32;
  const int64_t plain = (units + 3) / 4;
  int best = 0;
  int64_t best_rows = forced ? INT64_MAX : split_busiest_rows(rows_per_expert, E, nout, 0, rows1, nout1, cus);
  for (int64_t nts = plain + 1; units / nts >= 3 && nts <= plain + 8; ++nts) {
    const int64_t r = split_busiest_rows(rows_per_expert, E, nout, (int)nts, rows1, nout1, cus);
    if (r < best_rows) {
      best_rows = r;
      best = (int)nts;
    }
  }
  return best;
}

template <bool SWIGLU>
static moge_status_t launch_ggemm(const moge_shape_t& s, const GemmOperands& p0, const int32_t* offsets, int e_lo,
                                  int E, int64_t rows_cap, const GemmOperands& p1, int rows1, hipStream_t stream) {
  if (wide_tiles(s, SWIGLU, E, p0.NOUT, rows1, p1.NOUT))
    return launch_ggemm_shape<SWIGLU, 1>(p0, offsets, e_lo, E, rows_cap, p1, rows1, 0, stream);
  const int nts0 = SWIGLU ? gate_up_split(s, E, p0.NOUT, rows1, p1.NOUT) : 0;
  return launch_ggemm_shape<SWIGLU, 2>(p0, offsets, e_lo, E, rows_cap, p1, rows1, nts0, stream);
}

static GemmOperands operands(const void* A, const void* B0, const void* B1, void* C, int NOUT, int KD,
                             int amode = 0, const int32_t* perm = nullptr, int64_t arows = 0, int64_t prows = 0) {
  return GemmOperands{static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B0),
                      static_cast<const uint16_t*>(B1), static_cast<uint16_t*>(C), NOUT,
                      (int)round_up(KD, kTileCols), amode, perm, arows, prows, nullptr, nullptr, 0, 0};
}

}  // namespace moge

using namespace moge;

static moge_status_t ffn_common_checks(const moge_shape_t* shape, int32_t e_lo, int32_t e_hi, int64_t rows_cap) {
  moge_status_t st = validate_shape(shape);
  if (st != MOGE_OK) return st;
  if (shape->F <= 0) return fail(MOGE_ERR_SHAPE, "the expert FFN needs F > 0");
  if (e_lo < 0 || e_hi > shape->N || e_lo >= e_hi) return fail(MOGE_ERR_ARG, "need 0 <= e_lo < e_hi <= N");
  if (rows_cap < 1) return fail(MOGE_ERR_CAPACITY, "rows_cap must be >= 1");
  if (rows_cap >= (int64_t(1) << 31) - kMaxBM) return fail(MOGE_ERR_CAPACITY, "rows_cap must be < 2^31 - 320");
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
    const GemmOperands none{};
    st = launch_ggemm<true>(s, operands(x_perm, w_gate, w_up, h, s.F, s.d), offsets, e_lo, e_hi - e_lo, rows_cap, none,
                            0, stream);
  } else {
    hipLaunchKernelGGL(ffn_f32_gateup_kernel, dim3((unsigned)grid_1d(rows_cap * round_up(s.F, kTileCols))), dim3(256),
                       0, stream, static_cast<const float*>(x_perm), offsets, e_lo, e_hi - e_lo, rows_cap,
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
    const GemmOperands none{};
    st = launch_ggemm<false>(s, operands(h, w_down, nullptr, out, s.d, s.F), offsets, e_lo, e_hi - e_lo, rows_cap, none,
                             0, stream);
  } else {
    hipLaunchKernelGGL(ffn_f32_down_kernel, dim3((unsigned)grid_1d(rows_cap * s.d)), dim3(256), 0, stream,
                       static_cast<const float*>(h), offsets, e_lo, e_hi - e_lo, rows_cap,
                       static_cast<const float*>(w_down), s.d, s.F, static_cast<float*>(out));
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

// ---- routed experts and the shared expert in the same two launches
static moge_status_t shared_checks(const moge_shape_t* shape, int32_t F_shared, int32_t e_lo, int32_t e_hi,
                                   int64_t rows_cap) {
  moge_status_t st = ffn_common_checks(shape, e_lo, e_hi, rows_cap);
  if (st != MOGE_OK) return st;
  if (F_shared < 8 || F_shared % 8 != 0) return fail(MOGE_ERR_SHAPE, "F_shared must be a positive multiple of 8");
  if (shape->dtype != MOGE_BF16)
    return fail(MOGE_ERR_DTYPE, "the fused shared-expert calls are bf16 only; float32 uses moge_grouped_ffn twice");
  return MOGE_OK;
}

extern "C" moge_status_t moge_expert_gate_up_with_shared(const moge_shape_t* shape, int32_t F_shared,
                                                         const void* x_perm, const int32_t* offsets, int32_t e_lo,
                                                         int32_t e_hi, int64_t rows_cap, const void* w_gate,
                                                         const void* w_up, void* h, const void* x_tiled,
                                                         const void* ws_gate, const void* ws_up, void* hs,
                                                         hipStream_t stream) {
  moge_status_t st = shared_checks(shape, F_shared, e_lo, e_hi, rows_cap);
  if (st != MOGE_OK) return st;
  if (!x_perm || !offsets || !w_gate || !w_up || !h || !x_tiled || !ws_gate || !ws_up || !hs)
    return fail(MOGE_ERR_NULL, "every operand is required");
  const moge_shape_t& s = *shape;
  st = launch_ggemm<true>(s, operands(x_perm, w_gate, w_up, h, s.F, s.d), offsets, e_lo, e_hi - e_lo, rows_cap,
                          operands(x_tiled, ws_gate, ws_up, hs, F_shared, s.d), s.T, stream);
  return st == MOGE_OK ? ok() : st;
}

extern "C" moge_status_t moge_expert_down_with_shared(const moge_shape_t* shape, int32_t F_shared, const void* h,
                                                      const int32_t* offsets, int32_t e_lo, int32_t e_hi,
                                                      int64_t rows_cap, const void* w_down, void* out, const void* hs,
                                                      const void* ws_down, void* out_shared, hipStream_t stream) {
  moge_status_t st = shared_checks(shape, F_shared, e_lo, e_hi, rows_cap);
  if (st != MOGE_OK) return st;
  if (!h || !offsets || !w_down || !out || !hs || !ws_down || !out_shared)
    return fail(MOGE_ERR_NULL, "every operand is required");
  const moge_shape_t& s = *shape;
  st = launch_ggemm<false>(s, operands(h, w_down, nullptr, out, s.d, s.F), offsets, e_lo, e_hi - e_lo, rows_cap,
                           operands(hs, ws_down, nullptr, out_shared, s.d, F_shared), s.T, stream);
  return st == MOGE_OK ? ok() : st;
}

extern "C" moge_status_t moge_expert_gate_up_gather(const moge_shape_t* shape, const void* x, const int32_t* perm,
                                                    const int32_t* offsets, int32_t e_lo, int32_t e_hi,
                                                    int64_t rows_cap, const void* w_gate, const void* w_up, void* h,
                                                    int32_t F_shared, const void* ws_gate, const void* ws_up, void* hs,
                                                    hipStream_t stream) {
  moge_status_t st = ffn_common_checks(shape, e_lo, e_hi, rows_cap);
  if (st != MOGE_OK) return st;
  const moge_shape_t& s = *shape;
  if (s.dtype != MOGE_BF16) return fail(MOGE_ERR_DTYPE, "moge_expert_gate_up_gather is bf16 only");
  if (s.d % kTileCols != 0) return fail(MOGE_ERR_SHAPE, "moge_expert_gate_up_gather needs d % 32 == 0");
  if (!x || !perm || !offsets || !w_gate || !w_up || !h)
    return fail(MOGE_ERR_NULL, "x, perm, offsets, w_gate, w_up and h are required");
  if (F_shared < 0 || (F_shared > 0 && F_shared % 8 != 0))
    return fail(MOGE_ERR_SHAPE, "F_shared must be 0 or a positive multiple of 8");
  if (F_shared > 0 && (!ws_gate || !ws_up || !hs))
    return fail(MOGE_ERR_NULL, "ws_gate, ws_up and hs are required when F_shared > 0");
  if (F_shared == 0 && (ws_gate || ws_up || hs)) return fail(MOGE_ERR_ARG, "F_shared == 0 takes no shared operands");
  const GemmOperands none{};
  st = launch_ggemm<true>(s, operands(x, w_gate, w_up, h, s.F, s.d, kAGather, perm, s.T, rows_cap), offsets, e_lo, e_hi - e_lo,
                          rows_cap,
                          F_shared ? operands(x, ws_gate, ws_up, hs, F_shared, s.d, kARows, nullptr, s.T) : none,
                          F_shared ? s.T : 0, stream);
  return st == MOGE_OK ? ok() : st;
}

extern "C" moge_status_t moge_expert_down_combine(const moge_shape_t* shape, const void* h, const int32_t* offsets,
                                                  int32_t e_lo, int32_t e_hi, int64_t rows_cap, const void* w_down,
                                                  const int32_t* perm, const float* gate, float* y,
                                                  hipStream_t stream) {
  moge_status_t st = ffn_common_checks(shape, e_lo, e_hi, rows_cap);
  if (st != MOGE_OK) return st;
  const moge_shape_t& s = *shape;
  if (s.dtype != MOGE_BF16) return fail(MOGE_ERR_DTYPE, "moge_expert_down_combine is bf16 only");
  const int G = s.N / s.M;
  if (s.k_per_group != 1 || e_lo % G != 0 || e_hi != e_lo + G)
    return fail(MOGE_ERR_ARG, "moge_expert_down_combine needs k_per_group == 1 and [e_lo, e_hi) one whole group");
  if (!h || !offsets || !w_down || !perm || !gate || !y)
    return fail(MOGE_ERR_NULL, "h, offsets, w_down, perm, gate and y are required");
  GemmOperands p = operands(h, w_down, nullptr, nullptr, s.d, s.F);
  p.perm = perm;
  p.arows = s.T;
  p.Y = y;
  p.gate = gate;
  p.gstride = s.M;       // K = M slots per token (k_per_group == 1)
  p.gslot = e_lo / G;    // the slot of this group
  const GemmOperands none{};
  st = launch_ggemm<false>(s, p, offsets, e_lo, e_hi - e_lo, rows_cap, none, 0, stream);
  return st == MOGE_OK ? ok() : st;
}

extern "C" int32_t moge_tile_choice(const moge_shape_t* shape, int32_t gemm, int32_t e_lo, int32_t e_hi,
                                    int32_t F_shared) {
  if (validate_shape(shape) != MOGE_OK || shape->F <= 0) return -1;
  if ((gemm != 1 && gemm != 2) || e_lo < 0 || e_hi > shape->N || e_lo >= e_hi || F_shared < 0) return -1;
  const moge_shape_t& s = *shape;
  const bool swiglu = gemm == 1;
  const int64_t nout = swiglu ? s.F : s.d, nout1 = swiglu ? F_shared : s.d;
  const int64_t rows1 = F_shared > 0 ? s.T : 0;
  if (wide_tiles(s, swiglu, e_hi - e_lo, nout, rows1, nout1)) return MOGE_TILES_WIDE;
  return swiglu && gate_up_split(s, e_hi - e_lo, nout, rows1, nout1) > 0 ? MOGE_TILES_BALANCED : MOGE_TILES_TALL;
}
