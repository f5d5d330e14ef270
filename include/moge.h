/*
 * moge.h -- C ABI of libmoge, the forward pass of one MoGE (Mixture of Grouped
 * Experts) layer on an AMD Instinct MI355X (gfx950).
 *
 * Method sources (web pages about "Pangu Pro MoE: Mixture of Grouped Experts
 * for Efficient Sparsity", arXiv 2505.21411):
 *   [P1] lsdiaocha.cn long-form summary of the paper, section 1 (architecture):
 *        N experts split evenly into M groups of N/M, one group per device;
 *        each token takes a softmax over all N experts and then keeps the
 *        K' = K/M best experts inside every group; the imbalance score is the
 *        workload gap between the busiest and the idlest device, and is zero
 *        for MoGE by construction.
 *   [P5] hyper.ai page with the paper's abstract: tokens activate an equal
 *        number of experts in each predefined group.
 *   [P4] reportify.cn digests of Pangu Ultra MoE (dropless training, one
 *        always-on shared expert).
 * The expert is a SwiGLU feed-forward block without biases:
 *   FFN_e(x) = W_down[e] . ( silu(W_gate[e] . x) * (W_up[e] . x) ).
 *
 * Conventions for every call
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates or frees device memory and keeps no state between calls
 *     (every setting, such as the expert GEMMs' tile shape, travels with the
 *     call in moge_shape_t).  The one exception is moge_dispatch_noalloc's fixed
 *     device array, described there.
 *   - Tensors are contiguous.  x, logits, idx, gate, inv, the expert outputs
 *     and y are row-major; the operands of the expert GEMMs use the tiled
 *     layout described at moge_tiled_elems.  Weights come in the
 *     (out_features, in_features) layout of a linear layer:
 *       w_router [N][d];  w_gate, w_up [E][F][d];  w_down [E][d][F]
 *     where E is the number of experts the array holds; the expert weights are
 *     packed once into the tiled layout (moge_pack_weights) before use.
 *   - dtype MOGE_BF16: x, weights, x_perm, h and expert outputs are bf16
 *     (uint16 bit patterns); logits, gates and y are float32; bf16 matrix
 *     products use MFMA with float32 accumulation.
 *     dtype MOGE_F32: every tensor is float32 and products use plain float32
 *     vector arithmetic.
 *   - Every call validates its arguments on the host BEFORE any launch and
 *     returns a status; on error nothing is launched and moge_last_error()
 *     (per thread) describes the problem.  On success the work is enqueued on
 *     `stream` and the call returns without waiting for it (moge_check_finite,
 *     a checking call, is the one that waits).
 *   - Calls on different streams are independent; the library is re-entrant.
 */
#ifndef MOGE_H
#define MOGE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOGE_OK = 0,
  MOGE_ERR_ARG = 1,        /* an argument is out of range (mode, expert range, ...) */
  MOGE_ERR_SHAPE = 2,      /* the shape breaks a rule listed at moge_shape_t */
  MOGE_ERR_NULL = 3,       /* a required pointer is NULL */
  MOGE_ERR_WORKSPACE = 4,  /* workspace missing or smaller than moge_workspace_size() */
  MOGE_ERR_DTYPE = 5,      /* unknown dtype */
  MOGE_ERR_HIP = 6,        /* a HIP launch failed (message has the HIP error) */
  MOGE_ERR_CAPACITY = 7,   /* rows_cap is below the row bound of the call */
  MOGE_ERR_NONFINITE = 8   /* moge_check_finite found a NaN or an infinity */
} moge_status_t;

typedef enum { MOGE_BF16 = 0, MOGE_F32 = 1 } moge_dtype_t;

/* MOGE_ROUTE_GROUPED: MoGE, top-K' inside each of the M groups ([P1] section 1).
 * MOGE_ROUTE_GLOBAL:  the conventional router, top-K over all N experts with
 *                     K = M*K' ([P1] section 1 contrasts MoGE with it). */
typedef enum { MOGE_ROUTE_GROUPED = 0, MOGE_ROUTE_GLOBAL = 1 } moge_route_mode_t;

/* Workspace stages for moge_workspace_size(). */
typedef enum { MOGE_STAGE_DISPATCH = 1, MOGE_STAGE_CHECK = 2, MOGE_STAGE_ROUTE = 3 } moge_stage_t;

/* Tile shape of the bf16 expert GEMMs (moge_shape_t.tiles).  Every output is
 * bit-identical under all of them (same reduction order per output element).
 *   MOGE_TILES_AUTO  the library's choice for each GEMM from its shape (the
 *                    default, 0): the tile table of moge_tile_choice, which plays
 *                    the part of the grouped matmul's tiling cache and its switch
 *                    of mode by workload ([P1] section 3, SwiftGMM);
 *   MOGE_TILES_TALL  320 token rows x 256 weight rows;
 *   MOGE_TILES_WIDE  96 token rows x 512 weight rows (few rows per expert);
 *   MOGE_TILES_BALANCED  the tall tiles, with the gate/up GEMM's columns of each
 *                    routed expert split into tiles of 128 and 96 columns (256
 *                    and 192 weight rows) so that the tiles fill whole rounds of
 *                    the CUs (few rows per expert, e.g. 1408 columns as 8 x 128 +
 *                    4 x 96); the down GEMM as MOGE_TILES_TALL. */
#define MOGE_TILES_AUTO 0
#define MOGE_TILES_TALL 1
#define MOGE_TILES_WIDE 2
#define MOGE_TILES_BALANCED 3

/*
 * Layer shape.  Rules checked by moge_validate():
 *   T >= 1 tokens; d >= 8 hidden, d % 8 == 0; 1 <= M <= N experts, N % M == 0;
 *   1 <= k_per_group (K') <= N/M; K = M*K' slots per token (so K <= N);
 *   F expert width: F == 0 (routing only) or F >= 8 with F % 8 == 0;
 *   T*K < 2^31;  N <= 256 (both dtypes);  dtype in moge_dtype_t;
 *   tiles: MOGE_TILES_AUTO, _TALL, _WIDE or _BALANCED (a zero-initialised
 *   struct: AUTO).
 * Groups are contiguous blocks of expert ids: group(e) = e / (N/M).
 */
typedef struct {
  int32_t T;
  int32_t d;
  int32_t N;
  int32_t M;
  int32_t k_per_group;
  int32_t F;
  int32_t dtype;
  int32_t tiles;
} moge_shape_t;

/* Host-only shape check (no device call; usable without a GPU). */
moge_status_t moge_validate(const moge_shape_t* shape);

/*
 * Tiled layout.  The operands of the expert GEMMs (x_perm, h, the shared
 * expert's copy of x and the packed expert weights) are stored in tiles of
 * 16 rows x 32 columns.  With Cp = cols rounded up to a multiple of 32,
 * element (r, c) of such a matrix is at element index
 *     ((r / 16) * (Cp / 32) + c / 32) * 512 + (r % 16) * 32 + (c % 32),
 * i.e. each 16 x 32 tile is one contiguous block of 512 elements (1 KiB in
 * bf16) and the tiles of a 16-row band follow each other.  Columns cols .. Cp-1
 * hold zeros.  A GEMM step reads whole tiles: one contiguous burst per 16 rows
 * instead of 16 separate 64-byte pieces of long rows.
 *
 * Row numbering of the permuted rows (x_perm, h and the expert outputs).
 * Expert e in [e_lo, e_hi) owns local rows P(e) .. P(e) + counts[e] - 1, where
 *     P(e_lo) = 0,   P(e + 1) = P(e) + 16 * ceil(counts[e] / 16),
 * so every expert's segment starts on a 16-row boundary and no tile holds rows
 * of two experts.  The up to 15 padding rows after a segment are never written
 * into a live output; perm marks them -1.
 */

/* Largest number of (padded) rows that (t, slot) pairs of experts in [e_lo, e_hi)
 * can occupy under `mode`: the assignment bound (GROUPED -> T * sum_g min(K',
 * |[e_lo,e_hi) & group g|); GLOBAL -> T * min(K, e_hi - e_lo)) plus 15 padding
 * rows per expert of the range.  Returns -1 on invalid arguments.  perm, x_perm,
 * h and the expert outputs need this many rows. */
int64_t moge_rows_bound(const moge_shape_t* shape, int32_t mode, int32_t e_lo, int32_t e_hi);

/* Elements of one tiled matrix of `rows` activation rows: ceil16(rows) * ceil32(cols). */
int64_t moge_tiled_elems(int64_t rows, int64_t cols);

/* Elements of one packed expert weight matrix: ceil32(rows) * ceil32(cols). */
int64_t moge_packed_weight_elems(int64_t rows, int64_t cols);

/* Bytes of device workspace a stage needs (0 if none; (size_t)-1 if invalid). */
size_t moge_workspace_size(const moge_shape_t* shape, int32_t stage);

/*
 * moge_pack_weights -- E row-major matrices src [E][rows][cols] (dtype) into the
 * tiled layout, rows padded with zero rows to a multiple of 32 and columns with
 * zeros to a multiple of 32: dst holds E * moge_packed_weight_elems(rows, cols)
 * elements, expert after expert.  Weights are packed once, when they are
 * loaded; the expert GEMMs read packed weights only.  For an expert's SwiGLU
 * block: w_gate and w_up have rows = F, cols = d; w_down has rows = d, cols = F.
 * src and dst must not overlap.  Requires cols % 8 == 0 and rows >= 1.
 */
moge_status_t moge_pack_weights(int32_t dtype, int64_t E, int64_t rows, int64_t cols, const void* src, void* dst,
                                hipStream_t stream);

/*
 * moge_round_bf16 -- y[i] = x[i] rounded to bf16 (round to nearest, ties to even;
 * infinities kept; a NaN stays a NaN, made quiet), the rounding the library
 * applies where the layer stores bf16 values: h before the down projection and
 * the expert outputs.  For callers that prepare bf16 activations with the same
 * rounding, and to check it.
 *   x  [n] float32 device;  y [n] bf16 bit patterns (uint16) device, not
 *      overlapping x;  n >= 0 (0: nothing is launched).
 * Errors: MOGE_ERR_SHAPE (n < 0), MOGE_ERR_NULL (x or y NULL with n > 0).
 */
moge_status_t moge_round_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t stream);

/*
 * moge_route -- router scores, global softmax, top-K' per group ([P1] section 1).
 *   x        [T][d] (dtype) or NULL; w_router [N][d] (dtype); bias [N] f32 or NULL.
 *   logits   [T][N] f32.  If x != NULL: scores are computed as x.w_router^T (+bias)
 *            with float32 accumulation and, when logits != NULL, also stored.
 *            If x == NULL: logits is the INPUT (bias must then be NULL).
 *   idx      [T][K] int32 out: chosen expert ids.
 *   gate     [T][K] f32 out: the chosen experts' probabilities under the softmax
 *            over all N scores (not renormalised over the chosen experts).
 *   ws       device workspace of moge_workspace_size(shape, MOGE_STAGE_ROUTE)
 *            bytes: the partial sums of a reduction split over slices of d, for
 *            bf16 scores from x with N > 128, or with N <= 128, d >= 128 and
 *            fewer than 256 token tiles (tiles of 128 tokens for N <= 64, of 64
 *            for N <= 128: T <= 32640 or T <= 16320); 0 bytes (NULL allowed) for
 *            every other call.  MOGE_ERR_WORKSPACE if missing or too small.
 * Slot order: GROUPED -> slot = g*K' + rank inside group g; GLOBAL -> slot = rank.
 * rank orders experts by score, higher first, equal scores -> lower expert id
 * (-0 and +0 are equal).
 * Scores are meant to be finite (moge_check_finite tests them).  A NaN score
 * ranks as -inf (below every finite score; ties by the lower id as above), so
 * the choice keeps exactly K' distinct experts of every group whatever the
 * scores; a token with a NaN or infinite score may get NaN gates.
 */
moge_status_t moge_route(const moge_shape_t* shape, int32_t mode, const void* x, const void* w_router,
                         const float* bias, float* logits, int32_t* idx, float* gate, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/*
 * moge_route_pair -- both routers on the same scores in one pass: the MoGE choice
 * (idx, gate: MOGE_ROUTE_GROUPED) and the conventional global top-K with K = M*K'
 * (gidx, ggate: MOGE_ROUTE_GLOBAL) that [P1] section 1 compares it with.  Each
 * result equals moge_route's for that mode; the scores are computed (or read) once
 * and need not be stored for the second router.  Arguments as moge_route; all four
 * outputs are required.
 */
moge_status_t moge_route_pair(const moge_shape_t* shape, const void* x, const void* w_router, const float* bias,
                              float* logits, int32_t* idx, float* gate, int32_t* gidx, float* ggate, void* ws,
                              size_t ws_bytes, hipStream_t stream);


/*
 * moge_dispatch -- per-expert counts and the token permutation (dropless: every
 * (token, slot) pair gets a row; [P4]), plus the gather of x into expert order.
 *   idx      [T][K] int32 from moge_route with the same `mode`.
 *   x        [T][d] (dtype), row-major.
 *   [e_lo, e_hi) experts whose rows are materialised (a device's share, e.g.
 *            one group); 0 <= e_lo < e_hi <= N.
 *   rows_cap rows available in perm / x_perm; must be >= moge_rows_bound().
 *   counts   [N] int32 out: rows per expert (all N experts).
 *   offsets  [N+1] int32 out: exclusive prefix sum of counts (all N experts).
 *   inv      [T][K] int32 out: local row of (t, slot) = P(e) + #{t' < t that
 *            chose e} (P as defined at the tiled layout above); -1 when the
 *            expert is outside [e_lo, e_hi).
 *   perm     [rows_cap] int32 out: token of each local row, -1 on the padding
 *            rows of a segment (rows past P(e_hi) are left untouched).
 *   x_perm   tiled, rows_cap rows x d columns (dtype) out: row r = x[perm[r]]
 *            for live rows; padding rows are left unspecified.
 *   x_tiled  tiled, T rows x d columns (dtype) out, or NULL: x in token order
 *            (the input of the always-on shared expert).  Needs x.
 *   ws       device workspace of moge_workspace_size(shape, MOGE_STAGE_DISPATCH) bytes.
 * Rows of one expert are in ascending token order, so the result is unique and
 * deterministic.  Expert ids outside [0, N) in idx are ignored (memory-safe).
 * Lighter forms: x and x_perm both NULL -> no row copies; additionally inv and
 * perm both NULL -> counts and offsets only (rows_cap is then not checked), e.g.
 * for the load of the global top-K comparator.
 */
moge_status_t moge_dispatch(const moge_shape_t* shape, int32_t mode, const int32_t* idx, const void* x,
                            int32_t e_lo, int32_t e_hi, int64_t rows_cap, int32_t* counts, int32_t* offsets,
                            int32_t* inv, int32_t* perm, void* x_perm, void* x_tiled, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/*
 * moge_dispatch_noalloc -- moge_dispatch for callers that cannot allocate device
 * memory (code recorded into a HIP graph, tight serving loops, harnesses that
 * forbid allocation): the same arguments and results, without ws / ws_bytes.
 * Its workspace is a fixed 4 MiB array in device memory that the library holds
 * on every GPU it runs on until the process ends; the call allocates and frees
 * nothing.  Limit: moge_workspace_size(shape, MOGE_STAGE_DISPATCH) <= 4 MiB,
 * i.e. N * ceil(T / 64) <= 524288 (256 experts up to T = 131072 tokens, 64
 * experts up to T = 524288); larger shapes get MOGE_ERR_WORKSPACE before any
 * launch.  All calls on one GPU share that array: calls that overlap in time on
 * one GPU (different streams, or threads without ordering) race and must not be
 * made; calls in order on one stream are safe.  The array keeps the last call's
 * contents, and no part of it needs clearing between calls.
 */
moge_status_t moge_dispatch_noalloc(const moge_shape_t* shape, int32_t mode, const int32_t* idx, const void* x,
                                    int32_t e_lo, int32_t e_hi, int64_t rows_cap, int32_t* counts, int32_t* offsets,
                                    int32_t* inv, int32_t* perm, void* x_perm, void* x_tiled, hipStream_t stream);

/*
 * moge_grouped_ffn -- the SwiGLU expert applied to every expert's row segment
 * (a grouped GEMM pair).  [P1] section 1: each token's rows go to the experts it
 * chose, whose groups sit on separate devices; section 3: the grouped matmul
 * (GroupMatmul, SwiftGMM) that multiplies every expert's rows by that expert's
 * weights is the dominant kernel of inference.  The expert form itself (SwiGLU,
 * no biases) is not on the pages; it is the form stated at the top of this file.
 *   x_perm   tiled, rows_cap rows x d columns: local rows P(e) .. P(e)+counts[e]-1
 *            belong to expert e (counts[e] = offsets[e+1] - offsets[e]).
 *   offsets  [N+1] int32 device (from moge_dispatch).
 *   w_gate, w_up: packed (moge_pack_weights) [e_hi-e_lo] x (F rows x d cols);
 *   w_down:  packed [e_hi-e_lo] x (d rows x F cols): the arrays hold experts
 *            e_lo .. e_hi-1 only (a device's share of the weights).
 *   h        tiled, rows_cap rows x F columns, scratch (dtype): silu(x.Wg^T) *
 *            (x.Wu^T), rounded to dtype before the down projection.
 *   out      [rows_cap][d] (dtype), row-major: FFN_e(x_perm[r]) for every live row.
 * The always-on shared expert is the same call with a one-expert shape
 * (N = M = k_per_group = 1, F = shared width), offsets = {0, T} and x_perm = the
 * x_tiled copy written by moge_dispatch.
 */
moge_status_t moge_grouped_ffn(const moge_shape_t* shape, const void* x_perm, const int32_t* offsets,
                               int32_t e_lo, int32_t e_hi, int64_t rows_cap, const void* w_gate,
                               const void* w_up, const void* w_down, void* h, void* out, hipStream_t stream);

/*
 * The two halves of moge_grouped_ffn, for callers that schedule or time them
 * separately (same arguments and rules as moge_grouped_ffn):
 *   moge_expert_gate_up: h   = silu(x_perm . Wg^T) * (x_perm . Wu^T)  per expert segment
 *   moge_expert_down:    out = h . Wd^T                               per expert segment
 */
moge_status_t moge_expert_gate_up(const moge_shape_t* shape, const void* x_perm, const int32_t* offsets,
                                  int32_t e_lo, int32_t e_hi, int64_t rows_cap, const void* w_gate, const void* w_up,
                                  void* h, hipStream_t stream);
moge_status_t moge_expert_down(const moge_shape_t* shape, const void* h, const int32_t* offsets, int32_t e_lo,
                               int32_t e_hi, int64_t rows_cap, const void* w_down, void* out, hipStream_t stream);

/*
 * The routed experts' SwiGLU blocks and the always-on shared expert's block over
 * all T tokens ([P4]: one shared expert), in the same launches: one persistent
 * tile list per GEMM holds the routed tiles followed by the shared expert's, so
 * the shared tiles fill the last round of routed tiles instead of running as
 * launches of their own with half-empty rounds.  bf16 only.
 *   Routed arguments as moge_expert_gate_up / moge_expert_down.
 *   F_shared  the shared expert's width (F_shared % 8 == 0).
 *   x_tiled   tiled, T rows x d columns (moge_dispatch's x_tiled).
 *   ws_gate, ws_up: packed F_shared x d; ws_down: packed d x F_shared.
 *   hs        tiled, T rows x F_shared columns (scratch: the shared expert's h).
 *   out_shared [T][d] (dtype), row-major: the shared expert's output.
 * Each output element is computed exactly as by the separate calls (bit-identical).
 */
moge_status_t moge_expert_gate_up_with_shared(const moge_shape_t* shape, int32_t F_shared, const void* x_perm,
                                              const int32_t* offsets, int32_t e_lo, int32_t e_hi, int64_t rows_cap,
                                              const void* w_gate, const void* w_up, void* h, const void* x_tiled,
                                              const void* ws_gate, const void* ws_up, void* hs, hipStream_t stream);
moge_status_t moge_expert_down_with_shared(const moge_shape_t* shape, int32_t F_shared, const void* h,
                                           const int32_t* offsets, int32_t e_lo, int32_t e_hi, int64_t rows_cap,
                                           const void* w_down, void* out, const void* hs, const void* ws_down,
                                           void* out_shared, hipStream_t stream);

/*
 * moge_expert_gate_up_gather -- moge_expert_gate_up (and, when F_shared > 0, the
 * shared expert's gate/up over all T tokens in the same launch) reading the
 * token rows straight from x through perm instead of from a tiled x_perm, so
 * that moge_dispatch needs no row copy (call it with x = x_perm = NULL and
 * inv/perm given).  bf16 only, d % 32 == 0.
 *   x         [T][d] bf16 row-major (the layer input).
 *   perm      [rows_cap] int32 from moge_dispatch (same e_lo, e_hi, rows_cap): the
 *             token of each local row, -1 on padding rows.
 *   offsets, e_lo, e_hi, rows_cap, w_gate, w_up, h: as moge_expert_gate_up.
 *   F_shared  0 (no shared expert; ws_gate, ws_up, hs must be NULL) or the shared
 *             expert's width (% 8 == 0) with ws_gate, ws_up packed F_shared x d
 *             and hs tiled T x F_shared, as moge_expert_gate_up_with_shared.
 * h (and hs) are bit-identical to moge_expert_gate_up(_with_shared) on the
 * dispatched x_perm (x_tiled).  Errors: MOGE_ERR_DTYPE for float32,
 * MOGE_ERR_SHAPE for d % 32 != 0 or a bad F_shared, MOGE_ERR_NULL / MOGE_ERR_ARG
 * for missing or unexpected operands, plus those of moge_expert_gate_up.
 */
moge_status_t moge_expert_gate_up_gather(const moge_shape_t* shape, const void* x, const int32_t* perm,
                                         const int32_t* offsets, int32_t e_lo, int32_t e_hi, int64_t rows_cap,
                                         const void* w_gate, const void* w_up, void* h, int32_t F_shared,
                                         const void* ws_gate, const void* ws_up, void* hs, hipStream_t stream);

/*
 * moge_expert_down_combine -- moge_expert_down followed by moge_combine, in one
 * launch, for a device's share of exactly one group with k_per_group == 1 (the
 * expert-parallel layout that places one group per device: [P1] section 1).
 * Then every token has exactly one row in [e_lo, e_hi), and GEMM 2's epilogue
 * writes y[t] = gate[t][g] * o[row of t] itself (g = e_lo / (N/M), o rounded to
 * bf16 first, then one float32 multiply), so o is never stored and no combine
 * pass runs.  bf16 only; no shared expert (add it with moge_combine's form if
 * needed).
 *   h, offsets, e_lo, e_hi, rows_cap, w_down: as moge_expert_down.
 *   perm [rows_cap] int32 from moge_dispatch; gate [T][K] float32 from moge_route.
 *   y    [T][d] float32, every row written.
 * y is bit-identical to moge_expert_down + moge_combine(shared_out = NULL).
 * Errors: MOGE_ERR_DTYPE for float32; MOGE_ERR_ARG unless k_per_group == 1 and
 * [e_lo, e_hi) is one whole group; MOGE_ERR_NULL for a missing operand; plus
 * those of moge_expert_down.
 */
moge_status_t moge_expert_down_combine(const moge_shape_t* shape, const void* h, const int32_t* offsets,
                                       int32_t e_lo, int32_t e_hi, int64_t rows_cap, const void* w_down,
                                       const int32_t* perm, const float* gate, float* y, hipStream_t stream);

/*
 * moge_combine -- gate-weighted sum of the expert outputs back in token order.
 * [P1] section 1: the weights are the chosen experts' probabilities under the
 * softmax over all N experts, taken before the per-group choice, so they are not
 * renormalised; [P4]: the always-on shared expert is added to every token.
 *   y[t] = sum over slots s (in slot order) with inv[t][s] >= 0 of
 *          gate[t][s] * o[inv[t][s]]   (+ shared_out[t] when not NULL), in float32.
 *   o [rows_cap][d] (dtype), inv/gate [T][K], shared_out [T][d] (dtype) or NULL,
 *   y [T][d] f32.  Rows inv >= rows_cap are ignored (memory-safe).
 */
moge_status_t moge_combine(const moge_shape_t* shape, const void* o, const int32_t* inv, const float* gate,
                           int64_t rows_cap, const void* shared_out, float* y, hipStream_t stream);

/*
 * moge_imbalance -- per-device (per-group) load and the imbalance score ([P1]
 * section 1: busiest minus idlest device in the batch).
 *   counts [N] int32 (from moge_dispatch); group_load [M] int32 out =
 *   sum of counts over the group's experts; is_raw [1] int32 out = max - min;
 *   is_norm [1] double out = is_raw / T.  All device pointers.
 */
moge_status_t moge_imbalance(const moge_shape_t* shape, const int32_t* counts, int32_t* group_load,
                             int32_t* is_raw, double* is_norm, hipStream_t stream);

/*
 * moge_imbalance_batches -- the imbalance score of each of B batches routed in one
 * call: the setting in which [P1] (section 1) compares the routers by Monte-Carlo
 * simulation.  Batch b holds tokens b*Tb .. (b+1)*Tb - 1 of idx.
 *   shape   the shape of the routing call: T = B * Tb tokens, N, M, k_per_group
 *           (idx has K = M*k_per_group slots per token in both route modes).
 *   idx     [T][K] int32 (device) from moge_route; ids outside [0, N) are ignored.
 *   tokens_per_batch  Tb, must divide T.
 *   group_load [B][M] int32 out: assignments per group (group(e) = e / (N/M)).
 *   is_raw  [B] int32 out: busiest minus idlest group of the batch.
 */
moge_status_t moge_imbalance_batches(const moge_shape_t* shape, const int32_t* idx, int64_t tokens_per_batch,
                                     int32_t* group_load, int32_t* is_raw, hipStream_t stream);

/*
 * moge_check_finite -- a checking call: tests n values for NaN and infinities
 * and WAITS for the result (it synchronises `stream`), for callers that want
 * the router scores (moge_route's logits) or any other input checked before
 * trusting a result.  The pages define no outcome for non-finite scores, so the
 * layer's own calls do not test for them.
 *   dtype  MOGE_F32 (a: float32) or MOGE_BF16 (a: bf16 bit patterns).
 *   a      [n] device;  n >= 0.
 *   ws     device workspace of moge_workspace_size(any valid shape,
 *          MOGE_STAGE_CHECK) bytes.
 * Returns MOGE_OK if every value is finite, MOGE_ERR_NONFINITE otherwise (the
 * message gives the count and the first index), MOGE_ERR_HIP if the stream
 * fails, MOGE_ERR_DTYPE / MOGE_ERR_SHAPE / MOGE_ERR_NULL / MOGE_ERR_WORKSPACE
 * for bad arguments.  Not for use while `stream` is being captured into a graph.
 */
moge_status_t moge_check_finite(int32_t dtype, const void* a, int64_t n, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/*
 * moge_tile_choice -- the tile shape MOGE_TILES_AUTO gives one expert GEMM of a call
 * with this shape: gemm 1 = gate/up (output width F), 2 = down (output width d), for
 * the routed experts [e_lo, e_hi) and, when F_shared > 0, the shared expert's tiles in
 * the same launch.  The table keys on the rows per expert under MoGE routing
 * (T*K' / (N/M)), the experts, the output width and the device's CU count, and takes
 * the shape whose busiest CU streams the fewest weight rows: ceil(tiles / CUs) times
 * the tile's weight rows (the wide shape on a tie).  For gate/up with the tall shape
 * and at most 64 rows per expert it also weighs the balanced column splits (each
 * tile i on CU i mod CUs) and takes one that lowers the busiest CU's weight rows.  A
 * forced shape.tiles is returned as the shape that GEMM runs (BALANCED forced on the
 * down GEMM: TALL).  Host-only (the CU count is queried once; 256 without a device).
 * Returns MOGE_TILES_TALL, MOGE_TILES_WIDE or MOGE_TILES_BALANCED, or -1 for invalid
 * arguments.
 */
int32_t moge_tile_choice(const moge_shape_t* shape, int32_t gemm, int32_t e_lo, int32_t e_hi, int32_t F_shared);

/* Library version string and the calling thread's last error message. */
const char* moge_version(void);
const char* moge_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOGE_H */
