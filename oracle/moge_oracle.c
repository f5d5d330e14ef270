/*
 * moge_oracle.c -- plain, slow CPU oracle for the forward pass of one MoGE
 * (Mixture of Grouped Experts) layer.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  It shares no code, header, table or
 * helper with the GPU library; the two meet only in the seeded inputs.
 *
 * Sources (web pages about "Pangu Pro MoE: Mixture of Grouped Experts for
 * Efficient Sparsity", arXiv 2505.21411):
 *   [P1] the lsdiaocha.cn long-form summary of the paper;
 *   [P5] the hyper.ai page carrying the paper's abstract.
 *
 * Every floating-point quantity is computed in binary64 from inputs that are
 * exactly representable (bf16 or binary32 values widened without rounding).
 * The only rounding to binary32 is the router logit, because the selection
 * key is the binary32 logit (see oracle_logits).
 *
 * Parity: every function here is pinned by the CPU tests against closed forms,
 * invariants, library routines (NumPy/SciPy) or brute-force enumeration.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BF16 0
#define ORACLE_F32 1

/* Exact widening of one stored element to binary64. */
static double load_elem(const void* base, int dtype, int64_t i) {
  if (dtype == ORACLE_BF16) {
    uint32_t u = ((uint32_t)((const uint16_t*)base)[i]) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[i];
}

/*
 * Router scores.  [P1] section 1 (architecture): MoGE first scores all N
 * experts for each token.  The score of expert e for token t is the linear
 * router output
 *     l[t][e] = sum_i x[t][i] * w[e][i]  (+ bias[e])
 * summed in binary64 and rounded once to binary32.  x is [T][d], w is [N][d].
 */
void oracle_logits(int64_t T, int64_t d, int64_t N, int dtype, const void* x, const void* w, const float* bias,
                   float* logits) {
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t e = 0; e < N; ++e) {
      double acc = 0.0;
      for (int64_t i = 0; i < d; ++i) acc += load_elem(x, dtype, t * d + i) * load_elem(w, dtype, e * d + i);
      if (bias) acc += (double)bias[e];
      logits[t * N + e] = (float)acc;
    }
  }
}

/*
 * Grouped selection.  [P1] section 1: the N experts are split evenly into
 * n_groups groups of N/n_groups (contiguous blocks of expert ids here); each
 * token takes a softmax over ALL N experts (the global softmax) and then keeps
 * the k best experts INSIDE every group ([P5]: an equal number of experts is
 * activated in each predefined group).  With n_groups = 1 and k = K this is the
 * conventional global top-K router that [P1] section 1 contrasts with MoGE.
 *
 * Outputs, per token t, K = n_groups * k slots, slot = g * k + rank:
 *   idx[t][slot]  = chosen expert id,
 *   gate[t][slot] = its global softmax probability (binary64, no renormalisation),
 *   gap[t]        = min over groups of p(rank k-1) - p(rank k); +inf when k = group size.
 * rank(e) = #{e' in group(e) : l[e'] > l[e]  or  (l[e'] == l[e] and e' < e)},
 * comparing the binary32 logits: the exponential is strictly increasing, so this
 * is the order of the exact softmax, and equal logits go to the lower index.
 */
void oracle_route(int64_t T, int64_t N, int64_t n_groups, int64_t k, const float* logits, int32_t* idx,
                  double* gate, double* gap) {
  const int64_t G = N / n_groups;
  const int64_t K = n_groups * k;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * N;
    double* p = (double*)malloc(sizeof(double) * (size_t)N);
    double m = (double)l[0];
    for (int64_t e = 1; e < N; ++e)
      if ((double)l[e] > m) m = (double)l[e];
    double z = 0.0;
    for (int64_t e = 0; e < N; ++e) z += exp((double)l[e] - m);
    for (int64_t e = 0; e < N; ++e) p[e] = exp((double)l[e] - m) / z;
    double gmin = INFINITY;
    for (int64_t g = 0; g < n_groups; ++g) {
      double p_last = 0.0, p_next = 0.0;
      int have_next = 0;
      for (int64_t e = g * G; e < (g + 1) * G; ++e) {
        int64_t rank = 0;
        for (int64_t e2 = g * G; e2 < (g + 1) * G; ++e2)
          if (l[e2] > l[e] || (l[e2] == l[e] && e2 < e)) ++rank;
        if (rank < k) {
          idx[t * K + g * k + rank] = (int32_t)e;
          gate[t * K + g * k + rank] = p[e];
        }
        if (rank == k - 1) p_last = p[e];
        if (rank == k) {
          p_next = p[e];
          have_next = 1;
        }
      }
      if (have_next && p_last - p_next < gmin) gmin = p_last - p_next;
    }
    gap[t] = gmin;
    free(p);
  }
}

/*
 * Token dispatch (dropless: every (token, slot) pair gets a row).
 *   counts[e]  = number of (t, s) with idx[t][s] == e       (N entries)
 *   offsets[e] = counts[0] + ... + counts[e-1]              (N+1 entries)
 * Rows of expert e are ordered by ascending token id: the pair (t, s) with
 * idx[t][s] == e gets global row offsets[e] + #{t' < t : t' chose e}.
 * Only experts in [e_lo, e_hi) get rows in the output numbering, which starts
 * at offsets[e_lo]:
 *   inv[t][s] = global row - offsets[e_lo]   (or -1 when e is out of range)
 *   perm[r]   = the token of local row r.
 */
void oracle_dispatch(int64_t T, int64_t K, int64_t N, const int32_t* idx, int64_t e_lo, int64_t e_hi,
                     int32_t* counts, int32_t* offsets, int32_t* inv, int32_t* perm) {
  int64_t* seen = (int64_t*)calloc((size_t)N, sizeof(int64_t));
  for (int64_t e = 0; e < N; ++e) counts[e] = 0;
  for (int64_t j = 0; j < T * K; ++j) counts[idx[j]] += 1;
  offsets[0] = 0;
  for (int64_t e = 0; e < N; ++e) offsets[e + 1] = offsets[e] + counts[e];
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t s = 0; s < K; ++s) {
      const int64_t e = idx[t * K + s];
      const int64_t row = offsets[e] + seen[e];
      seen[e] += 1;
      if (e >= e_lo && e < e_hi) {
        inv[t * K + s] = (int32_t)(row - offsets[e_lo]);
        perm[row - offsets[e_lo]] = (int32_t)t;
      } else {
        inv[t * K + s] = -1;
      }
    }
  }
  free(seen);
}

/*
 * One expert applied to one token row: the SwiGLU feed-forward block
 *   a_f = sum_i x_i * wg[f][i],   b_f = sum_i x_i * wu[f][i]
 *   h_f = silu(a_f) * b_f,        silu(z) = z / (1 + exp(-z))
 *   out_j = sum_f h_f * wd[j][f]
 * with wg, wu of shape [F][d] and wd of shape [d][F] (output-major, like a
 * linear layer's weight).  Everything in binary64.
 */
void oracle_ffn_row(int64_t d, int64_t F, int dtype, const void* x, const void* wg, const void* wu, const void* wd,
                    double* out) {
  double* h = (double*)malloc(sizeof(double) * (size_t)F);
#pragma omp parallel for schedule(static)
  for (int64_t f = 0; f < F; ++f) {
    double a = 0.0, b = 0.0;
    for (int64_t i = 0; i < d; ++i) {
      const double xi = load_elem(x, dtype, i);
      a += xi * load_elem(wg, dtype, f * d + i);
      b += xi * load_elem(wu, dtype, f * d + i);
    }
    h[f] = a / (1.0 + exp(-a)) * b;
  }
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < d; ++j) {
    double acc = 0.0;
    for (int64_t f = 0; f < F; ++f) acc += h[f] * load_elem(wd, dtype, j * F + f);
    out[j] = acc;
  }
  free(h);
}

/*
 * Per-device load and the imbalance score.  [P1] section 1: experts of one
 * group sit on one device; the imbalance score is the gap in workload between
 * the busiest and the idlest device in a batch.  Workload = number of
 * (token, expert) assignments that land in the group.
 */
void oracle_imbalance(int64_t N, int64_t M, const int32_t* counts, int32_t* group_load, int32_t* is_raw) {
  const int64_t G = N / M;
  int32_t lo = 0, hi = 0;
  for (int64_t g = 0; g < M; ++g) {
    int32_t s = 0;
    for (int64_t e = g * G; e < (g + 1) * G; ++e) s += counts[e];
    group_load[g] = s;
    if (g == 0 || s < lo) lo = s;
    if (g == 0 || s > hi) hi = s;
  }
  *is_raw = hi - lo;
}

/* Number of OpenMP threads the oracle's parallel loops use. */
int oracle_threads(void) { return omp_get_max_threads(); }
