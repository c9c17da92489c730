/*
 * cce_oracle.c -- plain, slow, fp64 CPU oracle for Cut Cross-Entropy.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table
 * or helper with the HIP path and must never be called from the product path.
 *
 * What it computes (sources: "Cut Your Losses in Large-Vocabulary Language
 * Models" paper digest, section "The Mathematical Decomposition" and
 * Algorithms 2-4; the blog post "Cut Cross-Entropy: Training Loss Without the
 * Logit Matrix ...", sections "The decomposition" and "Gradient filtering";
 * the kernel card "cut-cross-entropy", sections "Method" and "Correctness"):
 *
 *   A[n][v]  = sum_d E[n][d] * C[v][d]                  (logit of vocab v for token n)
 *   lse[n]   = log sum_v exp(A[n][v])                    (linear-log-sum-exp)
 *   loss[n]  = lse[n] - A[n][x[n]]   for valid rows, 0 for ignored rows
 *   G[n][v]  = exp(A[n][v] - lse[n]) - [v == x[n]]       (gradient of loss w.r.t. the logits)
 *   filter:  a unit of unit_rows x unit_cols entries of G (aligned at 0,
 *            clipped to N and V; with `compact`, rows counted among the
 *            valid rows only) whose every |G| < eps is set to zero, in
 *            the G of both contractions or (digest, "Numerical Stability
 *            Variants") of dE only (FullC) or of dC only (FullE)
 *   dE[n]    = s[n] * sum_v G[n][v] * C[v]
 *   dC[v]    = sum_n s[n] * G[n][v] * E[n]
 *
 * with s[n] the per-row upstream scale: g / max(N_valid, 1) for the mean,
 * g for the sum, g[n] for no reduction, and 0 on ignored rows.
 *
 * Everything is done in double precision on the given arrays.  The logits
 * are materialised one row (forward) or one block of unit_rows rows
 * (backward) at a time, never all N x V at once.
 *
 * Parity unpinned: none of the functions below (every one is pinned by the
 * CPU tests against closed forms, a library log-softmax, finite differences
 * and invariants).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* The number of threads the OpenMP loops below use. */
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NO_MEMORY 2

#define RED_NONE 0
#define RED_MEAN 1
#define RED_SUM 2

#define FILTER_BOTH 0   /* dE and dC from the filtered G */
#define FILTER_FULL_C 1 /* dC from the unfiltered G */
#define FILTER_FULL_E 2 /* dE from the unfiltered G */

/* One row of logits: A[v] = E_row . C[v]. */
static void logits_row(const double *E_row, const double *C, int64_t V,
                       int64_t D, double *A) {
  for (int64_t v = 0; v < V; ++v) {
    const double *c = C + v * D;
    double acc = 0.0;
    for (int64_t d = 0; d < D; ++d) acc += E_row[d] * c[d];
    A[v] = acc;
  }
}

/* Max, sum of exp(A - max), and log-sum-exp of one row of logits. */
static double row_lse(const double *A, int64_t V, double *max_out) {
  double m = -INFINITY;
  for (int64_t v = 0; v < V; ++v)
    if (A[v] > m) m = A[v];
  double s = 0.0;
  for (int64_t v = 0; v < V; ++v) s += exp(A[v] - m);
  if (max_out) *max_out = m;
  return m + log(s);
}

/* loss = lse - t, written as (m - t) + log(exp(t - m) + sum_{v != x} exp(A - m)).
   The two forms are equal; the second keeps full relative accuracy when the
   target is the row maximum and the loss is tiny (then it is log1p of the
   off-target mass). */
static double row_loss(const double *A, int64_t V, int64_t x, double m) {
  double t = A[x];
  double off = 0.0;
  for (int64_t v = 0; v < V; ++v)
    if (v != x) off += exp(A[v] - m);
  if (t >= m) return log1p(off); /* target is the maximum: m == t */
  return (m - t) + log(exp(t - m) + off);
}

static int targets_ok(const int64_t *x, int64_t N, int64_t V, int64_t ignore) {
  for (int64_t n = 0; n < N; ++n)
    if (x[n] != ignore && (x[n] < 0 || x[n] >= V)) return 0;
  return 1;
}

/* Forward: per-row lse (0 on ignored rows), per-row loss, reduced loss.
   loss_out has N entries for RED_NONE, 1 entry otherwise. */
int oracle_forward(const double *E, const double *C, const int64_t *x,
                   int64_t N, int64_t V, int64_t D, int64_t ignore_index,
                   int reduction, double *loss_out, double *lse_out,
                   int64_t *n_valid_out) {
  if (N < 0 || V < 1 || D < 1) return ORACLE_BAD_ARG;
  if (reduction != RED_NONE && reduction != RED_MEAN && reduction != RED_SUM)
    return ORACLE_BAD_ARG;
  if (!targets_ok(x, N, V, ignore_index)) return ORACLE_BAD_ARG;

  double *row_loss_v = (double *)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
  if (!row_loss_v) return ORACLE_NO_MEMORY;
  int failed = 0;

#pragma omp parallel
  {
    double *A = (double *)malloc((size_t)V * sizeof(double));
    if (!A) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t n = 0; n < N; ++n) {
      if (!A) continue;
      if (x[n] == ignore_index) {
        if (lse_out) lse_out[n] = 0.0;
        row_loss_v[n] = 0.0;
        continue;
      }
      logits_row(E + n * D, C, V, D, A);
      double m;
      double lse = row_lse(A, V, &m);
      if (lse_out) lse_out[n] = lse;
      row_loss_v[n] = row_loss(A, V, x[n], m);
    }
    free(A);
  }
  if (failed) {
    free(row_loss_v);
    return ORACLE_NO_MEMORY;
  }

  int64_t n_valid = 0;
  double total = 0.0;
  for (int64_t n = 0; n < N; ++n) {
    if (x[n] == ignore_index) continue;
    ++n_valid;
    total += row_loss_v[n];
  }
  if (n_valid_out) *n_valid_out = n_valid;
  if (reduction == RED_NONE) {
    for (int64_t n = 0; n < N; ++n) loss_out[n] = row_loss_v[n];
  } else if (reduction == RED_SUM) {
    loss_out[0] = total;
  } else {
    loss_out[0] = total / (double)(n_valid > 0 ? n_valid : 1);
  }
  free(row_loss_v);
  return ORACLE_OK;
}

/* G for every row: exp(A - lse) - onehot on valid rows, 0 on ignored rows.
   G is N x V, row-major.  For small problems (tests of the invariants). */
int oracle_grad_logits(const double *E, const double *C, const int64_t *x,
                       int64_t N, int64_t V, int64_t D, int64_t ignore_index,
                       double *G) {
  if (N < 0 || V < 1 || D < 1) return ORACLE_BAD_ARG;
  if (!targets_ok(x, N, V, ignore_index)) return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t n = 0; n < N; ++n) {
    double *g = G + n * V;
    if (x[n] == ignore_index) {
      for (int64_t v = 0; v < V; ++v) g[v] = 0.0;
      continue;
    }
    logits_row(E + n * D, C, V, D, g);
    double lse = row_lse(g, V, NULL);
    for (int64_t v = 0; v < V; ++v) g[v] = exp(g[v] - lse);
    g[x[n]] -= 1.0;
  }
  return ORACLE_OK;
}

/* Backward: dE (N x D) and dC (V x D), both overwritten.
   grad has 1 entry (mean, sum) or N entries (none).  eps <= 0 turns the
   filter off.  units_total / units_skipped count the filter units.
   compact != 0 cuts the filter units from the valid rows only (see rowid).
   filter_mode picks the contractions that take the filtered G ("Cut Your
   Losses" digest, "Numerical Stability Variants"): FILTER_BOTH (basic CCE),
   FILTER_FULL_C (dC from the unfiltered G, dE filtered: the FullC variant)
   or FILTER_FULL_E (dE unfiltered, dC filtered: FullE).  The Kahan part of
   those variants is about bf16 accumulation and has no counterpart here:
   everything is fp64. */
int oracle_backward(const double *E, const double *C, const int64_t *x,
                    int64_t N, int64_t V, int64_t D, int64_t ignore_index,
                    int reduction, const double *grad, double eps,
                    int filter_mode, int compact, int64_t unit_rows,
                    int64_t unit_cols, double *dE, double *dC,
                    int64_t *units_total, int64_t *units_skipped) {
  if (N < 0 || V < 1 || D < 1 || unit_rows < 1 || unit_cols < 1)
    return ORACLE_BAD_ARG;
  if (filter_mode != FILTER_BOTH && filter_mode != FILTER_FULL_C &&
      filter_mode != FILTER_FULL_E)
    return ORACLE_BAD_ARG;
  if (reduction != RED_NONE && reduction != RED_MEAN && reduction != RED_SUM)
    return ORACLE_BAD_ARG;
  if (!(eps == eps)) return ORACLE_BAD_ARG; /* NaN */
  if (!targets_ok(x, N, V, ignore_index)) return ORACLE_BAD_ARG;

  int64_t n_valid = 0;
  for (int64_t n = 0; n < N; ++n)
    if (x[n] != ignore_index) ++n_valid;

  memset(dE, 0, (size_t)(N * D) * sizeof(double));
  memset(dC, 0, (size_t)(V * D) * sizeof(double));

  /* The rows the blocks are cut from: every row, or with `compact` the valid
     rows only, in their order (the ignored rows removed before the gradient
     is computed, as in the digest's Table A1 ablation); an ignored row's dE
     stays 0 and it adds nothing to dC either way. */
  int64_t *rowid = (int64_t *)malloc((size_t)(N > 0 ? N : 1) * sizeof(int64_t));
  if (!rowid) return ORACLE_NO_MEMORY;
  int64_t nrows = 0;
  for (int64_t n = 0; n < N; ++n)
    if (!compact || x[n] != ignore_index) rowid[nrows++] = n;

  int64_t row_blocks = (nrows + unit_rows - 1) / unit_rows;
  int64_t col_units = (V + unit_cols - 1) / unit_cols;
  int64_t total = row_blocks * col_units, skipped = 0;

  double *G = (double *)malloc((size_t)(unit_rows * V) * sizeof(double));
  double *s = (double *)malloc((size_t)unit_rows * sizeof(double));
  /* the unfiltered G of the block, for the contraction a variant leaves
     unfiltered */
  double *Gu = (filter_mode != FILTER_BOTH)
                   ? (double *)malloc((size_t)(unit_rows * V) * sizeof(double))
                   : NULL;
  if (!G || !s || (filter_mode != FILTER_BOTH && !Gu)) {
    free(G);
    free(s);
    free(Gu);
    free(rowid);
    return ORACLE_NO_MEMORY;
  }
  const double *GE = (filter_mode == FILTER_FULL_E) ? Gu : G; /* G of dE */
  const double *GC = (filter_mode == FILTER_FULL_C) ? Gu : G; /* G of dC */

  for (int64_t b = 0; b < row_blocks; ++b) {
    int64_t r0 = b * unit_rows;
    int64_t rows = (nrows - r0 < unit_rows) ? nrows - r0 : unit_rows;

    /* per-row scale */
    for (int64_t i = 0; i < rows; ++i) {
      int64_t n = rowid[r0 + i];
      if (x[n] == ignore_index) {
        s[i] = 0.0;
      } else if (reduction == RED_NONE) {
        s[i] = grad[n];
      } else if (reduction == RED_SUM) {
        s[i] = grad[0];
      } else {
        s[i] = grad[0] / (double)(n_valid > 0 ? n_valid : 1);
      }
    }

    /* G rows of this block */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < rows; ++i) {
      int64_t n = rowid[r0 + i];
      double *g = G + i * V;
      if (x[n] == ignore_index) {
        for (int64_t v = 0; v < V; ++v) g[v] = 0.0;
        continue;
      }
      logits_row(E + n * D, C, V, D, g);
      double lse = row_lse(g, V, NULL);
      for (int64_t v = 0; v < V; ++v) g[v] = exp(g[v] - lse);
      g[x[n]] -= 1.0;
    }

    if (Gu) memcpy(Gu, G, (size_t)(rows * V) * sizeof(double));

    /* filter: zero every unit whose entries are all below eps in magnitude */
    if (eps > 0.0) {
      for (int64_t u = 0; u < col_units; ++u) {
        int64_t c0 = u * unit_cols;
        int64_t cols = (V - c0 < unit_cols) ? V - c0 : unit_cols;
        double mx = 0.0;
        for (int64_t i = 0; i < rows; ++i)
          for (int64_t j = 0; j < cols; ++j) {
            double a = fabs(G[i * V + c0 + j]);
            if (a > mx) mx = a;
          }
        if (mx < eps) {
          ++skipped;
          for (int64_t i = 0; i < rows; ++i)
            for (int64_t j = 0; j < cols; ++j) G[i * V + c0 + j] = 0.0;
        }
      }
    }

    /* dE rows of this block: s[n] * sum_v G[n][v] C[v] */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
      double *de = dE + rowid[r0 + i] * D;
      const double *g = GE + i * V;
      for (int64_t v = 0; v < V; ++v) {
        double w = g[v];
        if (w == 0.0) continue;
        const double *c = C + v * D;
        for (int64_t d = 0; d < D; ++d) de[d] += w * c[d];
      }
      for (int64_t d = 0; d < D; ++d) de[d] *= s[i];
    }

    /* dC rows: each vocab row gathers this block's contribution */
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < V; ++v) {
      double *dc = dC + v * D;
      for (int64_t i = 0; i < rows; ++i) {
        double w = s[i] * GC[i * V + v];
        if (w == 0.0) continue;
        const double *e = E + rowid[r0 + i] * D;
        for (int64_t d = 0; d < D; ++d) dc[d] += w * e[d];
      }
    }
  }

  free(G);
  free(s);
  free(Gu);
  free(rowid);
  if (units_total) *units_total = total;
  if (units_skipped) *units_skipped = (eps > 0.0) ? skipped : 0;
  return ORACLE_OK;
}
