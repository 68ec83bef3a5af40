/*
 * CPU oracle for the decomposed tensor-parallel collective matmuls.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, helper or
 * constant with the GPU library.
 *
 * What it computes is the monolithic definition that the decomposed method
 * must reproduce exactly (up to floating-point summation order):
 *
 *   AllGather -> GEMM   (column-parallel linear after a sequence-sharded
 *                        activation; "Hiding Tensor-Parallel Collectives:
 *                        AG/RS Overlap in Megatron", sections 1-2):
 *       Xfull = concat_r X_r   (rows, rank order)
 *       Y_r   = Xfull . W_r^T  for every rank r
 *
 *   GEMM -> ReduceScatter (row-parallel linear; same page, section 4):
 *       Z_r   = H_r . W_r^T
 *       Out_q = sum_r Z_r[q*m:(q+1)*m, :]   (sum taken in rank order)
 *
 *   AllReduce (used only as an invariant: "Tensor Parallelism > Communication
 *   Patterns", the paragraph on all-reduce being a reduce-scatter followed by
 *   an all-gather):
 *       AR = sum_r Z_r
 *
 * The decomposition page ("Overlap Communication with Dependent Computation
 * via Decomposition in Large Deep Learning Models", sections "The idea" and
 * "Why it works") states that the decomposed computation equals this
 * monolithic one because concatenation and summation are linear, so the
 * oracle is the definition written out, with no blocking or reordering.
 *
 * Conventions
 *   - Inputs are bf16 bit patterns (uint16).  A bf16 value is by definition
 *     the upper 16 bits of an IEEE binary32, so each converts exactly to
 *     float and then to double.
 *   - Weights are stored [n][k] (row j of W_r holds output feature j, its k
 *     entries contiguous), so Y[i][j] = sum_k A[i][k] * W[j][k].
 *   - All accumulation is fp64, in increasing k.
 *   - "mag" outputs, when not NULL, receive sum_k |a_ik| * |w_jk| over the
 *     same (full) contraction, which scales the floating-point error bound.
 *
 *   GEMM -> ReduceScatter with a bf16 bucket (the same bucket hand-off, the
 *   bucket stored in bf16 between hops): the definition above with the
 *   bucket rounded to bf16 after every addition, in ring order.
 *
 *   The transformer layer around them (attention, LayerNorm, GELU): see the
 *   section at the end of this file; the chained layer is composed in
 *   oracle/__init__.py.
 *
 * Parity pins: see the tests (brute force on tiny shapes, closed forms,
 * N = 1 against a library matmul, the AllReduce invariant, planted
 * mistakes).  The bf16 rounding routine is pinned by hand-derived tie cases;
 * the bf16-bucket chain by a hand-derived fixture with rounding ties, a
 * brute force in Python integers and its reduction to the fp32 definition
 * where no rounding can act.
 */
#include <math.h>
#include <stdlib.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* out[j] = sum_kk a[kk] * w[j][kk] for one activation row a (length k)
 * against every row j of one weight matrix w ([n][k]); mag likewise with
 * absolute values. */
static void row_times_weight(const uint16_t *a, const uint16_t *w, int k, int n,
                             double *out, double *mag) {
  for (int j = 0; j < n; ++j) {
    const uint16_t *wj = w + (size_t)j * k;
    double acc = 0.0;
    for (int kk = 0; kk < k; ++kk) acc += bf16_value(a[kk]) * bf16_value(wj[kk]);
    out[j] = acc;
    if (mag) {
      double accabs = 0.0;
      for (int kk = 0; kk < k; ++kk) accabs += fabs(bf16_value(a[kk])) * fabs(bf16_value(wj[kk]));
      mag[j] = accabs;
    }
  }
}

int orc_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Row i (0 <= i < N*m) of Xfull = concat_r X_r: shard i / m, local row i % m. */
static const uint16_t *xfull_row(const uint16_t *x, int m, int k, int i) {
  int shard = i / m;
  int local = i % m;
  return x + ((size_t)shard * m + local) * k;
}

/*
 * AllGather -> GEMM, monolithic.
 *   x   [N][m][k]     shard r = X_r
 *   w   [N][n][k]     W_r
 *   y   [N][N*m][n]   Y_r = Xfull . W_r^T
 *   mag same shape as y, or NULL
 */
void orc_ag_gemm(int N, int m, int k, int n, const uint16_t *x, const uint16_t *w,
                 double *y, double *mag) {
  const int T = N * m;
#pragma omp parallel for collapse(2) schedule(static)
  for (int r = 0; r < N; ++r)
    for (int i = 0; i < T; ++i) {
      size_t o = ((size_t)r * T + i) * n;
      row_times_weight(xfull_row(x, m, k, i), w + (size_t)r * n * k, k, n, y + o,
                       mag ? mag + o : NULL);
    }
}

/*
 * The same definition evaluated only at selected (rank, row) pairs, for
 * checking sampled outputs of full-size runs and for timing a bounded sample.
 *   rank[s], row[s]: rank r and row i of Y_r (0 <= i < N*m)
 *   y   [ns][n], mag [ns][n] or NULL
 */
void orc_ag_gemm_rows(int N, int m, int k, int n, const uint16_t *x, const uint16_t *w,
                      int ns, const int *rank, const int *row, double *y, double *mag) {
  (void)N;
#pragma omp parallel for schedule(dynamic)
  for (int s = 0; s < ns; ++s)
    row_times_weight(xfull_row(x, m, k, row[s]), w + (size_t)rank[s] * n * k, k, n,
                     y + (size_t)s * n, mag ? mag + (size_t)s * n : NULL);
}

/* Out_q row i: sum over ranks r (in rank order) of Z_r[q*m + i][:]. */
static void rs_row(int N, int m, int k, int n, const uint16_t *h, const uint16_t *w, int q,
                   int i, double *out, double *mag, double *zrow, double *zmag) {
  const size_t T = (size_t)N * m;
  for (int j = 0; j < n; ++j) {
    out[j] = 0.0;
    if (mag) mag[j] = 0.0;
  }
  for (int r = 0; r < N; ++r) {
    const uint16_t *hrow = h + ((size_t)r * T + (size_t)q * m + i) * k;
    row_times_weight(hrow, w + (size_t)r * n * k, k, n, zrow, zmag);
    for (int j = 0; j < n; ++j) {
      out[j] += zrow[j];
      if (mag) mag[j] += zmag[j];
    }
  }
}

/*
 * GEMM -> ReduceScatter, monolithic.
 *   h   [N][N*m][k]   H_r (rank r's full-sequence activation, its k = f/N slice)
 *   w   [N][n][k]     W_r
 *   out [N][m][n]     Out_q
 *   mag same shape as out, or NULL (sum over all ranks' contraction)
 */
void orc_gemm_rs(int N, int m, int k, int n, const uint16_t *h, const uint16_t *w, double *out,
                 double *mag) {
#pragma omp parallel
  {
    double *zrow = (double *)malloc(sizeof(double) * 2 * (size_t)n);
    double *zmag = zrow + n;
#pragma omp for collapse(2) schedule(static)
    for (int q = 0; q < N; ++q)
      for (int i = 0; i < m; ++i) {
        size_t o = ((size_t)q * m + i) * n;
        rs_row(N, m, k, n, h, w, q, i, out + o, mag ? mag + o : NULL, zrow, mag ? zmag : NULL);
      }
    free(zrow);
  }
}

/* Sampled form: owner[s] = q, row[s] = i (0 <= i < m); out [ns][n]. */
void orc_gemm_rs_rows(int N, int m, int k, int n, const uint16_t *h, const uint16_t *w, int ns,
                      const int *owner, const int *row, double *out, double *mag) {
#pragma omp parallel
  {
    double *zrow = (double *)malloc(sizeof(double) * 2 * (size_t)n);
    double *zmag = zrow + n;
#pragma omp for schedule(dynamic)
    for (int s = 0; s < ns; ++s)
      rs_row(N, m, k, n, h, w, owner[s], row[s], out + (size_t)s * n,
             mag ? mag + (size_t)s * n : NULL, zrow, mag ? zmag : NULL);
    free(zrow);
  }
}

/*
 * AllReduce of the row-parallel partials: ar [N*m][n] = sum_r H_r . W_r^T,
 * over whole T-row matrices (no bucketing), ranks summed in order.
 */
void orc_allreduce(int N, int m, int k, int n, const uint16_t *h, const uint16_t *w, double *ar) {
  const int T = N * m;
#pragma omp parallel
  {
    double *zrow = (double *)malloc(sizeof(double) * (size_t)n);
#pragma omp for schedule(static)
    for (int i = 0; i < T; ++i) {
      double *dst = ar + (size_t)i * n;
      for (int j = 0; j < n; ++j) dst[j] = 0.0;
      for (int r = 0; r < N; ++r) {
        row_times_weight(h + ((size_t)r * T + i) * k, w + (size_t)r * n * k, k, n, zrow, NULL);
        for (int j = 0; j < n; ++j) dst[j] += zrow[j];
      }
    }
    free(zrow);
  }
}

/*
 * Round a double to the nearest bfloat16 value, ties to the value whose last
 * significand bit is zero (round-half-to-even).  bfloat16: 1 sign bit, 8
 * exponent bits (bias 127), 7 stored significand bits; normal values carry 8
 * significant bits, so the spacing of values in [2^e, 2^(e+1)) is 2^(e-7);
 * below 2^-126 the spacing is fixed at 2^-133.  Magnitudes that round above
 * the largest finite value become infinity.  Written from that definition
 * (nearbyint rounds ties to even under the default rounding mode), not from
 * any bit-manipulation shortcut.
 */
static double bf16_round(double v) {
  const double max_finite = ldexp(255.0, 127 - 7); /* (2 - 2^-7) * 2^127 */
  if (v == 0.0 || isnan(v) || isinf(v)) return v;
  double a = fabs(v);
  int e;
  frexp(a, &e); /* a = f * 2^e with f in [0.5, 1): a in [2^(e-1), 2^e) */
  int exp2 = e - 1;
  if (exp2 < -126) exp2 = -126; /* subnormal spacing */
  double quantum = ldexp(1.0, exp2 - 7);
  double q = nearbyint(a / quantum) * quantum;
  if (q > max_finite) q = INFINITY;
  return v < 0 ? -q : q;
}

/* The same rounding as bit patterns. */
void orc_round_bf16(const double *in, uint16_t *out, size_t count) {
  for (size_t t = 0; t < count; ++t) {
    double r = bf16_round(in[t]);
    float f = (float)r; /* exact: r is a bf16 value, representable in binary32 */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (isnan(r)) u = 0x7FC00000u;
    out[t] = (uint16_t)(u >> 16);
  }
}

/*
 * GEMM -> ReduceScatter with the circulating bucket held in bfloat16 between
 * hops (half the bytes per hop of an fp32 bucket).  The bucket owned by q is
 * the accumulator that travels the ring ("The idea" on the decomposition
 * page; the bucket hand-off of section 4 of the Megatron page): each rank it
 * visits adds its partial product Z_r[q*m + i, :] and sends it on, so the sum
 * is stored, and here rounded to bf16, after every addition.  The owner adds
 * its own partial last; that final sum is returned unrounded (the caller
 * rounds to the output type).  Partial products are exact (fp64).
 *   dir 0, one ring:  the bucket visits ranks q+1, q+2, ..., q-1 (mod N).
 *   dir 1, both ring directions: two buckets, clockwise over ranks q-L, ...,
 *     q-1 and counter-clockwise over ranks q+R, ..., q+1 (mod N), with
 *     L = ceil((N-1)/2) and R = floor((N-1)/2); the owner adds its partial
 *     and both arrivals (the realigning addition).
 *   owner[s], row[s]: the output row Out_q[i] of sample s; out [ns][n].
 *   mag [ns][n] or NULL: sum_k |a|*|w| over every rank's contraction.
 *   rmag [ns][n] or NULL: the sum of |bucket| over every rounded bucket value
 *     (each rounding moves the value by at most half a bf16 spacing).
 */
void orc_gemm_rs_bf16_bucket_rows(int N, int m, int k, int n, const uint16_t *h, const uint16_t *w,
                                  int dir, int ns, const int *owner, const int *row, double *out,
                                  double *mag, double *rmag) {
  const size_t T = (size_t)N * m;
  const int L = N / 2, R = (N - 1) / 2; /* L = ceil((N-1)/2) */
#pragma omp parallel
  {
    double *z = (double *)malloc(sizeof(double) * 4 * (size_t)n);
    double *zm = z + n, *b0 = z + 2 * (size_t)n, *b1 = z + 3 * (size_t)n;
#pragma omp for schedule(dynamic)
    for (int s = 0; s < ns; ++s) {
      const int q = owner[s], i = row[s];
      double *o = out + (size_t)s * n;
      double *mg = mag ? mag + (size_t)s * n : NULL;
      double *rm = rmag ? rmag + (size_t)s * n : NULL;
      for (int j = 0; j < n; ++j) {
        b0[j] = b1[j] = 0.0;
        if (mg) mg[j] = 0.0;
        if (rm) rm[j] = 0.0;
      }
      /* one bucket visiting `len` ranks first, first + step, ... */
      for (int chain = 0; chain < (dir ? 2 : 1); ++chain) {
        int first, len, step;
        if (!dir) { first = q + 1; len = N - 1; step = 1; }
        else if (chain == 0) { first = q - L; len = L; step = 1; }
        else { first = q + R; len = R; step = -1; }
        double *b = chain == 0 ? b0 : b1;
        for (int t = 0; t < len; ++t) {
          const int r = ((first + t * step) % N + N) % N;
          row_times_weight(h + ((size_t)r * T + (size_t)q * m + i) * k, w + (size_t)r * n * k, k, n, z,
                           mg ? zm : NULL);
          for (int j = 0; j < n; ++j) {
            b[j] = bf16_round(b[j] + z[j]);
            if (rm) rm[j] += fabs(b[j]);
            if (mg) mg[j] += zm[j];
          }
        }
      }
      row_times_weight(h + ((size_t)q * T + (size_t)q * m + i) * k, w + (size_t)q * n * k, k, n, z,
                       mg ? zm : NULL);
      for (int j = 0; j < n; ++j) {
        o[j] = z[j] + b0[j] + b1[j];
        if (mg) mg[j] += zm[j];
      }
    }
    free(z);
  }
}

/* ------------------------------------------------------------------------
 * The sequence-parallel transformer layer around the collective matmuls
 * (attention between the AllGather->QKV projection and the output projection's
 * ReduceScatter; LayerNorm on the sequence shard between that ReduceScatter and
 * the next AllGather, the "do per-token work on the small shard" point of the
 * all-reduce paragraph of "Tensor Parallelism > Communication Patterns"; the
 * MLP activation between fc1 and fc2).  The pages name these stages but give
 * no formulas for them; the definitions below are the textbook ones:
 *
 *   attention (one head, query row t):
 *       s_j   = (q_t . k_j) / sqrt(D)     for j <= t (causal) or all j
 *       p_j   = exp(s_j - max_j s_j)
 *       out_t = sum_j p_j v_j / sum_j p_j
 *   LayerNorm (one row x of length n):
 *       mu = sum x / n,  var = sum (x - mu)^2 / n   (population variance)
 *       y  = (x - mu) / sqrt(var + eps) * gamma + beta
 *   GELU (exact form): gelu(x) = x * Phi(x) = 0.5 * x * (1 + erf(x / sqrt 2))
 * ------------------------------------------------------------------------ */

/*
 * Attention at selected (rank, head, query row) triples.
 *   qkv  [N][T][3*H*D] bf16: rank r's projection output; columns h*D.. hold
 *        the query of head h, H*D + h*D.. its key, 2*H*D + h*D.. its value
 *   out  [ns][D]: the head's output row
 *   mag  [ns][D] or NULL: sum_j p_j |v_jd| / sum_j p_j (the error scale of the
 *        weighted sum)
 */
void orc_attention_rows(int N, int T, int H, int D, int causal, const uint16_t *qkv, int ns,
                        const int *rank, const int *head, const int *row, double *out, double *mag) {
  (void)N;
  const size_t ld = (size_t)3 * H * D;
  const double scale = 1.0 / sqrt((double)D);
#pragma omp parallel
  {
    double *s = (double *)malloc(sizeof(double) * (size_t)T);
#pragma omp for schedule(dynamic)
    for (int t = 0; t < ns; ++t) {
      const int r = rank[t], h = head[t], i = row[t];
      const uint16_t *base = qkv + (size_t)r * T * ld;
      const uint16_t *q = base + (size_t)i * ld + (size_t)h * D;
      const int nk = causal ? i + 1 : T;
      double mx = -INFINITY;
      for (int j = 0; j < nk; ++j) {
        const uint16_t *kj = base + (size_t)j * ld + (size_t)H * D + (size_t)h * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += bf16_value(q[d]) * bf16_value(kj[d]);
        s[j] = dot * scale;
        if (s[j] > mx) mx = s[j];
      }
      double z = 0.0;
      for (int j = 0; j < nk; ++j) {
        s[j] = exp(s[j] - mx);
        z += s[j];
      }
      double *o = out + (size_t)t * D;
      double *mg = mag ? mag + (size_t)t * D : NULL;
      for (int d = 0; d < D; ++d) {
        double acc = 0.0, accabs = 0.0;
        for (int j = 0; j < nk; ++j) {
          const double v = bf16_value(base[(size_t)j * ld + (size_t)2 * H * D + (size_t)h * D + d]);
          acc += s[j] * v;
          accabs += s[j] * fabs(v);
        }
        o[d] = acc / z;
        if (mg) mg[d] = accabs / z;
      }
    }
    free(s);
  }
}

/*
 * LayerNorm of every row of x [rows][cols] (fp64 values) into y; gamma and
 * beta [cols] or NULL (1 and 0).
 */
void orc_layernorm(int rows, int cols, const double *x, double eps, const double *gamma,
                   const double *beta, double *y) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < rows; ++i) {
    const double *xi = x + (size_t)i * cols;
    double *yi = y + (size_t)i * cols;
    double sum = 0.0;
    for (int j = 0; j < cols; ++j) sum += xi[j];
    const double mu = sum / cols;
    double ss = 0.0;
    for (int j = 0; j < cols; ++j) ss += (xi[j] - mu) * (xi[j] - mu);
    const double inv = 1.0 / sqrt(ss / cols + eps);
    for (int j = 0; j < cols; ++j) {
      double v = (xi[j] - mu) * inv;
      if (gamma) v *= gamma[j];
      if (beta) v += beta[j];
      yi[j] = v;
    }
  }
}

/* GELU, exact (erf) form, elementwise. */
void orc_gelu(const double *x, double *y, size_t count) {
  for (size_t t = 0; t < count; ++t) y[t] = 0.5 * x[t] * (1.0 + erf(x[t] / sqrt(2.0)));
}

/* ------------------------------------------------------------------------
 * The backward pass of the two collective matmuls.  "Tensor Parallelism >
 * Communication Patterns" states that the backward communication pattern is
 * the dual of the forward one: the gradient of an AllGather->GEMM's input is
 * reduce-scattered, the gradient of a GEMM->ReduceScatter's input is
 * all-gathered.  With the forward definitions above:
 *
 *   column-parallel (forward Y_r = Xfull . W_r^T), given dY_r [T][n]:
 *       dX_q  = sum_r (dY_r . W_r)[q*m:(q+1)*m, :]      [m][k], ranks in order
 *       dW_r  = dY_r^T . Xfull                            [n][k]
 *   row-parallel (forward Out_q = sum_r (H_r . W_r^T)[q rows]), given dOut_q [m][n]:
 *       dH_r  = dOutfull . W_r                            [T][k], dOutfull = concat_q dOut_q
 *       dW_r  = dOutfull^T . H_r                          [n][k]
 *
 * These are the gradients of the scalar sum_r <dY_r, Y_r> (resp.
 * sum_q <dOut_q, Out_q>) with respect to X (resp. H) and W_r.  fp64, summed in
 * increasing index order; mag outputs (or NULL) receive the same sums of
 * absolute values.
 * ------------------------------------------------------------------------ */

/* out[i][j] = sum_t a[t*lda + i] * b[t*ldb + j] over t < T (a contraction over
 * the leading index of both operands), i < ni, j < nj. */
static void at_b(const uint16_t *a, int lda, const uint16_t *b, int ldb, int T, int ni, int nj, double *out,
                 double *mag) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < ni; ++i)
    for (int j = 0; j < nj; ++j) {
      double acc = 0.0, accabs = 0.0;
      for (int t = 0; t < T; ++t) {
        const double p = bf16_value(a[(size_t)t * lda + i]) * bf16_value(b[(size_t)t * ldb + j]);
        acc += p;
        accabs += fabs(p);
      }
      out[(size_t)i * nj + j] = acc;
      if (mag) mag[(size_t)i * nj + j] = accabs;
    }
}

/* out[t][j] = sum_c a[t][c] * w[c][j] (w stored [nc][nj], its leading index
 * contracted), t < rows. */
static void a_w(const uint16_t *a, const uint16_t *w, int rows, int nc, int nj, double *out, double *mag) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < rows; ++t)
    for (int j = 0; j < nj; ++j) {
      double acc = 0.0, accabs = 0.0;
      for (int c = 0; c < nc; ++c) {
        const double p = bf16_value(a[(size_t)t * nc + c]) * bf16_value(w[(size_t)c * nj + j]);
        acc += p;
        accabs += fabs(p);
      }
      out[(size_t)t * nj + j] = acc;
      if (mag) mag[(size_t)t * nj + j] = accabs;
    }
}

/*
 * Column-parallel backward.
 *   x  [N][m][k], w [N][n][k], dy [N][N*m][n]   (bf16)
 *   dx [N][m][k], dw [N][n][k]                  (fp64; mags or NULL)
 */
void orc_col_backward(int N, int m, int k, int n, const uint16_t *x, const uint16_t *w, const uint16_t *dy,
                      double *dx, double *dw, double *dx_mag, double *dw_mag) {
  const size_t T = (size_t)N * m;
  double *part = (double *)malloc(sizeof(double) * T * k);
  double *pmag = dx_mag ? (double *)malloc(sizeof(double) * T * k) : NULL;
  for (size_t i = 0; i < (size_t)N * m * k; ++i) {
    dx[i] = 0.0;
    if (dx_mag) dx_mag[i] = 0.0;
  }
  for (int r = 0; r < N; ++r) {
    /* dY_r . W_r over all T rows, then each owner q takes rows q*m.. */
    a_w(dy + (size_t)r * T * n, w + (size_t)r * n * k, (int)T, n, k, part, pmag);
    for (size_t i = 0; i < T * k; ++i) {
      dx[i] += part[i]; /* dx [N][m][k] is the row-major [T][k] of the owners' blocks */
      if (dx_mag) dx_mag[i] += pmag[i];
    }
    /* dW_r = dY_r^T . Xfull (Xfull rows = x read as [T][k]) */
    at_b(dy + (size_t)r * T * n, n, x, k, (int)T, n, k, dw + (size_t)r * n * k, dw_mag ? dw_mag + (size_t)r * n * k : NULL);
  }
  free(part);
  free(pmag);
}

/*
 * Row-parallel backward.
 *   h [N][N*m][k], w [N][n][k], dout [N][m][n]  (bf16)
 *   dh [N][N*m][k], dw [N][n][k]                (fp64; mags or NULL)
 */
void orc_row_backward(int N, int m, int k, int n, const uint16_t *h, const uint16_t *w, const uint16_t *dout,
                      double *dh, double *dw, double *dh_mag, double *dw_mag) {
  const size_t T = (size_t)N * m;
  for (int r = 0; r < N; ++r) {
    /* dH_r = dOutfull . W_r (dOutfull rows = dout read as [T][n]) */
    a_w(dout, w + (size_t)r * n * k, (int)T, n, k, dh + (size_t)r * T * k, dh_mag ? dh_mag + (size_t)r * T * k : NULL);
    /* dW_r = dOutfull^T . H_r */
    at_b(dout, n, h + (size_t)r * T * k, k, (int)T, n, k, dw + (size_t)r * n * k, dw_mag ? dw_mag + (size_t)r * n * k : NULL);
  }
}
