/*
 * CPU oracle for causal linear attention, its non-causal and RNN (decode) forms,
 * the same forms with other feature maps, the fast-weight delta rule and the
 * softmax decode baseline.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The GPU library never
 * links, loads or calls it, and the two share no code.
 *
 * Everything here is plain fp64 loops in the order the method states its
 * steps; there is no blocking, chunking or reordering.  Parallelism is only
 * over independent (batch, head) problems.
 *
 * Sources (the pages this follows):
 *   [TR]  "Transformers are RNNs: Fast Autoregressive Transformers with Linear
 *         Attention" (Katharopoulos et al., 2020), Chinese translation page
 *         "線性變換器": §3.1 eq.(3), §3.2 eq.(4)-(7), §3.3 eq.(8)-(12),
 *         §3.4 eq.(16)-(20).
 *   [FWP] News summary of "Linear Transformers Are Secretly Fast Weight
 *         Programmers" (Schlag, Irie, Schmidhuber, 2021): the paragraphs on the
 *         capacity limit, on the new update rule ("改進與更新") and on
 *         normalisation ("歸一化").
 *
 * The oracle_fmap_* functions repeat the causal and non-causal forms with the
 * other feature maps the pages name: DPFP-nu ([FWP], the DPFP paragraph) and
 * the degree-2 polynomial map ([TR] §3.2.1); the definitions are stated above
 * oracle_fmap_dim.
 *
 * The softmax decode step (oracle_softmax_decode) is the comparison baseline the
 * first page measures the recurrent form against: softmax attention, [TR] §3.1
 * eq.(2), evaluated for one new token over a cache of the earlier tokens' keys
 * and values ([TR] Appendix C.1, "stateful softmax").
 *
 * Layouts (row-major, contiguous, double precision):
 *   q, k : [BH, N, D]     v, o : [BH, N, M]
 *   S    : [BH, D, M]     z    : [BH, D]        W : [BH, M, D]
 *   beta : [BH, N]
 * BH = batch * heads; every (batch, head) pair is an independent problem.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef int64_t i64;

/* [TR] §3.2.1 eq.(7): phi(x) = elu(x) + 1 with alpha = 1.
 * For x > 0: x + 1.  For x <= 0: (exp(x) - 1) + 1 = exp(x); the exp form is
 * used directly so that very negative x keeps full relative accuracy. */
double oracle_phi(double x) { return x > 0.0 ? x + 1.0 : exp(x); }

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int oracle_get_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Explicit (quadratic) causal form, [TR] §3.3 eq.(8) with the kernel
 * similarity sim(q,k) = phi(q)^T phi(k) of eq.(4):
 *   o_i = sum_{j<=i} sim(q_i,k_j) v_j / sum_{j<=i} sim(q_i,k_j).
 * Computed only for the requested rows (0-based, per head: rows[h*nrows + r]),
 * out: [BH, nrows, M].  With rows = 0..N-1 it is the whole output. */
void oracle_causal_explicit_rows(const double* q, const double* k, const double* v,
                                 i64 BH, i64 N, i64 D, i64 M,
                                 const i64* rows, i64 nrows, double* out) {
#pragma omp parallel for schedule(dynamic)
  for (i64 h = 0; h < BH; ++h) {
    const double* qh = q + h * N * D;
    const double* kh = k + h * N * D;
    const double* vh = v + h * N * M;
    double* num = (double*)malloc(sizeof(double) * (size_t)M);
    for (i64 r = 0; r < nrows; ++r) {
      i64 i = rows[h * nrows + r];
      double den = 0.0;
      for (i64 m = 0; m < M; ++m) num[m] = 0.0;
      for (i64 j = 0; j <= i; ++j) {
        double sim = 0.0;
        for (i64 d = 0; d < D; ++d) sim += oracle_phi(qh[i * D + d]) * oracle_phi(kh[j * D + d]);
        for (i64 m = 0; m < M; ++m) num[m] += sim * vh[j * M + m];
        den += sim;
      }
      double* oh = out + (h * nrows + r) * M;
      for (i64 m = 0; m < M; ++m) oh[m] = num[m] / den;
    }
    free(num);
  }
}

/* Recurrent causal form, [TR] §3.3 eq.(10)-(12) (equivalently the RNN of
 * §3.4 eq.(16)-(20) without f_l and the residual):
 *   S_i = S_{i-1} + phi(k_i) v_i^T,  z_i = z_{i-1} + phi(k_i),
 *   o_i = phi(q_i)^T S_i / phi(q_i)^T z_i.
 * The state starts from (S0, z0) when given, else from zero (eq.(16)-(17)).
 * o may be NULL (state only).  S_out/z_out may be NULL. */
void oracle_causal_recurrent(const double* q, const double* k, const double* v,
                             i64 BH, i64 N, i64 D, i64 M,
                             const double* S0, const double* z0,
                             double* o, double* S_out, double* z_out) {
#pragma omp parallel for schedule(dynamic)
  for (i64 h = 0; h < BH; ++h) {
    double* S = (double*)malloc(sizeof(double) * (size_t)(D * M));
    double* z = (double*)malloc(sizeof(double) * (size_t)D);
    double* pk = (double*)malloc(sizeof(double) * (size_t)D);
    double* pq = (double*)malloc(sizeof(double) * (size_t)D);
    for (i64 e = 0; e < D * M; ++e) S[e] = S0 ? S0[h * D * M + e] : 0.0;
    for (i64 d = 0; d < D; ++d) z[d] = z0 ? z0[h * D + d] : 0.0;
    for (i64 i = 0; i < N; ++i) {
      const double* ki = k + (h * N + i) * D;
      const double* vi = v + (h * N + i) * M;
      const double* qi = q + (h * N + i) * D;
      for (i64 d = 0; d < D; ++d) pk[d] = oracle_phi(ki[d]);
      /* eq.(10)/(18): add the outer product phi(k_i) v_i^T */
      for (i64 d = 0; d < D; ++d)
        for (i64 m = 0; m < M; ++m) S[d * M + m] += pk[d] * vi[m];
      /* eq.(11)/(19) */
      for (i64 d = 0; d < D; ++d) z[d] += pk[d];
      if (o) {
        /* eq.(12)/(20): read with the state that already holds token i */
        for (i64 d = 0; d < D; ++d) pq[d] = oracle_phi(qi[d]);
        double den = 0.0;
        for (i64 d = 0; d < D; ++d) den += pq[d] * z[d];
        double* oi = o + (h * N + i) * M;
        for (i64 m = 0; m < M; ++m) {
          double num = 0.0;
          for (i64 d = 0; d < D; ++d) num += pq[d] * S[d * M + m];
          oi[m] = num / den;
        }
      }
    }
    if (S_out) memcpy(S_out + h * D * M, S, sizeof(double) * (size_t)(D * M));
    if (z_out) memcpy(z_out + h * D, z, sizeof(double) * (size_t)D);
    free(S); free(z); free(pk); free(pq);
  }
}

/* Explicit non-causal form, [TR] §3.2 eq.(4): the sums run over all j = 1..N.
 * Only the requested rows are produced: out [BH, nrows, M]. */
void oracle_noncausal_explicit_rows(const double* q, const double* k, const double* v,
                                    i64 BH, i64 N, i64 D, i64 M,
                                    const i64* rows, i64 nrows, double* out) {
#pragma omp parallel for schedule(dynamic)
  for (i64 h = 0; h < BH; ++h) {
    const double* qh = q + h * N * D;
    const double* kh = k + h * N * D;
    const double* vh = v + h * N * M;
    double* num = (double*)malloc(sizeof(double) * (size_t)M);
    for (i64 r = 0; r < nrows; ++r) {
      i64 i = rows[h * nrows + r];
      double den = 0.0;
      for (i64 m = 0; m < M; ++m) num[m] = 0.0;
      for (i64 j = 0; j < N; ++j) {
        double sim = 0.0;
        for (i64 d = 0; d < D; ++d) sim += oracle_phi(qh[i * D + d]) * oracle_phi(kh[j * D + d]);
        for (i64 m = 0; m < M; ++m) num[m] += sim * vh[j * M + m];
        den += sim;
      }
      double* oh = out + (h * nrows + r) * M;
      for (i64 m = 0; m < M; ++m) oh[m] = num[m] / den;
    }
    free(num);
  }
}

/* Non-causal form by associativity, [TR] §3.2 eq.(5)-(6):
 *   S = sum_j phi(k_j) v_j^T,  z = sum_j phi(k_j),  o_i = phi(q_i)^T S / phi(q_i)^T z.
 * S_out/z_out may be NULL. */
void oracle_noncausal(const double* q, const double* k, const double* v,
                      i64 BH, i64 N, i64 D, i64 M, double* o,
                      double* S_out, double* z_out) {
#pragma omp parallel for schedule(dynamic)
  for (i64 h = 0; h < BH; ++h) {
    double* S = (double*)calloc((size_t)(D * M), sizeof(double));
    double* z = (double*)calloc((size_t)D, sizeof(double));
    double* p = (double*)malloc(sizeof(double) * (size_t)D);
    for (i64 j = 0; j < N; ++j) {
      const double* kj = k + (h * N + j) * D;
      const double* vj = v + (h * N + j) * M;
      for (i64 d = 0; d < D; ++d) p[d] = oracle_phi(kj[d]);
      for (i64 d = 0; d < D; ++d)
        for (i64 m = 0; m < M; ++m) S[d * M + m] += p[d] * vj[m];
      for (i64 d = 0; d < D; ++d) z[d] += p[d];
    }
    for (i64 i = 0; i < N; ++i) {
      const double* qi = q + (h * N + i) * D;
      for (i64 d = 0; d < D; ++d) p[d] = oracle_phi(qi[d]);
      double den = 0.0;
      for (i64 d = 0; d < D; ++d) den += p[d] * z[d];
      double* oi = o + (h * N + i) * M;
      for (i64 m = 0; m < M; ++m) {
        double num = 0.0;
        for (i64 d = 0; d < D; ++d) num += p[d] * S[d * M + m];
        oi[m] = num / den;
      }
    }
    if (S_out) memcpy(S_out + h * D * M, S, sizeof(double) * (size_t)(D * M));
    if (z_out) memcpy(z_out + h * D, z, sizeof(double) * (size_t)D);
    free(S); free(z); free(p);
  }
}

/* One RNN step, [TR] §3.4 eq.(18)-(20) without f_l and the residual, applied
 * in place to every (batch, head) state:
 *   s <- s + phi(k) v^T,  z <- z + phi(k),  o = phi(q)^T s / phi(q)^T z.
 * q, k: [BH, D]; v, o: [BH, M]; S: [BH, D, M]; z: [BH, D]. */
void oracle_decode_step(const double* q, const double* k, const double* v,
                        i64 BH, i64 D, i64 M, double* S, double* z, double* o) {
#pragma omp parallel for schedule(static)
  for (i64 h = 0; h < BH; ++h) {
    double* Sh = S + h * D * M;
    double* zh = z + h * D;
    const double* kh = k + h * D;
    const double* qh = q + h * D;
    const double* vh = v + h * M;
    for (i64 d = 0; d < D; ++d) {
      double pk = oracle_phi(kh[d]);
      for (i64 m = 0; m < M; ++m) Sh[d * M + m] += pk * vh[m];
      zh[d] += pk;
    }
    double den = 0.0;
    for (i64 d = 0; d < D; ++d) den += oracle_phi(qh[d]) * zh[d];
    for (i64 m = 0; m < M; ++m) {
      double num = 0.0;
      for (i64 d = 0; d < D; ++d) num += oracle_phi(qh[d]) * Sh[d * M + m];
      o[h * M + m] = num / den;
    }
  }
}

/* Fast-weight memory with the delta update rule, [FWP] paragraphs on the
 * update rule and on normalisation.  For each token i, in order:
 *   kh = phi(k_i) / sum_c phi(k_i)_c,   qh = phi(q_i) / sum_c phi(q_i)_c
 *        (the keys and queries are divided by the sum of their components);
 *   vbar = W kh                          (retrieve the value now bound to k_i);
 *   vnew = beta_i v_i + (1 - beta_i) vbar (convex combination, 0 <= beta_i <= 1);
 *   W <- W - vbar kh^T + vnew kh^T       (remove the old pair, write the new one);
 *   o_i = W qh                           (read after the write, as in [TR] eq.(12)).
 * W starts from W0 when given, else zero.  W: [BH, M, D].  W_out may be NULL. */
void oracle_deltanet(const double* q, const double* k, const double* v, const double* beta,
                     i64 BH, i64 N, i64 D, i64 M, const double* W0,
                     double* o, double* W_out) {
#pragma omp parallel for schedule(dynamic)
  for (i64 h = 0; h < BH; ++h) {
    double* W = (double*)malloc(sizeof(double) * (size_t)(M * D));
    double* kh = (double*)malloc(sizeof(double) * (size_t)D);
    double* qh = (double*)malloc(sizeof(double) * (size_t)D);
    double* vbar = (double*)malloc(sizeof(double) * (size_t)M);
    for (i64 e = 0; e < M * D; ++e) W[e] = W0 ? W0[h * M * D + e] : 0.0;
    for (i64 i = 0; i < N; ++i) {
      const double* ki = k + (h * N + i) * D;
      const double* qi = q + (h * N + i) * D;
      const double* vi = v + (h * N + i) * M;
      const double b = beta[h * N + i];
      double sk = 0.0, sq = 0.0;
      for (i64 d = 0; d < D; ++d) { kh[d] = oracle_phi(ki[d]); sk += kh[d]; }
      for (i64 d = 0; d < D; ++d) { qh[d] = oracle_phi(qi[d]); sq += qh[d]; }
      for (i64 d = 0; d < D; ++d) { kh[d] /= sk; qh[d] /= sq; }
      for (i64 m = 0; m < M; ++m) {
        double acc = 0.0;
        for (i64 d = 0; d < D; ++d) acc += W[m * D + d] * kh[d];
        vbar[m] = acc;
      }
      for (i64 m = 0; m < M; ++m) {
        const double vnew = b * vi[m] + (1.0 - b) * vbar[m];
        for (i64 d = 0; d < D; ++d)
          W[m * D + d] = W[m * D + d] - vbar[m] * kh[d] + vnew * kh[d];
      }
      double* oi = o + (h * N + i) * M;
      for (i64 m = 0; m < M; ++m) {
        double acc = 0.0;
        for (i64 d = 0; d < D; ++d) acc += W[m * D + d] * qh[d];
        oi[m] = acc;
      }
    }
    if (W_out) memcpy(W_out + h * M * D, W, sizeof(double) * (size_t)(M * D));
    free(W); free(kh); free(qh); free(vbar);
  }
}

/* Softmax attention for one new token over a key/value cache: the "stateful
 * softmax" of [TR] Appendix C.1 (the keys and values of earlier tokens are kept
 * rather than recomputed), with the attention of [TR] §3.1 eq.(2),
 *   o = softmax(q K^T / sqrt(D)) V,
 * over rows 0..L of the cache, where row L holds the new token's key and value
 * (the caller appends them).  The largest score is subtracted before the
 * exponentials, which leaves the weights unchanged.
 * q: [BH, D]; Kc: [BH, Lmax, D]; Vc: [BH, Lmax, M]; o: [BH, M]. */
void oracle_softmax_decode(const double* q, const double* Kc, const double* Vc, i64 BH, i64 L, i64 Lmax, i64 D,
                           i64 M, double* o) {
#pragma omp parallel for schedule(static)
  for (i64 h = 0; h < BH; ++h) {
    const double* qh = q + h * D;
    const double* Kh = Kc + h * Lmax * D;
    const double* Vh = Vc + h * Lmax * M;
    double* w = (double*)malloc(sizeof(double) * (size_t)(L + 1));
    double mx = -INFINITY;
    for (i64 j = 0; j <= L; ++j) {
      double s = 0.0;
      for (i64 d = 0; d < D; ++d) s += qh[d] * Kh[j * D + d];
      w[j] = s / sqrt((double)D);
      if (w[j] > mx) mx = w[j];
    }
    double tot = 0.0;
    for (i64 j = 0; j <= L; ++j) {
      w[j] = exp(w[j] - mx);
      tot += w[j];
    }
    for (i64 m = 0; m < M; ++m) {
      double acc = 0.0;
      for (i64 j = 0; j <= L; ++j) acc += w[j] * Vh[j * M + m];
      o[h * M + m] = acc / tot;
    }
    free(w);
  }
}

/* ---- Other feature maps ---------------------------------------------------
 * [TR] §3.2.1 allows any feature map phi: R^D -> R^C in place of elu + 1; the
 * cost becomes O(N C M).  Two maps the pages name are built:
 *
 * fmap = 1, DPFP-nu ([FWP], the DPFP paragraph and the figure it describes:
 *   a deterministic, parameter-free map that raises the dot-product dimension;
 *   in two dimensions each input has one non-zero output among four, and the
 *   four quadrants land on mutually orthogonal directions).  The formula is
 *   not printed; the reading taken is
 *     r = (relu(x_0..x_{D-1}), relu(-x_0..-x_{D-1}))              in R^{2D},
 *     phi(x)_{(n-1) 2D + i} = r_i * r_{(i + n) mod 2D},  i < 2D,  n = 1..nu,
 *   so C = 2 nu D.
 * fmap = 2, degree-2 polynomial kernel ([TR] §3.2.1: an exact finite feature
 *   map, cost O(N D^2 M)): phi(x)_{a D + b} = x_a x_b, C = D^2, so that
 *   phi(q).phi(k) = (q.k)^2.
 *
 * With phi of dimension C the causal and non-causal forms are eq.(8)-(12) and
 * eq.(5)-(6) unchanged: S has shape [C, M] and z [C]. */

i64 oracle_fmap_dim(int fmap, int nu, i64 D) {
  if (fmap == 1) return 2 * (i64)nu * D;
  if (fmap == 2) return D * D;
  return 0;
}

void oracle_fmap(const double* x, i64 D, int fmap, int nu, double* out) {
  if (fmap == 1) {
    const i64 R = 2 * D;
    for (int n = 1; n <= nu; ++n)
      for (i64 i = 0; i < R; ++i) {
        const i64 j = (i + n) % R;
        const double ri = i < D ? (x[i] > 0.0 ? x[i] : 0.0) : (x[i - D] < 0.0 ? -x[i - D] : 0.0);
        const double rj = j < D ? (x[j] > 0.0 ? x[j] : 0.0) : (x[j - D] < 0.0 ? -x[j - D] : 0.0);
        out[(n - 1) * R + i] = ri * rj;
      }
  } else if (fmap == 2) {
    for (i64 a = 0; a < D; ++a)
      for (i64 b = 0; b < D; ++b) out[a * D + b] = x[a] * x[b];
  }
}

/* Recurrent causal form, eq.(10)-(12), with the feature map fmap:
 *   S_i = S_{i-1} + phi(k_i) v_i^T,  z_i = z_{i-1} + phi(k_i),
 *   o_i = phi(q_i)^T S_i / phi(q_i)^T z_i.
 * S0/z0 ([BH, C, M], [BH, C]) may be NULL (zero start); o, S_out, z_out may be NULL. */
void oracle_fmap_causal(const double* q, const double* k, const double* v, i64 BH, i64 N, i64 D, i64 M,
                        int fmap, int nu, const double* S0, const double* z0,
                        double* o, double* S_out, double* z_out) {
  const i64 C = oracle_fmap_dim(fmap, nu, D);
#pragma omp parallel for schedule(dynamic)
  for (i64 h = 0; h < BH; ++h) {
    double* S = (double*)malloc(sizeof(double) * (size_t)(C * M));
    double* z = (double*)malloc(sizeof(double) * (size_t)C);
    double* pk = (double*)malloc(sizeof(double) * (size_t)C);
    double* pq = (double*)malloc(sizeof(double) * (size_t)C);
    for (i64 e = 0; e < C * M; ++e) S[e] = S0 ? S0[h * C * M + e] : 0.0;
    for (i64 c = 0; c < C; ++c) z[c] = z0 ? z0[h * C + c] : 0.0;
    for (i64 i = 0; i < N; ++i) {
      const double* vi = v + (h * N + i) * M;
      oracle_fmap(k + (h * N + i) * D, D, fmap, nu, pk);
      for (i64 c = 0; c < C; ++c)
        for (i64 m = 0; m < M; ++m) S[c * M + m] += pk[c] * vi[m];
      for (i64 c = 0; c < C; ++c) z[c] += pk[c];
      if (o) {
        oracle_fmap(q + (h * N + i) * D, D, fmap, nu, pq);
        double den = 0.0;
        for (i64 c = 0; c < C; ++c) den += pq[c] * z[c];
        double* oi = o + (h * N + i) * M;
        for (i64 m = 0; m < M; ++m) {
          double num = 0.0;
          for (i64 c = 0; c < C; ++c) num += pq[c] * S[c * M + m];
          oi[m] = num / den;
        }
      }
    }
    if (S_out) memcpy(S_out + h * C * M, S, sizeof(double) * (size_t)(C * M));
    if (z_out) memcpy(z_out + h * C, z, sizeof(double) * (size_t)C);
    free(S); free(z); free(pk); free(pq);
  }
}

/* Non-causal form, eq.(5)-(6), with the feature map fmap: S = sum_j phi(k_j) v_j^T,
 * z = sum_j phi(k_j) over all N tokens, then o_i = phi(q_i)^T S / phi(q_i)^T z. */
void oracle_fmap_noncausal(const double* q, const double* k, const double* v, i64 BH, i64 N, i64 D, i64 M,
                           int fmap, int nu, double* o, double* S_out, double* z_out) {
  const i64 C = oracle_fmap_dim(fmap, nu, D);
#pragma omp parallel for schedule(dynamic)
  for (i64 h = 0; h < BH; ++h) {
    double* S = (double*)calloc((size_t)(C * M), sizeof(double));
    double* z = (double*)calloc((size_t)C, sizeof(double));
    double* p = (double*)malloc(sizeof(double) * (size_t)C);
    for (i64 j = 0; j < N; ++j) {
      const double* vj = v + (h * N + j) * M;
      oracle_fmap(k + (h * N + j) * D, D, fmap, nu, p);
      for (i64 c = 0; c < C; ++c)
        for (i64 m = 0; m < M; ++m) S[c * M + m] += p[c] * vj[m];
      for (i64 c = 0; c < C; ++c) z[c] += p[c];
    }
    for (i64 i = 0; i < N; ++i) {
      oracle_fmap(q + (h * N + i) * D, D, fmap, nu, p);
      double den = 0.0;
      for (i64 c = 0; c < C; ++c) den += p[c] * z[c];
      double* oi = o + (h * N + i) * M;
      for (i64 m = 0; m < M; ++m) {
        double num = 0.0;
        for (i64 c = 0; c < C; ++c) num += p[c] * S[c * M + m];
        oi[m] = num / den;
      }
    }
    if (S_out) memcpy(S_out + h * C * M, S, sizeof(double) * (size_t)(C * M));
    if (z_out) memcpy(z_out + h * C, z, sizeof(double) * (size_t)C);
    free(S); free(z); free(p);
  }
}
