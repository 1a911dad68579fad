/*
 * CPU oracle for the edge-aware attention layer (FlexAttentionGT layer).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do. It shares no code, header, table or helper with the
 * HIP path.
 *
 * What it computes is the plain definition of one layer forward plus the
 * residual edge update, written out as loops in double precision. Source:
 * "Efficient Edge-aware Attention Network for Graph Generation"
 * (ai-frontier-tracker digest, full-text summary): standard scaled dot-product
 * attention replaces the per-channel outer product; head-wise FiLM injects the
 * edge features and the global feature into the scores inside score_mod; the
 * graph mask is respected; softmax gives normalized coefficients; the value is
 * augmented with the identity so one pass returns the node aggregation and the
 * attention map; the edge representation then takes a residual update from the
 * attention map. The English abstract on the same page and on the arXiv
 * listing page states the same structure (head-wise score modulation, graph
 * masks, a lightweight residual edge update that depends on attention scores);
 * the kongchang.com explainer ("Head-wise score modulation") states that the
 * modulation is per head and acts on the scores only.
 *
 * Readings taken where the pages are silent (the pages give no formulas):
 *   - score scale 1/sqrt(dh) (standard scaled dot product);
 *   - FiLM: gamma = 1 + linear(feature), beta = linear(feature), applied as
 *     s*gamma + beta; edge FiLM first, then global FiLM:
 *       u = (s * gamma_e + beta_e) * gamma_y + beta_y;
 *   - pair mask m_i AND m_j; a row with no real key gives A = 0 and O = 0;
 *   - head split: feature c = h*dh + t; weights in [out, in] layout;
 *   - edge update E'_ij = E_ij + W_e A_ij + b_e with W_e [de, H], on real
 *     pairs; every masked output is +0.0;
 *   - bf16 mode: Q, K, V are rounded to bfloat16 after their projection, A is
 *     rounded to bfloat16 and that rounded A is what A*V and the edge update
 *     use; everything else stays in double here (the oracle does not round
 *     its outputs).
 *
 * Ablation variants (dims.variant bits). The summary section of the same page
 * reports ablations of the layer: without the per-edge modulation ("Light
 * Edge") the model does not learn, neither the edge update nor the score
 * modulation can be dropped, and normalized attention coefficients converge
 * more stably than unnormalized ones. Readings taken, each the plainest one:
 *   - 1, light edge: no per-edge FiLM, gamma_e = 1 and beta_e = 0 (the
 *     global FiLM stays): u = s * gamma_y + beta_y;
 *   - 2, no score modulation: neither FiLM, u = s (masked SDPA);
 *   - 4, unnormalized update: the edge update takes the coefficients before
 *     normalization, i.e. the masked logits u themselves (0 at masked pairs),
 *     E'_ij = E_ij + W_e u_ij + b_e; O and A stay normalized. In bf16 mode
 *     that operand is rounded to bfloat16 like A is.
 *
 * Parity status: every function below is pinned by the CPU test suite
 * (closed forms, a hand-worked example, library SDPA special cases, mask
 * enumeration, invariants). Absolute agreement with the authors' trained layer
 * is not pinned by anything on the pages (they print no formulas or values).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int32_t B, n, d, de, dy, H, dh;
  int32_t bf16;    /* 1: apply the bfloat16 rounding points */
  int32_t variant; /* ablation bits: 1 light edge, 2 no score modulation, 4 unnormalized update */
} eao_dims;

enum { EAO_LIGHT_EDGE = 1, EAO_NO_SCORE_MOD = 2, EAO_UNNORMALIZED = 4 };

/* All weights float32 in nn.Linear layout [out, in]; any bias may be NULL. */
typedef struct {
  const float *w_q, *w_k, *w_v, *b_q, *b_k, *b_v;     /* [d,d], [d]   */
  const float *w_emul, *w_eadd, *b_emul, *b_eadd;     /* [H,de], [H]  */
  const float *w_ymul, *w_yadd, *b_ymul, *b_yadd;     /* [H,dy], [H]  */
  const float *w_e, *b_e;                             /* [de,H], [de] */
} eao_params;

static double bias_at(const float* b, int k) { return b ? (double)b[k] : 0.0; }

/*
 * Round a double to the nearest bfloat16 value (8 significant bits, float32
 * exponent range), ties to even. NaN stays NaN, overflow goes to +-inf.
 */
double eao_bf16_round(double x) {
  if (isnan(x) || isinf(x) || x == 0.0) return x;
  const double sub_min = ldexp(1.0, -126);          /* smallest normal      */
  if (fabs(x) < sub_min) {                          /* subnormal: grid 2^-133 */
    return nearbyint(x * ldexp(1.0, 133)) * ldexp(1.0, -133);
  }
  int e;
  double m = frexp(x, &e);                          /* |m| in [0.5, 1)     */
  double r = ldexp(nearbyint(ldexp(m, 8)), e - 8);  /* keep 8 bits, RNE    */
  const double maxv = ldexp(255.0, 127 - 7);        /* (2 - 2^-7) * 2^127  */
  if (fabs(r) > maxv) return x > 0 ? INFINITY : -INFINITY;
  return r;
}

/*
 * Node projections for one graph b: out[i][c] = b[c] + sum_k X[b,i,k] W[c][k].
 * Padded nodes (mask 0) get a zero row; they are never read by the layer.
 */
static void project_graph(const eao_dims* dm, const float* X, const uint8_t* mask,
                          int b, const float* W, const float* bias, double* out) {
  const int n = dm->n, d = dm->d;
  for (int i = 0; i < n; ++i) {
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      if (mask[(size_t)b * n + i]) {
        acc = bias_at(bias, c);
        const float* x = X + ((size_t)b * n + i) * d;
        const float* w = W + (size_t)c * d;
        for (int k = 0; k < d; ++k) acc += (double)x[k] * (double)w[k];
        if (dm->bf16) acc = eao_bf16_round(acc);
      }
      out[(size_t)i * d + c] = acc;
    }
  }
}

/* Exported projection (all graphs) so that tests can check this step alone. */
void eao_project(const eao_dims* dm, const float* X, const uint8_t* mask,
                 const float* W, const float* bias, double* out /*[B,n,d]*/) {
  for (int b = 0; b < dm->B; ++b)
    project_graph(dm, X, mask, b, W, bias, out + (size_t)b * dm->n * dm->d);
}

/* Global FiLM of graph b: gamma_y[h] = 1 + lin_mul(y), beta_y[h] = lin_add(y). */
static void global_film(const eao_dims* dm, const float* y, int b, const eao_params* p,
                        double* gamma_y, double* beta_y) {
  for (int h = 0; h < dm->H; ++h) {
    if (dm->variant & EAO_NO_SCORE_MOD) { gamma_y[h] = 1.0; beta_y[h] = 0.0; continue; }
    double gm = bias_at(p->b_ymul, h), ga = bias_at(p->b_yadd, h);
    for (int c = 0; c < dm->dy; ++c) {
      double yc = y[(size_t)b * dm->dy + c];
      gm += yc * (double)p->w_ymul[(size_t)h * dm->dy + c];
      ga += yc * (double)p->w_yadd[(size_t)h * dm->dy + c];
    }
    gamma_y[h] = 1.0 + gm;
    beta_y[h] = ga;
  }
}

/*
 * One query row (b, i): logits u[h][j], attention A[h][j], lse[h], node
 * output O[c] and edge output Ep[j][c]. Q, K, V are the graph's projections.
 */
static void layer_row(const eao_dims* dm, const float* E, const uint8_t* mask,
                      const eao_params* p, int b, int i,
                      const double* Q, const double* K, const double* V,
                      const double* gamma_y, const double* beta_y,
                      double* O, double* A, double* Ep, double* U, double* lse) {
  const int n = dm->n, d = dm->d, de = dm->de, H = dm->H, dh = dm->dh;
  const uint8_t* m = mask + (size_t)b * n;
  const double r = 1.0 / sqrt((double)dh);
  const float* Erow = E + ((size_t)b * n + i) * (size_t)n * de;

  for (int h = 0; h < H; ++h) {
    double* u = U + (size_t)h * n;
    double* a = A + (size_t)h * n;
    /* scores, FiLM and mask */
    for (int j = 0; j < n; ++j) {
      if (!(m[i] && m[j])) { u[j] = -INFINITY; continue; }
      const float* e = Erow + (size_t)j * de;
      double gm = 0.0, ga = 0.0;
      if (!(dm->variant & (EAO_LIGHT_EDGE | EAO_NO_SCORE_MOD))) {
        gm = bias_at(p->b_emul, h);
        ga = bias_at(p->b_eadd, h);
        for (int c = 0; c < de; ++c) {
          gm += (double)e[c] * (double)p->w_emul[(size_t)h * de + c];
          ga += (double)e[c] * (double)p->w_eadd[(size_t)h * de + c];
        }
      }
      const double gamma_e = 1.0 + gm, beta_e = ga;
      double s = 0.0;
      for (int t = 0; t < dh; ++t)
        s += Q[(size_t)i * d + h * dh + t] * K[(size_t)j * d + h * dh + t];
      s *= r;
      u[j] = (s * gamma_e + beta_e) * gamma_y[h] + beta_y[h];
    }
    /* masked softmax over j */
    double M = -INFINITY;
    for (int j = 0; j < n; ++j) if (u[j] > M) M = u[j];
    if (M == -INFINITY) {
      for (int j = 0; j < n; ++j) a[j] = 0.0;
      lse[h] = -INFINITY;
    } else {
      double L = 0.0;
      for (int j = 0; j < n; ++j) {
        a[j] = (u[j] == -INFINITY) ? 0.0 : exp(u[j] - M);
        L += a[j];
      }
      for (int j = 0; j < n; ++j) {
        a[j] = a[j] / L;
        if (dm->bf16) a[j] = eao_bf16_round(a[j]);
      }
      lse[h] = M + log(L);
    }
    /* node aggregation O = A V for this head */
    for (int t = 0; t < dh; ++t) {
      double acc = 0.0;
      for (int j = 0; j < n; ++j) acc += a[j] * V[(size_t)j * d + h * dh + t];
      O[h * dh + t] = acc;
    }
  }
  /* residual edge update, from A (or, unnormalized variant, from u) */
  const int unnorm = (dm->variant & EAO_UNNORMALIZED) != 0;
  for (int j = 0; j < n; ++j) {
    double* ep = Ep + (size_t)j * de;
    if (!(m[i] && m[j])) { for (int c = 0; c < de; ++c) ep[c] = 0.0; continue; }
    const float* e = Erow + (size_t)j * de;
    double coef[64];
    for (int h = 0; h < H; ++h) {
      coef[h] = A[(size_t)h * n + j];
      if (unnorm) coef[h] = dm->bf16 ? eao_bf16_round(U[(size_t)h * n + j]) : U[(size_t)h * n + j];
    }
    for (int c = 0; c < de; ++c) {
      double acc = (double)e[c] + bias_at(p->b_e, c);
      for (int h = 0; h < H; ++h) acc += (double)p->w_e[(size_t)c * H + h] * coef[h];
      ep[c] = acc;
    }
  }
}

/*
 * Forward + edge update for a list of query rows (row_b[r], row_i[r]).
 * Outputs are compact, one slot per requested row:
 *   O  [nrows][d], A [nrows][H][n], Ep [nrows][n][de],
 *   U  [nrows][H][n] (logits, may be NULL), lse [nrows][H] (may be NULL).
 * Rows must be grouped by graph (all rows of one graph contiguous) so that a
 * graph's projections are computed once. Returns 0, or -1 on bad arguments.
 */
int eao_forward_rows(const eao_dims* dm, const float* X, const float* E, const float* y,
                     const uint8_t* mask, const eao_params* p,
                     int nrows, const int32_t* row_b, const int32_t* row_i,
                     double* O, double* A, double* Ep, double* U, double* lse) {
  if (!dm || !X || !E || !y || !mask || !p || !O || !A || !Ep) return -1;
  if (dm->d != dm->H * dm->dh || dm->n < 1 || dm->B < 1 || dm->H > 64) return -1;
  const int n = dm->n, d = dm->d, de = dm->de, H = dm->H;
  const size_t nd = (size_t)n * d;
  double* Q = (double*)malloc(sizeof(double) * nd);
  double* K = (double*)malloc(sizeof(double) * nd);
  double* V = (double*)malloc(sizeof(double) * nd);
  double* Uall = U ? NULL : (double*)malloc(sizeof(double) * (size_t)nrows * H * n);
  double* Lall = lse ? NULL : (double*)malloc(sizeof(double) * (size_t)nrows * H);
  double* Uo = U ? U : Uall;
  double* Lo = lse ? lse : Lall;
  if (!Q || !K || !V || !Uo || !Lo) { free(Q); free(K); free(V); free(Uall); free(Lall); return -1; }

  int start = 0;
  while (start < nrows) {
    const int b = row_b[start];
    int end = start;
    while (end < nrows && row_b[end] == b) ++end;
    if (b < 0 || b >= dm->B) { start = end; continue; }
    project_graph(dm, X, mask, b, p->w_q, p->b_q, Q);
    project_graph(dm, X, mask, b, p->w_k, p->b_k, K);
    project_graph(dm, X, mask, b, p->w_v, p->b_v, V);
    double gamma_y[64], beta_y[64];
    global_film(dm, y, b, p, gamma_y, beta_y);
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = start; r < end; ++r) {
      const int i = row_i[r];
      if (i < 0 || i >= n) continue;
      layer_row(dm, E, mask, p, b, i, Q, K, V, gamma_y, beta_y,
                O + (size_t)r * d, A + (size_t)r * H * n, Ep + (size_t)r * n * de,
                Uo + (size_t)r * H * n, Lo + (size_t)r * H);
      if (!mask[(size_t)b * n + i]) {
        for (int c = 0; c < d; ++c) O[(size_t)r * d + c] = 0.0;
      }
    }
    start = end;
  }
  free(Q); free(K); free(V); free(Uall); free(Lall);
  return 0;
}

/*
 * The literal [V | I] aggregation for one row: out[h][0..dh) = sum_j A_ij V_j
 * and out[h][dh + k] = sum_j A_ij * [j == k], i.e. attention times the value
 * matrix augmented with the n x n identity (the single-call trick that returns
 * node aggregation and attention map together). Used only to check that
 * writing A directly is the same result.
 */
void eao_vi_product(const eao_dims* dm, const double* A_row /*[H][n]*/, const double* V /*[n][d]*/,
                    double* out /*[H][dh+n]*/) {
  const int n = dm->n, d = dm->d, H = dm->H, dh = dm->dh, w = dh + n;
  for (int h = 0; h < H; ++h) {
    for (int col = 0; col < w; ++col) {
      double acc = 0.0;
      for (int j = 0; j < n; ++j) {
        const double vij = col < dh ? V[(size_t)j * d + h * dh + col] : (j == col - dh ? 1.0 : 0.0);
        acc += A_row[(size_t)h * n + j] * vij;
      }
      out[(size_t)h * w + col] = acc;
    }
  }
}

/* Threads the row loop uses (1 without OpenMP). */
int eao_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads the row loop uses from now on (timing legs: 1 thread, all cores);
   returns the previous count. No effect without OpenMP. */
int eao_set_num_threads(int t) {
#ifdef _OPENMP
  const int prev = omp_get_max_threads();
  if (t >= 1) omp_set_num_threads(t);
  return prev;
#else
  (void)t;
  return 1;
#endif
}
