/*
 * moe_oracle.c -- plain, slow CPU oracle of the routed-experts layer (TEST INFRASTRUCTURE ONLY).
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg use this file. It shares
 * no code, header, table or helper with the GPU library, and the GPU library never calls it.
 *
 * What it computes is the definition of the layer, written out element by element:
 *
 *   Dist-MoE 0.1.0 (PyPI page), "Understand the execution model": caller routing (x, expert ids,
 *   scores) goes through route -> W13 -> SwiGLU -> W2 -> combine; forward GEMMs are FPROP, the
 *   input-gradient GEMMs DGRAD and the weight-gradient GEMMs WGRAD.
 *   Dist-MoE, "BF16 Quickstart": x[T,D], ids[T,K] in [0,E), scores[T,K], w13[E,2,F,D] (the gate/up
 *   axis explicit; same bytes as [E,2F,D]) and w2[E,D,F].
 *   Dist-MoE, "Choose a precision and pipeline / BF16": activations and weights enter the expert
 *   GEMMs in BF16 and the products accumulate in FP32.
 *   TeraMoE README, worker list: compute = gate/up projection, activation, down projection;
 *   combine applies the weighted accumulation of the routed results; gather reduces several
 *   expert results of one token.
 *   MegaMoE (ROCm Primus technical guide), introduction and "Configuration": gated SwiGLU with SiLU
 *   between the two grouped GEMMs, and the score-weighted reduce happens at combine.
 *
 * Readings taken where the pages leave a step open (each is also listed with the design notes):
 *   - w13[e,0] is the gate, w13[e,1] the up projection; weights are [out,in] (y = W x).
 *   - SwiGLU: a = silu(g) * u with silu(z) = z * sigmoid(z), sigmoid(z) = 1/(1+exp(-z)).
 *   - scores weight the expert outputs after W2, at combine.
 *   - slot i = t*K + k; expert-grouped row order is a stable counting sort of the flat slots.
 *   - out-of-range ids: the slot is dropped (no row, contributes nothing) and counted.
 *   - bf16 storage points (round_bf16 = 1): every GEMM output that is stored (h13 = [g|u], y,
 *     dxg, dW13, dW2) and every GEMM operand produced by element-wise math (a, dy, dh13), and the
 *     combined outputs out and dx, are rounded once to bf16 (nearest-even). SwiGLU and its
 *     derivative read the rounded g and u. dscores and the transient da are not rounded.
 *   - sums are evaluated in double precision in ascending index order: the value that the FP32
 *     accumulation of the pages approximates. round_bf16 = 0 gives the exact (unrounded) layer.
 *
 * Inputs may be bf16 bit patterns (uint16) or doubles (in_dtype); every intermediate and output is
 * an array of doubles (bf16-representable values when round_bf16 = 1).
 *
 * Error scales (optional outputs, test infrastructure): for every output that is a sum of terms
 * (out and dx over the K slots, dscores over D, dW13 and dW2 over an expert's rows), the
 * root-sum-square of its terms, sqrt(sum term^2). It is not part of the layer; the parity tests use
 * it as the size scale of a reduction whose terms cancel, since a one-ulp difference in a bf16
 * operand moves a sum by at most 2^-7 of that term.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_IN_BF16 0
#define ORACLE_IN_F64 1

typedef struct oracle_shape {
  int64_t T, D, F, E, K;
  int32_t round_bf16; /* 1: bf16 storage points; 0: exact evaluation */
  int32_t in_dtype;   /* ORACLE_IN_BF16 or ORACLE_IN_F64 for x, w13, w2, dout */
  int32_t wgrad_f32;  /* 1: dW13, dW2 are stored in fp32 (no bf16 rounding at that point) */
} oracle_shape;

/* ------------------------------------------------------------------------------------------- */
/* scalar helpers                                                                                */

/* Round a double to the nearest bf16 value (8 significant bits, ties to even, fp32 exponent range
 * with gradual underflow at 2^-133 spacing, overflow to infinity). Written from the format: scale
 * so that one bf16 unit in the last place is 1, round to the nearest integer (ties to even, the
 * default floating-point rounding mode), scale back. */
double oracle_round_bf16(double v) {
  if (isnan(v)) return NAN;
  if (isinf(v) || v == 0.0) return v;
  int ex;
  frexp(fabs(v), &ex); /* |v| = m * 2^ex, m in [0.5, 1) */
  int q = ex - 8;      /* exponent of one bf16 ulp at this magnitude */
  if (q < -133) q = -133;
  double r = ldexp(nearbyint(ldexp(v, -q)), q);
  if (fabs(r) > 0x1.FCp127) r = copysign(INFINITY, v); /* above the largest finite bf16 */
  return r;
}

static inline double bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static inline double ld(const void* p, int64_t i, int32_t dt) {
  if (dt == ORACLE_IN_BF16) return bits_to_double(((const uint16_t*)p)[i]);
  return ((const double*)p)[i];
}

static inline double R(const oracle_shape* s, double v) {
  return s->round_bf16 ? oracle_round_bf16(v) : v;
}

/* Storage point of a weight gradient: bf16 unless the gradients are kept in fp32 (Dist-MoE, "In-place
 * WGRAD accumulation": gradients in BF16 or FP32, the same dtype for W13 and W2). With an initial
 * gradient (accumulation into existing storage) the new contribution is added to it before that
 * single rounding. */
static inline double RW(const oracle_shape* s, double v) { return s->wgrad_f32 ? v : R(s, v); }

static inline double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* threads the OpenMP loops below use */
int oracle_num_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------------------------- */
/* routing plan: a stable counting sort of the flat slots i = t*K + k by expert id               */

/* counts[e] = #{i : ids_i = e}; offsets[0] = 0, offsets[e+1] = offsets[e] + counts[e];
 * pos[i] = offsets[ids_i] + #{j < i : ids_j = ids_i}; src[pos[i]] = i.
 * Slots whose id is outside [0,E) get pos = -1 and no row; src entries past the last row are -1.
 * Returns the number of such slots. */
int64_t oracle_plan(int64_t T, int64_t K, int64_t E, const int64_t* ids, int64_t* counts,
                    int64_t* offsets, int64_t* pos, int64_t* src) {
  const int64_t N = T * K;
  int64_t bad = 0;
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t i = 0; i < N; ++i) {
    if (ids[i] >= 0 && ids[i] < E)
      counts[ids[i]] += 1;
    else
      bad += 1;
  }
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int64_t* seen = (int64_t*)calloc((size_t)(E > 0 ? E : 1), sizeof(int64_t));
  for (int64_t r = 0; r < N; ++r) src[r] = -1;
  for (int64_t i = 0; i < N; ++i) {
    int64_t e = ids[i];
    if (e < 0 || e >= E) {
      pos[i] = -1;
      continue;
    }
    pos[i] = offsets[e] + seen[e];
    seen[e] += 1;
    src[pos[i]] = i;
  }
  free(seen);
  return bad;
}

/* ------------------------------------------------------------------------------------------- */
/* one routed row through one expert                                                              */

/* h[j] = R(sum_d W13[e][j][d] * xrow[d]) for j in [0, 2F): W13[e] viewed as [2F, D]; j < F is the
 * gate g, j >= F the up projection u. */
static double h_elem(const oracle_shape* s, const void* w13, int64_t e, int64_t j,
                     const double* xrow) {
  const int64_t D = s->D, F = s->F;
  const int64_t base = (e * 2 * F + j) * D;
  double acc = 0.0;
  for (int64_t d = 0; d < D; ++d) acc += ld(w13, base + d, s->in_dtype) * xrow[d];
  return R(s, acc);
}

/* a = R(silu(g) * u) */
static double act_elem(const oracle_shape* s, double g, double u) {
  return R(s, g * sigmoid(g) * u);
}

/* y[d] = R(sum_f W2[e][d][f] * arow[f]) */
static double y_elem(const oracle_shape* s, const void* w2, int64_t e, int64_t d,
                     const double* arow) {
  const int64_t D = s->D, F = s->F;
  const int64_t base = (e * D + d) * F;
  double acc = 0.0;
  for (int64_t f = 0; f < F; ++f) acc += ld(w2, base + f, s->in_dtype) * arow[f];
  return R(s, acc);
}

/* da[f] = sum_d W2[e][d][f] * dyrow[d] (transient, not rounded) */
static double da_elem(const oracle_shape* s, const void* w2, int64_t e, int64_t f,
                      const double* dyrow) {
  const int64_t D = s->D, F = s->F;
  double acc = 0.0;
  for (int64_t d = 0; d < D; ++d) acc += ld(w2, (e * D + d) * F + f, s->in_dtype) * dyrow[d];
  return acc;
}

/* derivative of a = silu(g) * u:  dg = R(da * u * sig * (1 + g*(1 - sig))),  du = R(da * g * sig) */
static void swiglu_grad(const oracle_shape* s, double da, double g, double u, double* dg,
                        double* du) {
  const double sg = sigmoid(g);
  *dg = R(s, da * u * sg * (1.0 + g * (1.0 - sg)));
  *du = R(s, da * g * sg);
}

/* dxg[d] = R(sum_j W13[e][j][d] * dh[j]) over j in [0, 2F), for every d. The loop runs over j
 * outside and d inside so that W13[e] is read along its rows; every dxg[d] still adds its terms in
 * ascending j. */
static void dxg_row(const oracle_shape* s, const void* w13, int64_t e, const double* dh,
                    double* dxg) {
  const int64_t D = s->D, F = s->F;
  for (int64_t d = 0; d < D; ++d) dxg[d] = 0.0;
  for (int64_t j = 0; j < 2 * F; ++j) {
    const double v = dh[j];
    const int64_t base = (e * 2 * F + j) * D;
    for (int64_t d = 0; d < D; ++d) dxg[d] += ld(w13, base + d, s->in_dtype) * v;
  }
  for (int64_t d = 0; d < D; ++d) dxg[d] = R(s, dxg[d]);
}

/* da[f] = sum_d W2[e][d][f] * dyrow[d] for every f (transient, not rounded). Loop order as in
 * dxg_row: d outside, f inside; every da[f] adds its terms in ascending d, the same sum as
 * da_elem. */
static void da_row(const oracle_shape* s, const void* w2, int64_t e, const double* dyrow,
                   double* da) {
  const int64_t D = s->D, F = s->F;
  for (int64_t f = 0; f < F; ++f) da[f] = 0.0;
  for (int64_t d = 0; d < D; ++d) {
    const double v = dyrow[d];
    const int64_t base = (e * D + d) * F;
    for (int64_t f = 0; f < F; ++f) da[f] += ld(w2, base + f, s->in_dtype) * v;
  }
}

/* Forward of one routed row: h[2F], a[F], y[D] from xrow[D] through expert e. */
static void row_forward(const oracle_shape* s, const void* w13, const void* w2, int64_t e,
                        const double* xrow, double* h, double* a, double* y) {
  const int64_t D = s->D, F = s->F;
  for (int64_t j = 0; j < 2 * F; ++j) h[j] = h_elem(s, w13, e, j, xrow);
  for (int64_t f = 0; f < F; ++f) a[f] = act_elem(s, h[f], h[F + f]);
  for (int64_t d = 0; d < D; ++d) y[d] = y_elem(s, w2, e, d, a);
}

/* Input-gradient part of the backward of one routed row: dy[D] = R(score * dout_t), dh[2F],
 * dxg[D]; h is the row's forward [g|u]. */
static void row_backward(const oracle_shape* s, const void* w13, const void* w2, int64_t e,
                         double score, const double* doutrow, const double* h, double* dy,
                         double* dh, double* dxg) {
  const int64_t D = s->D, F = s->F;
  double* da = (double*)malloc(sizeof(double) * F);
  for (int64_t d = 0; d < D; ++d) dy[d] = R(s, score * doutrow[d]);
  da_row(s, w2, e, dy, da);
  for (int64_t f = 0; f < F; ++f) swiglu_grad(s, da[f], h[f], h[F + f], &dh[f], &dh[F + f]);
  dxg_row(s, w13, e, dh, dxg);
  free(da);
}

static void load_row(const oracle_shape* s, const void* p, int64_t row, double* dst) {
  for (int64_t d = 0; d < s->D; ++d) dst[d] = ld(p, row * s->D + d, s->in_dtype);
}

/* ------------------------------------------------------------------------------------------- */
/* full layer (small shapes)                                                                      */

/* Forward over all rows. Needs the plan (pos, src). Outputs: xg[N,D], h13[N,2F], a[N,F], y[N,D],
 * out[T,D]; rows past the last routed row are zero. */
int oracle_forward(const oracle_shape* s, const void* x, const int64_t* ids, const double* scores,
                   const void* w13, const void* w2, const int64_t* pos, const int64_t* src,
                   double* xg, double* h13, double* a, double* y, double* out, double* out_rss) {
  const int64_t T = s->T, D = s->D, F = s->F, K = s->K, N = T * K;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < N; ++r) {
    double* xr = xg + r * D;
    if (src[r] < 0) {
      memset(xr, 0, sizeof(double) * D);
      memset(h13 + r * 2 * F, 0, sizeof(double) * 2 * F);
      memset(a + r * F, 0, sizeof(double) * F);
      memset(y + r * D, 0, sizeof(double) * D);
      continue;
    }
    const int64_t i = src[r], t = i / K, e = ids[i];
    load_row(s, x, t, xr); /* permute: xg[r] = x[t] */
    row_forward(s, w13, w2, e, xr, h13 + r * 2 * F, a + r * F, y + r * D);
  }
  /* combine: out[t,d] = R(sum_k score[t,k] * y[pos[t,k], d]), k ascending */
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t d = 0; d < D; ++d) {
      double acc = 0.0, sq = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const int64_t p = pos[t * K + k];
        if (p >= 0) {
          const double term = scores[t * K + k] * y[p * D + d];
          acc += term;
          sq += term * term;
        }
      }
      out[t * D + d] = R(s, acc);
      if (out_rss) out_rss[t * D + d] = sqrt(sq);
    }
  }
  return 0;
}

/* Backward over all rows, from the forward's saved xg, h13, a, y. Outputs: dy[N,D], dscores[T,K],
 * dh13[N,2F], dxg[N,D], dx[T,D], dw13[E,2F,D], dw2[E,D,F]. */
int oracle_backward(const oracle_shape* s, const void* dout, const int64_t* ids,
                    const double* scores, const void* w13, const void* w2, const int64_t* offsets,
                    const int64_t* pos, const int64_t* src, const double* xg, const double* h13,
                    const double* a, const double* y, double* dy, double* dscores, double* dh13,
                    double* dxg, double* dx, double* dw13, double* dw2, const double* dw13_init,
                    const double* dw2_init, double* dscores_rss, double* dx_rss, double* dw13_rss,
                    double* dw2_rss) {
  const int64_t T = s->T, D = s->D, F = s->F, E = s->E, K = s->K, N = T * K;
  /* dscores[t,k] = sum_d dout[t,d] * y[pos[t,k], d]; 0 for a dropped slot */
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < N; ++i) {
    const int64_t t = i / K, p = pos[i];
    double acc = 0.0, sq = 0.0;
    if (p >= 0)
      for (int64_t d = 0; d < D; ++d) {
        const double term = ld(dout, t * D + d, s->in_dtype) * y[p * D + d];
        acc += term;
        sq += term * term;
      }
    dscores[i] = acc;
    if (dscores_rss) dscores_rss[i] = sqrt(sq);
  }
  /* per-row input gradients */
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < N; ++r) {
    if (src[r] < 0) {
      memset(dy + r * D, 0, sizeof(double) * D);
      memset(dh13 + r * 2 * F, 0, sizeof(double) * 2 * F);
      memset(dxg + r * D, 0, sizeof(double) * D);
      continue;
    }
    const int64_t i = src[r], t = i / K, e = ids[i];
    double* drow = (double*)malloc(sizeof(double) * D);
    load_row(s, dout, t, drow);
    row_backward(s, w13, w2, e, scores[i], drow, h13 + r * 2 * F, dy + r * D, dh13 + r * 2 * F,
                 dxg + r * D);
    free(drow);
  }
  /* dW2[e,d,f] = R(init + sum_{r in segment e} dy[r,d] * a[r,f]), rows ascending (init = 0 unless
   * accumulating); an empty expert's sum is 0 */
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t e = 0; e < E; ++e)
    for (int64_t d = 0; d < D; ++d)
      for (int64_t f = 0; f < F; ++f) {
        double acc = 0.0, sq = 0.0;
        for (int64_t r = offsets[e]; r < offsets[e + 1]; ++r) {
          const double term = dy[r * D + d] * a[r * F + f];
          acc += term;
          sq += term * term;
        }
        const int64_t o = (e * D + d) * F + f;
        dw2[o] = RW(s, (dw2_init ? dw2_init[o] : 0.0) + acc);
        if (dw2_rss) dw2_rss[o] = sqrt(sq);
      }
  /* dW13[e,j,d] = R(init + sum_{r in segment e} dh13[r,j] * xg[r,d]) */
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t e = 0; e < E; ++e)
    for (int64_t j = 0; j < 2 * F; ++j)
      for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0, sq = 0.0;
        for (int64_t r = offsets[e]; r < offsets[e + 1]; ++r) {
          const double term = dh13[r * 2 * F + j] * xg[r * D + d];
          acc += term;
          sq += term * term;
        }
        const int64_t o = (e * 2 * F + j) * D + d;
        dw13[o] = RW(s, (dw13_init ? dw13_init[o] : 0.0) + acc);
        if (dw13_rss) dw13_rss[o] = sqrt(sq);
      }
  /* dx[t,d] = R(sum_k dxg[pos[t,k], d]), k ascending */
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t d = 0; d < D; ++d) {
      double acc = 0.0, sq = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const int64_t p = pos[t * K + k];
        if (p >= 0) {
          acc += dxg[p * D + d];
          sq += dxg[p * D + d] * dxg[p * D + d];
        }
      }
      dx[t * D + d] = R(s, acc);
      if (dx_rss) dx_rss[t * D + d] = sqrt(sq);
    }
  return 0;
}

/* ------------------------------------------------------------------------------------------- */
/* sampled outputs (any shape)                                                                    */

/* For each token in toks[0..n): out[t,:], and when dout is given dscores[t,:] and dx[t,:].
 * These depend only on the token's own K slots. y_rows (optional, [n,K,D]) receives the routed
 * rows' y (zero for a dropped slot). */
int oracle_tokens(const oracle_shape* s, const void* x, const int64_t* ids, const double* scores,
                  const void* w13, const void* w2, const void* dout, int64_t n, const int64_t* toks,
                  double* out_rows, double* dscore_rows, double* dx_rows, double* y_rows,
                  double* out_rss, double* dscore_rss, double* dx_rss) {
  const int64_t D = s->D, F = s->F, K = s->K, E = s->E;
  int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t q = 0; q < n; ++q) {
    const int64_t t = toks[q];
    double* xrow = (double*)malloc(sizeof(double) * D);
    double* h = (double*)malloc(sizeof(double) * 2 * F * K);
    double* a = (double*)malloc(sizeof(double) * F);
    double* y = (double*)calloc((size_t)(K * D), sizeof(double));
    double* drow = (double*)malloc(sizeof(double) * D);
    double* dy = (double*)malloc(sizeof(double) * D);
    double* dh = (double*)malloc(sizeof(double) * 2 * F);
    double* dxg = (double*)calloc((size_t)(K * D), sizeof(double));
    load_row(s, x, t, xrow);
    for (int64_t k = 0; k < K; ++k) {
      const int64_t e = ids[t * K + k];
      if (e < 0 || e >= E) continue;
      row_forward(s, w13, w2, e, xrow, h + k * 2 * F, a, y + k * D);
    }
    for (int64_t d = 0; d < D; ++d) {
      double acc = 0.0, sq = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const int64_t e = ids[t * K + k];
        if (e >= 0 && e < E) {
          const double term = scores[t * K + k] * y[k * D + d];
          acc += term;
          sq += term * term;
        }
      }
      out_rows[q * D + d] = R(s, acc);
      if (out_rss) out_rss[q * D + d] = sqrt(sq);
    }
    if (y_rows) memcpy(y_rows + q * K * D, y, sizeof(double) * K * D);
    if (dout) {
      load_row(s, dout, t, drow);
      for (int64_t k = 0; k < K; ++k) {
        const int64_t e = ids[t * K + k];
        double acc = 0.0, sq = 0.0;
        if (e >= 0 && e < E) {
          for (int64_t d = 0; d < D; ++d) {
            const double term = drow[d] * y[k * D + d];
            acc += term;
            sq += term * term;
          }
          row_backward(s, w13, w2, e, scores[t * K + k], drow, h + k * 2 * F, dy, dh,
                       dxg + k * D);
        }
        dscore_rows[q * K + k] = acc;
        if (dscore_rss) dscore_rss[q * K + k] = sqrt(sq);
      }
      for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0, sq = 0.0;
        for (int64_t k = 0; k < K; ++k) {
          const int64_t e = ids[t * K + k];
          if (e >= 0 && e < E) {
            acc += dxg[k * D + d];
            sq += dxg[k * D + d] * dxg[k * D + d];
          }
        }
        dx_rows[q * D + d] = R(s, acc);
        if (dx_rss) dx_rss[q * D + d] = sqrt(sq);
      }
    }
    free(xrow); free(h); free(a); free(y); free(drow); free(dy); free(dh); free(dxg);
  }
  return status;
}

/* Selected entries of the weight gradients of expert e:
 *   dw13_vals[p] = dW13[e, jd[2p], jd[2p+1]]  (j in [0,2F), d in [0,D)),
 *   dw2_vals[p]  = dW2[e, df[2p], df[2p+1]]   (d in [0,D), f in [0,F)).
 * The sums run over the expert's rows in ascending row order, i.e. the slots i with ids_i = e in
 * ascending i (the stable grouped order). Each needed column f of the intermediate is evaluated per
 * row from its definition. dw13_rss / dw2_rss (optional): the root-sum-square of each entry's
 * terms, as for the whole-layer evaluation. */
int oracle_wgrad_entries(const oracle_shape* s, const void* x, const int64_t* ids,
                         const double* scores, const void* w13, const void* w2, const void* dout,
                         int64_t e, int64_t n13, const int64_t* jd, double* dw13_vals, int64_t n2,
                         const int64_t* df, double* dw2_vals, const double* dw13_init,
                         const double* dw2_init, double* dw13_rss, double* dw2_rss) {
  const int64_t D = s->D, F = s->F, K = s->K, N = s->T * s->K;
  /* distinct intermediate columns f that the requested entries need */
  int64_t* fl = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n13 + n2 + 1));
  int64_t nf = 0;
  for (int64_t p = 0; p < n13 + n2; ++p) {
    const int64_t f = p < n13 ? jd[2 * p] % F : df[2 * (p - n13) + 1];
    int64_t found = 0;
    for (int64_t q = 0; q < nf; ++q) found |= (fl[q] == f);
    if (!found) fl[nf++] = f;
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t q = 0; q < nf; ++q) {
    const int64_t f = fl[q];
    int need13 = 0;
    for (int64_t p = 0; p < n13; ++p) need13 |= (jd[2 * p] % F == f);
    double* acc13 = (double*)calloc((size_t)(n13 + 1), sizeof(double));
    double* acc2 = (double*)calloc((size_t)(n2 + 1), sizeof(double));
    double* sq13 = (double*)calloc((size_t)(n13 + 1), sizeof(double));
    double* sq2 = (double*)calloc((size_t)(n2 + 1), sizeof(double));
    double* xrow = (double*)malloc(sizeof(double) * D);
    double* dyrow = (double*)malloc(sizeof(double) * D);
    for (int64_t i = 0; i < N; ++i) {
      if (ids[i] != e) continue;
      const int64_t t = i / K;
      load_row(s, x, t, xrow);
      const double g = h_elem(s, w13, e, f, xrow);
      const double u = h_elem(s, w13, e, F + f, xrow);
      const double av = act_elem(s, g, u);
      for (int64_t d = 0; d < D; ++d)
        dyrow[d] = R(s, scores[i] * ld(dout, t * D + d, s->in_dtype));
      for (int64_t p = 0; p < n2; ++p)
        if (df[2 * p + 1] == f) {
          const double term = dyrow[df[2 * p]] * av;
          acc2[p] += term;
          sq2[p] += term * term;
        }
      if (need13) {
        const double da = da_elem(s, w2, e, f, dyrow);
        double dg, du;
        swiglu_grad(s, da, g, u, &dg, &du);
        for (int64_t p = 0; p < n13; ++p) {
          const int64_t j = jd[2 * p];
          if (j % F != f) continue;
          const double term = (j < F ? dg : du) * xrow[jd[2 * p + 1]];
          acc13[p] += term;
          sq13[p] += term * term;
        }
      }
    }
    for (int64_t p = 0; p < n2; ++p)
      if (df[2 * p + 1] == f) {
        dw2_vals[p] = RW(s, (dw2_init ? dw2_init[p] : 0.0) + acc2[p]);
        if (dw2_rss) dw2_rss[p] = sqrt(sq2[p]);
      }
    for (int64_t p = 0; p < n13; ++p)
      if (jd[2 * p] % F == f) {
        dw13_vals[p] = RW(s, (dw13_init ? dw13_init[p] : 0.0) + acc13[p]);
        if (dw13_rss) dw13_rss[p] = sqrt(sq13[p]);
      }
    free(acc13); free(acc2); free(sq13); free(sq2); free(xrow); free(dyrow);
  }
  free(fl);
  return 0;
}

/* Element-wise steps over arrays, for the whole-expert evaluation in oracle/__init__.py (which
 * forms the expert's contractions with a library matmul): the same rounding, SwiGLU and SwiGLU
 * derivative as the row functions above.
 *   oracle_store_array: out[i] = R(v[i]), or RW(v[i]) when wgrad is set (weight-gradient storage);
 *   oracle_swiglu_array: a[i] = R(silu(g[i]) * u[i]);
 *   oracle_swiglu_grad_array: dg[i], du[i] from da[i], g[i], u[i] as swiglu_grad. */
void oracle_store_array(const oracle_shape* s, int64_t n, int32_t wgrad, const double* v,
                        double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = wgrad ? RW(s, v[i]) : R(s, v[i]);
}

void oracle_swiglu_array(const oracle_shape* s, int64_t n, const double* g, const double* u,
                         double* a) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) a[i] = act_elem(s, g[i], u[i]);
}

void oracle_swiglu_grad_array(const oracle_shape* s, int64_t n, const double* da, const double* g,
                              const double* u, double* dg, double* du) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) swiglu_grad(s, da[i], g[i], u[i], &dg[i], &du[i]);
}

/* ------------------------------------------------------------------------------------------- */
/* router: score function and (group-limited) top-k                                             */
/*
 * MegaMoE (ROCm Primus technical guide), introduction: the expert path is preceded by a router made
 * of a score function and a group-limited top-k. Primus, "Router force load balancing", `uniform`:
 * the router then works on random logits. The pages name the pieces but give no formulas; the
 * readings taken here:
 *   - scores: softmax over the E logits of a token, or the elementwise logistic sigmoid;
 *   - both are strictly increasing in a token's own logit, so the experts with the largest scores
 *     are the experts with the largest logits: selection compares logits (ties: lower index
 *     first; NaN counts as below every number);
 *   - group-limited: the E experts form n_group equal groups of consecutive ids; a group's score is
 *     its largest logit; the topk_group best groups are kept (ties: lower group first) and the K
 *     experts are chosen among the kept groups' experts only;
 *   - weights: renormalize = 0 gives the chosen experts' scores as computed over all E experts
 *     (softmax) or per expert (sigmoid); renormalize = 1 divides them by their sum over the K
 *     chosen, which for softmax equals the softmax of the K chosen logits;
 *   - ids are written in selection order (descending logit).
 */
#define ORACLE_SCORE_SOFTMAX 0
#define ORACLE_SCORE_SIGMOID 1

/* a ranks before b: larger value, or equal value and lower index; NaN below every number */
static int ranks_before(double va, int64_t ia, double vb, int64_t ib) {
  const int na = isnan(va), nb = isnan(vb);
  if (na != nb) return nb;
  if (!na && va != vb) return va > vb;
  return ia < ib;
}

int oracle_route(int64_t T, int64_t E, int64_t K, const float* logits, int32_t score_fn,
                 int32_t renormalize, int64_t n_group, int64_t topk_group, int64_t* ids,
                 double* weights) {
  if (E < 1 || K < 1 || K > E || n_group < 1 || E % n_group != 0 || topk_group < 1 ||
      topk_group > n_group || K > topk_group * (E / n_group))
    return -1;
  const int64_t gs = E / n_group;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    char* allowed = (char*)calloc((size_t)E, 1);
    char* taken = (char*)calloc((size_t)E, 1);
    char* gtaken = (char*)calloc((size_t)n_group, 1);
    /* groups */
    for (int64_t r = 0; r < topk_group; ++r) {
      int64_t best = -1;
      double bestv = 0.0;
      for (int64_t g = 0; g < n_group; ++g) {
        if (gtaken[g]) continue;
        int64_t gi = g * gs;  /* the group's best expert, compared like experts */
        for (int64_t e = g * gs + 1; e < (g + 1) * gs; ++e)
          if (ranks_before((double)l[e], e, (double)l[gi], gi)) gi = e;
        if (best < 0 || ranks_before((double)l[gi], g, bestv, best)) {
          best = g;
          bestv = (double)l[gi];
        }
      }
      gtaken[best] = 1;
      for (int64_t e = best * gs; e < (best + 1) * gs; ++e) allowed[e] = 1;
    }
    /* experts */
    for (int64_t k = 0; k < K; ++k) {
      int64_t best = -1;
      for (int64_t e = 0; e < E; ++e) {
        if (!allowed[e] || taken[e]) continue;
        if (best < 0 || ranks_before((double)l[e], e, (double)l[best], best)) best = e;
      }
      taken[best] = 1;
      ids[t * K + k] = best;
    }
    /* weights */
    double* w = weights + t * K;
    if (score_fn == ORACLE_SCORE_SOFTMAX) {
      double m = -INFINITY, z = 0.0;
      if (renormalize) {
        for (int64_t k = 0; k < K; ++k) m = fmax(m, (double)l[ids[t * K + k]]);
        for (int64_t k = 0; k < K; ++k) z += exp((double)l[ids[t * K + k]] - m);
      } else {
        for (int64_t e = 0; e < E; ++e) m = fmax(m, (double)l[e]);
        for (int64_t e = 0; e < E; ++e) z += exp((double)l[e] - m);
      }
      for (int64_t k = 0; k < K; ++k) w[k] = exp((double)l[ids[t * K + k]] - m) / z;
    } else {
      double z = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        w[k] = 1.0 / (1.0 + exp(-(double)l[ids[t * K + k]]));
        z += w[k];
      }
      if (renormalize)
        for (int64_t k = 0; k < K; ++k) w[k] /= z;
    }
    free(allowed);
    free(taken);
    free(gtaken);
  }
  return 0;
}
