/*
 * FP64 CPU oracle for the weight-stationary skinny GEMM and the AttnRes decode
 * epilogue.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it. It shares no code with the HIP library.
 *
 * Everything is written out plainly: bfloat16 values are widened exactly to
 * double, every sum runs in ascending index order in double precision, the
 * transcendental functions are the C library's exp and sqrt, and the single
 * rounding to bfloat16 is round-to-nearest-even from the exact double value.
 *
 * Sources (vLLM API pages of the Kimi-K3 specialized decode, CuTe DSL):
 *  - attn_res.kernel page, ClusterAttnRes (module summary and the methods pre,
 *    weights, post) and the helper rstd: what AttnRes computes per token.
 *  - gemm.ws_gemm page, WsGemm (module summary: y[M, N] = x[M, K] W[N, K]^T)
 *    and positive_zero (-0.0 halves are stored as +0.0).
 *  - oproj.prepared page, module summary and PreparedOproj: the o-projection
 *    output is the AttnRes delta of the same layer.
 *
 * Readings where the pages leave a step open (all listed in the design notes):
 *  - "rounded to BF16" is round-to-nearest-even.
 *  - The fused call rounds the projection output to bfloat16 (with -0.0 made
 *    +0.0) before it is used as the delta.
 *  - eps values arrive as float32; 1/H is applied in double.
 *  - Saved blocks are scored with their values at launch; the written block
 *    slot, the prefix and the aux copy all receive the new prefix.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL -1

/* ---- bfloat16 <-> double ------------------------------------------------ */

/* Exact widening: a bfloat16 pattern is the top half of a float32 pattern. */
static double bf(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round a double to the nearest bfloat16 (ties to even). A normal bfloat16
 * carries 8 significant bits, so |z| in [2^(e-1), 2^e) is quantised to
 * multiples of 2^(e-8); below the normal range the quantum stays 2^-133. */
static uint16_t rn_bf16(double z) {
  if (isnan(z)) return 0x7FC0;
  uint16_t sign = signbit(z) ? 0x8000 : 0;
  double a = fabs(z);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);
  int q = e - 8;
  if (q < -133) q = -133;
  double r = nearbyint(ldexp(a, -q)); /* default mode: nearest, ties even */
  double v = ldexp(r, q);
  if (v >= 0x1p128) return sign | 0x7F80; /* overflow to infinity */
  float f = (float)v;                      /* exact: v has <= 8 bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

/* Reciprocal RMS of an H-wide row from its sum of squares (rstd helper on the
 * attn_res.kernel page), in double: 1 / sqrt(ss / H + eps). */
static double rrms(double ss, int H, double eps) { return 1.0 / sqrt(ss / (double)H + eps); }

/* ---- threading: contiguous index ranges, same code per index --------------- */

typedef void (*range_fn)(void* ctx, int lo, int hi);
typedef struct {
  range_fn fn;
  void* ctx;
  int lo, hi;
} range_job;

static void* run_job(void* p) {
  range_job* j = (range_job*)p;
  j->fn(j->ctx, j->lo, j->hi);
  return NULL;
}

/* Runs fn over [0, n) split into nthreads contiguous ranges. Every index is
 * computed by the same sequential code, so results do not depend on nthreads. */
static void parallel_ranges(range_fn fn, void* ctx, int n, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n) nthreads = n > 0 ? n : 1;
  if (nthreads == 1) {
    fn(ctx, 0, n);
    return;
  }
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  range_job* jobs = (range_job*)malloc(sizeof(range_job) * nthreads);
  for (int i = 0; i < nthreads; ++i) {
    jobs[i].fn = fn;
    jobs[i].ctx = ctx;
    jobs[i].lo = (int)((long long)n * i / nthreads);
    jobs[i].hi = (int)((long long)n * (i + 1) / nthreads);
    if (pthread_create(&th[i], NULL, run_job, &jobs[i]) != 0) {
      run_job(&jobs[i]);
      th[i] = 0;
    }
  }
  for (int i = 0; i < nthreads; ++i)
    if (th[i]) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
}

/* ---- GEMM: y[m, n] = sum_k x[m, k] W[n, k] --------------------------------- */

typedef struct {
  const uint16_t *x, *W;
  int64_t ldx, ldw, ldy;
  uint16_t* y;
  double* yexact;
  int N, K;
} gemm_ctx;

/* Output elements [lo, hi) in row-major (m, n) order: each one is the same
 * ascending-k sum whichever thread computes it, so the split over threads
 * (by element, so that a single token still spreads over every thread) does
 * not change any result. */
static void gemm_elems(void* p, int lo, int hi) {
  gemm_ctx* c = (gemm_ctx*)p;
  for (int i = lo; i < hi; ++i) {
    const int m = i / c->N, n = i % c->N;
    double s = 0.0;
    for (int k = 0; k < c->K; ++k) s += bf(c->x[m * c->ldx + k]) * bf(c->W[n * c->ldw + k]);
    if (c->yexact) c->yexact[(int64_t)m * c->N + n] = s;
    uint16_t r = rn_bf16(s);
    if (r == 0x8000) r = 0; /* -0.0 is stored as +0.0 (positive_zero) */
    c->y[m * c->ldy + n] = r;
  }
}

/* y [M, N] bf16 (row stride ldy) = round(x [M, K] (row stride ldx) . W [N, K]^T
 * (row stride ldw)); yexact [M, N] (optional) receives the unrounded sums. */
int oracle_gemm(const uint16_t* x, int64_t ldx, const uint16_t* W, int64_t ldw, uint16_t* y,
                int64_t ldy, double* yexact, int M, int N, int K, int nthreads) {
  if (!x || !W || !y || M < 0 || N < 0 || K < 0 || ldx < K || ldw < K || ldy < N) return OR_EINVAL;
  if ((int64_t)M * N > 0x7FFFFFFF) return OR_EINVAL;
  gemm_ctx c = {x, W, ldx, ldw, ldy, y, yexact, N, K};
  parallel_ranges(gemm_elems, &c, M * N, nthreads);
  return OR_OK;
}

/* ---- AttnRes, plain definition ------------------------------------------------ */

typedef struct {
  const uint16_t* delta;
  int64_t ld_delta;
  uint16_t* prefix;
  int64_t ld_prefix;
  uint16_t* blocks;
  int64_t bst_t, bst_b;
  const uint16_t *norm, *query, *out_norm;
  uint16_t* out;
  int64_t ld_out;
  uint16_t* aux;
  int64_t ld_aux;
  double eps, out_eps;
  int H, nb, write, has_delta, final;
  double *h_exact, *out_exact, *probs, *logits; /* optional diagnostics */
} attn_ctx;

/* One token of AttnRes (ClusterAttnRes.pre / .post as plain mathematics):
 *   w      = norm * query                               (weights)
 *   l_b    = (v_b . w) * rrms(sum v_b^2, eps)           saved blocks b < nb
 *   new    = bf16(prefix + delta)  or  delta            residual update
 *   l_n    = (new . w) * rrms(sum new^2, eps)
 *   p      = softmax(l_0 .. l_{nb-1}, l_n)              (nb > 0)
 *   h      = sum_b p_b v_b + p_n new, rounded to bf16 at a final boundary;
 *            h = new when nb == 0
 *   out    = bf16(h * rrms(sum h^2, out_eps) * out_norm)
 *   prefix, aux and blocks[write] receive new after every read. */
static void attn_token(const attn_ctx* c, int t) {
  const int H = c->H, nb = c->nb;
  double* w = (double*)malloc(sizeof(double) * H);
  double* v = (double*)malloc(sizeof(double) * (size_t)H * (nb > 0 ? nb : 1));
  double* nw = (double*)malloc(sizeof(double) * H);
  double* h = (double*)malloc(sizeof(double) * H);
  uint16_t* newbits = (uint16_t*)malloc(sizeof(uint16_t) * H);
  double lg[9], p[9];

  for (int i = 0; i < H; ++i) w[i] = bf(c->norm[i]) * bf(c->query[i]);

  /* saved blocks, launch-time values */
  for (int b = 0; b < nb; ++b) {
    const uint16_t* row = c->blocks + t * c->bst_t + b * c->bst_b;
    double ss = 0.0, d = 0.0;
    for (int i = 0; i < H; ++i) {
      double vi = bf(row[i]);
      v[(size_t)b * H + i] = vi;
      ss += vi * vi;
      d += vi * w[i];
    }
    lg[b] = d * rrms(ss, H, c->eps);
  }

  /* residual update */
  for (int i = 0; i < H; ++i) {
    double d = bf(c->delta[t * c->ld_delta + i]);
    uint16_t r;
    if (c->has_delta)
      r = rn_bf16(bf(c->prefix[t * c->ld_prefix + i]) + d);
    else
      r = c->delta[t * c->ld_delta + i]; /* already bf16: rounding is the identity */
    newbits[i] = r;
    nw[i] = bf(r);
  }

  if (nb == 0) {
    for (int i = 0; i < H; ++i) h[i] = nw[i];
    if (c->probs) c->probs[(int64_t)t * 9] = 1.0;
  } else {
    double ss = 0.0, d = 0.0;
    for (int i = 0; i < H; ++i) {
      ss += nw[i] * nw[i];
      d += nw[i] * w[i];
    }
    lg[nb] = d * rrms(ss, H, c->eps);
    double L = lg[0];
    for (int j = 1; j <= nb; ++j)
      if (lg[j] > L) L = lg[j];
    double Z = 0.0;
    for (int j = 0; j <= nb; ++j) {
      p[j] = exp(lg[j] - L);
      Z += p[j];
    }
    for (int j = 0; j <= nb; ++j) p[j] /= Z;
    for (int i = 0; i < H; ++i) {
      double s = 0.0;
      for (int b = 0; b < nb; ++b) s += p[b] * v[(size_t)b * H + i];
      s += p[nb] * nw[i];
      h[i] = s;
    }
    if (c->probs)
      for (int j = 0; j <= nb; ++j) c->probs[(int64_t)t * 9 + j] = p[j];
    if (c->logits)
      for (int j = 0; j <= nb; ++j) c->logits[(int64_t)t * 9 + j] = lg[j];
  }
  if (c->h_exact)
    for (int i = 0; i < H; ++i) c->h_exact[(int64_t)t * H + i] = h[i];
  if (c->final && nb > 0)
    for (int i = 0; i < H; ++i) h[i] = bf(rn_bf16(h[i]));

  double hs = 0.0;
  for (int i = 0; i < H; ++i) hs += h[i] * h[i];
  double s = rrms(hs, H, c->out_eps);
  for (int i = 0; i < H; ++i) {
    double o = h[i] * s * bf(c->out_norm[i]);
    if (c->out_exact) c->out_exact[(int64_t)t * H + i] = o;
    c->out[t * c->ld_out + i] = rn_bf16(o);
  }

  /* state writes, after all reads of this token */
  for (int i = 0; i < H; ++i) c->prefix[t * c->ld_prefix + i] = newbits[i];
  if (c->aux)
    for (int i = 0; i < H; ++i) c->aux[t * c->ld_aux + i] = newbits[i];
  if (c->write >= 0)
    for (int i = 0; i < H; ++i) c->blocks[t * c->bst_t + c->write * c->bst_b + i] = newbits[i];

  free(w);
  free(v);
  free(nw);
  free(h);
  free(newbits);
}

static void attn_tokens(void* p, int lo, int hi) {
  for (int t = lo; t < hi; ++t) attn_token((const attn_ctx*)p, t);
}

static int attn_check(const void* delta, const void* prefix, const void* blocks, const void* norm,
                      const void* query, const void* out_norm, const void* out, int cap, int T,
                      int H, int nb, int write) {
  if (!delta || !prefix || !norm || !query || !out_norm || !out) return OR_EINVAL;
  if (T < 0 || H < 1 || nb < 0 || nb > 8 || nb > cap || write < -1 || write >= cap) return OR_EINVAL;
  if ((nb > 0 || write >= 0) && !blocks) return OR_EINVAL;
  return OR_OK;
}

/* AttnRes over T tokens. Layouts (element strides): delta, prefix, out, aux
 * [T, H] with row strides ld_*; blocks [T, cap, H] with strides (bst_t, bst_b,
 * 1). aux may be NULL; write = -1 writes no block. The diagnostics
 * (h_exact [T, H] before the final rounding, out_exact [T, H] before rounding,
 * probs [T, 9], logits [T, 9]) may be NULL. */
int oracle_attnres(const uint16_t* delta, int64_t ld_delta, uint16_t* prefix, int64_t ld_prefix,
                   uint16_t* blocks, int64_t bst_t, int64_t bst_b, int cap, const uint16_t* norm,
                   const uint16_t* query, const uint16_t* out_norm, uint16_t* out, int64_t ld_out,
                   uint16_t* aux, int64_t ld_aux, float eps, float out_eps, int T, int H, int nb,
                   int write, int has_delta, int final_boundary, double* h_exact,
                   double* out_exact, double* probs, double* logits, int nthreads) {
  int rc = attn_check(delta, prefix, blocks, norm, query, out_norm, out, cap, T, H, nb, write);
  if (rc) return rc;
  attn_ctx c = {delta, ld_delta, prefix, ld_prefix, blocks, bst_t, bst_b, norm, query, out_norm,
                out, ld_out, aux, ld_aux, (double)eps, (double)out_eps, H, nb, write,
                has_delta != 0, final_boundary != 0, h_exact, out_exact, probs, logits};
  parallel_ranges(attn_tokens, &c, T, nthreads);
  return OR_OK;
}

/* ---- AttnRes, the pages' streaming formulation --------------------------------
 * A second, independent route to the same numbers, following the order of
 * ClusterAttnRes: pre() keeps the running maximum m of the block logits,
 * e_b = exp(l_b - m), S = sum e_b and the unnormalised mixture M = sum e_b v_b;
 * post() merges the new prefix online (top = max(m, l_n), alpha = exp(m - top),
 * eps_n = exp(l_n - top), D = alpha S + eps_n) and then either rounds
 * h = (alpha M + eps_n new) / D to bf16 and normalises it (final boundary) or
 * normalises the unrounded mixture analytically from the three sums
 * sum M^2, sum M.new and sum new^2. */
static void attn_token_streaming(const attn_ctx* c, int t) {
  const int H = c->H, nb = c->nb;
  double* w = (double*)malloc(sizeof(double) * H);
  double* mix = (double*)calloc((size_t)H, sizeof(double));
  double* nw = (double*)malloc(sizeof(double) * H);
  uint16_t* newbits = (uint16_t*)malloc(sizeof(uint16_t) * H);
  double lg[9];
  for (int i = 0; i < H; ++i) w[i] = bf(c->norm[i]) * bf(c->query[i]);

  double m = 0.0, S = 0.0;
  for (int b = 0; b < nb; ++b) {
    const uint16_t* row = c->blocks + t * c->bst_t + b * c->bst_b;
    double ss = 0.0, d = 0.0;
    for (int i = 0; i < H; ++i) {
      ss += bf(row[i]) * bf(row[i]);
      d += bf(row[i]) * w[i];
    }
    lg[b] = d * rrms(ss, H, c->eps);
  }
  if (nb > 0) {
    m = lg[0];
    for (int b = 1; b < nb; ++b) m = fmax(m, lg[b]);
    for (int b = 0; b < nb; ++b) {
      const uint16_t* row = c->blocks + t * c->bst_t + b * c->bst_b;
      double e = exp(lg[b] - m);
      S += e;
      for (int i = 0; i < H; ++i) mix[i] += e * bf(row[i]);
    }
  }
  for (int i = 0; i < H; ++i) {
    double d = bf(c->delta[t * c->ld_delta + i]);
    newbits[i] = c->has_delta ? rn_bf16(bf(c->prefix[t * c->ld_prefix + i]) + d)
                              : c->delta[t * c->ld_delta + i];
    nw[i] = bf(newbits[i]);
  }
  double ssn = 0.0, dn = 0.0, mn = 0.0, mm = 0.0;
  for (int i = 0; i < H; ++i) {
    ssn += nw[i] * nw[i];
    dn += nw[i] * w[i];
    mn += mix[i] * nw[i];
    mm += mix[i] * mix[i];
  }
  const double oe = c->out_eps;
  if (nb == 0) {
    double s = rrms(ssn, H, oe);
    for (int i = 0; i < H; ++i) {
      double o = nw[i] * s * bf(c->out_norm[i]);
      if (c->out_exact) c->out_exact[(int64_t)t * H + i] = o;
      c->out[t * c->ld_out + i] = rn_bf16(o);
    }
  } else {
    double ln = dn * rrms(ssn, H, c->eps);
    double top = fmax(m, ln);
    double alpha = exp(m - top), en = exp(ln - top);
    double D = alpha * S + en;
    if (c->final) {
      double* hr = (double*)malloc(sizeof(double) * H);
      double hs = 0.0;
      for (int i = 0; i < H; ++i) {
        hr[i] = bf(rn_bf16((alpha * mix[i] + en * nw[i]) / D));
        hs += hr[i] * hr[i];
      }
      double s = rrms(hs, H, oe);
      for (int i = 0; i < H; ++i) {
        double o = hr[i] * s * bf(c->out_norm[i]);
        if (c->out_exact) c->out_exact[(int64_t)t * H + i] = o;
        c->out[t * c->ld_out + i] = rn_bf16(o);
      }
      free(hr);
    } else {
      double Q = alpha * alpha * mm + 2.0 * alpha * en * mn + en * en * ssn;
      double s = 1.0 / sqrt(Q / (double)H + oe * D * D);
      for (int i = 0; i < H; ++i) {
        double o = (alpha * s * mix[i] + en * s * nw[i]) * bf(c->out_norm[i]);
        if (c->out_exact) c->out_exact[(int64_t)t * H + i] = o;
        c->out[t * c->ld_out + i] = rn_bf16(o);
      }
    }
  }
  for (int i = 0; i < H; ++i) c->prefix[t * c->ld_prefix + i] = newbits[i];
  if (c->aux)
    for (int i = 0; i < H; ++i) c->aux[t * c->ld_aux + i] = newbits[i];
  if (c->write >= 0)
    for (int i = 0; i < H; ++i) c->blocks[t * c->bst_t + c->write * c->bst_b + i] = newbits[i];
  free(w);
  free(mix);
  free(nw);
  free(newbits);
}

static void attn_tokens_streaming(void* p, int lo, int hi) {
  for (int t = lo; t < hi; ++t) attn_token_streaming((const attn_ctx*)p, t);
}

/* Same arguments and outputs as oracle_attnres (h_exact, probs and logits are
 * not produced by this form). */
int oracle_attnres_streaming(const uint16_t* delta, int64_t ld_delta, uint16_t* prefix,
                             int64_t ld_prefix, uint16_t* blocks, int64_t bst_t, int64_t bst_b,
                             int cap, const uint16_t* norm, const uint16_t* query,
                             const uint16_t* out_norm, uint16_t* out, int64_t ld_out,
                             uint16_t* aux, int64_t ld_aux, float eps, float out_eps, int T, int H,
                             int nb, int write, int has_delta, int final_boundary,
                             double* out_exact, int nthreads) {
  int rc = attn_check(delta, prefix, blocks, norm, query, out_norm, out, cap, T, H, nb, write);
  if (rc) return rc;
  attn_ctx c = {delta, ld_delta, prefix, ld_prefix, blocks, bst_t, bst_b, norm, query, out_norm,
                out, ld_out, aux, ld_aux, (double)eps, (double)out_eps, H, nb, write,
                has_delta != 0, final_boundary != 0, NULL, out_exact, NULL, NULL};
  parallel_ranges(attn_tokens_streaming, &c, T, nthreads);
  return OR_OK;
}

/* ---- fused o-projection + AttnRes ----------------------------------------------
 * delta := bf16(x . W^T) with -0.0 stored as +0.0 (the o-projection output of the
 * oproj.prepared page is the AttnRes delta), then oracle_attnres. y [M, H]
 * receives that delta (caller-owned scratch, row stride H). */
int oracle_attnres_oproj(const uint16_t* x, int64_t ldx, const uint16_t* W, int64_t ldw, int K,
                         uint16_t* prefix, int64_t ld_prefix, uint16_t* blocks, int64_t bst_t,
                         int64_t bst_b, int cap, const uint16_t* norm, const uint16_t* query,
                         const uint16_t* out_norm, uint16_t* out, int64_t ld_out, uint16_t* aux,
                         int64_t ld_aux, float eps, float out_eps, int M, int H, int nb, int write,
                         int has_delta, int final_boundary, uint16_t* y, double* out_exact,
                         int nthreads) {
  if (!y) return OR_EINVAL;
  int rc = oracle_gemm(x, ldx, W, ldw, y, H, NULL, M, H, K, nthreads);
  if (rc) return rc;
  return oracle_attnres(y, H, prefix, ld_prefix, blocks, bst_t, bst_b, cap, norm, query,
                        out_norm, out, ld_out, aux, ld_aux, eps, out_eps, M, H, nb, write,
                        has_delta, final_boundary, NULL, out_exact, NULL, NULL, nthreads);
}

/* ---- saved-block statistics and the post step on given statistics ------------
 * The state ClusterAttnRes carries from pre() to post() (attn_res.kernel page,
 * method state: the mixture row and the two scalars maximum and exp_sum), which
 * the fused o-projection also stores for the next layer's AttnRes over the same
 * saved blocks (oproj.prepared page, PreparedOproj.bind_ahead and the `ahead`
 * rows of compile_oproj). Plain definitions, per token t:
 *   l_b      = (v_b . w) * rrms(sum v_b^2, eps)        b < nb, w = norm * query
 *   m        = max_b l_b                                (0 when nb == 0)
 *   S        = sum_b exp(l_b - m)                       (0 when nb == 0)
 *   mix_i    = sum_b exp(l_b - m) v_b,i                 (0 when nb == 0)
 * mixture [T, H] (row stride ld_mix) and scal [T, 2] = (m, S) are doubles. */
typedef struct {
  const uint16_t* blocks;
  int64_t bst_t, bst_b;
  const uint16_t *norm, *query;
  double eps;
  int H, nb;
  double* mixture;
  int64_t ld_mix;
  double* scal;
} pre_ctx;

static void pre_tokens(void* p, int lo, int hi) {
  const pre_ctx* c = (const pre_ctx*)p;
  const int H = c->H, nb = c->nb;
  double lg[8];
  for (int t = lo; t < hi; ++t) {
    double* mix = c->mixture + (int64_t)t * c->ld_mix;
    for (int i = 0; i < H; ++i) mix[i] = 0.0;
    for (int b = 0; b < nb; ++b) {
      const uint16_t* row = c->blocks + t * c->bst_t + b * c->bst_b;
      double ss = 0.0, d = 0.0;
      for (int i = 0; i < H; ++i) {
        double vi = bf(row[i]);
        ss += vi * vi;
        d += vi * (bf(c->norm[i]) * bf(c->query[i]));
      }
      lg[b] = d * rrms(ss, H, c->eps);
    }
    double m = 0.0, S = 0.0;
    if (nb > 0) {
      m = lg[0];
      for (int b = 1; b < nb; ++b)
        if (lg[b] > m) m = lg[b];
      for (int b = 0; b < nb; ++b) {
        const uint16_t* row = c->blocks + t * c->bst_t + b * c->bst_b;
        double e = exp(lg[b] - m);
        S += e;
        for (int i = 0; i < H; ++i) mix[i] += e * bf(row[i]);
      }
    }
    c->scal[2 * t] = m;
    c->scal[2 * t + 1] = S;
  }
}

int oracle_attnres_pre(const uint16_t* blocks, int64_t bst_t, int64_t bst_b, int cap,
                       const uint16_t* norm, const uint16_t* query, float eps, int T, int H,
                       int nb, double* mixture, int64_t ld_mix, double* scal, int nthreads) {
  if (!norm || !query || !mixture || !scal || T < 0 || H < 1 || nb < 0 || nb > 8 || nb > cap ||
      ld_mix < H || (nb > 0 && !blocks))
    return OR_EINVAL;
  pre_ctx c = {blocks, bst_t, bst_b, norm, query, (double)eps, H, nb, mixture, ld_mix, scal};
  parallel_ranges(pre_tokens, &c, T, nthreads);
  return OR_OK;
}

/* post() on given statistics (m, S, mix) of nb saved blocks, per token t:
 *   new  = bf16(prefix + delta)  or  delta
 *   l_n  = (new . w) * rrms(sum new^2, eps)
 *   nb == 0: h = new (the statistics are not read)
 *   else: top = max(m, l_n), alpha = exp(m - top), e_n = exp(l_n - top),
 *         D = alpha S + e_n, h = (alpha mix + e_n new) / D,
 *         rounded to bf16 at a final boundary
 *   out  = bf16(h * rrms(sum h^2, out_eps) * out_norm)
 *   prefix, aux and blocks[write] receive new.
 * With (m, S, mix) from oracle_attnres_pre this is exactly the softmax over
 * the nb blocks and the new prefix: alpha e_b / D = p_b and e_n / D = p_n. */
typedef struct {
  attn_ctx a;
  const double* mixture;
  int64_t ld_mix;
  const double* scal;
} post_ctx;

static void post_tokens(void* p, int lo, int hi) {
  const post_ctx* pc = (const post_ctx*)p;
  const attn_ctx* c = &pc->a;
  const int H = c->H, nb = c->nb;
  double* nw = (double*)malloc(sizeof(double) * H);
  double* h = (double*)malloc(sizeof(double) * H);
  uint16_t* newbits = (uint16_t*)malloc(sizeof(uint16_t) * H);
  for (int t = lo; t < hi; ++t) {
    for (int i = 0; i < H; ++i) {
      double d = bf(c->delta[t * c->ld_delta + i]);
      newbits[i] = c->has_delta ? rn_bf16(bf(c->prefix[t * c->ld_prefix + i]) + d)
                                : c->delta[t * c->ld_delta + i];
      nw[i] = bf(newbits[i]);
    }
    if (nb == 0) {
      for (int i = 0; i < H; ++i) h[i] = nw[i];
    } else {
      double ss = 0.0, d = 0.0;
      for (int i = 0; i < H; ++i) {
        ss += nw[i] * nw[i];
        d += nw[i] * (bf(c->norm[i]) * bf(c->query[i]));
      }
      const double ln = d * rrms(ss, H, c->eps);
      const double m = pc->scal[2 * t], S = pc->scal[2 * t + 1];
      const double top = m > ln ? m : ln;
      const double alpha = exp(m - top), en = exp(ln - top);
      const double D = alpha * S + en;
      const double* mix = pc->mixture + (int64_t)t * pc->ld_mix;
      for (int i = 0; i < H; ++i) h[i] = (alpha * mix[i] + en * nw[i]) / D;
      if (c->final)
        for (int i = 0; i < H; ++i) h[i] = bf(rn_bf16(h[i]));
    }
    double hs = 0.0;
    for (int i = 0; i < H; ++i) hs += h[i] * h[i];
    const double s = rrms(hs, H, c->out_eps);
    for (int i = 0; i < H; ++i) {
      double o = h[i] * s * bf(c->out_norm[i]);
      if (c->out_exact) c->out_exact[(int64_t)t * H + i] = o;
      c->out[t * c->ld_out + i] = rn_bf16(o);
    }
    for (int i = 0; i < H; ++i) c->prefix[t * c->ld_prefix + i] = newbits[i];
    if (c->aux)
      for (int i = 0; i < H; ++i) c->aux[t * c->ld_aux + i] = newbits[i];
    if (c->write >= 0)
      for (int i = 0; i < H; ++i) c->blocks[t * c->bst_t + c->write * c->bst_b + i] = newbits[i];
  }
  free(nw);
  free(h);
  free(newbits);
}

/* Arguments as oracle_attnres, with the saved-block statistics given: mixture
 * [T, H] (row stride ld_mix) and scal [T, 2] = (m, S), doubles (statistics a
 * GPU stored as float32 are widened exactly by the caller). blocks is only
 * written (slot write) and may be NULL when write == -1. */
int oracle_attnres_post(const uint16_t* delta, int64_t ld_delta, uint16_t* prefix,
                        int64_t ld_prefix, uint16_t* blocks, int64_t bst_t, int64_t bst_b,
                        int cap, const uint16_t* norm, const uint16_t* query,
                        const uint16_t* out_norm, uint16_t* out, int64_t ld_out, uint16_t* aux,
                        int64_t ld_aux, const double* mixture, int64_t ld_mix, const double* scal,
                        float eps, float out_eps, int T, int H, int nb, int write, int has_delta,
                        int final_boundary, double* out_exact, int nthreads) {
  if (!delta || !prefix || !norm || !query || !out_norm || !out || T < 0 || H < 1 || nb < 0 ||
      nb > 8 || nb > cap || write < -1 || write >= cap || (write >= 0 && !blocks))
    return OR_EINVAL;
  if (nb > 0 && (!mixture || !scal || ld_mix < H)) return OR_EINVAL;
  post_ctx c = {{delta, ld_delta, prefix, ld_prefix, blocks, bst_t, bst_b, norm, query, out_norm,
                 out, ld_out, aux, ld_aux, (double)eps, (double)out_eps, H, nb, write,
                 has_delta != 0, final_boundary != 0, NULL, out_exact, NULL, NULL},
                mixture, ld_mix, scal};
  parallel_ranges(post_tokens, &c, T, nthreads);
  return OR_OK;
}

/* ---- the MoE-front epilogue of WsGemm ------------------------------------------
 * gemm.ws_gemm page, WsGemm.epilogue (and the module summary): the output rows
 * of y = x W^T are split into a router shard, padding and a latent shard.
 * Per token m and output row c (the GEMM's column):
 *   c <  valid          : FP32 word of y[m, c] (-0.0 stored as +0.0,
 *                         positive_zero32) at bf16 column
 *                         router_base + 2 (slot + c) of out row m;
 *   valid <= c < split  : dropped;
 *   c >= split          : bf16 of y[m, c] (-0.0 -> +0.0, positive_zero) at bf16
 *                         column base + c - split of out row m.
 * The FP32 word is y rounded once from its exact sum (the plain definition;
 * the GPU's FP32 accumulation matches it exactly on integer data). out is
 * [M, ld_out] bf16 patterns; nothing else is written. */
static uint32_t rn_f32_bits(double z) {
  float f = (float)z; /* IEEE conversion: round to nearest, ties to even */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u == 0x80000000u ? 0u : u;
}

int oracle_moe_front(const uint16_t* x, int64_t ldx, const uint16_t* W, int64_t ldw, int M, int N,
                     int K, uint16_t* out, int64_t ld_out, int router_base, int slot, int base,
                     int valid, int split) {
  if (!x || !W || !out || M < 0 || N < 0 || K < 0 || valid < 0 || valid > split || split > N)
    return OR_EINVAL;
  for (int m = 0; m < M; ++m) {
    for (int c = 0; c < N; ++c) {
      if (c >= valid && c < split) continue;
      double s = 0.0;
      for (int k = 0; k < K; ++k) s += bf(x[m * ldx + k]) * bf(W[c * ldw + k]);
      if (c < valid) {
        const uint32_t u = rn_f32_bits(s);
        const int64_t col = (int64_t)router_base + 2 * ((int64_t)slot + c);
        out[m * ld_out + col] = (uint16_t)(u & 0xFFFF); /* little-endian word */
        out[m * ld_out + col + 1] = (uint16_t)(u >> 16);
      } else {
        uint16_t r = rn_bf16(s);
        if (r == 0x8000) r = 0;
        out[m * ld_out + base + (c - split)] = r;
      }
    }
  }
  return OR_OK;
}

/* Exposed for the pins of the rounding rule. */
uint16_t oracle_round_bf16(double z) { return rn_bf16(z); }

/* The same rounding over n values (the parity tests build the bounds of a
 * bfloat16 sum from it). */
void oracle_round_bf16_n(const double* z, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = rn_bf16(z[i]);
}
