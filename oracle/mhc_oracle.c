/*
 * mhc_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU oracle for the per-token, per-site mHC
 * (manifold-constrained hyper-connections) residual program.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load this
 * library.  It shares no code, header, table or helper with the GPU library:
 * it is written from the method's description alone.
 *
 * Source of the method: docs.rs page "memra_engine 0.125.0
 * src/memra_engine/hyper.rs", module documentation, the "ARITHMETIC CONTRACT"
 * block and the "MEMORY LAYOUT" paragraph; the row order of the mixes comes
 * from the doc comment of HyperTopology::rows on the same page; the post mix
 * from the doc comment of the page's `post` function.
 *
 * Per token t of x[T][S][H] (token-major, element (t,k,i) at (t*S+k)*H+i):
 *   n = S*H, R = (2+S)*S
 *   O1  ss = sum_i x[t,i]^2 ;  rinv = 1/sqrt(ss/n + eps)     (mean over the slab)
 *   O2  m_r = rinv * sum_i fn_w[r,i]*x[t,i]                   (fn_w row-major [R][n])
 *   O3  z_r = scale[g(r)]*m_r + base[r]; g = 0 for the S pre rows, 1 for the
 *       S post rows, 2 for the S*S comb rows
 *   O4  pre_c = 1/(1+exp(-z_c)); post_k = 2/(1+exp(-z_{S+k}));
 *       C[j][k] = exp(z_{2S+j*S+k})   (j = source stream, k = target stream)
 *   O5  iters rounds of: row pass C[j][k] /= (sum_k C[j][k] + eps), then
 *       column pass C[j][k] /= (sum_j C[j][k] + eps); comb = C
 *   O6  y[t,i] = sum_c pre_c * x[t,c,i]
 *   O7  x'[t,k,i] = post[t,k]*f[t,i] + sum_j comb[t,j,k]*x[t,j,i]
 *
 * The page does not spell out the gate nonlinearities or what one Sinkhorn
 * iteration is.  Readings taken (and why) are stated beside each function.
 *
 * Every sum runs in ascending index order, in double precision; nothing is
 * blocked, fused or reordered.  Build without -ffast-math.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* Group of mixes row r: the page orders the rows as the S pre gates, the S
 * post gates, then the S x S combination block, with exactly three scales. */
static int row_group(int r, int S) {
  if (r < S) return 0;
  if (r < 2 * S) return 1;
  return 2;
}

/* O1 + O2 for one token: the RMS-rescaled mixes m[R].  The mean of the squares
 * is taken over the whole streams*hidden slab and eps sits inside the square
 * root (hyper.rs module doc, second line of the arithmetic contract). */
static void token_mixes(const float *xt, const float *fn_w, int S, int H,
                        double eps, double *m) {
  const long n = (long)S * H;
  const int R = (2 + S) * S;
  double ss = 0.0;
  for (long i = 0; i < n; ++i) ss += (double)xt[i] * (double)xt[i];
  const double rinv = 1.0 / sqrt(ss / (double)n + eps);
  for (int r = 0; r < R; ++r) {
    const float *w = fn_w + (long)r * n;
    double acc = 0.0;
    for (long i = 0; i < n; ++i) acc += (double)w[i] * (double)xt[i];
    m[r] = rinv * acc;
  }
}

/* O5: Sinkhorn-Knopp normalisation of the S x S block held in c (row-major,
 * c[j*S+k]).  One iteration is one row pass followed by one column pass, so
 * the last pass of every call is a column pass.  Every denominator is the sum
 * plus eps, the first row pass included (this is the "softmax" step of the
 * page's phase labels, read as exp followed by the first row normalisation). */
static void sinkhorn(double *c, int S, int iters, double eps) {
  for (int it = 0; it < iters; ++it) {
    for (int j = 0; j < S; ++j) {
      double s = 0.0;
      for (int k = 0; k < S; ++k) s += c[j * S + k];
      for (int k = 0; k < S; ++k) c[j * S + k] = c[j * S + k] / (s + eps);
    }
    for (int k = 0; k < S; ++k) {
      double s = 0.0;
      for (int j = 0; j < S; ++j) s += c[j * S + k];
      for (int j = 0; j < S; ++j) c[j * S + k] = c[j * S + k] / (s + eps);
    }
  }
}

/* O3 + O4 + O5 for one token.  Gate forms: pre = sigmoid, post = 2*sigmoid,
 * comb = Sinkhorn of exp(z).  The sigmoid is written 1/(1+exp(-z)) so that
 * z -> -inf gives exactly 0 and z -> +inf exactly 1. */
static void token_gates(const double *m, const float *scale, const float *base,
                        int S, int iters, double eps, double *pre, double *post,
                        double *comb) {
  const int R = (2 + S) * S;
  double z[80];  /* R <= 80 for S <= 8; larger S handled by the caller check */
  for (int r = 0; r < R; ++r)
    z[r] = (double)scale[row_group(r, S)] * m[r] + (double)base[r];
  for (int c = 0; c < S; ++c) pre[c] = 1.0 / (1.0 + exp(-z[c]));
  for (int k = 0; k < S; ++k) post[k] = 2.0 / (1.0 + exp(-z[S + k]));
  for (int j = 0; j < S; ++j)
    for (int k = 0; k < S; ++k) comb[j * S + k] = exp(z[2 * S + j * S + k]);
  sinkhorn(comb, S, iters, eps);
}

/* O6: collapse the streams into the branch input. */
static void token_collapse(const float *xt, const double *pre, int S, int H,
                           double *y) {
  for (int i = 0; i < H; ++i) {
    double acc = 0.0;
    for (int c = 0; c < S; ++c) acc += pre[c] * (double)xt[(long)c * H + i];
    y[i] = acc;
  }
}

/* O7: the post mix.  post and comb are taken AS GIVEN (the fp32 arrays the
 * caller holds), so that the post check is isolated from the pre chain. */
static void token_post(const float *xt, const float *ft, const float *post,
                       const float *comb, int S, int H, double *out) {
  for (int k = 0; k < S; ++k) {
    for (int i = 0; i < H; ++i) {
      double acc = (double)post[k] * (double)ft[i];
      for (int j = 0; j < S; ++j)
        acc += (double)comb[j * S + k] * (double)xt[(long)j * H + i];
      out[(long)k * H + i] = acc;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Thread fan-out over tokens (tokens are independent: every stage above is a
 * function of one token's slab and the site's weights only).               */

typedef struct {
  int kind; /* 0 = pre, 1 = post */
  long t0, t1;
  const float *x, *fn_w, *scale, *base, *f, *post_in, *comb_in;
  int S, H, iters;
  double eps;
  double *mixes, *pre, *post, *comb, *y, *x_out;
} job_t;

static void run_range(const job_t *jb) {
  const int S = jb->S, H = jb->H;
  const long n = (long)S * H;
  const int R = (2 + S) * S;
  for (long t = jb->t0; t < jb->t1; ++t) {
    const float *xt = jb->x + t * n;
    if (jb->kind == 0) {
      double m[80];
      token_mixes(xt, jb->fn_w, S, H, jb->eps, m);
      if (jb->mixes) memcpy(jb->mixes + t * R, m, sizeof(double) * R);
      token_gates(m, jb->scale, jb->base, S, jb->iters, jb->eps,
                  jb->pre + t * S, jb->post + t * S, jb->comb + t * S * S);
      if (jb->y) token_collapse(xt, jb->pre + t * S, S, H, jb->y + t * H);
    } else {
      token_post(xt, jb->f + t * H, jb->post_in + t * S, jb->comb_in + t * S * S,
                 S, H, jb->x_out + t * n);
    }
  }
}

static void *thread_main(void *arg) {
  run_range((const job_t *)arg);
  return NULL;
}

static int fan_out(const job_t *proto, long T, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((long)nthreads > T) nthreads = (int)(T > 0 ? T : 1);
  if (nthreads == 1) {
    job_t jb = *proto;
    jb.t0 = 0;
    jb.t1 = T;
    run_range(&jb);
    return 0;
  }
  pthread_t th[256];
  job_t jobs[256];
  for (int w = 0; w < nthreads; ++w) {
    jobs[w] = *proto;
    jobs[w].t0 = T * w / nthreads;
    jobs[w].t1 = T * (w + 1) / nthreads;
    if (pthread_create(&th[w], NULL, thread_main, &jobs[w]) != 0) {
      /* fall back to running this slice on the calling thread */
      run_range(&jobs[w]);
      th[w] = 0;
    }
  }
  for (int w = 0; w < nthreads; ++w)
    if (th[w]) pthread_join(th[w], NULL);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Exported entry points.  Return 0 on success, 1 on invalid arguments.      */

/* The pre chain for T tokens.  Outputs are double precision; mixes (the
 * rescaled m[T][R], before scale/base) and y may be NULL. */
int mhc_oracle_pre(const float *x, const float *fn_w, const float *scale,
                   const float *base, long T, int S, int H, int iters, double eps,
                   double *mixes, double *pre, double *post, double *comb,
                   double *y, int nthreads) {
  if (T < 0 || S < 1 || S > 8 || H < 1 || iters < 1 || !(eps > 0.0)) return 1;
  if (T == 0) return 0;
  if (!x || !fn_w || !scale || !base || !pre || !post || !comb) return 1;
  job_t jb;
  memset(&jb, 0, sizeof jb);
  jb.kind = 0;
  jb.x = x;
  jb.fn_w = fn_w;
  jb.scale = scale;
  jb.base = base;
  jb.S = S;
  jb.H = H;
  jb.iters = iters;
  jb.eps = eps;
  jb.mixes = mixes;
  jb.pre = pre;
  jb.post = post;
  jb.comb = comb;
  jb.y = y;
  return fan_out(&jb, T, nthreads);
}

/* The post mix for T tokens. */
int mhc_oracle_post(const float *x, const float *f, const float *post,
                    const float *comb, long T, int S, int H, double *x_out,
                    int nthreads) {
  if (T < 0 || S < 1 || S > 8 || H < 1) return 1;
  if (T == 0) return 0;
  if (!x || !f || !post || !comb || !x_out) return 1;
  job_t jb;
  memset(&jb, 0, sizeof jb);
  jb.kind = 1;
  jb.x = x;
  jb.f = f;
  jb.post_in = post;
  jb.comb_in = comb;
  jb.S = S;
  jb.H = H;
  jb.x_out = x_out;
  return fan_out(&jb, T, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Branch-input epilogue (hc_fused_gate.rs page, the v4z timing block: the
 * served rms-norm-and-q8 launch that the fused v4z kernel folds into the pre
 * chain, with a norm weight nw and epsilon 1e-5, writing z, an int8 code
 * vector q[H] and fp32 scales d[H/32]).  The page names the buffers but not the
 * formulas; the readings taken are:
 *   O8  z[i] = y[i] * nw[i] / sqrt(mean_i(y^2) + norm_eps)      (RMS norm of y)
 *   O9  per block of 32 consecutive entries of z (a q8 block):
 *         amax = max |z|;  d = amax / 127;  id = 1/d (0 when d == 0);
 *         q[i] = z[i] * id rounded to nearest, ties away from zero.
 * O8 is computed in double precision.  O9 turns floats into integers, so it is
 * evaluated in the precision the kernel uses: fp32, on the fp32 z given. */

/* O8 for T tokens: y [T][H] (fp32), nw [H] -> z [T][H] (double). */
int mhc_oracle_rmsnorm(const float *y, const float *nw, long T, int H,
                       double norm_eps, double *z) {
  if (T < 0 || H < 1 || !(norm_eps > 0.0)) return 1;
  if (T == 0) return 0;
  if (!y || !nw || !z) return 1;
  for (long t = 0; t < T; ++t) {
    const float *yt = y + t * H;
    double ss = 0.0;
    for (int i = 0; i < H; ++i) ss += (double)yt[i] * (double)yt[i];
    const double r = 1.0 / sqrt(ss / (double)H + norm_eps);
    for (int i = 0; i < H; ++i) z[t * H + i] = (double)yt[i] * r * (double)nw[i];
  }
  return 0;
}

/* O9 for T tokens: z [T][H] (fp32, H a multiple of 32) -> q [T][H], d [T][H/32]. */
int mhc_oracle_q8(const float *z, long T, int H, signed char *q, float *d) {
  if (T < 0 || H < 32 || H % 32 != 0) return 1;
  if (T == 0) return 0;
  if (!z || !q || !d) return 1;
  for (long t = 0; t < T; ++t) {
    for (int b = 0; b < H / 32; ++b) {
      const float *zb = z + t * H + b * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) {
        const float a = fabsf(zb[i]);
        if (a > amax) amax = a;
      }
      const float db = amax / 127.0f;
      const float id = db != 0.0f ? 1.0f / db : 0.0f;
      d[t * (H / 32) + b] = db;
      for (int i = 0; i < 32; ++i) {
        const float v = zb[i] * id;
        q[t * H + b * 32 + i] = (signed char)roundf(v);
      }
    }
  }
  return 0;
}

/* Sinkhorn alone, on S x S logits z (row-major), for the structural checks:
 * comb = Sinkhorn(exp(z)). */
int mhc_oracle_sinkhorn(const double *z, int S, int iters, double eps,
                        double *comb) {
  if (S < 1 || S > 8 || iters < 1 || !(eps > 0.0) || !z || !comb) return 1;
  for (int i = 0; i < S * S; ++i) comb[i] = exp(z[i]);
  sinkhorn(comb, S, iters, eps);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Trunk entry and exit (hyper.rs page: the doc comments of `expand`,
 * `contract_mean` and `collapse`, and the HyperHead loader, which sizes the
 * head's weight [S][S*H], its bias [S] and a single scale).  The page gives the
 * shapes and the kernel names but not the formulas; the readings taken are:
 *   O10 expand: x[t,k,i] = e[t,i] for every stream k (the entry copies the
 *       embedding into each stream; the page calls the mean kernel its
 *       inverse, and the mean of S equal copies is the copy).
 *   O11 mean:   y[t,i] = (sum_k x[t,k,i]) / S, streams in ascending order.
 *   O12 gated head (the head's gates are sigmoids, and it has only the pre
 *       half: no post gates and no combination block): the pre half of a site
 *       with the head's own S rows, one scale and S biases:
 *         rinv = 1/sqrt(sum_i x[t,i]^2 / (S*H) + eps)          (as O1)
 *         m_c  = rinv * sum_i fn_h[c,i] * x[t,i]                c < S
 *         g_c  = 1/(1+exp(-(scale_h * m_c + base_c)))          (the pre gate form)
 *         y[t,i] = sum_c g_c * x[t,c,i]                         (as O6)
 */

/* O10: e [T][H] -> x [T][S][H]; a copy, exact. */
int mhc_oracle_expand(const float *e, long T, int S, int H, float *x) {
  if (T < 0 || S < 1 || H < 1) return 1;
  if (T == 0) return 0;
  if (!e || !x) return 1;
  for (long t = 0; t < T; ++t)
    for (int k = 0; k < S; ++k)
      for (int i = 0; i < H; ++i) x[(t * S + k) * H + i] = e[t * H + i];
  return 0;
}

/* O11: x [T][S][H] -> y [T][H] (double). */
int mhc_oracle_mean(const float *x, long T, int S, int H, double *y) {
  if (T < 0 || S < 1 || H < 1) return 1;
  if (T == 0) return 0;
  if (!x || !y) return 1;
  for (long t = 0; t < T; ++t)
    for (int i = 0; i < H; ++i) {
      double acc = 0.0;
      for (int k = 0; k < S; ++k) acc += (double)x[(t * S + k) * H + i];
      y[t * H + i] = acc / (double)S;
    }
  return 0;
}

/* O12: x [T][S][H], fn_h [S][S*H], scale_h [1], base_h [S] -> gates [T][S],
 * y [T][H] (double). */
int mhc_oracle_head(const float *x, const float *fn_h, const float *scale_h,
                    const float *base_h, long T, int S, int H, double eps,
                    double *gates, double *y) {
  if (T < 0 || S < 1 || S > 8 || H < 1 || !(eps > 0.0)) return 1;
  if (T == 0) return 0;
  if (!x || !fn_h || !scale_h || !base_h || !gates || !y) return 1;
  const long n = (long)S * H;
  for (long t = 0; t < T; ++t) {
    const float *xt = x + t * n;
    double ss = 0.0;
    for (long i = 0; i < n; ++i) ss += (double)xt[i] * (double)xt[i];
    const double rinv = 1.0 / sqrt(ss / (double)n + eps);
    double g[8];
    for (int c = 0; c < S; ++c) {
      const float *w = fn_h + (long)c * n;
      double acc = 0.0;
      for (long i = 0; i < n; ++i) acc += (double)xt[i] * (double)w[i];
      const double z = (double)scale_h[0] * (rinv * acc) + (double)base_h[c];
      g[c] = 1.0 / (1.0 + exp(-z));
      gates[t * S + c] = g[c];
    }
    token_collapse(xt, g, S, H, y + t * H);
  }
  return 0;
}
