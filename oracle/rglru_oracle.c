/*
 * rglru_oracle.c -- plain, slow fp64 CPU oracle for the Griffin recurrent-block hot path:
 * a causal depthwise temporal Conv1D of width 4 feeding the RG-LRU gated linear recurrence.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link or call this file.
 * Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py use it, through
 * oracle/__init__.py. It shares no code, header, table or constant with the HIP library.
 *
 * Sources (the pages are web pages about Griffin / RecurrentGemma):
 *  - "Soham De's Griffin thread" (muskviewer.com, sohamde_ tweet 1768346638286762045):
 *      the tweet on adding a Recurrent Gate to LRU (gate may discard the input at time t and keep
 *      the history: RG-LRU); the tweet on S4D/LRU using a diagonal recurrent matrix; the tweet
 *      on keeping the recurrent block simple, which names the temporal Conv1D.
 *  - "Beyond Transformer Architecture: Griffin and Google RecurrentGemma" (alby13 blog),
 *      section "Core Components of Griffin -- 1. RG-LRU": gating independent of the recurrent
 *      state, fixed-size state.
 *  - "Griffin - Mixing Gated Linear Recurrences with Local Attention for Efficient Language
 *      Models" (docshare.wps.com payload): abstract and Introduction name the RG-LRU layer; the
 *      table of contents lists "Model Architecture", whose text the page does not carry.
 *
 * The pages print no equations. The definition followed here is the RG-LRU with block-diagonal
 * gates (H heads of Dh x Dh), c = 8, written out term by term:
 *   conv   xc[t][d] = sum_{j=0..3} w[j][d] * x[t-3+j][d],  x[s<0][d] = 0 (causal, no bias)
 *   gates  pa[t][d] = b_a[d] + sum_i W_a[g][o][i] * xc[t][g*Dh+i]   (d = g*Dh + o)
 *          px[t][d] = b_x[d] + sum_i W_x[g][o][i] * xc[t][g*Dh+i]
 *          r = 1/(1+exp(-pa)),  i = 1/(1+exp(-px))
 *          sp = softplus(-Lambda[d]) = log(1+exp(-Lambda[d]))
 *          log a = -8 * r * sp,  a = exp(log a),  m = sqrt(1 - a*a)
 *   scan   h[t] = a[t]*h[t-1] + m[t]*(i[t]*xc[t]),  h[-1] = h0 (zeros if absent)
 *   output y[t] = h[t];  h_T = h[T-1]
 * Readings where the pages are silent (each is listed with its reason in the design notes):
 *  the gates and the i*x term read the conv output; conv_w[j] multiplies x[t-3+j] (tap 3 is the
 *  current token); W is stored [head][out][in] and applied as out = W * in; 1 - a*a is taken
 *  literally in fp64.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define RGLRU_ORACLE_C 8.0   /* the fixed gate scale c */
#define RGLRU_ORACLE_W 4     /* temporal Conv1D width */

/* Logistic sigmoid, straight from its definition. exp(1e4) = inf gives exactly 0; exp(-1e4) = 0
 * gives exactly 1. */
static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* softplus(z) = log(1 + e^z), evaluated as max(z,0) + log1p(e^{-|z|}) so that neither branch
 * overflows. */
static double softplus(double z) { return (z > 0.0 ? z : 0.0) + log1p(exp(-fabs(z))); }

/* One RG-LRU step for one channel, given the conv output xc and both pre-activations.
 * Returns the new state: the gate, decay and normaliser terms of the definition in this file's
 * header (recurrence gate r, input gate i, decay a = sigma(Lambda)^(c r) taken in log space,
 * normaliser sqrt(1 - a^2)). */
static double rglru_step(double h, double xc, double pa, double px, double lambda) {
  double r = sigmoid(pa);
  double ig = sigmoid(px);
  double log_a = -RGLRU_ORACLE_C * r * softplus(-lambda);
  double a = exp(log_a);
  double m = sqrt(1.0 - a * a);
  return a * h + m * (ig * xc);
}

/* Causal depthwise conv output for channel d at time t of one sequence xs ([T][D], channels
 * contiguous). Taps before the start of the sequence read zero. */
static double conv_at(const double *xs, const double *conv_w, int D, int t, int d) {
  double acc = 0.0;
  for (int j = 0; j < RGLRU_ORACLE_W; ++j) {
    int s = t - (RGLRU_ORACLE_W - 1) + j;
    if (s >= 0) acc += conv_w[(size_t)j * D + d] * xs[(size_t)s * D + d];
  }
  return acc;
}

/* Set the number of OpenMP threads later calls use (n >= 1); a timing control only. */
void rglru_oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int rglru_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Pre-activations of both gates, for testing the gate projection on its own.
 * pa, px: [B][T][D]. */
void rglru_oracle_preacts(int B, int T, int D, int H, const double *x, const double *conv_w,
                          const double *W_a, const double *b_a, const double *W_x,
                          const double *b_x, double *pa, double *px) {
  int Dh = D / H;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < H; ++g) {
      const double *xs = x + (size_t)b * T * D;
      double *xc = (double *)malloc(sizeof(double) * (size_t)Dh);
      for (int t = 0; t < T; ++t) {
        for (int i = 0; i < Dh; ++i) xc[i] = conv_at(xs, conv_w, D, t, g * Dh + i);
        for (int o = 0; o < Dh; ++o) {
          int d = g * Dh + o;
          const double *wa = W_a + ((size_t)g * Dh + o) * Dh;
          const double *wx = W_x + ((size_t)g * Dh + o) * Dh;
          double sa = b_a[d], sx = b_x[d];
          for (int i = 0; i < Dh; ++i) {
            sa += wa[i] * xc[i];
            sx += wx[i] * xc[i];
          }
          pa[((size_t)b * T + t) * D + d] = sa;
          px[((size_t)b * T + t) * D + d] = sx;
        }
      }
      free(xc);
    }
}

/* Full forward over x[B][T][D]. h0 may be NULL (zeros); h_T may be NULL (not written). */
void rglru_oracle_forward(int B, int T, int D, int H, const double *x, const double *conv_w,
                          const double *W_a, const double *b_a, const double *W_x,
                          const double *b_x, const double *Lambda, const double *h0, double *y,
                          double *h_T) {
  int Dh = D / H;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < H; ++g) {
      const double *xs = x + (size_t)b * T * D;
      double *xc = (double *)malloc(sizeof(double) * (size_t)Dh);
      double *h = (double *)malloc(sizeof(double) * (size_t)Dh);
      for (int o = 0; o < Dh; ++o) h[o] = h0 ? h0[(size_t)b * D + g * Dh + o] : 0.0;
      for (int t = 0; t < T; ++t) {
        for (int i = 0; i < Dh; ++i) xc[i] = conv_at(xs, conv_w, D, t, g * Dh + i);
        for (int o = 0; o < Dh; ++o) {
          int d = g * Dh + o;
          const double *wa = W_a + ((size_t)g * Dh + o) * Dh;
          const double *wx = W_x + ((size_t)g * Dh + o) * Dh;
          double sa = b_a[d], sx = b_x[d];
          for (int i = 0; i < Dh; ++i) {
            sa += wa[i] * xc[i];
            sx += wx[i] * xc[i];
          }
          h[o] = rglru_step(h[o], xc[o], sa, sx, Lambda[d]);
          y[((size_t)b * T + t) * D + d] = h[o];
        }
      }
      if (h_T)
        for (int o = 0; o < Dh; ++o) h_T[(size_t)b * D + g * Dh + o] = h[o];
      free(xc);
      free(h);
    }
}

/* One decode step for N independent rows. conv_state[N][3][D] holds the last three inputs,
 * oldest first; it stands in for x[t-3..t-1] in the conv and is then shifted to
 * (cs[1], cs[2], x_t). h[N][D] is updated in place; y_t[N][D] = new h.
 * (Fixed-size state: alby13 blog, "Core Components of Griffin -- 1. RG-LRU".) */
void rglru_oracle_decode_step(int N, int D, int H, const double *x_t, double *conv_state,
                              double *h, double *y_t, const double *conv_w, const double *W_a,
                              const double *b_a, const double *W_x, const double *b_x,
                              const double *Lambda) {
  int Dh = D / H;
  const int K = RGLRU_ORACLE_W - 1;
#pragma omp parallel for schedule(dynamic)
  for (int n = 0; n < N; ++n) {
    double *cs = conv_state + (size_t)n * K * D;
    const double *xt = x_t + (size_t)n * D;
    double *xc = (double *)malloc(sizeof(double) * (size_t)D);
    for (int d = 0; d < D; ++d) {
      double acc = conv_w[(size_t)K * D + d] * xt[d];
      for (int j = 0; j < K; ++j) acc += conv_w[(size_t)j * D + d] * cs[(size_t)j * D + d];
      xc[d] = acc;
    }
    for (int g = 0; g < H; ++g)
      for (int o = 0; o < Dh; ++o) {
        int d = g * Dh + o;
        const double *wa = W_a + ((size_t)g * Dh + o) * Dh;
        const double *wx = W_x + ((size_t)g * Dh + o) * Dh;
        double sa = b_a[d], sx = b_x[d];
        for (int i = 0; i < Dh; ++i) {
          sa += wa[i] * xc[g * Dh + i];
          sx += wx[i] * xc[g * Dh + i];
        }
        double hn = rglru_step(h[(size_t)n * D + d], xc[d], sa, sx, Lambda[d]);
        h[(size_t)n * D + d] = hn;
        y_t[(size_t)n * D + d] = hn;
      }
    for (int d = 0; d < D; ++d) {
      for (int j = 0; j + 1 < K; ++j) cs[(size_t)j * D + d] = cs[(size_t)(j + 1) * D + d];
      cs[(size_t)(K - 1) * D + d] = xt[d];
    }
    free(xc);
  }
}

/* Gradients of the forward above, by reverse-mode differentiation of the same definition, term by
 * term. The loss is L = sum_{b,t,d} dy[b][t][d] * y[b][t][d] + sum_{b,d} dh_T[b][d] * h_T[b][d]
 * (dh_T may be NULL: zero). Outputs (all fully written):
 *   dx [B][T][D], dconv_w [4][D], dW_a, dW_x [H][Dh][Dh] (out, in), db_a, db_x, dLambda [D],
 *   dh0 [B][D] (may be NULL: not written).
 * For one channel, with delta_t = dL/dh_t (dy_t plus a_{t+1} delta_{t+1} carried back in time):
 *   u = m*i*xc:      dm = delta*i*xc,  di = delta*m*xc,  dxc += delta*m*i
 *   h = a*hprev + u: da = delta*hprev,  carried back: delta*a
 *   m = sqrt(1-a^2), a = exp(z):  dz = da*a + dm*(-a*a/m)   (dm/dz = -a^2/m; where m == 0, that is
 *                                 a == 1 exactly, the term takes its limit, 0)
 *   z = -c*r*sp:     dr = -c*sp*dz,  dsp = -c*r*dz,  sp = softplus(-Lambda): dLambda += -sigmoid(-Lambda)*dsp
 *   r = sigmoid(pa): dpa = dr*r*(1-r);  i = sigmoid(px): dpx = di*i*(1-i)
 *   pa = b_a + W_a xc:  db_a += dpa,  dW_a[o][i] += dpa[o]*xc[i],  dxc[i] += W_a[o][i]*dpa[o]
 *   xc[t] = sum_j w_j x[t-3+j]:  dw_j += dxc[t]*x[t-3+j],  dx[t-3+j] += w_j*dxc[t]
 * Heads touch disjoint channels and parameters, so the loop over heads runs in parallel. */
void rglru_oracle_backward(int B, int T, int D, int H, const double *x, const double *conv_w,
                           const double *W_a, const double *b_a, const double *W_x,
                           const double *b_x, const double *Lambda, const double *h0,
                           const double *dy, const double *dh_T, double *dx, double *dconv_w,
                           double *dW_a, double *db_a, double *dW_x, double *db_x,
                           double *dLambda, double *dh0) {
  int Dh = D / H;
  const int K = RGLRU_ORACLE_W - 1;
  memset(dx, 0, sizeof(double) * (size_t)B * T * D);
  memset(dconv_w, 0, sizeof(double) * (size_t)RGLRU_ORACLE_W * D);
  memset(dW_a, 0, sizeof(double) * (size_t)H * Dh * Dh);
  memset(dW_x, 0, sizeof(double) * (size_t)H * Dh * Dh);
  memset(db_a, 0, sizeof(double) * (size_t)D);
  memset(db_x, 0, sizeof(double) * (size_t)D);
  memset(dLambda, 0, sizeof(double) * (size_t)D);
#pragma omp parallel for schedule(dynamic)
  for (int g = 0; g < H; ++g) {
    double *xc = (double *)malloc(sizeof(double) * (size_t)T * Dh);
    double *pa = (double *)malloc(sizeof(double) * (size_t)T * Dh);
    double *px = (double *)malloc(sizeof(double) * (size_t)T * Dh);
    double *hs = (double *)malloc(sizeof(double) * (size_t)T * Dh);
    double *dxc = (double *)malloc(sizeof(double) * (size_t)T * Dh);
    double *dpa = (double *)malloc(sizeof(double) * (size_t)Dh);
    double *dpx = (double *)malloc(sizeof(double) * (size_t)Dh);
    double *delta = (double *)malloc(sizeof(double) * (size_t)Dh);
    for (int b = 0; b < B; ++b) {
      const double *xs = x + (size_t)b * T * D;
      /* forward again, keeping xc, the pre-activations and the states */
      for (int t = 0; t < T; ++t) {
        for (int i = 0; i < Dh; ++i) xc[(size_t)t * Dh + i] = conv_at(xs, conv_w, D, t, g * Dh + i);
        for (int o = 0; o < Dh; ++o) {
          int d = g * Dh + o;
          const double *wa = W_a + ((size_t)g * Dh + o) * Dh;
          const double *wx = W_x + ((size_t)g * Dh + o) * Dh;
          double sa = b_a[d], sx = b_x[d];
          for (int i = 0; i < Dh; ++i) {
            sa += wa[i] * xc[(size_t)t * Dh + i];
            sx += wx[i] * xc[(size_t)t * Dh + i];
          }
          pa[(size_t)t * Dh + o] = sa;
          px[(size_t)t * Dh + o] = sx;
          double hprev = t > 0 ? hs[(size_t)(t - 1) * Dh + o] : (h0 ? h0[(size_t)b * D + d] : 0.0);
          hs[(size_t)t * Dh + o] = rglru_step(hprev, xc[(size_t)t * Dh + o], sa, sx, Lambda[d]);
        }
      }
      /* backward in time */
      for (int o = 0; o < Dh; ++o) delta[o] = dh_T ? dh_T[(size_t)b * D + g * Dh + o] : 0.0;
      for (int t = T - 1; t >= 0; --t) {
        for (int o = 0; o < Dh; ++o) {
          int d = g * Dh + o;
          double dl = delta[o] + dy[((size_t)b * T + t) * D + d];
          double r = sigmoid(pa[(size_t)t * Dh + o]);
          double ig = sigmoid(px[(size_t)t * Dh + o]);
          double sp = softplus(-Lambda[d]);
          double z = -RGLRU_ORACLE_C * r * sp;
          double a = exp(z);
          double m = sqrt(1.0 - a * a);
          double xcv = xc[(size_t)t * Dh + o];
          double hprev = t > 0 ? hs[(size_t)(t - 1) * Dh + o] : (h0 ? h0[(size_t)b * D + d] : 0.0);
          double dm = dl * ig * xcv;
          double di = dl * m * xcv;
          double da = dl * hprev;
          double dz = da * a + (m > 0.0 ? dm * (-a * a / m) : 0.0);
          double dr = -RGLRU_ORACLE_C * sp * dz;
          double dsp = -RGLRU_ORACLE_C * r * dz;
          dLambda[d] += -sigmoid(-Lambda[d]) * dsp;
          dpa[o] = dr * r * (1.0 - r);
          dpx[o] = di * ig * (1.0 - ig);
          dxc[(size_t)t * Dh + o] = dl * m * ig;
          delta[o] = dl * a;
        }
        for (int o = 0; o < Dh; ++o) {
          int d = g * Dh + o;
          db_a[d] += dpa[o];
          db_x[d] += dpx[o];
          double *gwa = dW_a + ((size_t)g * Dh + o) * Dh;
          double *gwx = dW_x + ((size_t)g * Dh + o) * Dh;
          const double *wa = W_a + ((size_t)g * Dh + o) * Dh;
          const double *wx = W_x + ((size_t)g * Dh + o) * Dh;
          for (int i = 0; i < Dh; ++i) {
            gwa[i] += dpa[o] * xc[(size_t)t * Dh + i];
            gwx[i] += dpx[o] * xc[(size_t)t * Dh + i];
            dxc[(size_t)t * Dh + i] += wa[i] * dpa[o] + wx[i] * dpx[o];
          }
        }
      }
      if (dh0)
        for (int o = 0; o < Dh; ++o) dh0[(size_t)b * D + g * Dh + o] = delta[o];
      /* through the conv */
      for (int t = 0; t < T; ++t)
        for (int i = 0; i < Dh; ++i) {
          int d = g * Dh + i;
          for (int j = 0; j <= K; ++j) {
            int s = t - K + j;
            if (s < 0) continue;
            dconv_w[(size_t)j * D + d] += dxc[(size_t)t * Dh + i] * xs[(size_t)s * D + d];
            dx[((size_t)b * T + s) * D + d] += conv_w[(size_t)j * D + d] * dxc[(size_t)t * Dh + i];
          }
        }
    }
    free(xc);
    free(pa);
    free(px);
    free(hs);
    free(dxc);
    free(dpa);
    free(dpx);
    free(delta);
  }
}
