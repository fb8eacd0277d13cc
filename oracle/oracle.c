/*
 * CPU oracle for one data-parallel worker's minibatch SGD step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * HIP path is checked against.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header or
 * constant with the HIP library: it has its own layer codes, its own NCHW
 * activation layout and its own loops.
 *
 * Every function is the definition of the operation written out directly:
 * convolution is the 7-deep loop over (n, co, oy, ox, ci, ky, kx) (no im2col,
 * no GEMM), fully connected layers are a naive triple loop, the update rules
 * are scalar loops with one rounding per statement.
 *
 * Precision.  The pages fix single precision (SGEMM, float32 training), so
 * the default build stores every tensor in float and rounds to float after
 * each layer, exactly where the GPU path rounds.  Every sum is accumulated in
 * double, in a fixed sequential order, so the oracle is not itself the error
 * source.  Built with -DOR_REAL=double it stores everything in double; that
 * build is used for the finite-difference checks.
 *
 * Sources (each function below cites the passage it follows):
 *  [SPRINT]  IPSJ SIG Technical Report Vol.2016-HPC-155 No.8 (the SPRINT
 *            asynchronous-SGD trainer and its performance model).
 *  [PIPE]    "Pipelined training with stale weights of deep convolutional
 *            neural networks" (Zhang & Abdelrahman), section 2, backprop.
 *  [CHAINER] Qiita multi-GPU Chainer tutorial (the 5000-unit MLP; the
 *            data-parallel step that sums half-batch gradients).
 *  [DISTBELIEF] blog review of "Large Scale Distributed Deep Networks"
 *            (parameter server, commutative additive gradients, Adagrad).
 *
 * Parity status: every function here is pinned by a CPU test (closed forms,
 * finite differences, library routines, invariants); none is unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef OR_REAL
#define OR_REAL float
#endif
typedef OR_REAL real;

#define IDX4(a, b, c, d, B, C, D) ((((int64_t)(a) * (B) + (b)) * (C) + (c)) * (D) + (d))

/* ------------------------------------------------------------------------ */
/* Convolution, stride 1, zero padding P, square c x c filter.              */
/* [SPRINT] sec. 3.2: a conv layer maps m_{l-1} channels of width x_{l-1} to  */
/* m_l channels with c x c filters; eq. (2) gives the width x_{l-1} - c + 1  */
/* for the unpadded case, generalised here to H + 2P - c + 1.               */
/* Layout: x[n][ci][y][x], w[co][ci][ky][kx], y[n][co][oy][ox] (NCHW).      */
/* ------------------------------------------------------------------------ */
void or_conv_fwd(int N, int Ci, int H, int W, int Co, int c, int P,
                 const real* x, const real* w, const real* b, real* y) {
  const int Ho = H + 2 * P - c + 1, Wo = W + 2 * P - c + 1;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int n = 0; n < N; ++n)
    for (int co = 0; co < Co; ++co)
      for (int oy = 0; oy < Ho; ++oy)
        for (int ox = 0; ox < Wo; ++ox) {
          double acc = (double)b[co];
          for (int ci = 0; ci < Ci; ++ci)
            for (int ky = 0; ky < c; ++ky) {
              const int iy = oy + ky - P;
              if (iy < 0 || iy >= H) continue;
              for (int kx = 0; kx < c; ++kx) {
                const int ix = ox + kx - P;
                if (ix < 0 || ix >= W) continue;
                acc += (double)x[IDX4(n, ci, iy, ix, Ci, H, W)] *
                       (double)w[IDX4(co, ci, ky, kx, Ci, c, c)];
              }
            }
          y[IDX4(n, co, oy, ox, Co, Ho, Wo)] = (real)acc;
        }
}

/* Backward of the convolution: given dy = dE/dy (NCHW),
 *   db[co]            = sum_{n,oy,ox} dy[n][co][oy][ox]
 *   dw[co][ci][ky][kx] = sum_{n,oy,ox} dy[n][co][oy][ox] * x[n][ci][oy+ky-P][ox+kx-P]
 *   dx[n][ci][iy][ix]  = sum_{co,ky,kx} dy[n][co][iy-ky+P][ix-kx+P] * w[co][ci][ky][kx]
 * (taps outside the image contribute nothing).  These are the dedb, dedw and
 * dedx_conv products of the [SPRINT] sec. 3.3 SGEMM table, written as sums.
 * dx may be NULL (no gradient for the image, as in that table). */
void or_conv_bwd(int N, int Ci, int H, int W, int Co, int c, int P,
                 const real* x, const real* w, const real* dy,
                 real* dw, real* db, real* dx) {
  const int Ho = H + 2 * P - c + 1, Wo = W + 2 * P - c + 1;
#pragma omp parallel for schedule(dynamic)
  for (int co = 0; co < Co; ++co) {
    double acc = 0.0;
    for (int n = 0; n < N; ++n)
      for (int oy = 0; oy < Ho; ++oy)
        for (int ox = 0; ox < Wo; ++ox) acc += (double)dy[IDX4(n, co, oy, ox, Co, Ho, Wo)];
    db[co] = (real)acc;
  }
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int co = 0; co < Co; ++co)
    for (int ci = 0; ci < Ci; ++ci)
      for (int ky = 0; ky < c; ++ky)
        for (int kx = 0; kx < c; ++kx) {
          double acc = 0.0;
          for (int n = 0; n < N; ++n)
            for (int oy = 0; oy < Ho; ++oy) {
              const int iy = oy + ky - P;
              if (iy < 0 || iy >= H) continue;
              for (int ox = 0; ox < Wo; ++ox) {
                const int ix = ox + kx - P;
                if (ix < 0 || ix >= W) continue;
                acc += (double)dy[IDX4(n, co, oy, ox, Co, Ho, Wo)] *
                       (double)x[IDX4(n, ci, iy, ix, Ci, H, W)];
              }
            }
          dw[IDX4(co, ci, ky, kx, Ci, c, c)] = (real)acc;
        }
  if (!dx) return;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int n = 0; n < N; ++n)
    for (int ci = 0; ci < Ci; ++ci)
      for (int iy = 0; iy < H; ++iy)
        for (int ix = 0; ix < W; ++ix) {
          double acc = 0.0;
          for (int co = 0; co < Co; ++co)
            for (int ky = 0; ky < c; ++ky) {
              const int oy = iy - ky + P;
              if (oy < 0 || oy >= Ho) continue;
              for (int kx = 0; kx < c; ++kx) {
                const int ox = ix - kx + P;
                if (ox < 0 || ox >= Wo) continue;
                acc += (double)dy[IDX4(n, co, oy, ox, Co, Ho, Wo)] *
                       (double)w[IDX4(co, ci, ky, kx, Ci, c, c)];
              }
            }
          dx[IDX4(n, ci, iy, ix, Ci, H, W)] = (real)acc;
        }
}

/* Single outputs of the same three sums, for spot checks on tensors too
 * large for the full loops.  Same definitions as above. */
double or_conv_fwd_point(int N, int Ci, int H, int W, int Co, int c, int P,
                         const real* x, const real* w, const real* b,
                         int n, int co, int oy, int ox) {
  (void)N; (void)Co;
  double acc = (double)b[co];
  for (int ci = 0; ci < Ci; ++ci)
    for (int ky = 0; ky < c; ++ky) {
      const int iy = oy + ky - P;
      if (iy < 0 || iy >= H) continue;
      for (int kx = 0; kx < c; ++kx) {
        const int ix = ox + kx - P;
        if (ix < 0 || ix >= W) continue;
        acc += (double)x[IDX4(n, ci, iy, ix, Ci, H, W)] * (double)w[IDX4(co, ci, ky, kx, Ci, c, c)];
      }
    }
  return acc;
}

double or_conv_dw_point(int N, int Ci, int H, int W, int Co, int c, int P,
                        const real* x, const real* dy, int co, int ci, int ky, int kx) {
  const int Ho = H + 2 * P - c + 1, Wo = W + 2 * P - c + 1;
  double acc = 0.0;
  for (int n = 0; n < N; ++n)
    for (int oy = 0; oy < Ho; ++oy) {
      const int iy = oy + ky - P;
      if (iy < 0 || iy >= H) continue;
      for (int ox = 0; ox < Wo; ++ox) {
        const int ix = ox + kx - P;
        if (ix < 0 || ix >= W) continue;
        acc += (double)dy[IDX4(n, co, oy, ox, Co, Ho, Wo)] * (double)x[IDX4(n, ci, iy, ix, Ci, H, W)];
      }
    }
  return acc;
}

double or_conv_db_point(int N, int Co, int Ho, int Wo, const real* dy, int co) {
  double acc = 0.0;
  for (int n = 0; n < N; ++n)
    for (int oy = 0; oy < Ho; ++oy)
      for (int ox = 0; ox < Wo; ++ox) acc += (double)dy[IDX4(n, co, oy, ox, Co, Ho, Wo)];
  return acc;
}

double or_conv_dx_point(int N, int Ci, int H, int W, int Co, int c, int P,
                        const real* w, const real* dy, int n, int ci, int iy, int ix) {
  (void)N;
  const int Ho = H + 2 * P - c + 1, Wo = W + 2 * P - c + 1;
  double acc = 0.0;
  for (int co = 0; co < Co; ++co)
    for (int ky = 0; ky < c; ++ky) {
      const int oy = iy - ky + P;
      if (oy < 0 || oy >= Ho) continue;
      for (int kx = 0; kx < c; ++kx) {
        const int ox = ix - kx + P;
        if (ox < 0 || ox >= Wo) continue;
        acc += (double)dy[IDX4(n, co, oy, ox, Co, Ho, Wo)] * (double)w[IDX4(co, ci, ky, kx, Ci, c, c)];
      }
    }
  return acc;
}

/* ------------------------------------------------------------------------ */
/* ReLU, as used after every hidden layer (the Chainer MLP applies F.relu   */
/* after each Linear but the last).  Derivative taken as 0 at 0.  The pages */
/* define it on numbers only; here a NaN input stays NaN (it is not <= 0),  */
/* so a diverged step shows up in the loss instead of being zeroed.         */
/* ------------------------------------------------------------------------ */
void or_relu_fwd(int64_t n, const real* y, real* a) {
#pragma omp parallel for
  for (int64_t i = 0; i < n; ++i) a[i] = y[i] <= (real)0 ? (real)0 : y[i];
}

/* dy = da where the forward output a was positive, else 0. */
void or_relu_bwd(int64_t n, const real* a, const real* da, real* dy) {
#pragma omp parallel for
  for (int64_t i = 0; i < n; ++i) dy[i] = a[i] > (real)0 ? da[i] : (real)0;
}

/* ------------------------------------------------------------------------ */
/* Max pooling, p x p windows with stride p ([SPRINT] sec. 3.2: layer l is  */
/* followed by pooling when p_l > 1, dividing the width by p_l).  The       */
/* window is scanned row-major and a strict '>' keeps the first maximum;    */
/* a NaN anywhere in the window makes the output NaN.  argmax holds the     */
/* window-local index ky*p + kx of the chosen input.                        */
/* ------------------------------------------------------------------------ */
void or_maxpool_fwd(int N, int C, int H, int W, int p, const real* x, real* y, int32_t* argmax) {
  const int Ho = H / p, Wo = W / p;
#pragma omp parallel for collapse(2)
  for (int n = 0; n < N; ++n)
    for (int ch = 0; ch < C; ++ch)
      for (int oy = 0; oy < Ho; ++oy)
        for (int ox = 0; ox < Wo; ++ox) {
          real best = x[IDX4(n, ch, oy * p, ox * p, C, H, W)];
          int bi = 0, nan = 0;
          for (int ky = 0; ky < p; ++ky)
            for (int kx = 0; kx < p; ++kx) {
              const real v = x[IDX4(n, ch, oy * p + ky, ox * p + kx, C, H, W)];
              if (v != v) nan = 1;
              if (v > best) { best = v; bi = ky * p + kx; }
            }
          y[IDX4(n, ch, oy, ox, C, Ho, Wo)] = nan ? (real)NAN : best;
          argmax[IDX4(n, ch, oy, ox, C, Ho, Wo)] = bi;
        }
}

/* dx = 0 everywhere except at each window's argmax, which receives dy. */
void or_maxpool_bwd(int N, int C, int H, int W, int p, const real* dy, const int32_t* argmax, real* dx) {
  const int Ho = H / p, Wo = W / p;
  memset(dx, 0, sizeof(real) * (size_t)N * C * H * W);
#pragma omp parallel for collapse(2)
  for (int n = 0; n < N; ++n)
    for (int ch = 0; ch < C; ++ch)
      for (int oy = 0; oy < Ho; ++oy)
        for (int ox = 0; ox < Wo; ++ox) {
          const int64_t o = IDX4(n, ch, oy, ox, C, Ho, Wo);
          const int ky = argmax[o] / p, kx = argmax[o] % p;
          dx[IDX4(n, ch, oy * p + ky, ox * p + kx, C, H, W)] += dy[o];
        }
}

/* ------------------------------------------------------------------------ */
/* Fully connected layer, z[n][o] = b[o] + sum_i a[n][i] w[o][i], w stored  */
/* [out][in] ([SPRINT] sec. 3.2 eq. (3): an fc layer holds m_l weights per  */
/* input value plus one bias each; the fc SGEMM row of sec. 3.3 has         */
/* m = N_Subbatch, n = m_l, k = x^2 m_{l-1}).  A conv input is flattened in */
/* (c, h, w) order, which is simply its NCHW memory order.                  */
/* ------------------------------------------------------------------------ */
void or_fc_fwd(int N, int In, int Out, const real* a, const real* w, const real* b, real* z) {
#pragma omp parallel for collapse(2)
  for (int n = 0; n < N; ++n)
    for (int o = 0; o < Out; ++o) {
      double acc = (double)b[o];
      for (int i = 0; i < In; ++i) acc += (double)a[(int64_t)n * In + i] * (double)w[(int64_t)o * In + i];
      z[(int64_t)n * Out + o] = (real)acc;
    }
}

/* db[o] = sum_n dz[n][o]; dw[o][i] = sum_n dz[n][o] a[n][i];
 * da[n][i] = sum_o dz[n][o] w[o][i] (skipped when da is NULL). */
void or_fc_bwd(int N, int In, int Out, const real* a, const real* w, const real* dz,
               real* dw, real* db, real* da) {
#pragma omp parallel for
  for (int o = 0; o < Out; ++o) {
    double acc = 0.0;
    for (int n = 0; n < N; ++n) acc += (double)dz[(int64_t)n * Out + o];
    db[o] = (real)acc;
  }
#pragma omp parallel for collapse(2)
  for (int o = 0; o < Out; ++o)
    for (int i = 0; i < In; ++i) {
      double acc = 0.0;
      for (int n = 0; n < N; ++n) acc += (double)dz[(int64_t)n * Out + o] * (double)a[(int64_t)n * In + i];
      dw[(int64_t)o * In + i] = (real)acc;
    }
  if (!da) return;
#pragma omp parallel for collapse(2)
  for (int n = 0; n < N; ++n)
    for (int i = 0; i < In; ++i) {
      double acc = 0.0;
      for (int o = 0; o < Out; ++o) acc += (double)dz[(int64_t)n * Out + o] * (double)w[(int64_t)o * In + i];
      da[(int64_t)n * In + i] = (real)acc;
    }
}

/* ------------------------------------------------------------------------ */
/* Softmax cross-entropy over C classes ([CHAINER] softmax_cross_entropy,   */
/* a batch mean; [SPRINT] eq. (1) sums per-sample gradients).               */
/*   lse_i = m_i + log sum_j exp(z_ij - m_i),  m_i = max_j z_ij             */
/*   loss  = s * sum_i (lse_i - z_{i,y_i})                                  */
/*   dz_ij = s * (exp(z_ij - lse_i) - [j == y_i])                           */
/* with s = 1/N for the mean reduction (reduce_sum == 0) and 1 for the sum. */
/* Computed in double from the stored logits; returns the loss in double.   */
/* ------------------------------------------------------------------------ */
double or_softmax_ce(int N, int C, const real* z, const int32_t* y, int reduce_sum, real* dz) {
  const double s = reduce_sum ? 1.0 : 1.0 / (double)N;
  double total = 0.0;
  for (int n = 0; n < N; ++n) {
    const real* zr = z + (int64_t)n * C;
    double m = (double)zr[0];
    for (int j = 1; j < C; ++j)
      if ((double)zr[j] > m) m = (double)zr[j];
    double se = 0.0;
    for (int j = 0; j < C; ++j) se += exp((double)zr[j] - m);
    const double lse = m + log(se);
    total += lse - (double)zr[y[n]];
    if (dz)
      for (int j = 0; j < C; ++j)
        dz[(int64_t)n * C + j] = (real)(s * (exp((double)zr[j] - lse) - (j == y[n] ? 1.0 : 0.0)));
  }
  return s * total;
}

/* ------------------------------------------------------------------------ */
/* GradBuf accumulation ([SPRINT] Algorithm 1: if the worker's GradBuf is   */
/* empty it takes the new gradient, otherwise the gradient is added to it;  */
/* Algorithm 2 folds the buffers t = 1..N_GPU in order into SendBuf).       */
/* *empty is the buffer's empty flag; it is cleared by the first call.      */
/* ------------------------------------------------------------------------ */
void or_accumulate(real* buf, int* empty, const real* g, int64_t n) {
  if (*empty) {
    for (int64_t i = 0; i < n; ++i) buf[i] = g[i];
    *empty = 0;
  } else {
    for (int64_t i = 0; i < n; ++i) buf[i] = buf[i] + g[i];
  }
}

/* ------------------------------------------------------------------------ */
/* Update rules, one rounding per statement (build with -ffp-contract=off). */
/* g == NULL means an empty GradBuf, i.e. a zero gradient ([SPRINT]         */
/* Algorithm 2: with no gradient in the first buffer the send buffer is 0). */
/* ------------------------------------------------------------------------ */

/* Weight decay ([PIPE] appendix A trains with weight decay; the pages give
 * no formula).  Read as the gradient of (decay/2)*|W|^2 added to the data
 * gradient before any rule, for every parameter:  wd = decay*W;  g = g + wd.
 * With decay == 0 the gradient is used as it is. */
static real decayed(real g, real w, real decay) {
  if (decay == (real)0) return g;
  const real wd = decay * w;
  return g + wd;
}

/* Plain SGD, [SPRINT] eq. (1): W(t+1) = W(t) - eta * sum of gradients. */
void or_apply_plain(real* W, const real* g, int64_t n, real eta, real decay) {
  if (!g && decay == (real)0) return;
  for (int64_t i = 0; i < n; ++i) {
    const real gi = decayed(g ? g[i] : (real)0, W[i], decay);
    const real t = eta * gi;
    W[i] = W[i] - t;
  }
}

/* Momentum ([SPRINT] sec. 2 design point (b) and Algorithm 2, where the
 * new weights add nu times the previous weight change).  With the change
 * kept in V:  V = mu*V - eta*g;  W = W + V. */
void or_apply_momentum(real* W, real* V, const real* g, int64_t n, real mu, real eta, real decay) {
  for (int64_t i = 0; i < n; ++i) {
    const real gi = decayed(g ? g[i] : (real)0, W[i], decay);
    const real t1 = mu * V[i];
    const real t2 = eta * gi;
    V[i] = t1 - t2;
    W[i] = W[i] + V[i];
  }
}

/* Nesterov momentum ([PIPE] appendix A trains AlexNet and VGG-16 with it;
 * the pages give no formula).  Read as the look-ahead form of the momentum
 * above: the change V is updated as for momentum, and the weights move by
 * mu times the new change plus the gradient step:
 *   V = mu*V - eta*g;  W = W + (mu*V - eta*g). */
void or_apply_nesterov(real* W, real* V, const real* g, int64_t n, real mu, real eta, real decay) {
  for (int64_t i = 0; i < n; ++i) {
    const real gi = decayed(g ? g[i] : (real)0, W[i], decay);
    const real t1 = mu * V[i];
    const real t2 = eta * gi;
    V[i] = t1 - t2;
    const real t3 = mu * V[i];
    const real u = t3 - t2;
    W[i] = W[i] + u;
  }
}

/* Adagrad, a separate adaptive rate per parameter on the parameter server
 * ([DISTBELIEF]: the server applies w' = w - eta_i * dw with Adagrad's rate).
 * The accumulator includes the current gradient before it is used:
 *   A = A + g*g;  r = eta / (sqrt(A) + eps);  W = W - r*g. */
void or_apply_adagrad(real* W, real* A, const real* g, int64_t n, real eta, real eps, real decay) {
  if (!g && decay == (real)0) return;
  for (int64_t i = 0; i < n; ++i) {
    const real gi = decayed(g ? g[i] : (real)0, W[i], decay);
    const real gg = gi * gi;
    A[i] = A[i] + gg;
#if defined(OR_REAL_IS_DOUBLE)
    const real d = sqrt(A[i]) + eps;
#else
    const real d = sqrtf(A[i]) + eps;
#endif
    const real r = eta / d;
    const real t = r * gi;
    W[i] = W[i] - t;
  }
}
