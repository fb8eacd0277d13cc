/*
 * TEST INFRASTRUCTURE ONLY.  A driver that runs every oracle function on
 * small ragged shapes with exactly sized heap buffers, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (an out-of-bounds index,
 * an overflow or a use of uninitialised memory in oracle.c then aborts the
 * run).  It checks that the outputs are finite; the values themselves are
 * pinned by the Python tests.  Built and run by tests/test_oracle_sanitize.py:
 *   gcc -fsanitize=address,undefined -fno-sanitize-recover=all oracle.c sanitize_check.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef float real; /* the default (single precision) build of oracle.c */

void or_conv_fwd(int, int, int, int, int, int, int, const real*, const real*, const real*, real*);
void or_conv_bwd(int, int, int, int, int, int, int, const real*, const real*, const real*, real*, real*, real*);
double or_conv_fwd_point(int, int, int, int, int, int, int, const real*, const real*, const real*, int, int, int, int);
double or_conv_dw_point(int, int, int, int, int, int, int, const real*, const real*, int, int, int, int);
double or_conv_db_point(int, int, int, int, const real*, int);
double or_conv_dx_point(int, int, int, int, int, int, int, const real*, const real*, int, int, int, int);
void or_relu_fwd(int64_t, const real*, real*);
void or_relu_bwd(int64_t, const real*, const real*, real*);
void or_maxpool_fwd(int, int, int, int, int, const real*, real*, int32_t*);
void or_maxpool_bwd(int, int, int, int, int, const real*, const int32_t*, real*);
void or_fc_fwd(int, int, int, const real*, const real*, const real*, real*);
void or_fc_bwd(int, int, int, const real*, const real*, const real*, real*, real*, real*);
double or_softmax_ce(int, int, const real*, const int32_t*, int, real*);
void or_accumulate(real*, int*, const real*, int64_t);
void or_apply_plain(real*, const real*, int64_t, real, real);
void or_apply_momentum(real*, real*, const real*, int64_t, real, real, real);
void or_apply_nesterov(real*, real*, const real*, int64_t, real, real, real);
void or_apply_adagrad(real*, real*, const real*, int64_t, real, real, real);

static uint32_t state = 12345u;
static real rnd(void) { /* xorshift32 in [-1, 1) */
  state ^= state << 13;
  state ^= state >> 17;
  state ^= state << 5;
  return (real)((double)state / 2147483648.0 - 1.0);
}
static real* fill(int64_t n) {
  real* p = (real*)malloc((size_t)(n > 0 ? n : 1) * sizeof(real));
  for (int64_t i = 0; i < n; ++i) p[i] = rnd();
  return p;
}
static int finite_all(const real* p, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}
#define CHECK(cond, what)                         \
  do {                                            \
    if (!(cond)) {                                \
      fprintf(stderr, "check failed: %s\n", what); \
      return 1;                                   \
    }                                             \
  } while (0)

static int conv_case(int N, int Ci, int H, int W, int Co, int c, int P) {
  const int Ho = H + 2 * P - c + 1, Wo = W + 2 * P - c + 1;
  const int64_t nx = (int64_t)N * Ci * H * W, nw = (int64_t)Co * Ci * c * c, ny = (int64_t)N * Co * Ho * Wo;
  real *x = fill(nx), *w = fill(nw), *b = fill(Co), *y = fill(ny), *dy = fill(ny);
  real *dw = fill(nw), *db = fill(Co), *dx = fill(nx);
  or_conv_fwd(N, Ci, H, W, Co, c, P, x, w, b, y);
  or_conv_bwd(N, Ci, H, W, Co, c, P, x, w, dy, dw, db, dx);
  double s = or_conv_fwd_point(N, Ci, H, W, Co, c, P, x, w, b, N - 1, Co - 1, Ho - 1, Wo - 1);
  s += or_conv_dw_point(N, Ci, H, W, Co, c, P, x, dy, Co - 1, Ci - 1, c - 1, c - 1);
  s += or_conv_db_point(N, Co, Ho, Wo, dy, Co - 1);
  s += or_conv_dx_point(N, Ci, H, W, Co, c, P, w, dy, N - 1, Ci - 1, H - 1, W - 1);
  const int ok = finite_all(y, ny) && finite_all(dw, nw) && finite_all(db, Co) && finite_all(dx, nx) && isfinite(s);
  free(x), free(w), free(b), free(y), free(dy), free(dw), free(db), free(dx);
  return ok;
}

int main(void) {
  CHECK(conv_case(2, 3, 7, 5, 4, 3, 1), "conv 3x3 pad 1");
  CHECK(conv_case(1, 2, 6, 6, 3, 5, 2), "conv 5x5 pad 2");
  CHECK(conv_case(3, 1, 9, 8, 2, 5, 0), "conv 5x5 pad 0");
  CHECK(conv_case(2, 5, 4, 3, 6, 1, 0), "conv 1x1");
  CHECK(conv_case(1, 2, 4, 4, 3, 4, 0), "conv covering the whole input");

  { /* relu, pooling */
    const int N = 2, C = 3, H = 6, W = 9, p = 3;
    const int64_t n = (int64_t)N * C * H * W, m = (int64_t)N * C * (H / p) * (W / p);
    real *x = fill(n), *a = fill(n), *da = fill(n), *dyr = fill(n), *y = fill(m), *dy = fill(m), *dx = fill(n);
    int32_t* am = (int32_t*)malloc((size_t)m * sizeof(int32_t));
    or_relu_fwd(n, x, a);
    or_relu_bwd(n, a, da, dyr);
    or_maxpool_fwd(N, C, H, W, p, x, y, am);
    or_maxpool_bwd(N, C, H, W, p, dy, am, dx);
    CHECK(finite_all(a, n) && finite_all(dyr, n) && finite_all(y, m) && finite_all(dx, n), "relu / pool");
    for (int64_t i = 0; i < m; ++i) CHECK(am[i] >= 0 && am[i] < p * p, "argmax in the window");
    free(x), free(a), free(da), free(dyr), free(y), free(dy), free(dx), free(am);
  }
  { /* fc and softmax-CE */
    const int N = 5, In = 13, Out = 7;
    real *a = fill((int64_t)N * In), *w = fill((int64_t)Out * In), *b = fill(Out), *z = fill((int64_t)N * Out);
    real *dz = fill((int64_t)N * Out), *dw = fill((int64_t)Out * In), *db = fill(Out), *da = fill((int64_t)N * In);
    int32_t* y = (int32_t*)malloc(N * sizeof(int32_t));
    for (int i = 0; i < N; ++i) y[i] = (i * 3) % Out;
    or_fc_fwd(N, In, Out, a, w, b, z);
    const double l1 = or_softmax_ce(N, Out, z, y, 0, dz);
    const double l2 = or_softmax_ce(N, Out, z, y, 1, dz);
    or_fc_bwd(N, In, Out, a, w, dz, dw, db, da);
    or_fc_bwd(N, In, Out, a, w, dz, dw, db, NULL);
    CHECK(isfinite(l1) && isfinite(l2) && finite_all(dw, (int64_t)Out * In) && finite_all(da, (int64_t)N * In),
          "fc / softmax");
    free(a), free(w), free(b), free(z), free(dz), free(dw), free(db), free(da), free(y);
  }
  { /* GradBuf and the update rules, ragged n */
    const int64_t n = 1003;
    real *buf = fill(n), *g = fill(n), *W = fill(n), *V = fill(n), *A = fill(n);
    for (int64_t i = 0; i < n; ++i) A[i] = A[i] * A[i] + 0.1f;
    int empty = 1;
    or_accumulate(buf, &empty, g, n);
    or_accumulate(buf, &empty, g, n);
    or_apply_plain(W, buf, n, 0.01f, 0.f);
    or_apply_plain(W, buf, n, 0.01f, 5e-4f);
    or_apply_momentum(W, V, buf, n, 0.9f, 0.01f, 5e-4f);
    or_apply_nesterov(W, V, buf, n, 0.9f, 0.01f, 0.f);
    or_apply_adagrad(W, A, buf, n, 0.01f, 1e-8f, 5e-4f);
    CHECK(!empty && finite_all(W, n) && finite_all(V, n) && finite_all(A, n), "updates");
    free(buf), free(g), free(W), free(V), free(A);
  }
  printf("oracle sanitizer run: ok\n");
  return 0;
}
