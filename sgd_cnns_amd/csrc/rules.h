// The weight-update rules, one parameter (or one float4 of parameters) at a
// time, shared by the standalone update kernels and the fused training-step
// epilogue so both compute bitwise-identical results.  Each statement rounds
// once (the library is built with -ffp-contract=off; HIP's single-precision
// division and square root are correctly rounded):
//   weight decay (any rule, when decay != 0): wd = decay*W; g = g + wd
//             (the PIPE report's appendix A trains with weight decay 5e-4)
//   plain:    t = eta*g;  W = W - t                       (SPRINT eq. (1))
//   momentum: t1 = mu*V; t2 = eta*g; V = t1 - t2; W = W + V
//             (SPRINT Algorithm 2: the new weights add nu times the last change)
//   adagrad:  A = A + g*g; d = sqrt(A) + eps; r = eta/d; t = r*g; W = W - t
//             (DistBelief review: a per-parameter adaptive rate on the server)
//   nesterov: t1 = mu*V; t2 = eta*g; V = t1 - t2; t3 = mu*V; u = t3 - t2;
//             W = W + u      (the look-ahead momentum of the PIPE report's
//             appendix A: the step adds mu times the new change plus the
//             gradient step)
#pragma once

#include "common.h"

namespace sgd {

template <int RULE, typename T>
__device__ __forceinline__ void rule1(T& w, T& st, T g, float eta, float mu, float eps, float decay) {
  if (decay != 0.f) {
    const T wd = decay * w;
    g = g + wd;
  }
  if (RULE == SGD_PLAIN) {
    const T t = eta * g;
    w = w - t;
  } else if (RULE == SGD_MOMENTUM) {
    const T t1 = mu * st;
    const T t2 = eta * g;
    st = t1 - t2;
    w = w + st;
  } else if (RULE == SGD_NESTEROV) {
    const T t1 = mu * st;
    const T t2 = eta * g;
    st = t1 - t2;
    const T t3 = mu * st;
    const T u = t3 - t2;
    w = w + u;
  } else {
    const T gg = g * g;
    st = st + gg;
    T d;
    if constexpr (sizeof(T) == sizeof(float)) {
      d = sqrtf(st) + eps;
    } else {
      d = T{sqrtf(st.x), sqrtf(st.y), sqrtf(st.z), sqrtf(st.w)} + eps;
    }
    const T r = eta / d;
    const T t = r * g;
    w = w - t;
  }
}

// Apply `rule` to the parameter at w (state at st; unused for plain) with
// gradient g.
__device__ __forceinline__ void apply_one(int rule, float* w, float* st, float g, float eta, float mu, float eps,
                                          float decay) {
  float wv = *w;
  float sv = rule == SGD_PLAIN ? 0.f : *st;
  if (rule == SGD_PLAIN) rule1<SGD_PLAIN>(wv, sv, g, eta, mu, eps, decay);
  else if (rule == SGD_MOMENTUM) rule1<SGD_MOMENTUM>(wv, sv, g, eta, mu, eps, decay);
  else if (rule == SGD_NESTEROV) rule1<SGD_NESTEROV>(wv, sv, g, eta, mu, eps, decay);
  else rule1<SGD_ADAGRAD>(wv, sv, g, eta, mu, eps, decay);
  *w = wv;
  if (rule != SGD_PLAIN) *st = sv;
}

}  // namespace sgd
