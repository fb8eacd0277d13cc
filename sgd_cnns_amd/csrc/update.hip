// GradBuf accumulation and the weight-update rules: streaming, HBM-bound
// elementwise kernels over the flat parameter vector.
//
// The arithmetic is one rounding per statement in a fixed order (the library
// is compiled with -ffp-contract=off, and HIP's default single-precision
// division and square root are correctly rounded), so results are bitwise
// reproducible and bitwise equal to a scalar loop written the same way:
//   plain:    t = eta*g;  W = W - t                       (SPRINT eq. (1))
//   momentum: t1 = mu*V; t2 = eta*g; V = t1 - t2; W = W + V
//             (SPRINT Algorithm 2: new weights add nu times the last change)
//   adagrad:  A = A + g*g; d = sqrt(A) + eps; r = eta/d; t = r*g; W = W - t
//             (DistBelief review: a per-parameter adaptive rate on the server)
// The gradient g is the left fold of k buffers g_0 + g_1 + ... + g_{k-1}
// (SPRINT Algorithm 2's SumGradient order); k = 0 is an empty GradBuf, i.e.
// a zero gradient.
//
// Each thread handles float4 groups (16-byte loads and stores); a scalar path
// covers misaligned pointers and the n % 4 tail.
#include "common.h"
#include "layers.h"

namespace sgd {
namespace {

constexpr int kMaxK = 16;
constexpr int kBlock = 256;

struct Ptrs {
  const float* g[kMaxK];
};

__device__ __forceinline__ float fold(const Ptrs& P, int k, int64_t i) {
  float s = P.g[0][i];
  for (int j = 1; j < k; ++j) s = s + P.g[j][i];
  return s;
}

__device__ __forceinline__ float4 fold4(const Ptrs& P, int k, int64_t i) {
  float4 s = reinterpret_cast<const float4*>(P.g[0])[i];
  for (int j = 1; j < k; ++j) {
    const float4 v = reinterpret_cast<const float4*>(P.g[j])[i];
    s.x = s.x + v.x;
    s.y = s.y + v.y;
    s.z = s.z + v.z;
    s.w = s.w + v.w;
  }
  return s;
}

// buf = (first_is_copy ? 0-term : buf) + g_0 + ... + g_{k-1}, left to right.
__global__ void accumulate_kernel(float* __restrict__ buf, Ptrs P, int k, int first_is_copy, int64_t n, int vec) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t done = 0;
  if (vec) {
    const int64_t n4 = n / 4;
    for (int64_t i = t0; i < n4; i += stride) {
      float4 s;
      if (first_is_copy) {
        s = fold4(P, k, i);
      } else {
        s = reinterpret_cast<const float4*>(buf)[i];
        for (int j = 0; j < k; ++j) {
          const float4 v = reinterpret_cast<const float4*>(P.g[j])[i];
          s.x = s.x + v.x;
          s.y = s.y + v.y;
          s.z = s.z + v.z;
          s.w = s.w + v.w;
        }
      }
      reinterpret_cast<float4*>(buf)[i] = s;
    }
    done = n4 * 4;
  }
  for (int64_t i = done + t0; i < n; i += stride) {
    float s;
    if (first_is_copy) {
      s = fold(P, k, i);
    } else {
      s = buf[i];
      for (int j = 0; j < k; ++j) s = s + P.g[j][i];
    }
    buf[i] = s;
  }
}

template <int RULE>
__device__ __forceinline__ void rule1(float& w, float* st, float g, float eta, float mu, float eps) {
  if (RULE == SGD_PLAIN) {
    const float t = eta * g;
    w = w - t;
  } else if (RULE == SGD_MOMENTUM) {
    const float t1 = mu * *st;
    const float t2 = eta * g;
    const float v = t1 - t2;
    *st = v;
    w = w + v;
  } else {
    const float gg = g * g;
    const float a = *st + gg;
    *st = a;
    const float d = sqrtf(a) + eps;
    const float r = eta / d;
    const float t = r * g;
    w = w - t;
  }
}

template <int RULE>
__global__ void apply_kernel(float* __restrict__ W, float* __restrict__ state, Ptrs P, int k, int64_t n, float eta,
                             float mu, float eps, int vec) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t done = 0;
  if (vec) {
    const int64_t n4 = n / 4;
    for (int64_t i = t0; i < n4; i += stride) {
      const float4 g = k > 0 ? fold4(P, k, i) : make_float4(0.f, 0.f, 0.f, 0.f);
      float4 w = reinterpret_cast<const float4*>(W)[i];
      float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
      if (RULE != SGD_PLAIN) s = reinterpret_cast<const float4*>(state)[i];
      rule1<RULE>(w.x, &s.x, g.x, eta, mu, eps);
      rule1<RULE>(w.y, &s.y, g.y, eta, mu, eps);
      rule1<RULE>(w.z, &s.z, g.z, eta, mu, eps);
      rule1<RULE>(w.w, &s.w, g.w, eta, mu, eps);
      reinterpret_cast<float4*>(W)[i] = w;
      if (RULE != SGD_PLAIN) reinterpret_cast<float4*>(state)[i] = s;
    }
    done = n4 * 4;
  }
  for (int64_t i = done + t0; i < n; i += stride) {
    const float g = k > 0 ? fold(P, k, i) : 0.f;
    float w = W[i];
    float s = RULE != SGD_PLAIN ? state[i] : 0.f;
    rule1<RULE>(w, &s, g, eta, mu, eps);
    W[i] = w;
    if (RULE != SGD_PLAIN) state[i] = s;
  }
}

bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int grid_for(int64_t n) {
  // Enough workgroups to fill 256 CUs several times over; each thread then
  // loops over float4 groups.
  const int64_t want = ceil_div(ceil_div(n, 4), kBlock);
  return (int)std::max<int64_t>(1, std::min<int64_t>(want, 256 * 16));
}

}  // namespace

int accumulate(float* buf, const float* const* grads, int k, bool first_is_copy, int64_t n, hipStream_t s) {
  Ptrs P{};
  bool vec = a16(buf);
  for (int j = 0; j < k; ++j) {
    P.g[j] = grads[j];
    vec = vec && a16(grads[j]);
  }
  hipLaunchKernelGGL(accumulate_kernel, dim3(grid_for(n)), dim3(kBlock), 0, s, buf, P, k, (int)first_is_copy, n,
                     (int)vec);
  return check_launch("accumulate");
}

int apply_rule(float* W, float* state, const float* const* grads, int k, int64_t n, int rule, float eta, float mu,
               float eps, hipStream_t s) {
  Ptrs P{};
  bool vec = a16(W) && (rule == SGD_PLAIN || a16(state));
  for (int j = 0; j < k; ++j) {
    P.g[j] = grads[j];
    vec = vec && a16(grads[j]);
  }
  const dim3 g(grid_for(n)), b(kBlock);
  switch (rule) {
    case SGD_PLAIN:
      hipLaunchKernelGGL(apply_kernel<SGD_PLAIN>, g, b, 0, s, W, state, P, k, n, eta, mu, eps, (int)vec);
      break;
    case SGD_MOMENTUM:
      hipLaunchKernelGGL(apply_kernel<SGD_MOMENTUM>, g, b, 0, s, W, state, P, k, n, eta, mu, eps, (int)vec);
      break;
    default:
      hipLaunchKernelGGL(apply_kernel<SGD_ADAGRAD>, g, b, 0, s, W, state, P, k, n, eta, mu, eps, (int)vec);
      break;
  }
  return check_launch("apply_rule");
}

}  // namespace sgd
