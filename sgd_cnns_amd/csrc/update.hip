// GradBuf accumulation and the weight-update rules: streaming, HBM-bound
// elementwise kernels over the flat parameter vector.
//
// The rules themselves are in rules.h (one rounding per statement, shared with
// the fused training-step epilogue).
// The gradient g is the left fold of k buffers g_0 + g_1 + ... + g_{k-1}
// (SPRINT Algorithm 2's SumGradient order); k = 0 is an empty GradBuf, i.e.
// a zero gradient.
//
// Each thread handles two float4 groups per iteration (16-byte loads and
// stores, all issued before the arithmetic so more bytes are in flight); the
// data are streamed with non-temporal loads and stores, since every byte is
// touched once.  A scalar path covers misaligned pointers and the n % 4 tail.
#include "common.h"
#include "layers.h"
#include "rules.h"

namespace sgd {
namespace {

constexpr int kMaxK = 16;
constexpr int kBlock = 256;
constexpr int kUnroll = 2;

typedef float v4f __attribute__((ext_vector_type(4)));

struct Ptrs {
  const float* g[kMaxK];
};

__device__ __forceinline__ v4f ld4(const float* p, int64_t i) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p) + i);
}
__device__ __forceinline__ void st4(float* p, int64_t i, v4f v) {
  __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(p) + i);
}

// Left fold g_0 + g_1 + ... + g_{k-1} (k >= 1), one rounding per addition.
__device__ __forceinline__ v4f fold4(const Ptrs& P, int k, int64_t i) {
  v4f s = ld4(P.g[0], i);
  for (int j = 1; j < k; ++j) s = s + ld4(P.g[j], i);
  return s;
}
__device__ __forceinline__ float fold1(const Ptrs& P, int k, int64_t i) {
  float s = P.g[0][i];
  for (int j = 1; j < k; ++j) s = s + P.g[j][i];
  return s;
}

// buf = (first_is_copy ? g_0 : buf + g_0) + g_1 + ... + g_{k-1}, left to right.
__global__ void accumulate_kernel(float* __restrict__ buf, Ptrs P, int k, int first_is_copy, int64_t n, int vec) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t done = 0;
  if (vec) {
    const int64_t n4 = n / 4;
    for (; i + (kUnroll - 1) * stride < n4; i += kUnroll * stride) {
      v4f s[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) s[u] = first_is_copy ? ld4(P.g[0], i + u * stride) : ld4(buf, i + u * stride);
      for (int j = first_is_copy ? 1 : 0; j < k; ++j)
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) s[u] = s[u] + ld4(P.g[j], i + u * stride);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) st4(buf, i + u * stride, s[u]);
    }
    for (; i < n4; i += stride) {
      v4f s = first_is_copy ? ld4(P.g[0], i) : ld4(buf, i);
      for (int j = first_is_copy ? 1 : 0; j < k; ++j) s = s + ld4(P.g[j], i);
      st4(buf, i, s);
    }
    done = n4 * 4;
    i = done + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  }
  for (; i < n; i += stride) {
    float s = first_is_copy ? P.g[0][i] : buf[i];
    for (int j = first_is_copy ? 1 : 0; j < k; ++j) s = s + P.g[j][i];
    buf[i] = s;
  }
}

template <int RULE>
__global__ void apply_kernel(float* __restrict__ W, float* __restrict__ state, Ptrs P, int k, int64_t n, float eta,
                             float mu, float eps, float decay, int vec) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  constexpr bool kState = RULE != SGD_PLAIN;
  if (vec) {
    const int64_t n4 = n / 4;
    for (; i + (kUnroll - 1) * stride < n4; i += kUnroll * stride) {
      v4f w[kUnroll], st[kUnroll], g[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        g[u] = k > 0 ? fold4(P, k, i + u * stride) : v4f{0.f, 0.f, 0.f, 0.f};
        w[u] = ld4(W, i + u * stride);
        st[u] = kState ? ld4(state, i + u * stride) : v4f{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        rule1<RULE>(w[u], st[u], g[u], eta, mu, eps, decay);
        st4(W, i + u * stride, w[u]);
        if (kState) st4(state, i + u * stride, st[u]);
      }
    }
    for (; i < n4; i += stride) {
      v4f g = k > 0 ? fold4(P, k, i) : v4f{0.f, 0.f, 0.f, 0.f};
      v4f w = ld4(W, i);
      v4f st = kState ? ld4(state, i) : v4f{0.f, 0.f, 0.f, 0.f};
      rule1<RULE>(w, st, g, eta, mu, eps, decay);
      st4(W, i, w);
      if (kState) st4(state, i, st);
    }
    i = n4 * 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  }
  for (; i < n; i += stride) {
    const float g = k > 0 ? fold1(P, k, i) : 0.f;
    float w = W[i];
    float st = kState ? state[i] : 0.f;
    rule1<RULE>(w, st, g, eta, mu, eps, decay);
    W[i] = w;
    if (kState) state[i] = st;
  }
}

bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// About one unrolled iteration per thread: many waves in flight per CU hide
// HBM latency better than a few long-running ones.
int grid_for(int64_t n) {
  const int64_t want = ceil_div(ceil_div(n, 4), (int64_t)kBlock * kUnroll);
  return (int)std::max<int64_t>(1, std::min<int64_t>(want, 1 << 16));
}

}  // namespace

int accumulate(float* buf, const float* const* grads, int k, bool first_is_copy, int64_t n, hipStream_t s) {
  Ptrs P{};
  bool vec = a16(buf);
  for (int j = 0; j < k; ++j) {
    P.g[j] = grads[j];
    vec = vec && a16(grads[j]);
  }
  const double streams = k + (first_is_copy ? 1 : 2);
  prof_begin(first_is_copy ? "accumulate_copy" : "accumulate_add", (double)(k - (first_is_copy ? 1 : 0)) * n,
             4.0 * streams * n, s);
  hipLaunchKernelGGL(accumulate_kernel, dim3(grid_for(n)), dim3(kBlock), 0, s, buf, P, k, (int)first_is_copy, n,
                     (int)vec);
  prof_end(s);
  return check_launch("accumulate");
}

int apply_rule(float* W, float* state, const float* const* grads, int k, int64_t n, int rule, float eta, float mu,
               float eps, float decay, hipStream_t s) {
  Ptrs P{};
  bool vec = a16(W) && (rule == SGD_PLAIN || a16(state));
  for (int j = 0; j < k; ++j) {
    P.g[j] = grads[j];
    vec = vec && a16(grads[j]);
  }
  const dim3 g(grid_for(n)), b(kBlock);
  static const char* const names[4] = {"apply_plain", "apply_momentum", "apply_adagrad", "apply_nesterov"};
  const double streams = k + (rule == SGD_PLAIN ? 2 : 4);
  prof_begin(names[rule], (double)n * (k + 4), 4.0 * streams * n, s);
  switch (rule) {
    case SGD_PLAIN:
      hipLaunchKernelGGL(apply_kernel<SGD_PLAIN>, g, b, 0, s, W, state, P, k, n, eta, mu, eps, decay, (int)vec);
      break;
    case SGD_MOMENTUM:
      hipLaunchKernelGGL(apply_kernel<SGD_MOMENTUM>, g, b, 0, s, W, state, P, k, n, eta, mu, eps, decay, (int)vec);
      break;
    case SGD_NESTEROV:
      hipLaunchKernelGGL(apply_kernel<SGD_NESTEROV>, g, b, 0, s, W, state, P, k, n, eta, mu, eps, decay, (int)vec);
      break;
    default:
      hipLaunchKernelGGL(apply_kernel<SGD_ADAGRAD>, g, b, 0, s, W, state, P, k, n, eta, mu, eps, decay, (int)vec);
      break;
  }
  prof_end(s);
  return check_launch("apply_rule");
}

}  // namespace sgd
