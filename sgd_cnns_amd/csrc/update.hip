// GradBuf accumulation and the weight-update rules: streaming, HBM-bound
// elementwise kernels over the flat parameter vector.
//
// The rules themselves are in rules.h (one rounding per statement, shared with
// the fused training-step epilogue).
// The gradient g is the left fold of k buffers g_0 + g_1 + ... + g_{k-1}
// (SPRINT Algorithm 2's SumGradient order); k = 0 is an empty GradBuf, i.e.
// a zero gradient.
//
// Memory shape (measured on MI355X with 8 gradient buffers + W + A, the
// parameter-server Adagrad apply): a block of 256 threads owns 1024
// consecutive float4 groups, i.e. 16 KiB of every stream, and each thread
// issues all of its loads -- 4 groups of every gradient buffer, W and the
// optimiser state -- before the first addition.  The number of buffers is a
// template parameter so the compiler can keep every load in flight; with a
// run-time count the loads of buffer j+1 wait for the sum of buffer j and the
// kernel ran at 70% of HBM peak instead of 75%.  Loads and stores are
// non-temporal: every byte is touched once.  Groups past the end re-read
// group 0 and store nothing; the last block's first n % 4 threads do the
// scalar tail.  Misaligned pointers take a scalar kernel.
#include "common.h"
#include "layers.h"
#include "rules.h"

namespace sgd {
namespace {

constexpr int kMaxK = 16;
constexpr int kBlock = 256;
constexpr int kGroups = 4;                      // float4 groups per thread
constexpr int kChunk = kBlock * kGroups;        // float4 groups per block
constexpr int kMaxUnrolledK = 8;                // K above this: run-time loop

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

// s[u] = x[u] + g_0[u] + ... + g_{k-1}[u] for the thread's groups idx[u], one
// rounding per addition, left to right.  K > 0: exactly K buffers (k == K),
// every load issued before the first addition; K < 0: k buffers, loaded one
// buffer at a time.  `init` says whether s already holds x (else s starts as
// g_0).
template <int K>
__device__ __forceinline__ void fold_groups(v4f (&s)[kGroups], const Ptrs& P, int k, bool init,
                                            const int64_t (&idx)[kGroups]) {
  if constexpr (K > 0) {
    v4f g[K][kGroups];
#pragma unroll
    for (int j = 0; j < K; ++j)
#pragma unroll
      for (int u = 0; u < kGroups; ++u) g[j][u] = ld4(P.g[j], idx[u]);
#pragma unroll
    for (int u = 0; u < kGroups; ++u) {
      v4f acc = init ? s[u] + g[0][u] : g[0][u];
#pragma unroll
      for (int j = 1; j < K; ++j) acc = acc + g[j][u];
      s[u] = acc;
    }
  } else {
    for (int j = 0; j < k; ++j) {
      v4f g[kGroups];
#pragma unroll
      for (int u = 0; u < kGroups; ++u) g[u] = ld4(P.g[j], idx[u]);
#pragma unroll
      for (int u = 0; u < kGroups; ++u) s[u] = (init || j > 0) ? s[u] + g[u] : g[u];
    }
  }
}

// Scalar left fold of the buffers j0..k-1 at element i onto s.
__device__ __forceinline__ float fold1(const Ptrs& P, int j0, int k, float s, int64_t i) {
  for (int j = j0; j < k; ++j) s = s + P.g[j][i];
  return s;
}

// buf = (COPY ? g_0 : buf + g_0) + g_1 + ... + g_{k-1}, left to right.
template <int K, bool COPY>
__global__ __launch_bounds__(kBlock) void accumulate_kernel(float* __restrict__ buf, Ptrs P, int k, int64_t n) {
  const int64_t n4 = n / 4;
  if (n4 > 0) {
    int64_t idx[kGroups], ld[kGroups];
#pragma unroll
    for (int u = 0; u < kGroups; ++u) {
      idx[u] = (int64_t)blockIdx.x * kChunk + u * kBlock + threadIdx.x;
      ld[u] = idx[u] < n4 ? idx[u] : 0;
    }
    v4f s[kGroups];
    if (!COPY) {
#pragma unroll
      for (int u = 0; u < kGroups; ++u) s[u] = ld4(buf, ld[u]);
    }
    fold_groups<K>(s, P, k, !COPY, ld);
#pragma unroll
    for (int u = 0; u < kGroups; ++u)
      if (idx[u] < n4) st4(buf, idx[u], s[u]);
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x < n - 4 * n4) {
    const int64_t i = 4 * n4 + threadIdx.x;
    buf[i] = COPY ? fold1(P, 1, k, P.g[0][i], i) : fold1(P, 0, k, buf[i], i);
  }
}

// The same for pointers that are not 16-byte aligned: one element per thread.
__global__ void accumulate_scalar_kernel(float* __restrict__ buf, Ptrs P, int k, int first_is_copy, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    buf[i] = first_is_copy ? fold1(P, 1, k, P.g[0][i], i) : fold1(P, 0, k, buf[i], i);
}

// W (and state) <- RULE(W, state, g_0 + ... + g_{k-1}); k = 0 is a zero
// gradient.  K as for fold_groups, 0 for no buffers.
template <int RULE, int K>
__global__ __launch_bounds__(kBlock) void apply_kernel(float* __restrict__ W, float* __restrict__ state, Ptrs P,
                                                       int k, int64_t n, float eta, float mu, float eps,
                                                       float decay) {
  constexpr bool kState = RULE != SGD_PLAIN;
  const int64_t n4 = n / 4;
  if (n4 > 0) {
    int64_t idx[kGroups], ld[kGroups];
#pragma unroll
    for (int u = 0; u < kGroups; ++u) {
      idx[u] = (int64_t)blockIdx.x * kChunk + u * kBlock + threadIdx.x;
      ld[u] = idx[u] < n4 ? idx[u] : 0;
    }
    v4f w[kGroups], st[kGroups], g[kGroups];
#pragma unroll
    for (int u = 0; u < kGroups; ++u) {
      w[u] = ld4(W, ld[u]);
      st[u] = kState ? ld4(state, ld[u]) : v4f{0.f, 0.f, 0.f, 0.f};
      g[u] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (K != 0) fold_groups<K>(g, P, k, false, ld);
#pragma unroll
    for (int u = 0; u < kGroups; ++u) {
      rule1<RULE>(w[u], st[u], g[u], eta, mu, eps, decay);
      if (idx[u] < n4) {
        st4(W, idx[u], w[u]);
        if (kState) st4(state, idx[u], st[u]);
      }
    }
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x < n - 4 * n4) {
    const int64_t i = 4 * n4 + threadIdx.x;
    const float g = k > 0 ? fold1(P, 1, k, P.g[0][i], i) : 0.f;
    float w = W[i];
    float st = kState ? state[i] : 0.f;
    rule1<RULE>(w, st, g, eta, mu, eps, decay);
    W[i] = w;
    if (kState) state[i] = st;
  }
}

template <int RULE>
__global__ void apply_scalar_kernel(float* __restrict__ W, float* __restrict__ state, Ptrs P, int k, int64_t n,
                                    float eta, float mu, float eps, float decay) {
  constexpr bool kState = RULE != SGD_PLAIN;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float g = k > 0 ? fold1(P, 1, k, P.g[0][i], i) : 0.f;
    float w = W[i];
    float st = kState ? state[i] : 0.f;
    rule1<RULE>(w, st, g, eta, mu, eps, decay);
    W[i] = w;
    if (kState) state[i] = st;
  }
}

// Reference streaming kernel: outs[j] = ins[0] + ... + ins[K-1] (left fold)
// for every output j < NOUT; with NOUT == 0 the sum is only kept live (a
// store that never fires).  G float4 groups per thread, block-contiguous as
// in the update kernels when G > 1, one float4 per thread when G == 1.  It
// has the memory shape of the update kernels without their arithmetic or
// state, and measures what that mix of read and write streams can reach.
template <int K, int NOUT, int G>
__global__ __launch_bounds__(kBlock) void stream_ref_kernel(Ptrs in, float* o0, float* o1,
                                                            int64_t n4) {
  int64_t idx[G];
#pragma unroll
  for (int u = 0; u < G; ++u) {
    idx[u] = (int64_t)blockIdx.x * kBlock * G + u * kBlock + threadIdx.x;
    if (idx[u] >= n4) idx[u] = -1;
  }
  v4f s[G];
  v4f g[K][G];
#pragma unroll
  for (int j = 0; j < K; ++j)
#pragma unroll
    for (int u = 0; u < G; ++u) g[j][u] = ld4(in.g[j], idx[u] < 0 ? 0 : idx[u]);
#pragma unroll
  for (int u = 0; u < G; ++u) {
    s[u] = g[0][u];
#pragma unroll
    for (int j = 1; j < K; ++j) s[u] = s[u] + g[j][u];
  }
#pragma unroll
  for (int u = 0; u < G; ++u) {
    if (idx[u] < 0) continue;
    if (NOUT >= 1) st4(o0, idx[u], s[u]);
    if (NOUT >= 2) st4(o1, idx[u], s[u]);
    if (NOUT == 0 && s[u].x == 1234567.f && s[u].y == -7654321.f) st4(o0, idx[u], s[u]);
  }
}

bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int vec_grid(int64_t n) { return (int)std::max<int64_t>(1, ceil_div(n / 4, kChunk)); }
int scalar_grid(int64_t n) { return (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(n, kBlock), 1 << 16)); }

// Calls f(std::integral_constant<int, K>) with K = k for k <= 8, else K = -1.
template <typename F>
void with_k(int k, F&& f) {
  switch (k) {
    case 0: f(std::integral_constant<int, 0>{}); break;
    case 1: f(std::integral_constant<int, 1>{}); break;
    case 2: f(std::integral_constant<int, 2>{}); break;
    case 3: f(std::integral_constant<int, 3>{}); break;
    case 4: f(std::integral_constant<int, 4>{}); break;
    case 5: f(std::integral_constant<int, 5>{}); break;
    case 6: f(std::integral_constant<int, 6>{}); break;
    case 7: f(std::integral_constant<int, 7>{}); break;
    case 8: f(std::integral_constant<int, 8>{}); break;
    default: f(std::integral_constant<int, -1>{}); break;
  }
  static_assert(kMaxUnrolledK == 8, "with_k unrolls k up to 8");
}

template <int RULE>
void launch_apply(bool vec, float* W, float* state, const Ptrs& P, int k, int64_t n, float eta, float mu, float eps,
                  float decay, hipStream_t s) {
  if (!vec) {
    hipLaunchKernelGGL(apply_scalar_kernel<RULE>, dim3(scalar_grid(n)), dim3(kBlock), 0, s, W, state, P, k, n, eta,
                       mu, eps, decay);
    return;
  }
  with_k(k, [&](auto K) {
    hipLaunchKernelGGL((apply_kernel<RULE, decltype(K)::value>), dim3(vec_grid(n)), dim3(kBlock), 0, s, W, state, P,
                       k, n, eta, mu, eps, decay);
  });
}

}  // namespace

int accumulate(float* buf, const float* const* grads, int k, bool first_is_copy, int64_t n, hipStream_t s) {
  if (k < 1 || k > kMaxK) {
    set_error("accumulate: k must be in 1..16");
    return SGD_EINVAL;
  }
  Ptrs P{};
  bool vec = a16(buf);
  for (int j = 0; j < k; ++j) {
    P.g[j] = grads[j];
    vec = vec && a16(grads[j]);
  }
  const double streams = k + (first_is_copy ? 1 : 2);
  prof_begin(first_is_copy ? "accumulate_copy" : "accumulate_add", (double)(k - (first_is_copy ? 1 : 0)) * n,
             4.0 * streams * n, s);
  if (!vec) {
    hipLaunchKernelGGL(accumulate_scalar_kernel, dim3(scalar_grid(n)), dim3(kBlock), 0, s, buf, P, k,
                       (int)first_is_copy, n);
  } else {
    with_k(k, [&](auto K) {
      constexpr int KK = decltype(K)::value;
      if constexpr (KK != 0) {
        if (first_is_copy)
          hipLaunchKernelGGL((accumulate_kernel<KK, true>), dim3(vec_grid(n)), dim3(kBlock), 0, s, buf, P, k, n);
        else
          hipLaunchKernelGGL((accumulate_kernel<KK, false>), dim3(vec_grid(n)), dim3(kBlock), 0, s, buf, P, k, n);
      }
    });
  }
  prof_end(s);
  return check_launch("accumulate");
}

int stream_ref(float* const* outs, int n_out, const float* const* ins, int n_in, int64_t n, int groups,
               hipStream_t s) {
  if (n <= 0 || n % 4) {
    set_error("stream_ref: n must be a positive multiple of 4");
    return SGD_EINVAL;
  }
  if (groups != 1 && groups != 4) {
    set_error("stream_ref: groups per thread must be 1 or 4");
    return SGD_EINVAL;
  }
  const bool shape_ok = (n_in == 1 && n_out == 1) || (n_in == 10 && (n_out == 0 || n_out == 2));
  if (!shape_ok) {
    set_error("stream_ref: supported (reads, writes): (1, 1), (10, 0), (10, 2)");
    return SGD_EINVAL;
  }
  Ptrs P{};
  for (int j = 0; j < n_in; ++j) {
    if (!ins[j] || !a16(ins[j])) {
      set_error("stream_ref: inputs must be 16-byte aligned device pointers");
      return SGD_EINVAL;
    }
    P.g[j] = ins[j];
  }
  for (int j = 0; j < n_out; ++j)
    if (!outs[j] || !a16(outs[j])) {
      set_error("stream_ref: outputs must be 16-byte aligned device pointers");
      return SGD_EINVAL;
    }
  float* o0 = n_out >= 1 ? outs[0] : const_cast<float*>(ins[0]);
  float* o1 = n_out >= 2 ? outs[1] : o0;
  const int64_t n4 = n / 4;
  const int grid = (int)ceil_div(n4, (int64_t)kBlock * groups);
  prof_begin("stream_ref", 0.0, 4.0 * (n_in + n_out) * (double)n, s);
  auto go = [&](auto kc, auto oc) {
    constexpr int K = decltype(kc)::value, NO = decltype(oc)::value;
    if (groups == 1)
      hipLaunchKernelGGL((stream_ref_kernel<K, NO, 1>), dim3(grid), dim3(kBlock), 0, s, P, o0, o1, n4);
    else
      hipLaunchKernelGGL((stream_ref_kernel<K, NO, 4>), dim3(grid), dim3(kBlock), 0, s, P, o0, o1, n4);
  };
  if (n_in == 1) go(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
  else if (n_out == 0) go(std::integral_constant<int, 10>{}, std::integral_constant<int, 0>{});
  else go(std::integral_constant<int, 10>{}, std::integral_constant<int, 2>{});
  prof_end(s);
  return check_launch("stream_ref");
}

int apply_rule(float* W, float* state, const float* const* grads, int k, int64_t n, int rule, float eta, float mu,
               float eps, float decay, hipStream_t s) {
  if (k < 0 || k > kMaxK) {
    set_error("apply_rule: k must be in 0..16");
    return SGD_EINVAL;
  }
  Ptrs P{};
  bool vec = a16(W) && (rule == SGD_PLAIN || a16(state));
  for (int j = 0; j < k; ++j) {
    P.g[j] = grads[j];
    vec = vec && a16(grads[j]);
  }
  static const char* const names[4] = {"apply_plain", "apply_momentum", "apply_adagrad", "apply_nesterov"};
  const double streams = k + (rule == SGD_PLAIN ? 2 : 4);
  prof_begin(names[rule], (double)n * (k + 4), 4.0 * streams * n, s);
  switch (rule) {
    case SGD_PLAIN: launch_apply<SGD_PLAIN>(vec, W, state, P, k, n, eta, mu, eps, decay, s); break;
    case SGD_MOMENTUM: launch_apply<SGD_MOMENTUM>(vec, W, state, P, k, n, eta, mu, eps, decay, s); break;
    case SGD_NESTEROV: launch_apply<SGD_NESTEROV>(vec, W, state, P, k, n, eta, mu, eps, decay, s); break;
    default: launch_apply<SGD_ADAGRAD>(vec, W, state, P, k, n, eta, mu, eps, decay, s); break;
  }
  prof_end(s);
  return check_launch("apply_rule");
}

}  // namespace sgd
