// fp32 matrix products on the CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// Every conv forward, fc, dedw, dedx_fc and dedx_conv product of the SPRINT
// report's section 3.3 SGEMM table is one call of gemm() below, in one of
// three operand forms:
//   forward  C = A * B^T   A [M][K], B [N][K]   (a_t = false, b_t = false)
//   dedw     C = A^T * B   A [K][M], B [K][N]   (a_t = true,  b_t = true)
//   dedx     C = A * B     A [M][K], B [K][N]   (a_t = false, b_t = true)
//
// Kernel shape: 256 threads = 4 wavefronts of 64 lanes in a 2x2 grid over a
// BM x BN output tile; each wavefront owns a (BM/2) x (BN/2) sub-tile made of
// 32x32 MFMA blocks accumulated in fp32.  K advances in BK = 16 slices
// staged through LDS with a two-buffer pipeline (the next slice is fetched
// into registers while the current one is multiplied).  LDS holds both
// operands K-major ([k][row]) so each MFMA operand is one conflict-free
// 32-float row segment; row strides are padded by 32 floats so the two
// half-wavefronts (k and k+1) read disjoint banks.
//
// Large-K products (conv dedw has K = N*Ho*Wo, up to 1.6M) are split along K;
// each slice writes its own partial tile and a second pass adds the slices in
// a fixed order, so results stay deterministic and the fp32 sums stay short.
#include "common.h"

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace sgd {
namespace {

constexpr int kBK = 16;
constexpr int kThreads = 256;

struct KArgs {
  const float* A;
  const float* B;
  float* C;
  int M, N, K;
  int64_t lda, ldb, ldc;
  int k_per_split;  // multiple of kBK
  int split;        // 1 -> write raw partials to C + z*M*N (row stride N)
  int epi;
  const float* bias;
  const float* mask;
  int64_t ldm;
  int a_vec, b_vec;  // float4 global loads allowed (aligned base, ld % 4 == 0)
  int tiles_n;       // number of tiles along N
  int tiles;         // tiles per split
};

// Fetch one operand slice (R rows x kBK) from global memory into registers.
//   T == false: stored [R][K] (row stride ld), 4 consecutive k per float4.
//   T == true:  stored [K][R], 4 consecutive rows per float4.
template <int R, bool T>
__device__ __forceinline__ void fetch(const float* __restrict__ X, int64_t ld, int r0, int rmax, int k0,
                                      int kend, bool vec, float4* regs) {
  constexpr int NL = R * kBK / 4 / kThreads;
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int i = threadIdx.x + kThreads * j;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!T) {
      const int r = i / (kBK / 4), k = (i % (kBK / 4)) * 4;
      const int gr = r0 + r, gk = k0 + k;
      if (gr < rmax) {
        const float* src = X + (int64_t)gr * ld + gk;
        if (vec && gk + 3 < kend) {
          v = *reinterpret_cast<const float4*>(src);
        } else {
          if (gk < kend) v.x = src[0];
          if (gk + 1 < kend) v.y = src[1];
          if (gk + 2 < kend) v.z = src[2];
          if (gk + 3 < kend) v.w = src[3];
        }
      }
    } else {
      const int k = i / (R / 4), r = (i % (R / 4)) * 4;
      const int gr = r0 + r, gk = k0 + k;
      if (gk < kend) {
        const float* src = X + (int64_t)gk * ld + gr;
        if (vec && gr + 3 < rmax) {
          v = *reinterpret_cast<const float4*>(src);
        } else {
          if (gr < rmax) v.x = src[0];
          if (gr + 1 < rmax) v.y = src[1];
          if (gr + 2 < rmax) v.z = src[2];
          if (gr + 3 < rmax) v.w = src[3];
        }
      }
    }
    regs[j] = v;
  }
}

// Write fetched registers into the K-major LDS slice S[k][row].
template <int R, int LD, bool T>
__device__ __forceinline__ void stash(float* S, const float4* regs) {
  constexpr int NL = R * kBK / 4 / kThreads;
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int i = threadIdx.x + kThreads * j;
    const float4 v = regs[j];
    if (!T) {
      const int r = i / (kBK / 4), k = (i % (kBK / 4)) * 4;
      S[(k + 0) * LD + r] = v.x;
      S[(k + 1) * LD + r] = v.y;
      S[(k + 2) * LD + r] = v.z;
      S[(k + 3) * LD + r] = v.w;
    } else {
      const int k = i / (R / 4), r = (i % (R / 4)) * 4;
      *reinterpret_cast<float4*>(&S[k * LD + r]) = v;
    }
  }
}

__device__ __forceinline__ float epilogue(float v, int epi, int row, int col, const KArgs& p, float old) {
  switch (epi) {
    case EPI_BIAS: return v + p.bias[col];
    case EPI_BIAS_RELU: {
      const float t = v + p.bias[col];
      return t <= 0.f ? 0.f : t;  // NaN passes through
    }
    case EPI_MASK: return p.mask[(int64_t)row * p.ldm + col] > 0.f ? v : 0.f;
    case EPI_ACCUM: return old + v;
    default: return v;
  }
}

template <int BM, int BN, bool AT, bool BT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(KArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int LDA = BM + 32, LDB = BN + 32;
  constexpr int NA = BM * kBK / 4 / kThreads, NB = BN * kBK / 4 / kThreads;
  static_assert(NA >= 1 && NB >= 1, "tile too small for 256 threads");
  __shared__ __align__(16) float As[2][kBK * LDA];
  __shared__ __align__(16) float Bs[2][kBK * LDB];

  // Tile order: consecutive workgroups are dealt round-robin to the 8 XCDs;
  // renumber so that each XCD walks a contiguous run of tiles (tiles in a run
  // share A row panels in that XCD's L2).
  const int nblk = gridDim.x;
  int b = blockIdx.x;
  if ((nblk & 7) == 0) b = (b & 7) * (nblk >> 3) + (b >> 3);
  const int z = b / p.tiles;
  const int t = b - z * p.tiles;
  const int tm_i = t / p.tiles_n, tn_i = t - tm_i * p.tiles_n;
  const int m0 = tm_i * BM, n0 = tn_i * BN;
  const int kbeg = z * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, lh = lane >> 5;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int c = 0; c < TN; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][c][r] = 0.f;

  float4 ra[NA], rb[NB];
  if (kbeg < kend) {
    fetch<BM, AT>(p.A, p.lda, m0, p.M, kbeg, kend, p.a_vec, ra);
    fetch<BN, BT>(p.B, p.ldb, n0, p.N, kbeg, kend, p.b_vec, rb);
    stash<BM, LDA, AT>(As[0], ra);
    stash<BN, LDB, BT>(Bs[0], rb);
  }
  __syncthreads();

  int cur = 0;
  for (int k0 = kbeg; k0 < kend; k0 += kBK) {
    const bool more = k0 + kBK < kend;
    if (more) {
      fetch<BM, AT>(p.A, p.lda, m0, p.M, k0 + kBK, kend, p.a_vec, ra);
      fetch<BN, BT>(p.B, p.ldb, n0, p.N, k0 + kBK, kend, p.b_vec, rb);
    }
    const float* as = As[cur] + wm * WM + li;
    const float* bs = Bs[cur] + wn * WN + li;
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 2) {
      float av[TM], bv[TN];
#pragma unroll
      for (int a = 0; a < TM; ++a) av[a] = as[(kk + lh) * LDA + a * 32];
#pragma unroll
      for (int c = 0; c < TN; ++c) bv[c] = bs[(kk + lh) * LDB + c * 32];
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int c = 0; c < TN; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a], bv[c], acc[a][c], 0, 0, 0);
    }
    if (more) {
      stash<BM, LDA, AT>(As[cur ^ 1], ra);
      stash<BN, LDB, BT>(Bs[cur ^ 1], rb);
    }
    __syncthreads();
    cur ^= 1;
  }

  // Result layout of a 32x32 block: lane (li, lh) holds column li and rows
  // 8*(r/4) + 4*lh + r%4 for r = 0..15.
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int c = 0; c < TN; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * WM + a * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        const int col = n0 + wn * WN + c * 32 + li;
        if (row < p.M && col < p.N) {
          const float v = acc[a][c][r];
          if (p.split) {
            p.C[(int64_t)z * p.M * p.N + (int64_t)row * p.N + col] = v;
          } else {
            float* dst = p.C + (int64_t)row * p.ldc + col;
            *dst = epilogue(v, p.epi, row, col, p, p.epi == EPI_ACCUM ? *dst : 0.f);
          }
        }
      }
}

// Sum split-K partial tiles in slice order, then apply the epilogue (or the
// permuted conv weight-gradient store).
__global__ void splitk_reduce_kernel(const float* __restrict__ part, int splits, int M, int N, KArgs p,
                                     int perm_c, int perm_ci, int perm_k) {
  const int64_t MN = (int64_t)M * N;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < MN;
       idx += (int64_t)gridDim.x * blockDim.x) {
    float v = part[idx];
    for (int s = 1; s < splits; ++s) v += part[(int64_t)s * MN + idx];
    const int row = (int)(idx / N), col = (int)(idx - (int64_t)row * N);
    if (perm_c > 0) {
      if (col < perm_k) {
        const int tap = col / perm_ci, ci = col - tap * perm_ci;
        p.C[(int64_t)row * p.ldc + (int64_t)ci * perm_c * perm_c + tap] = v;
      }
    } else {
      float* dst = p.C + (int64_t)row * p.ldc + col;
      *dst = epilogue(v, p.epi, row, col, p, p.epi == EPI_ACCUM ? *dst : 0.f);
    }
  }
}

template <int BM, int BN, bool AT, bool BT>
void launch(const KArgs& a, int splits, hipStream_t s) {
  const int blocks = a.tiles * splits;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, AT, BT>), dim3(blocks), dim3(kThreads), 0, s, a);
}

// Kernel names for profiling: tile shape and operand form (nt: forward,
// tn: dedw, nn: dedx).
const char* const kNames[4][3] = {
    {"gemm_128x128_nt", "gemm_128x128_tn", "gemm_128x128_nn"},
    {"gemm_128x64_nt", "gemm_128x64_tn", "gemm_128x64_nn"},
    {"gemm_64x128_nt", "gemm_64x128_tn", "gemm_64x128_nn"},
    {"gemm_64x64_nt", "gemm_64x64_tn", "gemm_64x64_nn"},
};

template <bool AT, bool BT>
void launch_cfg(int cfg, const KArgs& a, int splits, hipStream_t s) {
  switch (cfg) {
    case 0: launch<128, 128, AT, BT>(a, splits, s); break;
    case 1: launch<128, 64, AT, BT>(a, splits, s); break;
    case 2: launch<64, 128, AT, BT>(a, splits, s); break;
    default: launch<64, 64, AT, BT>(a, splits, s); break;
  }
}

const int kCfgBM[4] = {128, 128, 64, 64};
const int kCfgBN[4] = {128, 64, 128, 64};

int pick_cfg(int M, int N) {
  // Largest tile that still gives every CU a workgroup; else the smallest.
  for (int c = 0; c < 4; ++c) {
    if ((kCfgBM[c] > 64 && M <= 64) || (kCfgBN[c] > 64 && N <= 64)) continue;
    if (ceil_div(M, kCfgBM[c]) * ceil_div(N, kCfgBN[c]) >= 256) return c;
  }
  return 3;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

int gemm_pick_splits(int M, int N, int K) {
  const int cfg = pick_cfg(M, N);
  const int64_t tiles = ceil_div(M, kCfgBM[cfg]) * ceil_div(N, kCfgBN[cfg]);
  int s = 1;
  // Aim for >= 2 workgroups per CU while keeping each K slice >= 512 long.
  while (tiles * s < 512 && K / (2 * s) >= 512 && s < 256) s *= 2;
  return s;
}

int gemm(const GemmDesc& d, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0) return 0;
  const int cfg = pick_cfg(d.M, d.N);
  KArgs a{};
  a.A = d.A;
  a.B = d.B;
  a.M = d.M;
  a.N = d.N;
  a.K = d.K;
  a.lda = d.lda;
  a.ldb = d.ldb;
  a.epi = d.epi;
  a.bias = d.bias;
  a.mask = d.mask;
  a.ldm = d.ldm;
  a.a_vec = aligned16(d.A) && d.lda % 4 == 0;
  a.b_vec = aligned16(d.B) && d.ldb % 4 == 0;
  a.tiles_n = (int)ceil_div(d.N, kCfgBN[cfg]);
  a.tiles = (int)(ceil_div(d.M, kCfgBM[cfg]) * a.tiles_n);
  const int splits = d.splits < 1 ? 1 : d.splits;
  const bool via_partial = splits > 1 || d.perm_c > 0;
  a.k_per_split = (int)round_up(ceil_div(d.K, splits), kBK);
  if (via_partial) {
    a.C = d.partial;
    a.ldc = d.N;
    a.split = 1;
  } else {
    a.C = d.C;
    a.ldc = d.ldc;
    a.split = 0;
  }
  const int form = (!d.a_t && !d.b_t) ? 0 : (d.a_t && d.b_t) ? 1 : 2;
  const double flops = d.flops > 0 ? d.flops : 2.0 * d.M * d.N * (double)d.K;
  prof_begin(kNames[cfg][form], flops, 4.0 * ((double)d.M * d.K + (double)d.K * d.N + (double)d.M * d.N), s);
  if (!d.a_t && !d.b_t) launch_cfg<false, false>(cfg, a, splits, s);
  else if (d.a_t && d.b_t) launch_cfg<true, true>(cfg, a, splits, s);
  else if (!d.a_t && d.b_t) launch_cfg<false, true>(cfg, a, splits, s);
  else launch_cfg<true, false>(cfg, a, splits, s);
  prof_end(s);
  if (int e = check_launch("gemm")) return e;
  if (via_partial) {
    KArgs r = a;
    r.C = d.C;
    r.ldc = d.ldc;
    const int64_t mn = (int64_t)d.M * d.N;
    const int blocks = (int)std::min<int64_t>(ceil_div(mn, 256), 8192);
    prof_begin("splitk_reduce", (double)(splits - 1) * mn, 4.0 * (double)(splits + 1) * mn, s);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, d.partial, splits, d.M, d.N, r,
                       d.perm_c, d.perm_ci, d.perm_k);
    prof_end(s);
    if (int e = check_launch("splitk_reduce")) return e;
  }
  return 0;
}

}  // namespace sgd
