// fp32 matrix products on the CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// Every conv forward, fc, dedw, dedx_fc and dedx_conv product of the SPRINT
// report's section 3.3 SGEMM table is one call of gemm() below, in one of
// three operand forms:
//   forward  C = A * B^T   A [M][K], B [N][K]   (a_t = false, b_t = false)
//   dedw     C = A^T * B   A [K][M], B [K][N]   (a_t = true,  b_t = true)
//   dedx     C = A * B     A [M][K], B [K][N]   (a_t = false, b_t = true)
// The dedb row of that table (a product with a vector of ones) is folded into
// the dedw call: B gets an implicit extra column of ones, whose results are
// the bias gradient.
//
// Kernel shape: 256 threads = 4 wavefronts of 64 lanes in a 2x2 grid over a
// BM x BN output tile; each wavefront owns a (BM/2) x (BN/2) sub-tile of
// 32x32 MFMA blocks accumulated in fp32 registers.  K advances in BK-deep
// slices staged through LDS with two buffers: the next slice is fetched into
// registers while the current one is multiplied.
//
// LDS keeps each operand in its global orientation, so every LDS write is a
// 16-byte vector store:
//   K-contiguous operand   [row][BK + 4]  -> one ds_read_b128 feeds 4 MFMAs
//   row-contiguous operand [k][row + 8]   -> one ds_read_b32 per MFMA
// The reduction order inside a slice is permuted so that a lane's four
// consecutive k values feed four consecutive MFMAs: MFMA step e of group g
// uses k = 8g + 4h + e in lane half h (the 32x32x2 instruction takes k = h
// from lane half h).  The paddings keep both read patterns free of bank
// conflicts.
//
// Large-K products (conv dedw has K = N*Ho*Wo, up to 1.6M) are split along K:
// each slice writes its own partial tile and a second pass adds the slices in
// a fixed order, so results stay deterministic and the fp32 sums stay short.
// Tiles that lie wholly inside the matrices take an unchecked load path; edge
// tiles zero-fill out-of-range elements.
#include "common.h"

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace sgd {
namespace {

constexpr int kThreads = 256;

struct KArgs {
  const float* A;
  const float* B;
  float* C;
  int M, N, K;       // N excludes the ones column
  int Nt;            // columns computed: N, or N + 1 with the ones column
  int64_t lda, ldb, ldc;
  int k_per_split;   // multiple of BK
  int split;         // 1 -> raw partials to C + z*M*Nt (row stride Nt)
  int epi;
  const float* bias;
  const float* mask;
  int64_t ldm;
  float* ones_out;   // bias-gradient output for the ones column (final store)
  int accum;         // final stores add into the destination (GradBuf += grad)
  int a_vec, b_vec;  // float4 global loads allowed (aligned base, ld % 4 == 0)
  int tiles_n;       // tiles along Nt
  int tiles;         // tiles per split
};

// One operand slice: R rows (of the output) x BK values of k.
//   T == false: stored [R][K] (row stride ld)      LDS [R][BK + 4]
//   T == true:  stored [K][R] (row stride ld)      LDS [BK][R + 8]
template <int R, int BK, bool T>
struct Slice {
  static constexpr int LD = T ? (R + 8) : (BK + 4);
  static constexpr int SIZE = T ? BK * LD : R * LD;
  static constexpr int NL = R * BK / 4 / kThreads;
  static_assert(NL >= 1, "tile too small for 256 threads");

  __device__ static __forceinline__ void coords(int j, int& r, int& k) {
    const int i = threadIdx.x + kThreads * j;
    if (!T) {
      r = i / (BK / 4);
      k = (i % (BK / 4)) * 4;
    } else {
      k = i / (R / 4);
      r = (i % (R / 4)) * 4;
    }
  }

  // Whole slice in range and vector-aligned: no checks.
  __device__ static __forceinline__ void fetch_fast(const float* __restrict__ X, int64_t ld, int r0, int k0,
                                                    float4* regs) {
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      int r, k;
      coords(j, r, k);
      const float* src = T ? X + (int64_t)(k0 + k) * ld + (r0 + r) : X + (int64_t)(r0 + r) * ld + (k0 + k);
      regs[j] = *reinterpret_cast<const float4*>(src);
    }
  }

  // Edge slice: zero outside [0, rmax) x [k0, kend); `ones` adds an implicit
  // column of ones at row index rmax (only used with T == true).
  __device__ static __forceinline__ void fetch_checked(const float* __restrict__ X, int64_t ld, int r0, int rmax,
                                                       int k0, int kend, bool vec, bool ones, float4* regs) {
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      int r, k;
      coords(j, r, k);
      const int gr = r0 + r, gk = k0 + k;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (!T) {
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
      } else if (gk < kend) {
        const float* src = X + (int64_t)gk * ld + gr;
        if (vec && gr + 3 < rmax) {
          v = *reinterpret_cast<const float4*>(src);
        } else {
          if (gr < rmax) v.x = src[0];
          else if (ones && gr == rmax) v.x = 1.f;
          if (gr + 1 < rmax) v.y = src[1];
          else if (ones && gr + 1 == rmax) v.y = 1.f;
          if (gr + 2 < rmax) v.z = src[2];
          else if (ones && gr + 2 == rmax) v.z = 1.f;
          if (gr + 3 < rmax) v.w = src[3];
          else if (ones && gr + 3 == rmax) v.w = 1.f;
        }
      }
      regs[j] = v;
    }
  }

  __device__ static __forceinline__ void stash(float* S, const float4* regs) {
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      int r, k;
      coords(j, r, k);
      *reinterpret_cast<float4*>(&S[T ? k * LD + r : r * LD + k]) = regs[j];
    }
  }

  // The four k values 8g + 4h + (0..3) of output row `row` for lane half h.
  __device__ static __forceinline__ float4 operand(const float* S, int row, int g, int h) {
    if (!T) return *reinterpret_cast<const float4*>(&S[row * LD + 8 * g + 4 * h]);
    const float* p = S + (8 * g + 4 * h) * LD + row;
    return make_float4(p[0], p[LD], p[2 * LD], p[3 * LD]);
  }
};

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

template <int BM, int BN, int BK, bool AT, bool BT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(KArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  using SA = Slice<BM, BK, AT>;
  using SB = Slice<BN, BK, BT>;
  __shared__ __align__(16) float As[2][SA::SIZE];
  __shared__ __align__(16) float Bs[2][SB::SIZE];

  // Workgroups are dealt round-robin to the 8 XCDs; renumber so each XCD
  // walks a contiguous run of tiles (neighbouring tiles share operand panels
  // in that XCD's L2).
  const int nblk = gridDim.x;
  int b = blockIdx.x;
  if ((nblk & 7) == 0) b = (b & 7) * (nblk >> 3) + (b >> 3);
  const int z = b / p.tiles;
  const int t = b - z * p.tiles;
  const int tm_i = t / p.tiles_n, tn_i = t - tm_i * p.tiles_n;
  const int m0 = tm_i * BM, n0 = tn_i * BN;
  const int kbeg = z * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const bool ones = p.Nt > p.N;
  const bool interior = p.a_vec && p.b_vec && m0 + BM <= p.M && n0 + BN <= p.N;

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

  float4 ra[SA::NL], rb[SB::NL];
  auto fetch = [&](int k0) {
    if (interior && k0 + BK <= kend) {
      SA::fetch_fast(p.A, p.lda, m0, k0, ra);
      SB::fetch_fast(p.B, p.ldb, n0, k0, rb);
    } else {
      SA::fetch_checked(p.A, p.lda, m0, p.M, k0, kend, p.a_vec, false, ra);
      SB::fetch_checked(p.B, p.ldb, n0, p.N, k0, kend, p.b_vec, ones, rb);
    }
  };

  if (kbeg < kend) {
    fetch(kbeg);
    SA::stash(As[0], ra);
    SB::stash(Bs[0], rb);
  }
  __syncthreads();

  int cur = 0;
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
    const bool more = k0 + BK < kend;
    if (more) fetch(k0 + BK);
#pragma unroll
    for (int g = 0; g < BK / 8; ++g) {
      float4 av[TM], bv[TN];
#pragma unroll
      for (int a = 0; a < TM; ++a) av[a] = SA::operand(As[cur], wm * WM + a * 32 + li, g, lh);
#pragma unroll
      for (int c = 0; c < TN; ++c) bv[c] = SB::operand(Bs[cur], wn * WN + c * 32 + li, g, lh);
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int c = 0; c < TN; ++c) {
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a].x, bv[c].x, acc[a][c], 0, 0, 0);
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a].y, bv[c].y, acc[a][c], 0, 0, 0);
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a].z, bv[c].z, acc[a][c], 0, 0, 0);
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a].w, bv[c].w, acc[a][c], 0, 0, 0);
        }
    }
    if (more) {
      SA::stash(As[cur ^ 1], ra);
      SB::stash(Bs[cur ^ 1], rb);
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
        if (row >= p.M || col >= p.Nt) continue;
        const float v = acc[a][c][r];
        if (p.split) {
          p.C[(int64_t)z * p.M * p.Nt + (int64_t)row * p.Nt + col] = v;
        } else if (col == p.N) {
          p.ones_out[row] = p.accum ? p.ones_out[row] + v : v;
        } else {
          float* dst = p.C + (int64_t)row * p.ldc + col;
          *dst = epilogue(v, p.epi, row, col, p, p.epi == EPI_ACCUM ? *dst : 0.f);
        }
      }
}

// Sum split-K partial tiles in slice order, then store: the ones column to
// ones_out, the conv weight gradient permuted, anything else through the
// epilogue.
__global__ void splitk_reduce_kernel(const float* __restrict__ part, int splits, KArgs p, int perm_c, int perm_ci,
                                     int perm_k) {
  const int64_t MN = (int64_t)p.M * p.Nt;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < MN;
       idx += (int64_t)gridDim.x * blockDim.x) {
    float v = part[idx];
    for (int s = 1; s < splits; ++s) v += part[(int64_t)s * MN + idx];
    const int row = (int)(idx / p.Nt), col = (int)(idx - (int64_t)row * p.Nt);
    if (col == p.N) {
      p.ones_out[row] = p.accum ? p.ones_out[row] + v : v;
    } else if (perm_c > 0) {
      if (col < perm_k) {
        const int tap = col / perm_ci, ci = col - tap * perm_ci;
        float* dst = p.C + (int64_t)row * p.ldc + (int64_t)ci * perm_c * perm_c + tap;
        *dst = p.accum ? *dst + v : v;
      }
    } else {
      float* dst = p.C + (int64_t)row * p.ldc + col;
      *dst = epilogue(v, p.epi, row, col, p, p.epi == EPI_ACCUM ? *dst : 0.f);
    }
  }
}

struct Cfg {
  int bm, bn, bk;
};
// 0: 128x128x16  1: 256x128x16  2: 128x256x16  3: 128x64x32  4: 64x128x32
const Cfg kCfg[kGemmConfigs] = {{128, 128, 16}, {256, 128, 16}, {128, 256, 16}, {128, 64, 32}, {64, 128, 32}};

const char* const kNames[kGemmConfigs][3] = {
    {"gemm_128x128_nt", "gemm_128x128_tn", "gemm_128x128_nn"},
    {"gemm_256x128_nt", "gemm_256x128_tn", "gemm_256x128_nn"},
    {"gemm_128x256_nt", "gemm_128x256_tn", "gemm_128x256_nn"},
    {"gemm_128x64_nt", "gemm_128x64_tn", "gemm_128x64_nn"},
    {"gemm_64x128_nt", "gemm_64x128_tn", "gemm_64x128_nn"},
};

template <int BM, int BN, int BK, bool AT, bool BT>
void launch(const KArgs& a, int splits, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, AT, BT>), dim3(a.tiles * splits), dim3(kThreads), 0, s, a);
}

template <bool AT, bool BT>
void launch_cfg(int cfg, const KArgs& a, int splits, hipStream_t s) {
  switch (cfg) {
    case 0: launch<128, 128, 16, AT, BT>(a, splits, s); break;
    case 1: launch<256, 128, 16, AT, BT>(a, splits, s); break;
    case 2: launch<128, 256, 16, AT, BT>(a, splits, s); break;
    case 3: launch<128, 64, 32, AT, BT>(a, splits, s); break;
    default: launch<64, 128, 32, AT, BT>(a, splits, s); break;
  }
}

int64_t tiles_of(int cfg, int M, int N) { return ceil_div(M, kCfg[cfg].bm) * ceil_div(N, kCfg[cfg].bn); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

// Tile choice from measurements on the step's shapes: narrow outputs (64
// columns or rows) take the 128x64 / 64x128 tiles; very large outputs with
// both sides >= 1024 (the conv dedx products) the 256-wide tiles along their
// longer side; everything else 128x128.
int gemm_pick_cfg(int M, int Nt) {
  if (Nt <= 64) return 3;
  if (M <= 64) return 4;
  if (tiles_of(0, M, Nt) >= 4096 && M >= 1024 && Nt >= 1024) return M >= Nt ? 1 : 2;
  return 0;
}

int gemm_pick_splits(int M, int Nt, int K) {
  const int64_t tiles = tiles_of(gemm_pick_cfg(M, Nt), M, Nt);
  int s = 1;
  // Aim for >= 2 workgroups per CU while keeping each K slice >= 512 long.
  while (tiles * s < 512 && K / (2 * s) >= 512 && s < 256) s *= 2;
  return s;
}

int gemm(const GemmDesc& d, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0) return 0;
  const bool ones = d.ones_out != nullptr;
  KArgs a{};
  a.A = d.A;
  a.B = d.B;
  a.M = d.M;
  a.N = d.N;
  a.Nt = d.N + (ones ? 1 : 0);
  a.K = d.K;
  a.lda = d.lda;
  a.ldb = d.ldb;
  a.epi = d.accum ? EPI_ACCUM : d.epi;
  a.bias = d.bias;
  a.mask = d.mask;
  a.ldm = d.ldm;
  a.ones_out = d.ones_out;
  a.accum = d.accum ? 1 : 0;
  a.a_vec = aligned16(d.A) && d.lda % 4 == 0;
  a.b_vec = aligned16(d.B) && d.ldb % 4 == 0;
  const int cfg = (d.cfg >= 0 && d.cfg < kGemmConfigs) ? d.cfg : gemm_pick_cfg(d.M, a.Nt);
  a.tiles_n = (int)ceil_div(a.Nt, kCfg[cfg].bn);
  a.tiles = (int)(ceil_div(d.M, kCfg[cfg].bm) * a.tiles_n);
  const int splits = d.splits < 1 ? 1 : d.splits;
  const bool via_partial = splits > 1 || d.perm_c > 0;
  a.k_per_split = (int)round_up(ceil_div(d.K, splits), kCfg[cfg].bk);
  if (via_partial) {
    a.C = d.partial;
    a.ldc = a.Nt;
    a.split = 1;
  } else {
    a.C = d.C;
    a.ldc = d.ldc;
    a.split = 0;
  }
  const int form = (!d.a_t && !d.b_t) ? 0 : (d.a_t && d.b_t) ? 1 : 2;
  if (d.accum && d.epi != EPI_STORE) {
    set_error("gemm: accumulation is only defined for plain stores");
    return SGD_EINVAL;
  }
  const double flops = d.flops > 0 ? d.flops : 2.0 * d.M * d.N * (double)d.K;
  prof_begin(kNames[cfg][form], flops, 4.0 * ((double)d.M * d.K + (double)d.K * d.N + (double)d.M * a.Nt), s);
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
    const int64_t mn = (int64_t)d.M * a.Nt;
    const int blocks = (int)std::min<int64_t>(ceil_div(mn, 256), 8192);
    prof_begin("splitk_reduce", (double)(splits - 1) * mn, 4.0 * (double)(splits + 1) * mn, s);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, d.partial, splits, r, d.perm_c,
                       d.perm_ci, d.perm_k);
    prof_end(s);
    if (int e = check_launch("splitk_reduce")) return e;
  }
  return 0;
}

}  // namespace sgd
