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
// 32x32 MFMA blocks accumulated in fp32 registers.  K advances in 16-deep
// slices staged through LDS.  Two kernels share that shape:
//
// gemm_dma (the main path).  Each slice is copied global -> LDS directly by
// buffer_load_dwordx4 ... lds (16 bytes per lane, no register staging) into
// a ring of 3 LDS buffers, so two slices are in flight while the third is
// multiplied; one barrier per slice.  Lanes whose element lies outside the
// matrices get an out-of-range buffer offset and read zeros.  LDS layouts are
// XOR-swizzled so the MFMA operand reads are free of bank conflicts:
//   K-contiguous operand   [row][16], 16-byte quad q of row r stored at
//                          q ^ ((r>>1 ^ r>>3) & 3)   -> one ds_read_b128 per
//                          4 MFMAs
//   row-contiguous operand [k][R], column c of k-row k stored at
//                          c ^ (32 * ((k>>2) & 1))   -> ds_read_b32, the two
//                          lane halves (k and k+4) on disjoint banks
// Preconditions: 16-byte aligned operands and strides, K (for K-contiguous
// operands) and the row count (for row-contiguous ones) multiples of 4.
//
// gemm_staged (fallback for everything else).  Slices go through registers
// with per-element bounds checks into a padded two-buffer LDS layout.
//
// Both permute the reduction order inside a slice so a lane's four
// consecutive k values feed four consecutive MFMAs: step e of group g uses
// k = 8g + 4h + e in lane half h (the 32x32x2 instruction takes k = h from
// lane half h).
//
// Large-K products (conv dedw has K = N*Ho*Wo, up to 1.6M) are split along K:
// each slice writes its own partial tile and a second pass adds the slices in
// a fixed order, so results stay deterministic and the fp32 sums stay short.
#include <type_traits>

#include "common.h"
#include "rules.h"

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
  int perm_c, perm_ci, perm_k;  // conv weight-gradient store (see GemmDesc)
  int urule;         // >= 0: apply this update rule instead of storing the gradient
  float* ustate;     // rule state at the same offsets as C
  float* ustate_b;   // rule state of the ones column (bias)
  float eta, mu, eps;
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

// Final store of one result: the ones column to ones_out, the conv weight
// gradient permuted from [co][(ky,kx,ci)] to [co][ci][ky][kx], anything else
// through the epilogue.
// With urule >= 0 (the fused training step) the value is the parameter's
// final gradient and the update rule is applied to the parameter (and its
// state) in place of storing it.
__device__ __forceinline__ void finish(float v, int row, int col, const KArgs& p) {
  if (col == p.N) {
    if (p.urule >= 0) apply_one(p.urule, p.ones_out + row, p.ustate_b + row, v, p.eta, p.mu, p.eps);
    else p.ones_out[row] = p.accum ? p.ones_out[row] + v : v;
  } else if (p.perm_c > 0) {
    if (col < p.perm_k) {
      const int tap = col / p.perm_ci, ci = col - tap * p.perm_ci;
      const int64_t off = (int64_t)row * p.ldc + (int64_t)ci * p.perm_c * p.perm_c + tap;
      if (p.urule >= 0) apply_one(p.urule, p.C + off, p.ustate + off, v, p.eta, p.mu, p.eps);
      else p.C[off] = p.accum ? p.C[off] + v : v;
    }
  } else if (p.urule >= 0) {
    const int64_t off = (int64_t)row * p.ldc + col;
    apply_one(p.urule, p.C + off, p.ustate + off, v, p.eta, p.mu, p.eps);
  } else {
    float* dst = p.C + (int64_t)row * p.ldc + col;
    *dst = epilogue(v, p.epi, row, col, p, p.epi == EPI_ACCUM ? *dst : 0.f);
  }
}

// Write a wavefront's accumulators.  Result layout of a 32x32 block: lane
// (li, lh) holds column li and rows 8*(r/4) + 4*lh + r%4 for r = 0..15.
// Fused update of one 32x32 accumulator block whose columns are plain
// parameter columns: all 16 weight and state loads are issued before the
// rule is applied, so their latencies overlap.
template <int RULE>
__device__ __forceinline__ void update_block(const f32x16& g, const KArgs& p, int rb, int col, int lh) {
  float w[16], st[16];
  bool ok[16];
  int64_t off[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = rb + 8 * (r >> 2) + 4 * lh + (r & 3);
    ok[r] = row < p.M && col < p.N;
    off[r] = (int64_t)row * p.ldc + col;
    w[r] = ok[r] ? p.C[off[r]] : 0.f;
    st[r] = (ok[r] && RULE != SGD_PLAIN) ? p.ustate[off[r]] : 0.f;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) rule1<RULE>(w[r], st[r], g[r], p.eta, p.mu, p.eps);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (!ok[r]) continue;
    p.C[off[r]] = w[r];
    if (RULE != SGD_PLAIN) p.ustate[off[r]] = st[r];
  }
}

// FUSED: the launch applies an update rule to plain parameter columns (no
// split, no permutation); a separate instance so the other products keep
// their smaller register budget.
template <int TM, int TN, bool FUSED = false>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[TM][TN], const KArgs& p, int r0, int c0, int z, int li,
                                           int lh) {
  if (FUSED) {
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int c = 0; c < TN; ++c) {
        const int col = c0 + c * 32 + li;
        if (p.urule == SGD_PLAIN) update_block<SGD_PLAIN>(acc[a][c], p, r0 + a * 32, col, lh);
        else if (p.urule == SGD_MOMENTUM) update_block<SGD_MOMENTUM>(acc[a][c], p, r0 + a * 32, col, lh);
        else update_block<SGD_ADAGRAD>(acc[a][c], p, r0 + a * 32, col, lh);
        if (col == p.N) {  // the ones column: the bias
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = r0 + a * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
            if (row < p.M) finish(acc[a][c][r], row, col, p);
          }
        }
      }
    return;
  }
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int c = 0; c < TN; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = r0 + a * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        const int col = c0 + c * 32 + li;
        if (row >= p.M || col >= p.Nt) continue;
        const float v = acc[a][c][r];
        if (p.split) p.C[(int64_t)z * p.M * p.Nt + (int64_t)row * p.Nt + col] = v;
        else finish(v, row, col, p);
      }
}

template <int BM, int BN, int BK, bool AT, bool BT>
__global__ __launch_bounds__(kThreads) void gemm_staged(KArgs p) {
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

  store_tile<TM, TN>(acc, p, m0 + wm * WM, n0 + wn * WN, z, li, lh);
}

// ------------------------------------------------------------ gemm_dma ----
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr unsigned kOffBad = 0x80000000u;  // out-of-range buffer offset: the load returns zeros
constexpr int kDmaBK = 16;
constexpr int kDmaStages = 3;

// Buffer resource over [base, base + 2 GiB): 64-bit base, stride 0, record
// count, and the gfx9 data-format word.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = (int)(uint32_t)a;
  r.y = (int)(uint32_t)(a >> 32);
  r.z = (int)0x7ffffff0u;
  r.w = 0x00020000;
  return r;
}

// 16 bytes per lane from rsrc + voff into LDS at dst + 16 * lane.  Written as
// inline asm so the compiler's wait-count pass does not make every later LDS
// read wait for it; the kernel waits on vmcnt itself before using a stage.
__device__ __forceinline__ void dma16(i32x4 rsrc, const float* dst, uint32_t voff) {
  typedef __attribute__((address_space(3))) const float* lds_ptr_t;
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)dst);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// K-contiguous operand (stored [R][K]): LDS stage [R][16]; quad q of row r at
// slot q ^ swz(r).
template <int R>
struct DmaK {
  static constexpr int SIZE = R * kDmaBK;
  static constexpr int NI = R * (kDmaBK / 4) / 256;  // 16-byte loads per thread per stage
  __device__ static __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
  // Stage of slice kk (relative to the block's first k); rows >= rvalid and
  // k >= kvalid read zeros.
  __device__ static __forceinline__ void load(i32x4 rs, float* S, int64_t ld, int rvalid, int kk, int kvalid) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int qi = (wave * NI + j) * 64 + lane;
      const int r = qi >> 2, g = (qi & 3) ^ swz(r);
      const bool ok = r < rvalid && kk + 4 * g < kvalid;
      dma16(rs, S + (wave * NI + j) * 256, ok ? (uint32_t)(((int64_t)r * ld + kk + 4 * g) * 4) : kOffBad);
    }
  }
  __device__ static __forceinline__ float4 operand(const float* S, int row, int g, int h) {
    return *reinterpret_cast<const float4*>(&S[row * kDmaBK + 4 * ((2 * g + h) ^ swz(row))]);
  }
  __device__ static __forceinline__ void ones_fixup(float*, int, int, int, int) {}
};

// Row-contiguous operand (stored [K][R]): LDS stage [16][R]; column quad c of
// k-row k at quad c ^ swzT(k).
template <int R>
struct DmaT {
  static constexpr int Q = R / 4;
  static constexpr int SIZE = R * kDmaBK;
  static constexpr int NI = R * kDmaBK / 4 / 256;
  __device__ static __forceinline__ int swzT(int k) { return ((k >> 2) & 1) << 3; }
  __device__ static __forceinline__ void load(i32x4 rs, float* S, int64_t ld, int rvalid, int kk, int kvalid) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int qi = (wave * NI + j) * 64 + lane;
      const int k = qi / Q, c = (qi % Q) ^ swzT(k);
      const bool ok = kk + k < kvalid && 4 * c < rvalid;
      dma16(rs, S + (wave * NI + j) * 256, ok ? (uint32_t)(((int64_t)(kk + k) * ld + 4 * c) * 4) : kOffBad);
    }
  }
  __device__ static __forceinline__ float4 operand(const float* S, int col, int g, int h) {
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = 8 * g + 4 * h + e;
      v[e] = S[k * R + ((((col >> 2) ^ swzT(k))) << 2) + (col & 3)];
    }
    return make_float4(v[0], v[1], v[2], v[3]);
  }
  // The implicit ones column at tile-relative column `oc` (a multiple of 4, so
  // its quad was loaded as zeros): the lane that loaded that quad sets its
  // first element to 1 for the valid k of the stage.  Called after the lane's
  // own loads for the stage completed, before the barrier that publishes it.
  __device__ static __forceinline__ void ones_fixup(float* S, int oc, int kk, int kvalid, int /*unused*/) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int qi = (wave * NI + j) * 64 + lane;
      const int k = qi / Q, c = (qi % Q) ^ swzT(k);
      if (4 * c == oc && kk + k < kvalid) S[qi * 4] = 1.f;
    }
  }
};

template <int BM, int BN, bool AT, bool BT, bool FUSED = false>
__global__ __launch_bounds__(kThreads) void gemm_dma(KArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  using SA = typename std::conditional<AT, DmaT<BM>, DmaK<BM>>::type;
  using SB = typename std::conditional<BT, DmaT<BN>, DmaK<BN>>::type;
  constexpr int kLoads = SA::NI + SB::NI;
  __shared__ __align__(16) float As[kDmaStages][SA::SIZE];
  __shared__ __align__(16) float Bs[kDmaStages][SB::SIZE];

  // XCD-contiguous runs of tiles (see gemm_staged), tiles ordered along M
  // first so a run shares B panels.
  const int nblk = gridDim.x;
  int b = blockIdx.x;
  if ((nblk & 7) == 0) b = (b & 7) * (nblk >> 3) + (b >> 3);
  const int z = b / p.tiles;
  const int t = b - z * p.tiles;
  const int tiles_m = p.tiles / p.tiles_n;
  const int tn_i = t / tiles_m, tm_i = t - tn_i * tiles_m;
  const int m0 = tm_i * BM, n0 = tn_i * BN;
  const int kbeg = z * p.k_per_split;
  const int kval = max(0, min(p.K, kbeg + p.k_per_split) - kbeg);
  const i32x4 ra = buffer_rsrc(AT ? p.A + (int64_t)kbeg * p.lda + m0 : p.A + (int64_t)m0 * p.lda + kbeg);
  const i32x4 rb = buffer_rsrc(BT ? p.B + (int64_t)kbeg * p.ldb + n0 : p.B + (int64_t)n0 * p.ldb + kbeg);
  const int arows = p.M - m0, brows = p.N - n0;
  const int ones_col = (p.Nt > p.N && p.N >= n0 && p.N < n0 + BN) ? p.N - n0 : -1;
  const int nsl = (kval + kDmaBK - 1) / kDmaBK;

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

  // Prologue: stages 0 .. S-2 in flight.  Stages past the end of K read
  // zeros, which keeps the per-thread load count (and so the vmcnt
  // arithmetic) the same for every slice.
#pragma unroll
  for (int st = 0; st < kDmaStages - 1; ++st) {
    SA::load(ra, As[st], p.lda, arows, st * kDmaBK, kval);
    SB::load(rb, Bs[st], p.ldb, brows, st * kDmaBK, kval);
  }
  for (int i = 0; i < nsl; ++i) {
    const int cur = i % kDmaStages;
    wait_vmcnt<kLoads * (kDmaStages - 2)>();  // this thread's loads of slice i are in LDS
    if (ones_col >= 0) SB::ones_fixup(Bs[cur], ones_col, i * kDmaBK, kval, 0);
    lds_barrier();  // everyone's loads of slice i landed; everyone finished slice i-1
    const int nx = i + kDmaStages - 1;  // refill the buffer slice i-1 used
    SA::load(ra, As[nx % kDmaStages], p.lda, arows, nx * kDmaBK, kval);
    SB::load(rb, Bs[nx % kDmaStages], p.ldb, brows, nx * kDmaBK, kval);
#pragma unroll
    for (int g = 0; g < kDmaBK / 8; ++g) {
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
  }
  wait_vmcnt<0>();  // the trailing zero-fill loads must land before the workgroup ends
  store_tile<TM, TN, FUSED>(acc, p, m0 + wm * WM, n0 + wn * WN, z, li, lh);
}

// Sum split-K partial tiles in slice order, then store: the ones column to
// ones_out, the conv weight gradient permuted, anything else through the
// epilogue.
__global__ void splitk_reduce_kernel(const float* __restrict__ part, int splits, KArgs p) {
  const int64_t MN = (int64_t)p.M * p.Nt;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < MN;
       idx += (int64_t)gridDim.x * blockDim.x) {
    float v = part[idx];
    for (int s = 1; s < splits; ++s) v += part[(int64_t)s * MN + idx];
    const int row = (int)(idx / p.Nt), col = (int)(idx - (int64_t)row * p.Nt);
    finish(v, row, col, p);
  }
}

struct Cfg {
  int bm, bn, bk;
};
// gemm_staged configurations: 0: 128x128x16  1: 256x128x16  2: 128x256x16
// 3: 128x64x32  4: 64x128x32
constexpr int kStagedConfigs = 5;
const Cfg kCfg[kStagedConfigs] = {{128, 128, 16}, {256, 128, 16}, {128, 256, 16}, {128, 64, 32}, {64, 128, 32}};
// gemm_dma configurations: 0: 128x128  1: 256x128  2: 128x64  3: 64x128
constexpr int kDmaConfigs = 4;
const Cfg kDma[kDmaConfigs] = {{128, 128, kDmaBK}, {256, 128, kDmaBK}, {128, 64, kDmaBK}, {64, 128, kDmaBK}};

const char* const kNames[kStagedConfigs][3] = {
    {"gemm_staged_128x128_nt", "gemm_staged_128x128_tn", "gemm_staged_128x128_nn"},
    {"gemm_staged_256x128_nt", "gemm_staged_256x128_tn", "gemm_staged_256x128_nn"},
    {"gemm_staged_128x256_nt", "gemm_staged_128x256_tn", "gemm_staged_128x256_nn"},
    {"gemm_staged_128x64_nt", "gemm_staged_128x64_tn", "gemm_staged_128x64_nn"},
    {"gemm_staged_64x128_nt", "gemm_staged_64x128_tn", "gemm_staged_64x128_nn"},
};
const char* const kDmaNames[kDmaConfigs][3] = {
    {"gemm_dma_128x128_nt", "gemm_dma_128x128_tn", "gemm_dma_128x128_nn"},
    {"gemm_dma_256x128_nt", "gemm_dma_256x128_tn", "gemm_dma_256x128_nn"},
    {"gemm_dma_128x64_nt", "gemm_dma_128x64_tn", "gemm_dma_128x64_nn"},
    {"gemm_dma_64x128_nt", "gemm_dma_64x128_tn", "gemm_dma_64x128_nn"},
};

template <int BM, int BN, int BK, bool AT, bool BT>
void launch(const KArgs& a, int splits, hipStream_t s) {
  hipLaunchKernelGGL((gemm_staged<BM, BN, BK, AT, BT>), dim3(a.tiles * splits), dim3(kThreads), 0, s, a);
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

template <int BM, int BN, bool AT, bool BT, bool FUSED = false>
void launch_dma(const KArgs& a, int splits, hipStream_t s) {
  hipLaunchKernelGGL((gemm_dma<BM, BN, AT, BT, FUSED>), dim3(a.tiles * splits), dim3(kThreads), 0, s, a);
}

template <bool AT, bool BT, bool FUSED = false>
void launch_dma_cfg(int cfg, const KArgs& a, int splits, hipStream_t s) {
  switch (cfg) {
    case 0: launch_dma<128, 128, AT, BT, FUSED>(a, splits, s); break;
    case 1: launch_dma<256, 128, AT, BT, FUSED>(a, splits, s); break;
    case 2: launch_dma<128, 64, AT, BT, FUSED>(a, splits, s); break;
    default: launch_dma<64, 128, AT, BT, FUSED>(a, splits, s); break;
  }
}

int64_t tiles_of(const Cfg& c, int M, int N) { return ceil_div(M, c.bm) * ceil_div(N, c.bn); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Tile choice for gemm_staged, from measurements on the step's shapes.
int staged_cfg(int M, int Nt) {
  if (Nt <= 64) return 3;
  if (M <= 64) return 4;
  if (tiles_of(kCfg[0], M, Nt) >= 4096 && M >= 1024 && Nt >= 1024) return M >= Nt ? 1 : 2;
  return 0;
}

// Tile choice for gemm_dma: 128x128 unless one side of the output is narrow.
int dma_cfg(int M, int Nt) {
  if (Nt <= 64) return 2;
  if (M <= 64) return 3;
  return 0;
}

// gemm_dma preconditions: aligned operands and strides; K a multiple of 4 for
// a K-contiguous operand, the row count a multiple of 4 for a row-contiguous
// one (whole 16-byte quads are either in or out of range); the ones column at
// a quad boundary; every in-block offset below 2^31 bytes.
bool dma_ok(const GemmDesc& d, const Cfg& c, int kps) {
  auto operand_ok = [&](const float* X, int64_t ld, bool t, int rows, int tile) {
    if (!aligned16(X) || ld % 4) return false;
    if (t ? rows % 4 : d.K % 4) return false;
    const int64_t span = t ? ((int64_t)(kps - 1) * ld + tile) * 4 : ((int64_t)(tile - 1) * ld + kps) * 4;
    return span < (int64_t)kOffBad;
  };
  if (d.ones_out && d.N % 4) return false;
  return operand_ok(d.A, d.lda, d.a_t, d.M, c.bm) && operand_ok(d.B, d.ldb, d.b_t, d.N, c.bn);
}

}  // namespace

int gemm_pick_splits(int M, int Nt, int K) {
  const int64_t tiles = tiles_of(kDma[dma_cfg(M, Nt)], M, Nt);
  int s = 1;
  // Aim for >= 4 workgroups per CU while keeping each K slice >= 256 long
  // and the partial tiles' extra traffic ((s + 1) * M * Nt floats written
  // and read back) small next to the product: s <= K / 512.
  while (tiles * s < 1024 && K / (2 * s) >= 256 && 2 * s <= K / 512 && s < 256) s *= 2;
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
  a.perm_c = d.perm_c;
  a.perm_ci = d.perm_ci;
  a.perm_k = d.perm_k;
  a.urule = d.urule;
  a.ustate = d.ustate;
  a.ustate_b = d.ustate_b;
  a.eta = d.eta;
  a.mu = d.mu;
  a.eps = d.eps;
  if (d.urule >= 0 && (d.epi != EPI_STORE || d.accum)) {
    set_error("gemm: an update rule can only replace a plain store");
    return SGD_EINVAL;
  }
  a.a_vec = aligned16(d.A) && d.lda % 4 == 0;
  a.b_vec = aligned16(d.B) && d.ldb % 4 == 0;
  const int splits = d.splits < 1 ? 1 : d.splits;
  // d.cfg selects a gemm_dma configuration (0..3) or, as 4 + c, gemm_staged
  // configuration c; -1 picks from the shape, preferring gemm_dma.
  bool dma;
  int cfg;
  if (d.cfg >= 0 && d.cfg < kDmaConfigs) {
    dma = true;
    cfg = d.cfg;
  } else if (d.cfg >= kDmaConfigs && d.cfg < kDmaConfigs + kStagedConfigs) {
    dma = false;
    cfg = d.cfg - kDmaConfigs;
  } else {
    cfg = dma_cfg(d.M, a.Nt);
    dma = dma_ok(d, kDma[cfg], (int)round_up(ceil_div(d.K, splits), kDmaBK));
    if (!dma) cfg = staged_cfg(d.M, a.Nt);
  }
  const Cfg& c = dma ? kDma[cfg] : kCfg[cfg];
  a.k_per_split = (int)round_up(ceil_div(d.K, splits), c.bk);
  if (dma && !dma_ok(d, c, a.k_per_split)) {
    set_error("gemm: operands do not meet the direct-load preconditions");
    return SGD_EINVAL;
  }
  a.tiles_n = (int)ceil_div(a.Nt, c.bn);
  a.tiles = (int)(ceil_div(d.M, c.bm) * a.tiles_n);
  const bool via_partial = splits > 1;
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
  prof_begin(dma ? kDmaNames[cfg][form] : kNames[cfg][form], flops,
             4.0 * ((double)d.M * d.K + (double)d.K * d.N + (double)d.M * a.Nt), s);
  if (dma) {
    if (!d.a_t && !d.b_t) launch_dma_cfg<false, false>(cfg, a, splits, s);
    else if (d.a_t && d.b_t && d.urule >= 0 && !via_partial && d.perm_c == 0)
      launch_dma_cfg<true, true, true>(cfg, a, splits, s);
    else if (d.a_t && d.b_t) launch_dma_cfg<true, true>(cfg, a, splits, s);
    else if (!d.a_t && d.b_t) launch_dma_cfg<false, true>(cfg, a, splits, s);
    else launch_dma_cfg<true, false>(cfg, a, splits, s);
  } else {
    if (!d.a_t && !d.b_t) launch_cfg<false, false>(cfg, a, splits, s);
    else if (d.a_t && d.b_t) launch_cfg<true, true>(cfg, a, splits, s);
    else if (!d.a_t && d.b_t) launch_cfg<false, true>(cfg, a, splits, s);
    else launch_cfg<true, false>(cfg, a, splits, s);
  }
  prof_end(s);
  if (int e = check_launch("gemm")) return e;
  if (via_partial) {
    KArgs r = a;
    r.C = d.C;
    r.ldc = d.ldc;
    const int64_t mn = (int64_t)d.M * a.Nt;
    const int blocks = (int)std::min<int64_t>(ceil_div(mn, 256), 8192);
    prof_begin("splitk_reduce", (double)(splits - 1) * mn, 4.0 * (double)(splits + 1) * mn, s);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, d.partial, splits, r);
    prof_end(s);
    if (int e = check_launch("splitk_reduce")) return e;
  }
  return 0;
}

}  // namespace sgd
