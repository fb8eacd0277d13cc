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
//                          q ^ ((r>>2) & 3)          -> one ds_read_b128 per
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
// gemm_dma balances the machine with a stream-K schedule: its grid holds no
// more blocks than fit on the GPU at once, blocks take whole tiles first and
// then equal contiguous runs of the remaining tiles' k-slices, and tiles
// shared between runs are finished by a fixup pass that adds the partial
// products in k order -- deterministic, and the fp32 sums of large-K
// products (conv dedw has K = N*Ho*Wo, up to 1.6M) stay short.  gemm_staged
// splits large K into slices written as partial tiles and adds them in a
// fixed order in a second pass.
#include <algorithm>
#include <climits>
#include <cmath>
#include <map>
#include <mutex>
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
  float eta, mu, eps, decay;
  float gscale;      // every final gradient value is multiplied by this (1: none)
  int a_vec, b_vec;  // float4 global loads allowed (aligned base, ld % 4 == 0)
  int tiles_n;       // tiles along Nt
  int tiles;         // tiles per split
  ConvGather cv;     // implicit-GEMM operand (see GemmDesc::gather)
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
  v = v * p.gscale;
  if (col == p.N) {
    if (p.urule >= 0) apply_one(p.urule, p.ones_out + row, p.ustate_b + row, v, p.eta, p.mu, p.eps, p.decay);
    else p.ones_out[row] = p.accum ? p.ones_out[row] + v : v;
  } else if (p.perm_c > 0) {
    if (col < p.perm_k) {
      const int tap = col / p.perm_ci, ci = col - tap * p.perm_ci;
      const int64_t off = (int64_t)row * p.ldc + (int64_t)ci * p.perm_c * p.perm_c + tap;
      if (p.urule >= 0) apply_one(p.urule, p.C + off, p.ustate + off, v, p.eta, p.mu, p.eps, p.decay);
      else p.C[off] = p.accum ? p.C[off] + v : v;
    }
  } else if (p.urule >= 0) {
    const int64_t off = (int64_t)row * p.ldc + col;
    apply_one(p.urule, p.C + off, p.ustate + off, v, p.eta, p.mu, p.eps, p.decay);
  } else {
    float* dst = p.C + (int64_t)row * p.ldc + col;
    *dst = epilogue(v, p.epi, row, col, p, p.epi == EPI_ACCUM ? *dst : 0.f);
  }
}

// finish() for rows row .. row + nrow - 1 (nrow <= 4) of one column: every
// load the epilogue needs is issued before the first store.
__device__ __forceinline__ void finish4(const float (&v)[4], int row, int nrow, int col, const KArgs& p) {
  float *dst, *stt;
  int64_t base, ld;
  const bool plain = col != p.N && p.perm_c == 0;
  if (col == p.N) {
    dst = p.ones_out;
    stt = p.ustate_b;
    base = row;
    ld = 1;
  } else {
    int64_t cb = col;
    if (p.perm_c > 0) {
      if (col >= p.perm_k) return;
      const int tap = col / p.perm_ci, ci = col - tap * p.perm_ci;
      cb = (int64_t)ci * p.perm_c * p.perm_c + tap;
    }
    dst = p.C;
    stt = p.ustate;
    base = (int64_t)row * p.ldc + cb;
    ld = p.ldc;
  }
  const bool old_c = p.urule >= 0 || (plain ? p.epi == EPI_ACCUM : p.accum);
  float aux[4] = {0.f, 0.f, 0.f, 0.f}, sv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (e >= nrow) break;
    if (old_c) aux[e] = dst[base + e * ld];
    else if (plain && p.epi == EPI_MASK) aux[e] = p.mask[(int64_t)(row + e) * p.ldm + col];
    if (p.urule == SGD_MOMENTUM || p.urule == SGD_ADAGRAD || p.urule == SGD_NESTEROV) sv[e] = stt[base + e * ld];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (e >= nrow) break;
    float x = v[e] * p.gscale;
    if (p.urule >= 0) {
      if (p.urule == SGD_PLAIN) rule1<SGD_PLAIN>(aux[e], sv[e], x, p.eta, p.mu, p.eps, p.decay);
      else if (p.urule == SGD_MOMENTUM) rule1<SGD_MOMENTUM>(aux[e], sv[e], x, p.eta, p.mu, p.eps, p.decay);
      else if (p.urule == SGD_NESTEROV) rule1<SGD_NESTEROV>(aux[e], sv[e], x, p.eta, p.mu, p.eps, p.decay);
      else rule1<SGD_ADAGRAD>(aux[e], sv[e], x, p.eta, p.mu, p.eps, p.decay);
      dst[base + e * ld] = aux[e];
      if (p.urule != SGD_PLAIN) stt[base + e * ld] = sv[e];
      continue;
    }
    if (!plain) x = p.accum ? aux[e] + x : x;
    else if (p.epi == EPI_MASK) x = aux[e] > 0.f ? x : 0.f;
    else x = epilogue(x, p.epi, row + e, col, p, aux[e]);
    dst[base + e * ld] = x;
  }
}

// Epilogue variants of gemm_dma, fixed at compile time so each instance
// carries only the code (and registers) its products need:
enum EpiMode : int {
  EM_GENERIC = 0,  // finish() per element: any combination of the options
  EM_STORE = 1,    // C = v
  EM_BIAS = 2,     // C = v + bias[col], then ReLU when epi == EPI_BIAS_RELU
  EM_MASK = 3,     // C = mask > 0 ? v : 0
  EM_DW = 4,       // dedw: ones column to ones_out, permuted conv store, accum
  EM_UPDATE = 5,   // dedw with the update rule applied in place of the store
};

// Row of result register r inside a lane's 32x32 block (the MFMA layout:
// lane (li, lh) holds column li and rows 4*lh + 8*(r/4) + r%4).
__device__ __forceinline__ int blk_row(int r) { return 8 * (r >> 2) + (r & 3); }

// Epilogue memory goes through buffer instructions whose resource starts at
// the wavefront's first row and ends after its last valid row: rows past M
// fall outside the record range (loads read 0, stores are dropped) and lanes
// past the last column use an out-of-range offset, so no per-element branch
// is needed.  The host keeps 128 rows of any epilogue operand below 2^30
// bytes, so adding a row offset to an out-of-range offset cannot wrap.
typedef __amdgpu_buffer_rsrc_t brsrc;
constexpr uint32_t kOffOut = 0x80000000u;
__device__ __forceinline__ brsrc brsrc_rows(const float* base, int rows, uint32_t ld) {
  const int64_t bytes = rows > 0 ? (int64_t)rows * ld * 4 : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0,
                                           (int)std::min<int64_t>(bytes, 0x7ffffff0), 0x00020000);
}
__device__ __forceinline__ float bload(brsrc r, uint32_t vo) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)vo, 0, 0));
}
__device__ __forceinline__ void bstore(float v, brsrc r, uint32_t vo) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)vo, 0, 0);
}

// Keeps the scheduler from hoisting the next group's loads and arithmetic
// above this point, which bounds the values in flight (and the registers the
// epilogue needs) to one group.
__device__ __forceinline__ void sched_fence() { asm volatile("" ::: "memory"); }

// Specialised epilogues of one wavefront's TM x TN blocks; r0, c0 (its first
// row and column) are wavefront-uniform.
// Byte offset of lane (li, lh)'s first element (row 4*lh of the block, its column) in a dedw result
// whose wavefront block starts at column c0: the plain column, or the permuted conv weight position;
// kOffOut for a column past N (or past the permuted store's width).
__device__ __forceinline__ uint32_t dw_lane_offset(const KArgs& p, int col, int lh, uint32_t ldc) {
  bool ok = col < p.N;
  uint32_t cb = (uint32_t)col;
  if (p.perm_c > 0) {
    ok = ok && col < p.perm_k;
    const int tap = col / p.perm_ci, ci = col - tap * p.perm_ci;
    cb = (uint32_t)(ci * p.perm_c * p.perm_c + tap);
  }
  return ok ? (4u * lh * ldc + cb) * 4u : kOffOut;
}

// ONES_ONLY (dedw forms): only the ones column's results (the bias), when it falls in the wavefront's
// blocks; the weight block was stored by store_wave_pre.
template <int TM, int TN, int EM, bool ONES_ONLY = false>
__device__ __forceinline__ void store_wave(const f32x16 (&acc)[TM][TN], const KArgs& p, int r0, int c0, int li,
                                           int lh) {
  const int rows = min(p.M - r0, TM * 32);
  if (EM == EM_STORE || EM == EM_BIAS || EM == EM_MASK) {
    const uint32_t ldc = (uint32_t)p.ldc, ldm = (uint32_t)p.ldm;
    const brsrc rc = brsrc_rows(p.C + (int64_t)r0 * p.ldc + c0, rows, ldc);
    const brsrc rm = brsrc_rows(EM == EM_MASK ? p.mask + (int64_t)r0 * p.ldm + c0 : p.C, EM == EM_MASK ? rows : 0, ldm);
#pragma unroll
    for (int c = 0; c < TN; ++c) {
      const int col = c0 + c * 32 + li;
      const bool ok = col < p.N;
      const uint32_t vc = ok ? (4u * lh * ldc + c * 32 + li) * 4u : kOffOut;
      const uint32_t vm = ok ? (4u * lh * ldm + c * 32 + li) * 4u : kOffOut;
      const float bias = (EM == EM_BIAS && ok) ? p.bias[col] : 0.f;
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        float m[16];
        if (EM == EM_MASK) {
#pragma unroll
          for (int r = 0; r < 16; ++r) m[r] = bload(rm, vm + (a * 32 + blk_row(r)) * ldm * 4u);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = acc[a][c][r];
          if (EM == EM_BIAS) {
            x = x + bias;
            if (p.epi == EPI_BIAS_RELU) x = x <= 0.f ? 0.f : x;  // NaN passes through
          }
          if (EM == EM_MASK) x = m[r] > 0.f ? x : 0.f;
          bstore(x, rc, vc + (a * 32 + blk_row(r)) * ldc * 4u);
        }
        sched_fence();
      }
    }
  } else if (EM == EM_DW || EM == EM_UPDATE) {
    const uint32_t ldc = (uint32_t)p.ldc;
    const brsrc rd = brsrc_rows(p.C + (int64_t)r0 * p.ldc, rows, ldc);
    const bool st_on = EM == EM_UPDATE && p.ustate;
    const brsrc rs = brsrc_rows(st_on ? p.ustate + (int64_t)r0 * p.ldc : p.C, st_on ? rows : 0, ldc);
    const brsrc rdb = brsrc_rows(p.ones_out ? p.ones_out + r0 : p.C, p.ones_out ? rows : 0, 1);
    const brsrc rsb = brsrc_rows(EM == EM_UPDATE && p.ustate_b ? p.ustate_b + r0 : p.C,
                                 EM == EM_UPDATE && p.ustate_b ? rows : 0, 1);
    // Blocks of 8 rows of one lane's column: parameter (and state) loads
    // first, then the rule or the accumulation, then the stores.
    auto rows8 = [&](auto rule_c, const f32x16& v, int h, int a, brsrc d, brsrc st_r, uint32_t vo, uint32_t ld) {
      constexpr int RULE = decltype(rule_c)::value;  // -1: plain store (with accum)
      float w[8], st[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t o = vo + (a * 32 + blk_row(8 * h + e)) * ld * 4u;
        w[e] = (RULE >= 0 || p.accum) ? bload(d, o) : 0.f;
        st[e] = (RULE == SGD_MOMENTUM || RULE == SGD_ADAGRAD || RULE == SGD_NESTEROV) ? bload(st_r, o) : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (RULE >= 0) {
          rule1<(RULE >= 0 ? RULE : 0)>(w[e], st[e], v[8 * h + e], p.eta, p.mu, p.eps, p.decay);
        } else {
          const float x = v[8 * h + e] * p.gscale;
          w[e] = p.accum ? w[e] + x : x;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t o = vo + (a * 32 + blk_row(8 * h + e)) * ld * 4u;
        bstore(w[e], d, o);
        if (RULE == SGD_MOMENTUM || RULE == SGD_ADAGRAD || RULE == SGD_NESTEROV) bstore(st[e], st_r, o);
      }
      sched_fence();
    };
    auto block = [&](const f32x16& v, int a, brsrc d, brsrc st_r, uint32_t vo, uint32_t ld) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (EM == EM_DW) rows8(std::integral_constant<int, -1>{}, v, h, a, d, st_r, vo, ld);
        else if (p.urule == SGD_PLAIN) rows8(std::integral_constant<int, SGD_PLAIN>{}, v, h, a, d, st_r, vo, ld);
        else if (p.urule == SGD_MOMENTUM) rows8(std::integral_constant<int, SGD_MOMENTUM>{}, v, h, a, d, st_r, vo, ld);
        else if (p.urule == SGD_NESTEROV) rows8(std::integral_constant<int, SGD_NESTEROV>{}, v, h, a, d, st_r, vo, ld);
        else rows8(std::integral_constant<int, SGD_ADAGRAD>{}, v, h, a, d, st_r, vo, ld);
      }
    };
#pragma unroll
    for (int c = 0; c < TN; ++c) {
      const int col = c0 + c * 32 + li;
      // Plain or permuted conv weight columns.
      const uint32_t vo = dw_lane_offset(p, col, lh, ldc);
      if (!ONES_ONLY && c0 + c * 32 < p.N) {
#pragma unroll
        for (int a = 0; a < TM; ++a) block(acc[a][c], a, rd, rs, vo, ldc);
      }
      // The ones column (bias) when it falls in this block.
      if (p.ones_out && p.N >= c0 + c * 32 && p.N < c0 + c * 32 + 32) {
        const uint32_t vb = col == p.N ? 4u * lh * 4u : kOffOut;
#pragma unroll
        for (int a = 0; a < TM; ++a) block(acc[a][c], a, rdb, rsb, vb, 1);
      }
    }
  }
}

// Small-tile dedw epilogue with its memory operands loaded ahead (one 32x32 block per wavefront).
// When a weight-gradient product has only a few k-slices per tile (an fc layer's dedw has k = the
// batch), the product is short next to the round trips of its epilogue: the parameters and rule
// state the wavefront updates (or the GradBuf values it adds to) are therefore loaded by
// prefetch_params before the item's operand loads, so their latency overlaps the main loop, and
// store_wave_pre finishes the block from those registers.  The ones column (bias) is finished by
// store_wave<..., ONES_ONLY> with its own loads.
template <int EM>
__device__ __forceinline__ void prefetch_params(const KArgs& p, int r0, int c0, int li, int lh, float (&w)[16],
                                                float (&st)[16]) {
  const uint32_t ldc = (uint32_t)p.ldc;
  const int rows = min(p.M - r0, 32);
  const bool w_on = EM == EM_UPDATE || p.accum;
  const bool st_on = EM == EM_UPDATE && p.ustate &&
                     (p.urule == SGD_MOMENTUM || p.urule == SGD_ADAGRAD || p.urule == SGD_NESTEROV);
  const brsrc rd = brsrc_rows(p.C + (int64_t)r0 * p.ldc, w_on ? rows : 0, ldc);
  const brsrc rs = brsrc_rows(st_on ? p.ustate + (int64_t)r0 * p.ldc : p.C, st_on ? rows : 0, ldc);
  const uint32_t vo = c0 < p.N ? dw_lane_offset(p, c0 + li, lh, ldc) : kOffOut;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint32_t o = vo + blk_row(r) * ldc * 4u;
    w[r] = bload(rd, o);
    st[r] = bload(rs, o);
  }
}

template <int EM>
__device__ __forceinline__ void store_wave_pre(const f32x16 (&acc)[1][1], const KArgs& p, int r0, int c0, int li,
                                               int lh, float (&w)[16], float (&st)[16]) {
  if (c0 < p.N) {
    const uint32_t ldc = (uint32_t)p.ldc;
    const int rows = min(p.M - r0, 32);
    const bool st_on = EM == EM_UPDATE && p.ustate;
    const brsrc rd = brsrc_rows(p.C + (int64_t)r0 * p.ldc, rows, ldc);
    const brsrc rs = brsrc_rows(st_on ? p.ustate + (int64_t)r0 * p.ldc : p.C, st_on ? rows : 0, ldc);
    const uint32_t vo = dw_lane_offset(p, c0 + li, lh, ldc);
    const f32x16& v = acc[0][0];
    auto finish16 = [&](auto rule_c) {
      constexpr int RULE = decltype(rule_c)::value;  // -1: store (with accumulation)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t o = vo + blk_row(r) * ldc * 4u;
        if (RULE >= 0) {
          rule1<(RULE >= 0 ? RULE : 0)>(w[r], st[r], v[r], p.eta, p.mu, p.eps, p.decay);
        } else {
          const float x = v[r] * p.gscale;
          w[r] = p.accum ? w[r] + x : x;
        }
        bstore(w[r], rd, o);
        if (RULE == SGD_MOMENTUM || RULE == SGD_ADAGRAD || RULE == SGD_NESTEROV) bstore(st[r], rs, o);
      }
    };
    if (EM == EM_DW) finish16(std::integral_constant<int, -1>{});
    else if (p.urule == SGD_PLAIN) finish16(std::integral_constant<int, SGD_PLAIN>{});
    else if (p.urule == SGD_MOMENTUM) finish16(std::integral_constant<int, SGD_MOMENTUM>{});
    else if (p.urule == SGD_NESTEROV) finish16(std::integral_constant<int, SGD_NESTEROV>{});
    else finish16(std::integral_constant<int, SGD_ADAGRAD>{});
  }
  store_wave<1, 1, EM, true>(acc, p, r0, c0, li, lh);
}

// Generic epilogue: each 32x32 block of a wavefront is parked in the
// wavefront's own 1024 floats of LDS (`wl`) and finished by a short loop, so
// the code holds one finish() per block instead of one per element (an
// unrolled per-element finish() runs to tens of KiB of instructions that
// every wavefront fetches cold).  The caller makes sure no other wavefront
// still reads that LDS.
template <int TM, int TN>
__device__ __forceinline__ void store_tile_generic(const f32x16 (&acc)[TM][TN], const KArgs& p, int r0, int c0, int z,
                                                   int li, int lh, float* wl) {
  const int lane = li + 32 * lh;
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int c = 0; c < TN; ++c) {
#pragma unroll
      for (int r = 0; r < 16; ++r) wl[(4 * lh + blk_row(r)) * 32 + li] = acc[a][c][r];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the block is in LDS before any lane reads it
#pragma unroll 1
      for (int e = 0; e < 16; ++e) {
        const int k = e * 64 + lane;  // rows 2e, 2e+1 of the block: lanes cover 32 consecutive columns
        const int row = r0 + a * 32 + (k >> 5), col = c0 + c * 32 + (k & 31);
        const float v = wl[k];
        if (row < p.M && col < p.Nt) {
          if (p.split) p.C[(int64_t)z * p.M * p.Nt + (int64_t)row * p.Nt + col] = v;
          else finish(v, row, col, p);
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next block is parked
    }
}

template <int BM, int BN, int BK, bool AT, bool BT, int EM>
__global__ __launch_bounds__(kThreads) void gemm_staged(KArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  using SA = Slice<BM, BK, AT>;
  using SB = Slice<BN, BK, BT>;
  __shared__ __align__(16) float lds[2 * (SA::SIZE + SB::SIZE)];
  static_assert(2 * (SA::SIZE + SB::SIZE) >= 4 * 1024, "LDS too small for the generic epilogue");
  float(*As)[SA::SIZE] = reinterpret_cast<float(*)[SA::SIZE]>(lds);
  float(*Bs)[SB::SIZE] = reinterpret_cast<float(*)[SB::SIZE]>(lds + 2 * SA::SIZE);

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

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // uniform in the wavefront
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

  if (EM == EM_GENERIC) store_tile_generic<TM, TN>(acc, p, m0 + wm * WM, n0 + wn * WN, z, li, lh, lds + wave * 1024);
  else store_wave<TM, TN, EM>(acc, p, m0 + wm * WM, n0 + wn * WN, li, lh);
}

// ------------------------------------------------------------ gemm_dma ----
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr unsigned kOffBad = 0x80000000u;  // out-of-range buffer offset: the load returns zeros
constexpr int kDmaBK = 16;
constexpr int kDmaStages = 3;
// Schedule choices that can be switched off as a whole (each is measured against its absence in the
// design notes): the pipelined slice loop (gemm_dma), the grouped stream-K form (sk_group) and the
// edge-tiles-last order (edge_last_coords).  Results do not depend on the last, and the first keeps the
// products' order; grouping changes where k is cut.
constexpr bool pipe_slices = true;
// Weight gradients with at most this many k-slices per tile (k <= 128: an fc layer's dedw at batch
// <= 128) take 64x64 tiles and load their epilogue's memory operands ahead of the main loop.
constexpr int kPrefetchSlices = 8;

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
// slot q ^ swz(r).  `rs` addresses the work item's first element; the host
// keeps every offset inside an item below 2^31 bytes.
template <int R>
struct DmaK {
  static constexpr int SIZE = R * kDmaBK;
  static constexpr int NI = R * (kDmaBK / 4) / 256;  // 16-byte loads per thread per stage
  __device__ static __forceinline__ int swz(int r) { return (r >> 2) & 3; }
  // Slice at k offset kk of the item; rows >= rvalid and k >= kvalid read zeros.
  __device__ static __forceinline__ void load(i32x4 rs, float* S, uint32_t ld, int rvalid, int kk, int kvalid) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int qi = (wave * NI + j) * 64 + lane;
      const int r = qi >> 2, g = (qi & 3) ^ swz(r);
      const bool ok = r < rvalid && kk + 4 * g < kvalid;
      dma16(rs, S + (wave * NI + j) * 256, ok ? ((uint32_t)r * ld + (uint32_t)(kk + 4 * g)) * 4u : kOffBad);
    }
  }
  __device__ static __forceinline__ float4 operand(const float* S, int row, int g, int h) {
    return *reinterpret_cast<const float4*>(&S[row * kDmaBK + 4 * ((2 * g + h) ^ swz(row))]);
  }
  __device__ static __forceinline__ void ones_fixup(float*, int, int, int) {}
};

// Row-contiguous operand (stored [K][R]): LDS stage [16][R]; column quad c of
// k-row k at quad c ^ swzT(k).
template <int R>
struct DmaT {
  static constexpr int Q = R / 4;
  static constexpr int SIZE = R * kDmaBK;
  static constexpr int NI = R * kDmaBK / 4 / 256;
  __device__ static __forceinline__ int swzT(int k) { return ((k >> 2) & 1) << 3; }
  __device__ static __forceinline__ void load(i32x4 rs, float* S, uint32_t ld, int rvalid, int kk, int kvalid) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int qi = (wave * NI + j) * 64 + lane;
      const int k = qi / Q, c = (qi % Q) ^ swzT(k);
      const bool ok = kk + k < kvalid && 4 * c < rvalid;
      dma16(rs, S + (wave * NI + j) * 256, ok ? ((uint32_t)(kk + k) * ld + (uint32_t)(4 * c)) * 4u : kOffBad);
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
  // first element to 1 for the valid k of the slice.  Called after the lane's
  // own loads for the slice completed, before the barrier that publishes it.
  __device__ static __forceinline__ void ones_fixup(float* S, int oc, int kk, int kvalid) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int qi = (wave * NI + j) * 64 + lane;
      const int k = qi / Q, c = (qi % Q) ^ swzT(k);
      if (4 * c == oc && kk + k < kvalid) S[qi * 4] = 1.f;
    }
  }
};

// ---- implicit-GEMM operands: convolution windows gathered straight from an
// NHWC activation tensor (no im2col matrix in HBM).
//
// Row index q of the product runs over a pixel grid RH x RW (per image);
// column/k index (ky*c + kx)*SC + ch selects channel ch of source pixel
// (y + dy, x + dx) of the SH x SW x SC source, dy = ky - P (dy = P - ky when
// `flip`, the dedx gather), zero outside the source.

// q / d for 0 <= q < 2^22 from a float reciprocal, corrected to exact.
__device__ __forceinline__ int fdiv(int q, int d, float inv) {
  int r = (int)((float)q * inv);
  const int rem = q - r * d;
  r += (rem >= d) - (rem < 0);
  return r;
}

// K-contiguous gather (the A operand of conv forward and of dedx): LDS
// layout and operand reads as DmaK.  A 16-deep k-slice lies inside one tap
// (SC % 16 == 0), so each row's slice is 64 contiguous bytes of one source
// pixel.
template <int R>
struct DmaKg : DmaK<R> {
  using Base = DmaK<R>;
  static constexpr int NI = Base::NI;
  struct Item {
    i32x4 rs;
    int base[NI];  // first channel of the row's image in the source (floats)
    int y[NI], x[NI];
    int kbeg;
  };
  __device__ static __forceinline__ Item prep(const ConvGather& g, int m0, int rvalid, int kbeg) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    Item it;
    it.rs = buffer_rsrc(g.src);
    it.kbeg = kbeg;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int r = ((wave * NI + j) * 64 + lane) >> 2;
      const int q = m0 + r;
      const int t = fdiv(q, g.RW, g.inv_RW);
      const int n = fdiv(t, g.RH, g.inv_RH);
      it.x[j] = q - t * g.RW;
      it.y[j] = r < rvalid ? t - n * g.RH : -(1 << 20);  // rows past M read zeros
      it.base[j] = n * g.SH * g.SW * g.SC;
    }
    return it;
  }
  __device__ static __forceinline__ void load(const Item& it, const ConvGather& g, float* S, int kk, int kvalid) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ka = it.kbeg + kk;
    const int tap = ka / g.SC, ch0 = ka - tap * g.SC;
    const int ky = tap / g.c, kx = tap - ky * g.c;
    const int dy = g.flip ? g.P - ky : ky - g.P;
    const int dx = g.flip ? g.P - kx : kx - g.P;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int qi = (wave * NI + j) * 64 + lane;
      const int r = qi >> 2, q4 = (qi & 3) ^ Base::swz(r);
      const int sy = it.y[j] + dy, sx = it.x[j] + dx;
      const bool ok = kk + 4 * q4 < kvalid && (unsigned)sy < (unsigned)g.SH && (unsigned)sx < (unsigned)g.SW;
      const uint32_t off = (uint32_t)(it.base[j] + (sy * g.SW + sx) * g.SC + ch0 + 4 * q4) * 4u;
      dma16(it.rs, S + (wave * NI + j) * 256, ok ? off : kOffBad);
    }
  }
};

// Row-contiguous gather (the B operand of conv dedw, Col viewed as [pixel]
// [(ky,kx,ch)]): LDS layout, operand reads and the ones-column fix-up as
// DmaT.  A 4-column quad lies inside one tap (SC % 4 == 0).
template <int R>
struct DmaTg : DmaT<R> {
  using Base = DmaT<R>;
  static constexpr int NI = Base::NI;
  struct Item {
    i32x4 rs;
    int ch[NI], dy[NI], dx[NI];  // the quad's channel and tap offset; dy < -2^19: column past N
    int kbeg;
  };
  __device__ static __forceinline__ Item prep(const ConvGather& g, int n0, int rvalid, int kbeg) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    Item it;
    it.rs = buffer_rsrc(g.src);
    it.kbeg = kbeg;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int qi = (wave * NI + j) * 64 + lane;
      const int k = qi / Base::Q, c4 = (qi % Base::Q) ^ Base::swzT(k);
      const int col = n0 + 4 * c4;
      const int tap = col / g.SC;
      const int ky = tap / g.c, kx = tap - ky * g.c;
      it.ch[j] = col - tap * g.SC;
      it.dy[j] = 4 * c4 < rvalid ? ky - g.P : -(1 << 20);
      it.dx[j] = kx - g.P;
    }
    return it;
  }
  __device__ static __forceinline__ void load(const Item& it, const ConvGather& g, float* S, int kk, int kvalid) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int qi = (wave * NI + j) * 64 + lane;
      const int k = qi / Base::Q;
      const int q = it.kbeg + kk + k;  // pixel of this k-row
      const int t = fdiv(q, g.RW, g.inv_RW);
      const int n = fdiv(t, g.RH, g.inv_RH);
      const int sy = t - n * g.RH + it.dy[j], sx = q - t * g.RW + it.dx[j];
      const bool ok = kk + k < kvalid && (unsigned)sy < (unsigned)g.SH && (unsigned)sx < (unsigned)g.SW;
      const uint32_t off = (uint32_t)(((n * g.SH + sy) * g.SW + sx) * g.SC + it.ch[j]) * 4u;
      dma16(it.rs, S + (wave * NI + j) * 256, ok ? off : kOffBad);
    }
  }
};

// Stream-K schedule of one gemm_dma launch.  Blocks first take whole tiles
// round-robin (tiles [0, dp_tiles)); the k-slices of the remaining tiles,
// flattened tile by tile, are then cut into gridDim.x equal contiguous
// ranges, one per block, so every block ends after the same amount of work
// however the tile count divides the machine.  A range that covers a whole
// tile stores it directly; a tile shared by several ranges is written by
// each as a partial product to that block's slot (2b for the tile its range
// starts in, 2b + 1 for the tile it ends in) and gemm_sk_fixup adds the slots
// in k order before the epilogue, so results do not depend on timing.
//
// Grouped form (rg * cg > 1; no whole tiles first): a product only a few tiles
// tall (rg = its tile rows) is cut along k the same way, but the flattened
// space is (group of cg tile columns, k-slice), and gridDim.x / (rg * cg)
// ranges are each run by rg * cg blocks at once, one per tile of the group.
// The group's blocks are consecutive after the XCD renumbering, so they run
// on one XCD at the same time over the same k-slices: each A slice is read by
// cg blocks and each B slice by rg blocks, and all but the first read of a
// slice hit that XCD's L2 (the ungrouped order reads an operand panel once per
// tile, at a different time for each).  Slots and the fixup's k order follow
// the group's range, with the block's own index for the slot.
struct SkArgs {
  int ipt;           // k-slices per tile: ceil(K / 16)
  int dp_tiles;      // tiles done whole before the stream-K part (0 if grouped)
  int sk_iters;      // ungrouped: (tiles - dp_tiles) * ipt; grouped: tiles_n / cg * ipt.
                     // 0 or >= the number of ranges, and sk_iters * gridDim.x < 2^31
                     // (32-bit range arithmetic)
  float* part;       // 2 * gridDim.x slots of BM * BN floats
  int rg = 1, cg = 1;  // block group: rg tile rows (all of them) by cg tile columns
  int edge_last = 0;   // one block per tile: the ragged last tile row (bit 0) and column (bit 1) go last
};

__host__ __device__ inline int sk_start(int b, int S, int G) { return (int)((uint32_t)b * (uint32_t)S / (uint32_t)G); }

// The block whose range holds stream-K slice x.
__host__ __device__ inline int sk_block_of(int x, int S, int G) {
  int b = (int)(((uint32_t)x * (uint32_t)G + (uint32_t)G - 1u) / (uint32_t)S);
  while (b > 0 && sk_start(b, S, G) > x) --b;
  while (b + 1 < G && sk_start(b + 1, S, G) <= x) ++b;
  return b;
}

// Partial-slot layout: float4 (wave, a, c, q) of lane l at
// ((((wave * TM + a) * TN + c) * 4 + q) * 64 + l) * 4 -- every store and load
// instruction covers 1 KiB contiguously.
template <int TM, int TN>
__device__ __forceinline__ int64_t slot_index(int wave, int a, int c, int q, int lane) {
  return ((((int64_t)(wave * TM + a) * TN + c) * 4 + q) * 64 + lane) * 4;
}

// Tile t of a gemm_dma product.  A product more than kBandN tiles wide is
// ordered in bands of kBandN tile columns, along N first within a band, so
// an XCD's run of consecutive tiles (about 96 resident at once) reads about
// 12 A and 8 B panels rather than one A panel per tile.  Narrower products
// and conv weight gradients (permuted stores) run along M: the bands made
// the VGG networks' steps no faster and VGG-CIFAR's slower.  The stream-K
// fixup uses the same order.
constexpr int kBandN = 8;
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, bool banded, int& tm_i, int& tn_i) {
  if (!banded || tiles_n <= kBandN) {
    tn_i = t / tiles_m;
    tm_i = t - tn_i * tiles_m;
    return;
  }
  const int band = t / (tiles_m * kBandN);
  const int in_band = t - band * tiles_m * kBandN;
  const int cols = min(kBandN, tiles_n - band * kBandN);
  tm_i = in_band / cols;
  tn_i = band * kBandN + (in_band - tm_i * cols);
}

// Tile of block b in a launch of one block per tile with more tiles than
// resident blocks and a ragged last tile row and/or column (bits 0 and 1 of
// ragged).  The edge tiles carry a fraction of the matrix-core work (their
// blocks outside the output skip it), so each XCD's run of blocks takes its
// share of the interior tiles first, in tile_coords order over the interior,
// and its share of the edge tiles (last column, then last row) at the end:
// the launch's last, partly filled round of resident blocks then holds light
// tiles rather than full ones.
__device__ __forceinline__ void edge_last_coords(int b, int G, int tiles_m, int tiles_n, bool banded, int ragged,
                                                 int& tm_i, int& tn_i) {
  const int runs = (G & 7) == 0 ? 8 : 1, R = G / runs;  // the XCD runs of the renumbering below
  const int x = b / R, j = b - x * R;
  const int rowr = ragged & 1, colr = ragged >> 1;
  const int im = tiles_m - rowr, in_ = tiles_n - colr;
  const int ne = G - im * in_;
  const int e0 = x * ne / runs, ix = R - ((x + 1) * ne / runs - e0);
  if (j < ix) {
    tile_coords(x * R - e0 + j, im, in_, banded, tm_i, tn_i);
    return;
  }
  const int e = e0 + j - ix;
  if (e < colr * im) {
    tm_i = e;
    tn_i = tiles_n - 1;
  } else {
    tm_i = tiles_m - 1;
    tn_i = e - colr * im;
  }
}

// GA: the A operand is a K-contiguous convolution gather (DmaKg); GB: the B
// operand is a row-contiguous one (DmaTg).
// WR: rows of wavefronts (2: a 2 x 2 layout; 1: 1 x 4, each wavefront over all BM rows and a quarter of
// the columns, for products of at most 32 rows, whose second row of wavefronts would have no rows).
template <int BM, int BN, bool AT, bool BT, int EM, bool GA = false, bool GB = false, bool PIPE = false, int WR = 2>
__global__ __launch_bounds__(kThreads) void gemm_dma(KArgs p, SkArgs s) {
  constexpr int WC = 4 / WR;
  constexpr int WM = BM / WR, WN = BN / WC;
  constexpr int TM = WM / 32, TN = WN / 32;
  static_assert(!(GA && AT) && !(GB && !BT), "gathers: K-contiguous A, row-contiguous B");
  using SA = typename std::conditional<GA, DmaKg<BM>, typename std::conditional<AT, DmaT<BM>, DmaK<BM>>::type>::type;
  using SB = typename std::conditional<GB, DmaTg<BN>, typename std::conditional<BT, DmaT<BN>, DmaK<BN>>::type>::type;
  constexpr int kLoads = SA::NI + SB::NI;
  __shared__ __align__(16) float lds[kDmaStages * (SA::SIZE + SB::SIZE)];
  static_assert(kDmaStages * (SA::SIZE + SB::SIZE) >= 4 * 1024, "LDS too small for the generic epilogue");
  float(*As)[SA::SIZE] = reinterpret_cast<float(*)[SA::SIZE]>(lds);
  float(*Bs)[SB::SIZE] = reinterpret_cast<float(*)[SB::SIZE]>(lds + kDmaStages * SA::SIZE);

  // Blocks are dealt round-robin to the 8 XCDs; renumber so each XCD holds a
  // contiguous run of block indices, i.e. neighbouring tiles (which share
  // operand panels in that XCD's L2), in the band order of tile_coords.
  const int G = gridDim.x;
  int b = blockIdx.x;
  if ((G & 7) == 0) b = (b & 7) * (G >> 3) + (b >> 3);
  const int tiles_m = p.tiles / p.tiles_n;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // uniform in the wavefront
  const int wm = wave / WC, wn = wave % WC;
  const int li = lane & 31, lh = lane >> 5;
  f32x16 acc[TM][TN];

  // Work items: whole tiles b, b + G, ... below dp_tiles, then the block's
  // stream-K range, tile by tile.  One store site keeps the epilogue's code
  // (and registers) out of the pipelined loop.
  const int S = s.sk_iters;
  const int gsz = s.rg * s.cg;  // 1 when ungrouped
  const int grp = b / gsz, g_r = (b - grp * gsz) / s.cg, g_c = b - grp * gsz - g_r * s.cg;
  const int Q = G / gsz;
  int it = S > 0 ? sk_start(grp, S, Q) : 0;
  const int end = S > 0 ? sk_start(grp + 1, S, Q) : 0;
  int t_next = b;
  bool first_sk = true;
  for (;;) {
    int k0, k1, slot = -1;
    int tm_i, tn_i;
    if (t_next < s.dp_tiles) {
      if (s.edge_last) edge_last_coords(t_next, G, tiles_m, p.tiles_n, p.perm_c == 0, s.edge_last, tm_i, tn_i);
      else tile_coords(t_next, tiles_m, p.tiles_n, p.perm_c == 0, tm_i, tn_i);
      k0 = 0;
      k1 = s.ipt;
      t_next += G;
    } else if (it < end) {
      const int tt = (int)((uint32_t)it / (uint32_t)s.ipt);
      k0 = it - tt * s.ipt;
      k1 = min(s.ipt, k0 + (end - it));
      if (gsz == 1) {
        tile_coords(s.dp_tiles + tt, tiles_m, p.tiles_n, p.perm_c == 0, tm_i, tn_i);
      } else {
        tm_i = g_r;
        tn_i = tt * s.cg + g_c;
      }
      it += k1 - k0;
      slot = first_sk ? 2 * b : 2 * b + 1;
      first_sk = false;
    } else {
      break;
    }
    const int m0 = tm_i * BM, n0 = tn_i * BN;
    const int kbeg = k0 * kDmaBK;
    const int kval = min(p.K, k1 * kDmaBK) - kbeg;
    const int nsl = k1 - k0;
    const int arows = p.M - m0, brows = p.N - n0;
    const int ones_col = (p.Nt > p.N && p.N >= n0 && p.N < n0 + BN) ? p.N - n0 : -1;
    // The wavefront's 32 x 32 blocks that lie wholly outside the output (in the ragged last tile row
    // or column) skip their matrix-core work: nothing stores them, and the matrix cores they would
    // occupy are shared with the other resident blocks.  (128 x 128 tiles, and the 1 x 4 layout, whose
    // wavefronts all span the tile's rows: a product of at most 32 rows skips their second block.  In
    // the other narrow instances the second loop copy costs the registers of a fourth wavefront per SIMD.)
    constexpr bool kSkip = (TM == 2 && TN == 2) || (WR == 1 && TM == 2);
    constexpr bool kPipe = PIPE && kSkip && !AT && EM != EM_UPDATE && EM != EM_GENERIC;
    const int na = kSkip ? __builtin_amdgcn_readfirstlane(min(TM, max(0, (arows - wm * WM + 31) >> 5))) : TM;
    const int nc = kSkip ? __builtin_amdgcn_readfirstlane(min(TN, max(0, (p.Nt - n0 - wn * WN + 31) >> 5))) : TN;
    const i32x4 ra = buffer_rsrc(GA ? p.A : AT ? p.A + (int64_t)kbeg * p.lda + m0 : p.A + (int64_t)m0 * p.lda + kbeg);
    const i32x4 rb = buffer_rsrc(GB ? p.B : BT ? p.B + (int64_t)kbeg * p.ldb + n0 : p.B + (int64_t)n0 * p.ldb + kbeg);
    const uint32_t lda = (uint32_t)p.lda, ldb = (uint32_t)p.ldb;
    typename DmaKg<BM>::Item ga{};
    typename DmaTg<BN>::Item gb{};
    if constexpr (GA) ga = DmaKg<BM>::prep(p.cv, m0, arows, kbeg);
    if constexpr (GB) gb = DmaTg<BN>::prep(p.cv, n0, brows, kbeg);
    auto load_a = [&](float* S, int kk) {
      if constexpr (GA) DmaKg<BM>::load(ga, p.cv, S, kk, kval);
      else SA::load(ra, S, lda, arows, kk, kval);
    };
    auto load_b = [&](float* S, int kk) {
      if constexpr (GB) DmaTg<BN>::load(gb, p.cv, S, kk, kval);
      else SB::load(rb, S, ldb, brows, kk, kval);
    };

#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int c = 0; c < TN; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][c][r] = 0.f;
    // One 32x32 block per wavefront and a short reduction: the epilogue's parameter (and state)
    // loads are issued now, ahead of the operands (see prefetch_params).
    constexpr bool kPre = TM == 1 && TN == 1 && (EM == EM_UPDATE || EM == EM_DW);
    const bool whole = k0 == 0 && k1 == s.ipt;
    const bool pre = kPre && whole && s.ipt <= kPrefetchSlices && (EM == EM_UPDATE || p.accum);
    float pre_w[16], pre_s[16];
    if constexpr (kPre) {
      if (pre) prefetch_params<EM>(p, m0 + wm * WM, n0 + wn * WN, li, lh, pre_w, pre_s);
    }
    __syncthreads();  // every wave is done with the ring from the previous item
    // Prologue: slices 0 .. S-2 in flight.  Slices past the end of the item
    // read zeros, which keeps the per-thread load count (and so the vmcnt
    // arithmetic) the same for every slice.
#pragma unroll
    for (int st = 0; st < kDmaStages - 1; ++st) {
      load_a(As[st], st * kDmaBK);
      load_b(Bs[st], st * kDmaBK);
    }
    // The slice loop, once with every block's matrix-core work and once (edge tiles) without the
    // blocks outside the output; two copies so the interior tiles' loop has no branches.  The
    // narrower instances keep the plain loop written out below: compiled through the lambda they
    // take more registers and ran 3% slower (VGG-16's 128 x 64 and 64 x 128 products, same-box
    // comparison).
    // Pipelined form (kPipe): a slice's operands are all read from LDS before its first product, and
    // the wait and barrier that publish the next slice (and free this slice's buffer for the load two
    // slices ahead) sit between the slice's two operand groups, so the barrier and the next slice's
    // first LDS reads overlap products still in the matrix pipe rather than leaving it idle; with one
    // or two wavefronts per SIMD the other wavefronts cannot cover that gap.  Same products in the
    // same order; 16 more VGPRs (not for the update instances, which then lose their third block).
    auto slices_pipe = [&](auto skip_tag) {
      constexpr bool SKIP = decltype(skip_tag)::value;
      constexpr int NG = kDmaBK / 8;
      static_assert(NG == 2, "two operand groups per slice");
      wait_vmcnt<kLoads * (kDmaStages - 2)>();  // slice 0 is in LDS
      if (ones_col >= 0) SB::ones_fixup(Bs[0], ones_col, 0, kval);
      lds_barrier();
      load_a(As[(kDmaStages - 1) % kDmaStages], (kDmaStages - 1) * kDmaBK);
      load_b(Bs[(kDmaStages - 1) % kDmaStages], (kDmaStages - 1) * kDmaBK);
      for (int i = 0; i < nsl; ++i) {
        const int cur = i % kDmaStages;
        float4 av[NG][TM], bv[NG][TN];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
#pragma unroll
          for (int a = 0; a < TM; ++a) av[g][a] = SA::operand(As[cur], wm * WM + a * 32 + li, g, lh);
#pragma unroll
          for (int c = 0; c < TN; ++c) bv[g][c] = SB::operand(Bs[cur], wn * WN + c * 32 + li, g, lh);
        }
        __builtin_amdgcn_sched_barrier(0);  // the reads stay ahead of the products
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          if (g == 1) {
            // Publish slice i + 1 and refill this slice's buffer (all of its reads are done: the
            // barrier waits for them) with slice i + S.
            __builtin_amdgcn_sched_barrier(0);
            const int nxt = (i + 1) % kDmaStages;
            wait_vmcnt<kLoads * (kDmaStages - 2)>();
            if (ones_col >= 0) SB::ones_fixup(Bs[nxt], ones_col, (i + 1) * kDmaBK, kval);
            lds_barrier();
            const int nx = i + kDmaStages;
            load_a(As[cur], nx * kDmaBK);
            load_b(Bs[cur], nx * kDmaBK);
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int c = 0; c < TN; ++c) {
              if (SKIP && (a >= na || c >= nc)) continue;
              acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[g][a].x, bv[g][c].x, acc[a][c], 0, 0, 0);
              acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[g][a].y, bv[g][c].y, acc[a][c], 0, 0, 0);
              acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[g][a].z, bv[g][c].z, acc[a][c], 0, 0, 0);
              acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[g][a].w, bv[g][c].w, acc[a][c], 0, 0, 0);
            }
        }
      }
    };
    auto slices = [&](auto skip_tag) {
      constexpr bool SKIP = decltype(skip_tag)::value;
      for (int i = 0; i < nsl; ++i) {
        const int cur = i % kDmaStages;
        wait_vmcnt<kLoads * (kDmaStages - 2)>();  // this thread's loads of slice i are in LDS
        if (ones_col >= 0) SB::ones_fixup(Bs[cur], ones_col, i * kDmaBK, kval);
        lds_barrier();  // everyone's loads of slice i landed; everyone finished slice i-1
        const int nx = i + kDmaStages - 1;  // refill the buffer slice i-1 used
        load_a(As[nx % kDmaStages], nx * kDmaBK);
        load_b(Bs[nx % kDmaStages], nx * kDmaBK);
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
              if (SKIP && (a >= na || c >= nc)) continue;
              acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a].x, bv[c].x, acc[a][c], 0, 0, 0);
              acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a].y, bv[c].y, acc[a][c], 0, 0, 0);
              acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a].z, bv[c].z, acc[a][c], 0, 0, 0);
              acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a].w, bv[c].w, acc[a][c], 0, 0, 0);
            }
        }
      }
    };
    if constexpr (kSkip && kPipe) {
      if (na < TM || nc < TN) slices_pipe(std::true_type{});
      else slices_pipe(std::false_type{});
    } else if constexpr (kSkip) {
      if (na < TM || nc < TN) slices(std::true_type{});
      else slices(std::false_type{});
    } else if (__builtin_amdgcn_readfirstlane(arows <= wm * WM || p.Nt - n0 <= wn * WN)) {
      // The narrow tiles' wavefront whose whole 32-row (32-column) part lies outside the output -- columns
      // 32..63 of a 64-wide tile over a first conv layer's 29-column weight gradient, rows 32..63 of a
      // 64-row tile over a batch-32 fc layer -- only does its share of the loads: nothing stores its
      // accumulators (zeros) except as a zero partial tile.
      for (int i = 0; i < nsl; ++i) {
        const int cur = i % kDmaStages;
        wait_vmcnt<kLoads * (kDmaStages - 2)>();
        if (ones_col >= 0) SB::ones_fixup(Bs[cur], ones_col, i * kDmaBK, kval);
        lds_barrier();
        const int nx = i + kDmaStages - 1;
        load_a(As[nx % kDmaStages], nx * kDmaBK);
        load_b(Bs[nx % kDmaStages], nx * kDmaBK);
      }
    } else {
      for (int i = 0; i < nsl; ++i) {  // the same loop as `slices`, without the skip
        const int cur = i % kDmaStages;
        wait_vmcnt<kLoads * (kDmaStages - 2)>();
        if (ones_col >= 0) SB::ones_fixup(Bs[cur], ones_col, i * kDmaBK, kval);
        lds_barrier();
        const int nx = i + kDmaStages - 1;
        load_a(As[nx % kDmaStages], nx * kDmaBK);
        load_b(Bs[nx % kDmaStages], nx * kDmaBK);
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
    }
    wait_vmcnt<0>();  // the trailing zero-fill loads land before the ring is reused

    if (whole) {
      if (EM == EM_GENERIC) {
        __syncthreads();  // the ring is free for the epilogue's LDS blocks
        store_tile_generic<TM, TN>(acc, p, m0 + wm * WM, n0 + wn * WN, 0, li, lh, lds + wave * 1024);
      } else if constexpr (kPre) {
        if (pre) {
          store_wave_pre<EM>(reinterpret_cast<const f32x16(&)[1][1]>(acc), p, m0 + wm * WM, n0 + wn * WN, li, lh,
                             pre_w, pre_s);
        } else {
          store_wave<TM, TN, EM>(acc, p, m0 + wm * WM, n0 + wn * WN, li, lh);
        }
      } else {
        store_wave<TM, TN, EM>(acc, p, m0 + wm * WM, n0 + wn * WN, li, lh);
      }
    } else {
      float* dst = s.part + (int64_t)slot * (BM * BN);
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int c = 0; c < TN; ++c)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4*>(
                dst + (WR == 2 ? slot_index<TM, TN>(wave, a, c, q, lane)
                               // the 2 x 2 layout's slot of the same 32 x 32 block (the fixup's)
                               : slot_index<BM / 64, BN / 64>(((wm * TM + a) / (BM / 64)) * 2 + (wn * TN + c) / (BN / 64),
                                                              (wm * TM + a) % (BM / 64), (wn * TN + c) % (BN / 64), q,
                                                              lane))) =
                make_float4(acc[a][c][4 * q], acc[a][c][4 * q + 1], acc[a][c][4 * q + 2], acc[a][c][4 * q + 3]);
    }
  }
}

// Completes the stream-K tiles that were shared between blocks.  Block
// (j, y) takes 256 / TS float4s of stream-K tile j; the tile's slots (one per
// block whose range touched the tile, in block = k order) are split into TS
// contiguous groups, thread group g sums its group in order, and the TS
// group sums are added in group order -- a fixed two-level order, so the
// result depends only on the schedule.  Then finish4(), which computes what
// the gemm_dma epilogue variants compute.
constexpr int kFixChunk = 1024;  // elements a fixup block covers with one thread per float4
template <int BM, int BN>
__global__ __launch_bounds__(kThreads) void gemm_sk_fixup(KArgs p, SkArgs s, int G, int TS) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  __shared__ int slots[1024];
  __shared__ float4 part_sum[kThreads];
  const int j = blockIdx.x;
  const int S = s.sk_iters;
  const int tiles_m = p.tiles / p.tiles_n;
  // Stream-K tile j; grouped, it is tile (j % rg, j / rg) and its ranges are those of its column
  // group, run by the group member (j % rg) * cg + (column % cg) of each.
  const int gsz = s.rg * s.cg, Q = G / gsz;
  int tm_i, tn_i, u, member;
  if (gsz == 1) {
    tile_coords(s.dp_tiles + j, tiles_m, p.tiles_n, p.perm_c == 0, tm_i, tn_i);
    u = j;
    member = 0;
  } else {
    tm_i = j % s.rg;
    tn_i = j / s.rg;
    u = tn_i / s.cg;
    member = tm_i * s.cg + (tn_i - u * s.cg);
  }
  const int x0 = u * s.ipt;
  const int blo = sk_block_of(x0, S, Q), bhi = sk_block_of(x0 + s.ipt - 1, S, Q);
  if (blo == bhi) return;  // inside one range: stored by gemm_dma
  const int n = bhi - blo + 1;  // <= G <= 1024 (checked on the host)
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int qq = blo + i, bb = qq * gsz + member;
    slots[i] = sk_start(qq, S, Q) / s.ipt == u ? 2 * bb : 2 * bb + 1;
  }
  __syncthreads();
  const int m0 = tm_i * BM, n0 = tn_i * BN;
  const int grp = threadIdx.x % TS, v4 = threadIdx.x / TS;
  const int idx = (blockIdx.y * (kThreads / TS) + v4) * 4;  // the float4's first element in the slot
  const float4* src = reinterpret_cast<const float4*>(s.part + idx);
  constexpr int64_t kSlot4 = BM * BN / 4;
  const int i0 = grp * n / TS, i1 = (grp + 1) * n / TS;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  int i = i0;
  if (i < i1) v = src[(int64_t)slots[i++] * kSlot4];
  for (; i + 4 <= i1; i += 4) {
    float4 u[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) u[k] = src[(int64_t)slots[i + k] * kSlot4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v.x += u[k].x;
      v.y += u[k].y;
      v.z += u[k].z;
      v.w += u[k].w;
    }
  }
  for (; i < i1; ++i) {
    const float4 u = src[(int64_t)slots[i] * kSlot4];
    v.x += u.x;
    v.y += u.y;
    v.z += u.z;
    v.w += u.w;
  }
  if (TS > 1) {
    part_sum[threadIdx.x] = v;
    __syncthreads();
    if (grp != 0) return;
    for (int g = 1; g < TS; ++g) {
      const float4 u = part_sum[threadIdx.x + g];
      v.x += u.x;
      v.y += u.y;
      v.z += u.z;
      v.w += u.w;
    }
  }
  // Inverse of slot_index: float4 (wave, a, c, q) of lane l holds rows
  // 8q .. 8q+3 (plus 4 * lane half) of column l % 32 of block (a, c).
  const int lane = (idx >> 2) & 63;
  int rest = idx >> 8;
  const int q = rest & 3;
  rest >>= 2;
  const int c = rest % TN;
  rest /= TN;
  const int a = rest % TM, wave = rest / TM;
  const int row = m0 + (wave >> 1) * WM + a * 32 + 4 * (lane >> 5) + 8 * q;
  const int col = n0 + (wave & 1) * WN + c * 32 + (lane & 31);
  if (col < p.Nt && row < p.M) {
    const float r4[4] = {v.x, v.y, v.z, v.w};
    finish4(r4, row, min(4, p.M - row), col, p);
  }
}

// ---- Short-reduction weight gradients: dW = dY^T X with k <= 32 (an fc layer at a small batch).
//
// With so few k the product is a stream over W and the rule's state: the operands dY and X are a
// few MB that stay in the caches, and the matrix-core work is a small part of the time.  So there
// is no LDS ring.  A wavefront keeps its 32 rows of dY for the whole reduction in registers and
// walks a run of 32-column blocks of W; for NBLK blocks at a time it issues every load first
// (X's columns, and the W / state / GradBuf values it updates), then the products, the rule and
// the stores.  With no LDS and few registers many wavefronts are resident, and their loads keep
// HBM busy.  In the MFMA's result layout a lane holds one column of the block, so every load and
// store instruction covers two whole 128-byte runs of W rows.
constexpr int kShortK = 32;  // the largest reduction dw_short takes
struct ShortArgs {
  int MB, NB;  // 32-row blocks of W; 32-column blocks (the ones column included)
  int MG;      // groups of 4 row blocks: one workgroup of 4 wavefronts each
  int per;     // column blocks per workgroup
};

// KP: k pairs (k <= 2 KP); RULE: -1 stores (or accumulates) the gradient, else the update rule
// applied in place of the store.
template <int KP, int NBLK, int RULE>
__global__ __launch_bounds__(kThreads, KP * NBLK > 16 ? 3 : 4) void dw_short(KArgs p, ShortArgs s) {
  constexpr bool kState = RULE == SGD_MOMENTUM || RULE == SGD_ADAGRAD || RULE == SGD_NESTEROV;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int li = lane & 31, lh = lane >> 5;
  const int mb = (int)(blockIdx.x % (unsigned)s.MG) * 4 + wave;
  const int nb0 = (int)(blockIdx.x / (unsigned)s.MG) * s.per, nb1 = min(s.NB, nb0 + s.per);
  if (mb >= s.MB || nb0 >= nb1) return;
  const int m0 = mb * 32;
  const int rows = min(p.M - m0, 32);
  const uint32_t lda = (uint32_t)p.lda, ldb = (uint32_t)p.ldb, ldc = (uint32_t)p.ldc;
  const bool ones = p.ones_out != nullptr;
  const bool need_w = RULE >= 0 || p.accum;
  // Operands: dY [K][lda] and X [K][ldb]; k >= K lies past the records (reads 0).
  const brsrc ra = brsrc_rows(p.A, p.K, lda);
  const brsrc rb = brsrc_rows(p.B, p.K, ldb);
  // W (or the GradBuf) and the state from the wavefront's first row, and the ones column's bias
  // (and its state): rows past M lie past the records (read 0, stores dropped).
  const brsrc rw = brsrc_rows(p.C + (int64_t)m0 * p.ldc, rows, ldc);
  const brsrc rs = brsrc_rows(kState ? p.ustate + (int64_t)m0 * p.ldc : p.C, kState ? rows : 0, ldc);
  const brsrc rbw = brsrc_rows(ones ? p.ones_out + m0 : p.C, ones ? rows : 0, 1);
  const brsrc rbs = brsrc_rows(kState && p.ustate_b ? p.ustate_b + m0 : p.C, kState && p.ustate_b ? rows : 0, 1);
  float dy[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j)
    dy[j] = bload(ra, m0 + li < p.M ? ((uint32_t)(2 * j + lh) * lda + (uint32_t)(m0 + li)) * 4u : kOffOut);

  for (int nb = nb0; nb < nb1; nb += NBLK) {
    float xb[NBLK][KP], wv[NBLK][16], sv[NBLK][16];
    // Every load of the NBLK blocks first (a block past the run reads nothing).
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      const int n = nb + b < nb1 ? (nb + b) * 32 + li : INT_MAX;
#pragma unroll
      for (int j = 0; j < KP; ++j)
        xb[b][j] = bload(rb, n < p.N ? ((uint32_t)(2 * j + lh) * ldb + (uint32_t)n) * 4u : kOffOut);
      const uint32_t vo = n < p.N ? ((uint32_t)(4 * lh) * ldc + (uint32_t)n) * 4u : kOffOut;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t o = vo == kOffOut ? kOffOut : vo + (uint32_t)blk_row(r) * ldc * 4u;
        wv[b][r] = need_w ? bload(rw, o) : 0.f;
        sv[b][r] = kState ? bload(rs, o) : 0.f;
      }
    }
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      const int n0 = nb + b < nb1 ? (nb + b) * 32 : INT_MAX / 2;
      const int n = n0 + li;
      // The ones column (bias): X reads 1 for every k < K.
      const bool ones_blk = ones && p.N >= n0 && p.N < n0 + 32;
      if (ones_blk && n == p.N) {
#pragma unroll
        for (int j = 0; j < KP; ++j) xb[b][j] = 2 * j + lh < p.K ? 1.f : 0.f;
      }
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int j = 0; j < KP; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(dy[j], xb[b][j], acc, 0, 0, 0);
      // Lane (li, lh) holds column n of rows m0 + 4 lh + blk_row(r).
      const uint32_t vo = n < p.N ? ((uint32_t)(4 * lh) * ldc + (uint32_t)n) * 4u : kOffOut;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t o = vo == kOffOut ? kOffOut : vo + (uint32_t)blk_row(r) * ldc * 4u;
        float w = wv[b][r], st = sv[b][r];
        if constexpr (RULE >= 0) {
          rule1<(RULE >= 0 ? RULE : 0)>(w, st, acc[r], p.eta, p.mu, p.eps, p.decay);
        } else {
          const float x = acc[r] * p.gscale;
          w = p.accum ? w + x : x;
        }
        bstore(w, rw, o);
        if (kState) bstore(st, rs, o);
      }
      // The bias: the ones column's results, in the lane that holds column N.
      if (ones_blk) {
        const uint32_t ob = n == p.N ? (uint32_t)(4 * lh) * 4u : kOffOut;
        float bw[16], bs[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t o = ob == kOffOut ? kOffOut : ob + (uint32_t)blk_row(r) * 4u;
          bw[r] = (RULE >= 0 || p.accum) ? bload(rbw, o) : 0.f;
          bs[r] = kState ? bload(rbs, o) : 0.f;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t o = ob == kOffOut ? kOffOut : ob + (uint32_t)blk_row(r) * 4u;
          if constexpr (RULE >= 0) {
            rule1<(RULE >= 0 ? RULE : 0)>(bw[r], bs[r], acc[r], p.eta, p.mu, p.eps, p.decay);
          } else {
            const float x = acc[r] * p.gscale;
            bw[r] = p.accum ? bw[r] + x : x;
          }
          bstore(bw[r], rbw, o);
          if (kState) bstore(bs[r], rbs, o);
        }
      }
    }
  }
}

// ---- Skinny products: the logits layer's forward product (at most 16 outputs per row) and its
// input-gradient product (a reduction of at most 16).  Both are a pass over one large operand -- the
// layer's input, or its output gradient and ReLU mask -- next to which the tile kernels' prologue,
// stream-K split and fixup launch cost more than the arithmetic.
constexpr int kSkinny = 16;

// C[m][0..N) = epilogue(A[m][:] . B[n][:]) for N <= kSkinny, one block per row: thread t sums the
// float4 groups t, t + 256, ... of k for every output, then each output's 256 partial sums are added
// by a fixed tree in LDS.
__global__ __launch_bounds__(kThreads) void skinny_nt_kernel(KArgs p) {
  __shared__ float red[kSkinny][kThreads];
  const int row = blockIdx.x, t = threadIdx.x;
  const int N = p.N, K4 = p.K / 4;
  const float4* a = reinterpret_cast<const float4*>(p.A + (int64_t)row * p.lda);
  float acc[kSkinny];
#pragma unroll
  for (int n = 0; n < kSkinny; ++n) acc[n] = 0.f;
  for (int k4 = t; k4 < K4; k4 += kThreads) {
    // every load first (rows past N re-read row N - 1 and are not used), then the products
    const float4 av = a[k4];
    float4 bv[kSkinny];
#pragma unroll
    for (int n = 0; n < kSkinny; ++n)
      bv[n] = reinterpret_cast<const float4*>(p.B + (int64_t)min(n, N - 1) * p.ldb)[k4];
#pragma unroll
    for (int n = 0; n < kSkinny; ++n) {
      if (n < N) {
        acc[n] += av.x * bv[n].x;
        acc[n] += av.y * bv[n].y;
        acc[n] += av.z * bv[n].z;
        acc[n] += av.w * bv[n].w;
      }
    }
  }
#pragma unroll
  for (int n = 0; n < kSkinny; ++n) red[n][t] = acc[n];
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (t < o) {
#pragma unroll
      for (int n = 0; n < kSkinny; ++n) red[n][t] += red[n][t + o];
    }
    __syncthreads();
  }
  if (t < N) p.C[(int64_t)row * p.ldc + t] = epilogue(red[t][0], p.epi, row, t, p, 0.f);
}

// C[m][n..n+3] = epilogue(sum over k < K <= kSkinny of A[m][k] B[k][n..n+3]), one float4 of C per
// thread (N a multiple of 4), k in order.
__global__ __launch_bounds__(kThreads) void smallk_nn_kernel(KArgs p) {
  const int N4 = p.N / 4;
  const int64_t total = (int64_t)p.M * N4;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kThreads) {
    const int m = (int)(i / N4), n = (int)(i - (int64_t)m * N4) * 4;
    const float* ar = p.A + (int64_t)m * p.lda;
    // every load first (k past K re-reads row K - 1 and is not used), then the products in k order
    float4 mk = make_float4(1.f, 1.f, 1.f, 1.f);
    if (p.epi == EPI_MASK) mk = *reinterpret_cast<const float4*>(p.mask + (int64_t)m * p.ldm + n);
    float av[kSkinny];
    float4 bv[kSkinny];
#pragma unroll
    for (int k = 0; k < kSkinny; ++k) {
      const int kc = min(k, p.K - 1);
      av[k] = ar[kc];
      bv[k] = *reinterpret_cast<const float4*>(p.B + (int64_t)kc * p.ldb + n);
    }
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < kSkinny; ++k) {
      if (k < p.K) {
        acc.x += av[k] * bv[k].x;
        acc.y += av[k] * bv[k].y;
        acc.z += av[k] * bv[k].z;
        acc.w += av[k] * bv[k].w;
      }
    }
    if (p.epi == EPI_MASK) {
      acc.x = mk.x > 0.f ? acc.x : 0.f;
      acc.y = mk.y > 0.f ? acc.y : 0.f;
      acc.z = mk.z > 0.f ? acc.z : 0.f;
      acc.w = mk.w > 0.f ? acc.w : 0.f;
    }
    *reinterpret_cast<float4*>(p.C + (int64_t)m * p.ldc + n) = acc;
  }
}

// Split-K partials of a weight gradient A^T B (A stored [K][M], B [K][N]) with a small output and a
// long reduction whose rows miss the direct-load alignment (LeNet-5's first conv layer: 6 x 29
// outputs over 12544 pixels, rows of 6 floats).  Block z stages k-rows [z * kc, (z + 1) * kc) of both
// operands in LDS (dynamic, kc * (M + N) floats) and each thread sums its outputs over them in k
// order, the implicit ones column included; splitk_reduce_kernel adds the slices and runs the
// epilogue, as for gemm_staged's partials.  Each block reads its rows once, where the tiled kernel's
// k-loop makes a round trip per 32 rows.
constexpr int kLongMaxLds = 16384;  // floats
__global__ __launch_bounds__(256) void dw_long_kernel(KArgs p, float* __restrict__ part, int kc) {
  extern __shared__ float lds_long[];
  const int M = p.M, N = p.N, Nt = p.Nt;
  float* As = lds_long;           // [kc][M]
  float* Bs = lds_long + kc * M;  // [kc][N]
  const int k0 = (int)blockIdx.x * kc, nk = max(0, min(p.K, k0 + kc) - k0);
  for (int i = threadIdx.x; i < nk * M; i += 256) {
    const int kk = i / M, m = i - kk * M;
    As[i] = p.A[(int64_t)(k0 + kk) * p.lda + m];
  }
  for (int i = threadIdx.x; i < nk * N; i += 256) {
    const int kk = i / N, n = i - kk * N;
    Bs[i] = p.B[(int64_t)(k0 + kk) * p.ldb + n];
  }
  __syncthreads();
  const int64_t MN = (int64_t)M * Nt;
  for (int o = threadIdx.x; o < MN; o += 256) {
    const int m = o / Nt, n = o - m * Nt;
    float acc = 0.f;
    if (n < N) {
      for (int kk = 0; kk < nk; ++kk) acc += As[kk * M + m] * Bs[kk * N + n];
    } else {
      for (int kk = 0; kk < nk; ++kk) acc += As[kk * M + m];
    }
    part[(int64_t)blockIdx.x * MN + o] = acc;
  }
}

// Sum split-K partial tiles in slice order, then store: the ones column to
// ones_out, the conv weight gradient permuted, anything else through the
// epilogue.
// With TS > 1, TS threads share an element: each sums a contiguous group of
// slices and the group sums are added in group order (a fixed two-level
// order for products split many ways).
__global__ void splitk_reduce_kernel(const float* __restrict__ part, int splits, KArgs p, int TS) {
  __shared__ float gsum[256];
  const int64_t MN = (int64_t)p.M * p.Nt;
  const int grp = threadIdx.x % TS, per_block = blockDim.x / TS;
  const int s0 = grp * splits / TS, s1 = (grp + 1) * splits / TS;
  for (int64_t base = (int64_t)blockIdx.x * per_block; base < MN; base += (int64_t)gridDim.x * per_block) {
    const int64_t idx = base + threadIdx.x / TS;
    float v = 0.f;
    if (idx < MN) {
      v = part[(int64_t)s0 * MN + idx];
      for (int s = s0 + 1; s < s1; ++s) v += part[(int64_t)s * MN + idx];
    }
    if (TS > 1) {
      __syncthreads();  // the previous round's group sums were read
      gsum[threadIdx.x] = v;
      __syncthreads();
      if (grp == 0)
        for (int g = 1; g < TS; ++g) v += gsum[threadIdx.x + g];
    }
    if (grp == 0 && idx < MN) {
      const int row = (int)(idx / p.Nt), col = (int)(idx - (int64_t)row * p.Nt);
      finish(v, row, col, p);
    }
  }
}

struct Cfg {
  int bm, bn, bk;
};
// gemm_staged configurations: 0: 128x128x16  1: 128x64x32  2: 64x128x32
constexpr int kStagedConfigs = 3;
const Cfg kCfg[kStagedConfigs] = {{128, 128, 16}, {128, 64, 32}, {64, 128, 32}};
// gemm_dma configurations: 0: 128x128  1: 128x64  2: 64x128  3: 64x64 (weight
// gradients with both output sides <= 64 only: a first conv layer's)
constexpr int kDmaConfigs = 4;
const Cfg kDma[kDmaConfigs] = {{128, 128, kDmaBK}, {128, 64, kDmaBK}, {64, 128, kDmaBK}, {64, 64, kDmaBK}};

const char* const kNames[kStagedConfigs][4] = {
    {"gemm_staged_128x128_nt", "gemm_staged_128x128_tn", "gemm_staged_128x128_nn", "gemm_staged_128x128_tt"},
    {"gemm_staged_128x64_nt", "gemm_staged_128x64_tn", "gemm_staged_128x64_nn", "gemm_staged_128x64_tt"},
    {"gemm_staged_64x128_nt", "gemm_staged_64x128_tn", "gemm_staged_64x128_nn", "gemm_staged_64x128_tt"},
};
// Convolution gathers: forward, dedx (the flipped gather), dedw.
const char* const kConvNames[kDmaConfigs][3] = {
    {"gemm_conv_fwd_128x128", "gemm_conv_dx_128x128", "gemm_conv_dw_128x128"},
    {"gemm_conv_fwd_128x64", "gemm_conv_dx_128x64", "gemm_conv_dw_128x64"},
    {"gemm_conv_fwd_64x128", "gemm_conv_dx_64x128", "gemm_conv_dw_64x128"},
    {"gemm_conv_fwd_64x64", "gemm_conv_dx_64x64", "gemm_conv_dw_64x64"},
};
const char* const kDmaNames[kDmaConfigs][4] = {
    {"gemm_dma_128x128_nt", "gemm_dma_128x128_tn", "gemm_dma_128x128_nn", "gemm_dma_128x128_tt"},
    {"gemm_dma_128x64_nt", "gemm_dma_128x64_tn", "gemm_dma_128x64_nn", "gemm_dma_128x64_tt"},
    {"gemm_dma_64x128_nt", "gemm_dma_64x128_tn", "gemm_dma_64x128_nn", "gemm_dma_64x128_tt"},
    {"gemm_dma_64x64_nt", "gemm_dma_64x64_tn", "gemm_dma_64x64_nn", "gemm_dma_64x64_tt"},
};

typedef void (*StagedKernel)(KArgs);

// gemm_staged instances for a configuration, operand form and epilogue
// variant (the same variants as gemm_dma's; split partials use the generic
// path).
template <int BM, int BN, int BK>
StagedKernel staged_fn_of(int form, int em) {
  switch (form) {
    case 0:
      if (em == EM_BIAS) return gemm_staged<BM, BN, BK, false, false, EM_BIAS>;
      if (em == EM_STORE) return gemm_staged<BM, BN, BK, false, false, EM_STORE>;
      return gemm_staged<BM, BN, BK, false, false, EM_GENERIC>;
    case 1:
      if (em == EM_DW) return gemm_staged<BM, BN, BK, true, true, EM_DW>;
      if (em == EM_UPDATE) return gemm_staged<BM, BN, BK, true, true, EM_UPDATE>;
      if (em == EM_STORE) return gemm_staged<BM, BN, BK, true, true, EM_STORE>;
      return gemm_staged<BM, BN, BK, true, true, EM_GENERIC>;
    case 2:
      if (em == EM_MASK) return gemm_staged<BM, BN, BK, false, true, EM_MASK>;
      if (em == EM_STORE) return gemm_staged<BM, BN, BK, false, true, EM_STORE>;
      return gemm_staged<BM, BN, BK, false, true, EM_GENERIC>;
    default:
      return gemm_staged<BM, BN, BK, true, false, EM_GENERIC>;
  }
}
StagedKernel staged_fn(int cfg, int form, int em) {
  switch (cfg) {
    case 0: return staged_fn_of<128, 128, 16>(form, em);
    case 1: return staged_fn_of<128, 64, 32>(form, em);
    default: return staged_fn_of<64, 128, 32>(form, em);
  }
}

typedef void (*DmaKernel)(KArgs, SkArgs);
typedef void (*FixKernel)(KArgs, SkArgs, int, int);

// gemm_dma / gemm_sk_fixup instances for a configuration, operand form
// (0: A*B^T, 1: A^T*B, 2: A*B, 3: A^T*B^T) and epilogue variant; the
// variants instantiated per form are the ones the step uses, anything else
// runs the generic epilogue.
struct DmaFns {
  DmaKernel main;
  FixKernel fix;
  int bm, bn;
};
template <int BM, int BN, bool PIPE, bool AT, bool BT, int EM, bool GA = false, bool GB = false>
DmaFns dma_inst() {
  // else the plain instance; the weight-gradient form (A^T B, both operands read from LDS as single
  // floats) ran 3-8% slower pipelined alone (more LDS reads in flight than the counter holds).
  constexpr bool kPipe = PIPE && !AT && EM != EM_UPDATE && EM != EM_GENERIC;
  return {gemm_dma<BM, BN, AT, BT, EM, GA, GB, kPipe>, gemm_sk_fixup<BM, BN>, BM, BN};
}
template <int BM, int BN, bool PIPE = false>
DmaFns dma_fns_of(int form, int em, int gather) {
  if (gather == 1) {  // conv forward (bias) and dedx (mask or plain store)
    if (em == EM_BIAS) return dma_inst<BM, BN, PIPE, false, false, EM_BIAS, true>();
    if (em == EM_MASK) return dma_inst<BM, BN, PIPE, false, false, EM_MASK, true>();
    if (em == EM_STORE) return dma_inst<BM, BN, PIPE, false, false, EM_STORE, true>();
    return dma_inst<BM, BN, PIPE, false, false, EM_GENERIC, true>();
  }
  if (gather == 2) {  // conv dedw
    if (em == EM_DW) return dma_inst<BM, BN, PIPE, true, true, EM_DW, false, true>();
    if (em == EM_UPDATE) return dma_inst<BM, BN, PIPE, true, true, EM_UPDATE, false, true>();
    return dma_inst<BM, BN, PIPE, true, true, EM_GENERIC, false, true>();
  }
  switch (form) {
    case 0:
      if (em == EM_BIAS) return dma_inst<BM, BN, PIPE, false, false, EM_BIAS>();
      if (em == EM_STORE) return dma_inst<BM, BN, PIPE, false, false, EM_STORE>();
      return dma_inst<BM, BN, PIPE, false, false, EM_GENERIC>();
    case 1:
      if (em == EM_DW) return dma_inst<BM, BN, PIPE, true, true, EM_DW>();
      if (em == EM_UPDATE) return dma_inst<BM, BN, PIPE, true, true, EM_UPDATE>();
      if (em == EM_STORE) return dma_inst<BM, BN, PIPE, true, true, EM_STORE>();
      return dma_inst<BM, BN, PIPE, true, true, EM_GENERIC>();
    case 2:
      if (em == EM_MASK) return dma_inst<BM, BN, PIPE, false, true, EM_MASK>();
      if (em == EM_STORE) return dma_inst<BM, BN, PIPE, false, true, EM_STORE>();
      return dma_inst<BM, BN, PIPE, false, true, EM_GENERIC>();
    default:
      return dma_inst<BM, BN, PIPE, true, false, EM_GENERIC>();
  }
}
// 1 x 4 wavefront instances of the 64x128 tile for products of at most 32 rows (fc layers at a small
// batch): forward (bias) and input-gradient (mask) forms, and plain stores; nullptr otherwise.
DmaFns dma_fns_rows1(int form, int em, int gather) {
  constexpr DmaFns none{nullptr, nullptr, 0, 0};
  if (gather) return none;
  if (form == 0 && em == EM_BIAS) return {gemm_dma<64, 128, false, false, EM_BIAS, false, false, false, 1>, gemm_sk_fixup<64, 128>, 64, 128};
  if (form == 0 && em == EM_STORE) return {gemm_dma<64, 128, false, false, EM_STORE, false, false, false, 1>, gemm_sk_fixup<64, 128>, 64, 128};
  if (form == 2 && em == EM_MASK) return {gemm_dma<64, 128, false, true, EM_MASK, false, false, false, 1>, gemm_sk_fixup<64, 128>, 64, 128};
  if (form == 2 && em == EM_STORE) return {gemm_dma<64, 128, false, true, EM_STORE, false, false, false, 1>, gemm_sk_fixup<64, 128>, 64, 128};
  return none;
}
// 64x64 is instantiated for the one product dma_cfg gives it: dedw (A^T B,
// not gathered); anything else gets no kernel.
DmaFns dma_fns_64x64(int form, int em, int gather) {
  if (gather || form != 1) return {nullptr, nullptr, 0, 0};
  if (em == EM_DW) return dma_inst<64, 64, false, true, true, EM_DW>();
  if (em == EM_UPDATE) return dma_inst<64, 64, false, true, true, EM_UPDATE>();
  if (em == EM_STORE) return dma_inst<64, 64, false, true, true, EM_STORE>();
  return dma_inst<64, 64, false, true, true, EM_GENERIC>();
}
// pipe: the 128x128 instances with the pipelined slice loop (more VGPRs than three blocks per CU allow),
// for schedules of at most two blocks per CU.
DmaFns dma_fns(int cfg, int form, int em, int gather, bool pipe) {
  switch (cfg) {
    case 0: return pipe ? dma_fns_of<128, 128, true>(form, em, gather) : dma_fns_of<128, 128>(form, em, gather);
    case 1: return dma_fns_of<128, 64>(form, em, gather);
    case 2: return dma_fns_of<64, 128>(form, em, gather);
    default: return dma_fns_64x64(form, em, gather);
  }
}

// The epilogue variant for a product (see EpiMode).  The specialised ones
// address 128 rows of their output (and mask) from one buffer resource, so
// those must span less than 1 GiB.
int epi_mode(const GemmDesc& d, int form) {
  const int64_t kMaxLd = (int64_t)1 << 21;
  if (d.ldc >= kMaxLd || (d.epi == EPI_MASK && d.ldm >= kMaxLd)) return EM_GENERIC;
  const bool extra = d.ones_out || d.perm_c > 0 || d.accum || d.urule >= 0;
  if (form == 1) {
    if (d.epi != EPI_STORE) return EM_GENERIC;
    if (d.urule >= 0) return EM_UPDATE;
    return extra ? EM_DW : EM_STORE;
  }
  if (extra) return EM_GENERIC;
  if (form == 0 && (d.epi == EPI_BIAS || d.epi == EPI_BIAS_RELU)) return EM_BIAS;
  if ((form == 2 || (form == 0 && d.gather == 1)) && d.epi == EPI_MASK) return EM_MASK;
  if (d.epi == EPI_STORE && form != 3) return EM_STORE;
  return EM_GENERIC;
}

int64_t tiles_of(const Cfg& c, int M, int N) { return ceil_div(M, c.bm) * ceil_div(N, c.bn); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Compute units of the current device (cached per device; the MI355X's 256
// without a device, when a workspace is planned on a host without a GPU) and
// the gemm_dma blocks of a configuration that fit on one CU by their LDS ring
// (160 KiB per CU).  The schedule depends on nothing else, so a product
// rounds the same way whichever epilogue variant runs it.
struct Machine {
  int cus;
  int occ;
};
Machine machine_for(int cfg) {
  static std::mutex mu;
  static std::map<int, int> cus_of;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  (void)hipGetLastError();
  int cus = 256;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cus_of.find(dev);
    if (it != cus_of.end()) {
      cus = it->second;
    } else {
      int n = 0;
      if (dev >= 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
        cus = n;
      (void)hipGetLastError();
      cus_of[dev] = cus;
    }
  }
  const Cfg& c = kDma[cfg];
  const int lds = kDmaStages * kDmaBK * 4 * (c.bm + c.bn);
  return {cus, std::max(1, std::min(4, (160 * 1024) / lds))};
}

// Launch plan of one gemm_dma product: grid size, whole tiles first, then
// the stream-K part.  Chosen by a cost model in units of one 16-deep k-slice
// of one block at full occupancy:
//  * a block with k of the `occ` resident blocks per CU runs a slice in
//    k/occ of that time, scaled by the matrix-core efficiency measured at k
//    resident blocks (0.72, 0.85, 0.88 for 1, 2, 3+);
//  * each tile or stream-K segment costs a further kItemCost slices
//    (prologue latency and epilogue stores);
//  * the fixup pass moves the partial tiles through HBM at ~4 TB/s.
// Candidates: one block per tile, and stream-K on grids of 1 .. occ blocks
// per CU with the last one or two rounds of whole tiles given to stream-K.
struct SkPlan {
  int grid;
  int dp;
  int64_t sk_iters;
  int rg = 1, cg = 1;  // block group of the grouped form (see SkArgs)
  int edge_last = 0;   // see edge_last_coords
};
constexpr double kItemCost = 6.0;
SkPlan sk_choose(int64_t T, int64_t I, const Machine& m, int64_t tile_floats, int64_t cap_floats) {
  static const double eff[5] = {0.0, 0.72, 0.85, 0.88, 0.88};
  const int occ = std::max(1, std::min(m.occ, 4));
  auto slice_time = [&](int64_t k) {
    k = std::max<int64_t>(1, std::min<int64_t>(k, occ));
    return (double)k / occ * eff[occ] / eff[k];
  };
  const int64_t G3 = (int64_t)m.cus * occ;
  SkPlan best{(int)std::min<int64_t>(T, INT32_MAX), (int)std::min<int64_t>(T, INT32_MAX), 0};
  const int64_t full = T / G3, rem = T % G3;
  double best_cost = (double)full * (I + kItemCost) * slice_time(occ) +
                     (rem ? (I + kItemCost) * slice_time(ceil_div(rem, m.cus)) : 0.0);
  // Seconds per slice at full occupancy, for the fixup's memory time.
  const double unit_s = 2.0 * tile_floats * kDmaBK * (double)G3 / (eff[occ] * 157.3e12);
  for (int k = 1; k <= occ; ++k) {
    const int64_t g = (int64_t)m.cus * k;
    if (g > 1024 || 2 * g * tile_floats > cap_floats) continue;  // the fixup's slot list holds 1024
    for (int64_t r = std::max<int64_t>(0, T / g - 1); r <= T / g; ++r) {
      const int64_t dp = r * g;
      if (dp >= T) continue;
      const int64_t S = (T - dp) * I;
      if (S < g || S * g >= ((int64_t)1 << 31)) continue;
      const double per = (double)S / g;
      const double segs = std::ceil(per / I) + 1.0;
      const int64_t shared = std::min<int64_t>(T - dp, g);
      const double fix = 4.0 * tile_floats * (double)(2 * shared + g) / 4e12 / unit_s + 1.0;
      const double cost = ((double)r * (I + kItemCost) + per + segs * kItemCost) * slice_time(k) + fix;
      if (cost < best_cost) {
        best_cost = cost;
        best = {(int)g, (int)dp, S};
      }
    }
  }
  // Products with fewer k-slices than CUs: a few slices per block, one block
  // per CU.
  const int64_t S = T * I;
  for (int64_t per = 2; per <= 16; per *= 2) {
    const int64_t g = S / per;
    if (g < 2 || g >= m.cus || 2 * g * tile_floats > cap_floats) continue;
    const double fix = 4.0 * tile_floats * (double)(2 * T + g) / 4e12 / unit_s + 1.0;
    const double cost = ((double)S / g + (std::ceil((double)S / g / I) + 1.0) * kItemCost) * slice_time(1) + fix;
    if (cost < best_cost) {
      best_cost = cost;
      best = {(int)g, 0, S};
    }
  }
  return best;
}

// The grouped form for a pure stream-K plan of a product at most kGroupRows
// tile rows tall: rg = all of its tile rows, cg the widest divisor of its tile
// columns (up to kGroupCols) for which a group divides an XCD's run of G / 8
// blocks, so that the group's blocks share an XCD.  The per-block work, the
// number of ranges a tile is cut into and the slot count are those of the
// ungrouped plan.
constexpr int kGroupRows = 8, kGroupCols = 8;
constexpr bool group_sk = true;   // see pipe_slices
constexpr bool edge_last = true;  // see pipe_slices
void sk_group(SkPlan& p, int64_t tiles_m, int64_t tiles_n, int64_t ipt) {
  p.rg = p.cg = 1;
  if (p.dp != 0 || p.sk_iters <= 0 || p.grid % 8 || tiles_m > kGroupRows) return;
  const int run = p.grid / 8;
  if (run % tiles_m) return;
  int cg = 1;
  for (int c = kGroupCols; c > 1; --c)
    if (tiles_n % c == 0 && run % (tiles_m * c) == 0) {
      cg = c;
      break;
    }
  if (tiles_m * cg < 2) return;
  const int64_t S = tiles_n / cg * ipt, Q = p.grid / (tiles_m * cg);
  if (S < Q || S * p.grid >= ((int64_t)1 << 31)) return;
  p.rg = (int)tiles_m;
  p.cg = cg;
  p.sk_iters = S;
}

// Tile choice for gemm_staged, from measurements on the step's shapes.
int staged_cfg(int M, int Nt) {
  if (Nt <= 64) return 1;
  if (M <= 64) return 2;
  return 0;
}

// Tile choice for gemm_dma: 128x128 unless one side of the output is narrow.
// A weight gradient (form A^T B, not gathered) takes 64x64 when both sides
// are <= 64 -- a first conv layer's, 64 x (27 + 1) at VGG, where 128x64 would
// waste half the matrix-core work -- or when its reduction is short (an fc
// layer's dedw, k = the batch): then the product is bound by the epilogue's
// parameter traffic, 64x64 tiles keep four times as many of them in flight,
// and their epilogue operands are loaded ahead (prefetch_params).
int dma_cfg(int M, int Nt, int K, int form, bool gather) {
  if (form == 1 && !gather && ((M <= 64 && Nt <= 64) || ceil_div(K, kDmaBK) <= kPrefetchSlices)) return 3;
  if (Nt <= 64) return 1;
  if (M <= 64) return 2;
  return 0;
}

// gemm_dma preconditions: aligned operands and strides; K a multiple of 4 for
// a K-contiguous operand, the row count a multiple of 4 for a row-contiguous
// one (whole 16-byte quads are either in or out of range); the ones column at
// a quad boundary.
bool dma_ok(const GemmDesc& d) {
  auto operand_ok = [&](const float* X, int64_t ld, bool t, int rows) {
    if (!aligned16(X) || ld % 4) return false;
    return t ? rows % 4 == 0 : d.K % 4 == 0;
  };
  if (d.ones_out && d.N % 4) return false;
  return (d.gather == 1 || operand_ok(d.A, d.lda, d.a_t, d.M)) && (d.gather == 2 || operand_ok(d.B, d.ldb, d.b_t, d.N));
}

// Preconditions of a convolution gather: the form it is built for, channel
// counts that keep a slice (A) or a quad (B) inside one tap, an aligned
// source, 32-bit offsets into it and pixel indices below 2^22 (the float
// reciprocal division is exact there).
bool gather_ok(const GemmDesc& d) {
  const ConvGather& g = d.cv;
  if (d.gather == 0) return true;
  if (!g.src || !aligned16(g.src) || g.c < 1 || g.P < 0 || g.RH < 1 || g.RW < 1 || g.SH < 1 || g.SW < 1) return false;
  const int64_t pix = d.gather == 1 ? d.M : d.K;  // the gathered pixel index
  if (pix % ((int64_t)g.RH * g.RW) || pix + 256 >= ((int64_t)1 << 22)) return false;
  const int64_t imgs = pix / ((int64_t)g.RH * g.RW);
  if (imgs * g.SH * g.SW * g.SC * 4 + 64 >= (int64_t)kOffBad) return false;
  if (d.gather == 1) return !d.a_t && !d.b_t && g.SC % 16 == 0 && d.K == g.c * g.c * g.SC;
  return d.a_t && d.b_t && g.SC % 4 == 0 && d.N == g.c * g.c * g.SC;
}

// Every offset a work item of up to `slices` k-slices addresses from its
// buffer resource is below 2^31 bytes.
bool dma_span_ok(const GemmDesc& d, const Cfg& c, int64_t slices) {
  auto span = [&](int64_t ld, bool t, int tile) {
    const int64_t k = slices * kDmaBK;
    return (t ? (k - 1) * ld + tile : (int64_t)(tile - 1) * ld + k) * 4;
  };
  return (d.gather == 1 || span(d.lda, d.a_t, c.bm) < (int64_t)kOffBad) &&
         (d.gather == 2 || span(d.ldb, d.b_t, c.bn) < (int64_t)kOffBad);
}

int form_of(bool a_t, bool b_t) { return (!a_t && !b_t) ? 0 : (a_t && b_t) ? 1 : (!a_t && b_t) ? 2 : 3; }

}  // namespace

int gemm_pick_splits(int M, int Nt, int K) {
  const int64_t tiles = tiles_of(kCfg[staged_cfg(M, Nt)], M, Nt);
  int s = 1;
  // gemm_staged only (gemm_dma balances with stream-K): aim for >= 4
  // workgroups per CU while keeping each K slice >= 256 long and the partial
  // tiles' extra traffic ((s + 1) * M * Nt floats written and read back)
  // small next to the product: s <= K / 512.
  while (tiles * s < 1024 && K / (2 * s) >= 256 && 2 * s <= K / 512 && s < 256) s *= 2;
  // A product with few tiles is latency-bound: split while slices keep >= 64
  // k-values and the partial tiles stay small (<= 64 MiB).
  while (tiles * s < 256 && K / (2 * s) >= 64 && (int64_t)2 * s * M * Nt <= ((int64_t)1 << 24) && s < 256) s *= 2;
  return s;
}

int64_t gemm_scratch_floats(int M, int Nt, int K, bool a_t, bool b_t, bool fused, int splits) {
  const int64_t staged = splits > 1 ? (int64_t)splits * M * Nt : 0;
  (void)fused;
  const int cfg = dma_cfg(M, Nt, K, form_of(a_t, b_t), false);
  const Cfg& c = kDma[cfg];
  const SkPlan p = sk_choose(tiles_of(c, M, Nt), ceil_div(K, kDmaBK), machine_for(cfg), (int64_t)c.bm * c.bn, INT64_MAX);
  const int64_t sk = p.sk_iters > 0 ? 2 * (int64_t)p.grid * c.bm * c.bn : 0;
  return std::max(staged, sk);
}

int gemm_launch(const GemmDesc& d, hipStream_t s);

int gemm(const GemmDesc& d, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0) return 0;
  prof_set_shape(d.M, d.N + (d.ones_out ? 1 : 0), d.K);  // the ones column is computed too
  const int e = gemm_launch(d, s);
  prof_set_shape(0, 0, 0);
  return e;
}

// dw_short takes a weight gradient (A^T B, not gathered, plain store, accumulation or update rule)
// whose reduction is at most kShortK, with 16-byte-aligned rows of W (and of the state) and
// operand records within the 2 GiB a buffer resource addresses.
bool short_dw_ok(const GemmDesc& d, int form) {
  if (form != 1 || d.gather || d.perm_c > 0 || d.epi != EPI_STORE) return false;
  if (d.K < 1 || d.K > kShortK || d.M < 1 || d.N < 1) return false;
  if (d.lda < d.M || d.ldb < d.N || d.ldc < d.N) return false;
  if (d.N % 4 || d.ldc % 4 || !aligned16(d.C)) return false;
  const bool st = d.urule == SGD_MOMENTUM || d.urule == SGD_ADAGRAD || d.urule == SGD_NESTEROV;
  if (st && (!d.ustate || !aligned16(d.ustate))) return false;
  // Operand offsets are formed for every k < kShortK (those at k >= K fall past the records and
  // read 0), so kShortK rows of each operand must stay within 32-bit offsets below 2 GiB.
  const int64_t lim = 0x7ffffff0;
  return 4 * (int64_t)kShortK * d.lda <= lim && 4 * (int64_t)kShortK * d.ldb <= lim && 4 * 32 * d.ldc <= lim;
}

typedef void (*ShortKernel)(KArgs, ShortArgs);
// Blocks per batch of loads: one for the rules with a state array (their W and state loads fill
// the 128 registers of 4 wavefronts per SIMD), two for the others when a wavefront walks at
// least 4 blocks (at k = 32 that takes 3 wavefronts per SIMD; VGG-16's 4096 x 25088 fc weight
// gradient: 148 us against 157 with one), else one.
template <int KP>
ShortKernel short_fn(int urule, bool two) {
  switch (urule) {
    case SGD_PLAIN: return two ? dw_short<KP, 2, SGD_PLAIN> : dw_short<KP, 1, SGD_PLAIN>;
    case SGD_MOMENTUM: return dw_short<KP, 1, SGD_MOMENTUM>;
    case SGD_NESTEROV: return dw_short<KP, 1, SGD_NESTEROV>;
    case SGD_ADAGRAD: return dw_short<KP, 1, SGD_ADAGRAD>;
    default: return two ? dw_short<KP, 2, -1> : dw_short<KP, 1, -1>;
  }
}

// One workgroup covers 4 row blocks and a run of `per` column blocks; the runs are sized so the
// grid is about one round of the resident workgroups (one per wavefront slot of a SIMD).
int dw_short_launch(const GemmDesc& d, KArgs a, double flops, double bytes, hipStream_t s) {
  a.C = d.C;
  a.ldc = d.ldc;
  ShortArgs sa{};
  sa.MB = (int)ceil_div(d.M, 32);
  sa.NB = (int)ceil_div(a.Nt, 32);
  sa.MG = (int)ceil_div(sa.MB, 4);
  const int cus = machine_for(0).cus;
  const bool st = d.urule == SGD_MOMENTUM || d.urule == SGD_ADAGRAD || d.urule == SGD_NESTEROV;
  const int64_t blocks = (int64_t)sa.MG * sa.NB;  // per wavefront slot of a workgroup
  const bool two = !st && blocks >= 4 * 4 * (int64_t)cus;
  const int occ = two && d.K > 16 ? 3 : 4;  // wavefronts per SIMD the instance's registers allow
  sa.per = (int)std::max<int64_t>(1, ceil_div(blocks, (int64_t)cus * occ));
  const int64_t grid = (int64_t)sa.MG * ceil_div(sa.NB, sa.per);
  const bool k16 = d.K <= 16;
  const ShortKernel fn = k16 ? short_fn<8>(d.urule, two) : short_fn<16>(d.urule, two);
  prof_begin(k16 ? "gemm_dw_short_k16" : "gemm_dw_short_k32", flops, bytes, s);
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(kThreads), 0, s, a, sa);
  prof_end(s);
  return check_launch("gemm_dw_short");
}

// The skinny kernels take plain products (no gather, ones column, accumulation or update rule) whose
// vector operands are 16-byte aligned with row strides a multiple of 4 floats.
bool plain_product(const GemmDesc& d) {
  return d.skinny && !d.gather && !d.ones_out && !d.accum && d.urule < 0 && d.perm_c == 0 && d.M >= 1 && d.N >= 1 &&
         d.K >= 1;
}
// A block per row pays a 256-wide reduction tree whatever k is, so many rows over a short k (a 5x5
// conv layer's 12544 x 6 x 28 forward product as a plain product: 44 us against 8 on the tiles) stay
// on the tile kernels; a few rows (a logits layer at batch 16: k = 84) still take the row kernel.
bool skinny_nt_ok(const GemmDesc& d, int form) {
  return form == 0 && plain_product(d) && d.N <= kSkinny && d.K % 4 == 0 && d.lda % 4 == 0 && d.ldb % 4 == 0 &&
         (d.K >= 128 || d.M <= 1024) && aligned16(d.A) && aligned16(d.B) &&
         (d.epi == EPI_STORE || d.epi == EPI_BIAS || d.epi == EPI_BIAS_RELU);
}
// The small-k kernel reloads B's 16 rows for every output row, so it is used for outputs up to 2^20
// elements (LeNet-5's and VGG-CIFAR's logits dedx: 7.0 -> 6.0 and 10.9 -> 6.6 us); the MLP's 512 x 5000
// output stays on the tiled kernel, which shares B through LDS (11 us against 13).
bool smallk_nn_ok(const GemmDesc& d, int form) {
  return form == 2 && plain_product(d) && d.K <= kSkinny && (int64_t)d.M * d.N <= ((int64_t)1 << 20) &&
         d.N % 4 == 0 && d.ldb % 4 == 0 && d.ldc % 4 == 0 &&
         aligned16(d.B) && aligned16(d.C) &&
         (d.epi == EPI_STORE || (d.epi == EPI_MASK && d.ldm % 4 == 0 && aligned16(d.mask)));
}

// The automatic gemm_dma schedule of an M x Nt x K product on configuration cfg with cap floats of
// partial-tile scratch: the stream-K plan, its grouped form, and the edge-last tile order.
SkPlan auto_plan(int cfg, int M, int Nt, int K, int64_t cap) {
  const Cfg& c = kDma[cfg];
  const int64_t T = tiles_of(c, M, Nt), ipt = ceil_div(K, kDmaBK), tile = (int64_t)c.bm * c.bn;
  const Machine mc = machine_for(cfg);
  SkPlan plan = sk_choose(T, ipt, mc, tile, cap);
  if (group_sk) sk_group(plan, ceil_div(M, c.bm), ceil_div(Nt, c.bn), ipt);
  // One block per tile over more than one round of resident blocks: ragged edge tiles last.
  if (edge_last && plan.sk_iters == 0 && plan.dp == T && T == plan.grid && T > (int64_t)mc.cus * mc.occ)
    plan.edge_last = (M % c.bm ? 1 : 0) | (Nt % c.bn ? 2 : 0);
  return plan;
}

int gemm_launch(const GemmDesc& d, hipStream_t s) {
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
  a.decay = d.decay;
  a.gscale = d.gscale;
  if (d.urule >= 0 && (d.epi != EPI_STORE || d.accum || d.gscale != 1.f)) {
    set_error("gemm: an update rule can only replace a plain store");
    return SGD_EINVAL;
  }
  if (d.accum && d.epi != EPI_STORE) {
    set_error("gemm: accumulation is only defined for plain stores");
    return SGD_EINVAL;
  }
  a.a_vec = aligned16(d.A) && d.lda % 4 == 0;
  a.b_vec = aligned16(d.B) && d.ldb % 4 == 0;
  const int form = form_of(d.a_t, d.b_t);
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
    cfg = dma_cfg(d.M, a.Nt, d.K, form, d.gather != 0);
    dma = dma_ok(d);
    if (!dma) cfg = staged_cfg(d.M, a.Nt);
  }
  if (d.gather && (!dma || !gather_ok(d))) {
    set_error("gemm: the convolution gather's preconditions do not hold");
    return SGD_EINVAL;
  }
  if (dma && !dma_ok(d)) {
    set_error("gemm: operands do not meet the direct-load preconditions");
    return SGD_EINVAL;
  }
  a.cv = d.cv;
  const double flops = d.flops > 0 ? d.flops : 2.0 * d.M * d.N * (double)d.K;
  // Algorithmic bytes: both operands once, and the output: written once, read
  // too when accumulated, and with the fused update the parameters (and the
  // rule's state, if any) read and written in place of the store.
  const double out_words = (double)d.M * a.Nt;
  const double out_passes = d.urule >= 0 ? (d.urule == SGD_PLAIN ? 2.0 : 4.0) : d.accum ? 2.0 : 1.0;
  const double bytes = 4.0 * ((double)d.M * d.K + (double)d.K * d.N + out_passes * out_words);
  if (d.cfg < 0 && short_dw_ok(d, form)) return dw_short_launch(d, a, flops, bytes, s);
  if (d.cfg < 0 && (skinny_nt_ok(d, form) || smallk_nn_ok(d, form))) {
    a.C = d.C;
    a.ldc = d.ldc;
    if (form == 0) {
      prof_begin("gemm_skinny_nt", flops, bytes, s);
      hipLaunchKernelGGL(skinny_nt_kernel, dim3((unsigned)d.M), dim3(kThreads), 0, s, a);
    } else {
      const int64_t quads = (int64_t)d.M * (d.N / 4);
      prof_begin("gemm_smallk_nn", flops, bytes + (d.epi == EPI_MASK ? 4.0 * d.M * d.N : 0.0), s);
      hipLaunchKernelGGL(smallk_nn_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(quads, kThreads), 4096)),
                         dim3(kThreads), 0, s, a);
    }
    prof_end(s);
    return check_launch("gemm_skinny");
  }

  // gemm_dma schedule.  The plan depends only on the shape and the machine
  // (the instance without an update rule sets the occupancy), so a product
  // rounds the same way with and without the fused update.
  SkPlan plan{};
  if (dma) {
    const Cfg& c = kDma[cfg];
    const int64_t T = tiles_of(c, d.M, a.Nt), ipt = ceil_div(d.K, kDmaBK), tile = (int64_t)c.bm * c.bn;
    const int64_t cap = d.partial ? d.partial_floats : 0;
    if (d.sk_grid > 1024) {
      set_error("gemm: stream-K grid above 1024 blocks");
      return SGD_EINVAL;
    }
    if (d.sk_grid > 0) {  // forced schedule
      const int64_t dp = std::max<int64_t>(0, std::min<int64_t>(d.sk_dp, T));
      plan = {d.sk_grid, (int)dp, (T - dp) * ipt};
      if (plan.sk_iters > 0 && plan.sk_iters < plan.grid) {
        set_error("gemm: stream-K part has fewer k-slices than blocks");
        return SGD_EINVAL;
      }
    } else {
      plan = auto_plan(cfg, d.M, a.Nt, d.K, cap);
    }
    if (plan.sk_iters > 0 && plan.sk_iters * plan.grid >= ((int64_t)1 << 31)) {
      set_error("gemm: stream-K schedule too long for 32-bit range arithmetic");
      return SGD_EINVAL;
    }
    if (plan.sk_iters > 0 && 2 * (int64_t)plan.grid * tile > cap) {
      set_error("gemm: partial-tile buffer too small for the stream-K schedule");
      return SGD_EINVAL;
    }
    const int64_t item =
        plan.dp > 0 ? ipt : std::min<int64_t>(ipt, ceil_div(plan.sk_iters, plan.grid / (plan.rg * plan.cg)));
    if (!dma_span_ok(d, c, item)) {
      if (d.cfg >= 0 || d.gather) {
        set_error("gemm: a work item spans more than 2 GiB of an operand");
        return SGD_EINVAL;
      }
      dma = false;
      cfg = staged_cfg(d.M, a.Nt);
    }
  }
  const Cfg& c = dma ? kDma[cfg] : kCfg[cfg];
  a.tiles_n = (int)ceil_div(a.Nt, c.bn);
  a.tiles = (int)(ceil_div(d.M, c.bm) * a.tiles_n);

  if (dma) {
    a.C = d.C;
    a.ldc = d.ldc;
    a.split = 0;
    a.k_per_split = (int)round_up(d.K, kDmaBK);
    // The pipelined instances (two blocks per CU) for schedules of at most two blocks per CU, except
    // beside the side stream's products: there they made VGG-16's step 0.4% slower (same-box A/B), the
    // MLP's and VGG-CIFAR's no faster.
    DmaFns f{nullptr, nullptr, 0, 0};
    if (cfg == 2 && d.M <= 32) f = dma_fns_rows1(form, epi_mode(d, form), d.gather);
    if (!f.main)
      f = dma_fns(cfg, form, epi_mode(d, form), d.gather,
                  pipe_slices && !d.beside_side && cfg == 0 && plan.grid <= 2 * machine_for(cfg).cus);
    if (!f.main) {
      set_error("gemm: no 64x64 kernel for this product form");
      return SGD_EINVAL;
    }
    const int64_t T = a.tiles, ipt = ceil_div(d.K, kDmaBK), tile = (int64_t)c.bm * c.bn;
    const SkArgs sk{(int)ipt, plan.dp, (int)plan.sk_iters, d.partial, plan.rg, plan.cg, plan.edge_last};
    prof_begin(d.gather ? kConvNames[cfg][d.gather == 2 ? 2 : (d.cv.flip ? 1 : 0)] : kDmaNames[cfg][form], flops, bytes, s);
    hipLaunchKernelGGL(f.main, dim3(plan.grid), dim3(kThreads), 0, s, a, sk);
    prof_end(s);
    if (int e = check_launch("gemm")) return e;
    if (plan.sk_iters > 0) {
      // Partial tiles written and read back by the fixup (for the profile),
      // and the most slots a tile has.
      // (Grouped: the ranges of column group u cut each of its rg * cg tiles alike.)
      const int gsz = plan.rg * plan.cg, Q = plan.grid / gsz;
      int64_t shared = 0, slots = 0, most = 1;
      for (int64_t u = 0; u < sk.sk_iters / ipt; ++u) {
        const int blo = sk_block_of((int)(u * ipt), sk.sk_iters, Q);
        const int bhi = sk_block_of((int)(u * ipt + ipt - 1), sk.sk_iters, Q);
        if (blo != bhi) {
          shared += gsz;
          slots += (int64_t)gsz * (bhi - blo + 1);
          most = std::max<int64_t>(most, bhi - blo + 1);
        }
      }
      // Threads per float4: about 8 slots each, a power of two up to 16.
      int ts = 1;
      while (ts < 16 && most > 8 * ts) ts *= 2;
      prof_begin("gemm_sk_fixup", (double)(slots - shared) * tile, 4.0 * (double)(slots + shared) * tile, s);
      hipLaunchKernelGGL(f.fix, dim3((unsigned)(T - plan.dp), (unsigned)(tile * ts / kFixChunk)), dim3(kThreads), 0,
                         s, a, sk, plan.grid, ts);
      prof_end(s);
      if (int e = check_launch("gemm_sk_fixup")) return e;
    }
    return 0;
  }

  const int splits = d.splits < 1 ? 1 : d.splits;
  a.k_per_split = (int)round_up(ceil_div(d.K, splits), c.bk);
  const bool via_partial = splits > 1;
  if (via_partial && (!d.partial || (int64_t)splits * d.M * a.Nt > d.partial_floats)) {
    set_error("gemm: partial buffer too small for the split count");
    return SGD_EINVAL;
  }
  a.C = via_partial ? d.partial : d.C;
  a.ldc = via_partial ? a.Nt : d.ldc;
  a.split = via_partial ? 1 : 0;
  const int long_kc = (int)ceil_div(d.K, splits);
  if (via_partial && form == 1 && !d.gather && d.cfg < 0 && d.M <= 64 && d.N <= 64 &&
      (int64_t)long_kc * (d.M + d.N) <= kLongMaxLds) {
    prof_begin("gemm_staged_long_tn", flops, bytes, s);
    hipLaunchKernelGGL(dw_long_kernel, dim3((unsigned)splits), dim3(256),
                       (size_t)long_kc * (d.M + d.N) * sizeof(float), s, a, d.partial, long_kc);
  } else {
    prof_begin(kNames[cfg][form], flops, bytes, s);
    hipLaunchKernelGGL(staged_fn(cfg, form, via_partial ? EM_GENERIC : epi_mode(d, form)), dim3(a.tiles * splits),
                       dim3(kThreads), 0, s, a);
  }
  prof_end(s);
  if (int e = check_launch("gemm")) return e;
  if (via_partial) {
    KArgs r = a;
    r.C = d.C;
    r.ldc = d.ldc;
    const int64_t mn = (int64_t)d.M * a.Nt;
    int ts = 1;  // threads per element: about 8 slices each, a power of two up to 16
    while (ts < 16 && splits > 8 * ts) ts *= 2;
    const int blocks = (int)std::min<int64_t>(ceil_div(mn * ts, 256), 8192);
    prof_begin("splitk_reduce", (double)(splits - 1) * mn, 4.0 * (double)(splits + 1) * mn, s);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, d.partial, splits, r, ts);
    prof_end(s);
    if (int e = check_launch("splitk_reduce")) return e;
  }
  return 0;
}

int gemm_plan_query(int M, int Nt, int K, int form, int64_t* out) {
  const int cfg = dma_cfg(M, Nt, K, form, false);
  const Cfg& c = kDma[cfg];
  const SkPlan p = auto_plan(cfg, M, Nt, K, INT64_MAX);
  const int64_t v[12] = {c.bm, c.bn, p.grid, p.dp, p.sk_iters, p.rg, p.cg, p.edge_last,
                         ceil_div(M, c.bm), ceil_div(Nt, c.bn), ceil_div(K, kDmaBK), machine_for(cfg).cus};
  for (int i = 0; i < 12; ++i) out[i] = v[i];
  return 0;
}

}  // namespace sgd
