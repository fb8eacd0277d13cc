// Internal helpers shared by the HIP sources of libsgdstep (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>

#include "sgdstep.h"

namespace sgd {

// Thread-local error text behind sgd_last_error().
void set_error(const std::string& msg);

// A new net planned from the same input, layer list, reduction and
// settings (implicit convolution, dedw overlap) as `src`.
int clone_net(const sgd_net* src, sgd_net** out);
sgd_input net_input(const sgd_net* net);

// Records `what` plus the pending HIP error (if any) and returns SGD_EDEVICE,
// or returns 0 when the last launch succeeded.
int check_launch(const char* what);

// Optional per-launch timing (sgd_profile).  When a profiler is active on
// the calling thread, every launcher brackets its kernel with a HIP event
// pair and records the launch's algorithmic flops and HBM bytes.
void prof_begin(const char* kernel, double flops, double bytes, hipStream_t s);
void prof_end(hipStream_t s);
void prof_set_layer(int layer, int phase);
// The m x n x k of the product whose kernels are launched next (0 after it).
void prof_set_shape(int m, int n, int k);

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// ---------------------------------------------------------------- GEMM ----
// C[M][N] = op(A) * op(B) in fp32 on the matrix cores.
//   a_t == false: A stored [M][K] (row stride lda);  true: stored [K][M].
//   b_t == false: B stored [N][K] (row stride ldb);  true: stored [K][N].
// The epilogue is applied to each fp32 result v at (row, col):
enum Epilogue : int {
  EPI_STORE = 0,      // C = v
  EPI_BIAS = 1,       // C = v + bias[col]
  EPI_BIAS_RELU = 2,  // C = max(v + bias[col], 0)
  EPI_MASK = 3,       // C = mask[row*ldm + col] > 0 ? v : 0   (ReLU derivative)
  EPI_ACCUM = 4,      // C = C + v
};

// An implicit-GEMM operand: the rows (A) or k-rows (B) of the product run
// over a pixel grid RH x RW per image, and the index (ky*c + kx)*SC + ch over
// the c x c taps and SC channels of the NHWC source `src` (SH x SW pixels
// per image): channel ch of source pixel (y + dy, x + dx) with dy = ky - P,
// or dy = P - ky when `flip` (the dedx gather over the output gradient);
// zero outside the source.  inv_* are 1.0f/RW and 1.0f/RH.
struct ConvGather {
  const float* src;
  int RH, RW;
  int SH, SW, SC;
  int c, P, flip;
  float inv_RW, inv_RH;
};

struct GemmDesc {
  const float* A;
  const float* B;
  float* C;
  int M, N, K;
  int64_t lda, ldb, ldc;
  bool a_t, b_t;
  int epi;
  const float* bias;
  const float* mask;
  int64_t ldm;
  // Scratch for partial products (partial_floats floats).  gemm_dma
  // schedules work with stream-K and needs 2 * grid * tile floats when a
  // tile is shared between blocks (gemm_scratch_floats gives the need of a
  // shape).  gemm_staged splits K when splits > 1: the products of each K
  // slice go to partial[s][M][N] (row stride N) and a second pass sums the
  // slices in order s = 0..splits-1 before the epilogue.
  int splits;
  float* partial;
  int64_t partial_floats = 0;
  // Conv weight-gradient store: when perm_c > 0 the final value for
  // (row = co, col = kk) with kk = (ky*c + kx)*Ci + ci is written to
  // C[co*ldc + ci*c*c + ky*c + kx] (only kk < perm_k are stored).
  int perm_c, perm_ci, perm_k;
  // Algorithmic flops for profiling (0: 2*M*N*K).  Conv products pass the
  // unpadded reduction length here.
  double flops;
  // When set (dedw form only), B gets an implicit column of ones after its
  // last column and that column's results -- the row sums of op(A), i.e. the
  // bias gradient -- are written to ones_out[0..M).  Partial buffers then
  // hold splits*M*(N+1) floats.
  float* ones_out;
  // Add every final result into its destination instead of storing it
  // (with EPI_STORE only; used to accumulate a gradient into a GradBuf).
  bool accum = false;
  // Fused training step: when urule >= 0 the final values are gradients
  // and the rule (SGD_PLAIN / SGD_MOMENTUM / SGD_ADAGRAD) is applied to the
  // parameters at C (and the ones column's at ones_out) with state at the
  // same offsets in ustate (ustate_b for the ones column); nothing else is
  // stored.  Requires EPI_STORE and no accum.
  int urule = -1;
  float* ustate = nullptr;
  float* ustate_b = nullptr;
  float eta = 0.f, mu = 0.f, eps = 0.f, decay = 0.f;
  // Every final value is multiplied by gscale (one rounding) before it is
  // stored or accumulated: the worker-side gradient scaling of SPRINT
  // Algorithm 1.  Must be 1 with an update rule.
  float gscale = 1.f;
  // Kernel/tile override (-1: chosen from the shape and the operands).
  int cfg = -1;
  // gemm_dma schedule override: sk_grid > 0 forces that many blocks with
  // the first sk_dp tiles done whole and the rest by stream-K.
  int sk_grid = -1, sk_dp = 0;
  // The product may take the skinny kernels (a logits layer's forward and
  // input-gradient products): set for fc layers and standalone products,
  // not for convolutions, whose explicit and implicit paths keep one sum
  // order.
  bool skinny = false;
  // The product runs beside the side stream's weight-gradient products (an input-gradient product of the
  // overlapped backward pass): it keeps the instances that fit three blocks per CU, so those products
  // keep their share of each CU.
  bool beside_side = false;
  // Implicit GEMM: 1 = A (K-contiguous, not transposed) is gathered by cv
  // (A and lda are ignored); 2 = B (row-contiguous, transposed) is (B and
  // ldb are ignored).  Needs cv.SC % 16 == 0 for A, % 4 == 0 for B.
  int gather = 0;
  ConvGather cv{};
};

int gemm(const GemmDesc& d, hipStream_t s);

// Split count for gemm_staged for a product with an M x Nt output (Nt
// counts the ones column when there is one) and reduction length K.
int gemm_pick_splits(int M, int Nt, int K);

// Scratch floats gemm() needs in GemmDesc::partial for such a product on the
// current device (gemm_dma's stream-K slots, or gemm_staged's splits).
// `fused`: the dedw form with an update rule in the epilogue.
int64_t gemm_scratch_floats(int M, int Nt, int K, bool a_t, bool b_t, bool fused, int splits);

// The automatic direct-load (gemm_dma) schedule of an M x Nt x K product of the given form (0 nt, 1 tn,
// 2 nn, 3 tt), not gathered, with unlimited scratch: out[0..11] = tile rows, tile columns, grid, whole tiles
// first, stream-K k-slices, group rows, group columns, edge-last bits, tile rows count, tile columns count,
// k-slices per tile, compute units.  Host only.
int gemm_plan_query(int M, int Nt, int K, int form, int64_t* out);

}  // namespace sgd
