// Bandwidth-bound layer kernels of the SGD step: im2col / col2im, weight
// repacking, max-pooling forward and backward and softmax cross-entropy.
//
// Activation layout.  Every activation the library produces is NHWC
// (channels fastest), which is the natural row layout of the conv forward
// product (rows = pixels, columns = output channels).  Only the caller's
// images are NCHW, and the tensor feeding the first fc layer is written in
// NCHW order so that the fc input is flattened in (c, h, w) order.
//
// im2col column order is (ky, kx, ci): a row of the im2col matrix is c*c runs
// of Ci contiguous channels, so both its reads (NHWC) and writes are
// contiguous.  The weights are repacked to the same order once per step.
#include "common.h"
#include "layers.h"

namespace sgd {
namespace {

constexpr int kBlock = 256;

int grid_for(int64_t work) { return (int)std::min<int64_t>(std::max<int64_t>(ceil_div(work, kBlock), 1), 65536); }

#define GRID_STRIDE(i, n) \
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (n); i += (int64_t)gridDim.x * blockDim.x)

// ---------------------------------------------------------------- im2col ----
// Col[p][kk] = x[n][iy][ix][ci] with p = (n, oy, ox), kk = (ky*c + kx)*Ci + ci,
// iy = oy + ky - P, ix = ox + kx - P; 0 outside the image and for the pad
// columns K <= kk < ldk.
__global__ void im2col_nhwc_vec4(const float* __restrict__ x, float* __restrict__ col, int N, int Ci, int H,
                                 int W, int c, int P, int Ho, int Wo, int ldk) {
  const int cq = Ci / 4;
  const int64_t per_row = (int64_t)c * c * cq;
  const int64_t total = (int64_t)N * Ho * Wo * per_row;
  GRID_STRIDE(i, total) {
    const int64_t p = i / per_row;
    const int r = (int)(i - p * per_row);
    const int tap = r / cq, q = r - tap * cq;
    const int ky = tap / c, kx = tap - ky * c;
    const int ox = (int)(p % Wo);
    const int64_t t = p / Wo;
    const int oy = (int)(t % Ho);
    const int n = (int)(t / Ho);
    const int iy = oy + ky - P, ix = ox + kx - P;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (iy >= 0 && iy < H && ix >= 0 && ix < W)
      v = *reinterpret_cast<const float4*>(x + (((int64_t)n * H + iy) * W + ix) * Ci + 4 * q);
    *reinterpret_cast<float4*>(col + p * ldk + (int64_t)tap * Ci + 4 * q) = v;
  }
}

template <bool NCHW>
__global__ void im2col_scalar(const float* __restrict__ x, float* __restrict__ col, int N, int Ci, int H, int W,
                              int c, int P, int Ho, int Wo, int ldk) {
  const int K = c * c * Ci;
  const int64_t total = (int64_t)N * Ho * Wo * ldk;
  GRID_STRIDE(i, total) {
    const int64_t p = i / ldk;
    const int kk = (int)(i - p * ldk);
    float v = 0.f;
    if (kk < K) {
      const int tap = kk / Ci, ci = kk - tap * Ci;
      const int ky = tap / c, kx = tap - ky * c;
      const int ox = (int)(p % Wo);
      const int64_t t = p / Wo;
      const int oy = (int)(t % Ho);
      const int n = (int)(t / Ho);
      const int iy = oy + ky - P, ix = ox + kx - P;
      if (iy >= 0 && iy < H && ix >= 0 && ix < W)
        v = NCHW ? x[(((int64_t)n * Ci + ci) * H + iy) * W + ix] : x[(((int64_t)n * H + iy) * W + ix) * Ci + ci];
    }
    col[i] = v;
  }
}

// The general im2col one float4 of a column-matrix row per thread (ldk % 4
// == 0, fewer than 2^31 quads): thread i writes Col[p][4q .. 4q+3] with
// p = i / (ldk/4), q = i % (ldk/4), so consecutive threads store consecutive
// 16 bytes; the index math is 32-bit.  Same values as im2col_scalar.
template <bool NCHW>
__global__ void im2col_quad(const float* __restrict__ x, float4* __restrict__ col, int N, int Ci, int H, int W,
                            int c, int P, int Ho, int Wo, int ldk) {
  const int K = c * c * Ci;
  const int q4 = ldk / 4;
  const int total = N * Ho * Wo * q4;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    const int p = i / q4;
    const int q = i - p * q4;
    const int ox = p % Wo;
    const int t = p / Wo;
    const int oy = t % Ho;
    const int n = t / Ho;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kk = 4 * q + e;
      v[e] = 0.f;
      if (kk < K) {
        const int tap = kk / Ci, ci = kk - tap * Ci;
        const int ky = tap / c, kx = tap - ky * c;
        const int iy = oy + ky - P, ix = ox + kx - P;
        if (iy >= 0 && iy < H && ix >= 0 && ix < W)
          v[e] = NCHW ? x[(((int64_t)n * Ci + ci) * H + iy) * W + ix] : x[(((int64_t)n * H + iy) * W + ix) * Ci + ci];
      }
    }
    col[i] = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// ---------------------------------------------------------------- col2im ----
// dx[n][iy][ix][ci] = sum over (ky, kx) in row-major order of
// dcol[(n, iy - ky + P, ix - kx + P)][(ky*c + kx)*Ci + ci] (taps outside the
// output map skipped), then multiplied by the ReLU derivative [a > 0] of the
// conv's input activation when `a` is given.  A gather: each output is
// written once, no atomics.
__global__ void col2im_nhwc_vec4(const float* __restrict__ dcol, const float* __restrict__ a,
                                 float* __restrict__ dx, int N, int Ci, int H, int W, int c, int P, int Ho, int Wo,
                                 int ldk) {
  const int cq = Ci / 4;
  const int64_t total = (int64_t)N * H * W * cq;
  GRID_STRIDE(i, total) {
    const int q = (int)(i % cq);
    const int64_t pix = i / cq;
    const int ix = (int)(pix % W);
    const int64_t t = pix / W;
    const int iy = (int)(t % H);
    const int n = (int)(t / H);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int ky = 0; ky < c; ++ky) {
      const int oy = iy - ky + P;
      if (oy < 0 || oy >= Ho) continue;
      for (int kx = 0; kx < c; ++kx) {
        const int ox = ix - kx + P;
        if (ox < 0 || ox >= Wo) continue;
        const float4 v = *reinterpret_cast<const float4*>(
            dcol + (((int64_t)n * Ho + oy) * Wo + ox) * ldk + (int64_t)(ky * c + kx) * Ci + 4 * q);
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
      }
    }
    if (a) {
      const float4 m = *reinterpret_cast<const float4*>(a + i * 4);
      s.x = m.x > 0.f ? s.x : 0.f;
      s.y = m.y > 0.f ? s.y : 0.f;
      s.z = m.z > 0.f ? s.z : 0.f;
      s.w = m.w > 0.f ? s.w : 0.f;
    }
    *reinterpret_cast<float4*>(dx + i * 4) = s;
  }
}

__global__ void col2im_nhwc_scalar(const float* __restrict__ dcol, const float* __restrict__ a,
                                   float* __restrict__ dx, int N, int Ci, int H, int W, int c, int P, int Ho,
                                   int Wo, int ldk) {
  const int64_t total = (int64_t)N * H * W * Ci;
  GRID_STRIDE(i, total) {
    const int ci = (int)(i % Ci);
    const int64_t pix = i / Ci;
    const int ix = (int)(pix % W);
    const int64_t t = pix / W;
    const int iy = (int)(t % H);
    const int n = (int)(t / H);
    float s = 0.f;
    for (int ky = 0; ky < c; ++ky) {
      const int oy = iy - ky + P;
      if (oy < 0 || oy >= Ho) continue;
      for (int kx = 0; kx < c; ++kx) {
        const int ox = ix - kx + P;
        if (ox < 0 || ox >= Wo) continue;
        s += dcol[(((int64_t)n * Ho + oy) * Wo + ox) * ldk + (int64_t)(ky * c + kx) * Ci + ci];
      }
    }
    if (a) s = a[i] > 0.f ? s : 0.f;
    dx[i] = s;
  }
}

// ------------------------------------------------------- weight repacking ----
// Every conv layer's weights W[co][ci][ky][kx] are copied, once per step and
// in one launch for all layers, to
//   W'[co][(ky*c + kx)*Ci + ci]   rows of ldk floats, zero past c*c*Ci: the B
//                                 operand of the forward product (and of the
//                                 explicit dCol product), im2col's column order
//   W''[ci][(ky*c + kx)*Co + co]  the B operand of the gather-form dedx
//                                 product (each input pixel gathers its c*c
//                                 taps of the output gradient, Co channels each)
// The per-layer copies are small and latency-bound, so one launch replaces
// two per layer.  W'' is a transpose (neighbouring outputs come from sources
// Ci*c*c floats apart), so each block stages a tile of cot output channels x
// cit input channels x c*c taps in LDS: the tile is read as cot contiguous
// runs of cit*c*c floats and written as runs of cit floats (W') and cot
// floats (W'').  Blocks are numbered job by job.
constexpr int kMaxRepackJobs = 32;
constexpr int kRepackLds = 12800;  // floats of staged tile: cot * (cit*c*c + 1)
struct RepackJob {
  const float* w;
  float* wrep;
  float* wdx;        // nullptr: no W''
  int Co, Ci, c, ldk;
  int cot, cit;      // tile: output x input channels
  int tiles_ci;      // tiles along Ci
  int block0;        // first block of this job
  int vec;           // 3x3 kernel: Ci, Co multiples of 4 and w 16-byte aligned
};
struct RepackJobs {
  RepackJob j[kMaxRepackJobs];
  int n;
};

__global__ __launch_bounds__(kBlock) void repack_conv_weights_kernel(RepackJobs J) {
  __shared__ float T[kRepackLds];
  int l = 0;
  while (l + 1 < J.n && J.j[l + 1].block0 <= (int)blockIdx.x) ++l;
  const RepackJob b = J.j[l];
  const int bi = (int)blockIdx.x - b.block0;
  const int tco = bi / b.tiles_ci, tci = bi - tco * b.tiles_ci;
  const int co0 = tco * b.cot, ci0 = tci * b.cit;
  const int cc = b.c * b.c;
  const int nco = min(b.cot, b.Co - co0), nci = min(b.cit, b.Ci - ci0);
  const int seg = nci * cc;           // floats of one output channel in the tile
  const int ld = b.cit * cc + 1;      // LDS row stride (odd: reads along co are conflict-free)
  // T[co][ci*cc + tap] = W[co0 + co][ci0 + ci][tap]: one contiguous run per row.
  for (int t = threadIdx.x; t < nco * seg; t += kBlock) {
    const int co = t / seg, r = t - co * seg;
    T[co * ld + r] = b.w[((int64_t)(co0 + co) * b.Ci + ci0) * cc + r];
  }
  __syncthreads();
  // W'[co][tap*Ci + ci0 + ci]: runs of nci floats.
  for (int t = threadIdx.x; t < nco * cc * nci; t += kBlock) {
    const int r = t / nci, ci = t - r * nci;
    const int co = r / cc, tap = r - co * cc;
    b.wrep[(int64_t)(co0 + co) * b.ldk + tap * b.Ci + ci0 + ci] = T[co * ld + ci * cc + tap];
  }
  // The zero columns [c*c*Ci, ldk) of W' rows, written by the last tile along Ci.
  if (tci == b.tiles_ci - 1) {
    const int pad = b.ldk - cc * b.Ci;
    for (int t = threadIdx.x; t < nco * pad; t += kBlock) {
      const int co = t / pad, q = t - co * pad;
      b.wrep[(int64_t)(co0 + co) * b.ldk + cc * b.Ci + q] = 0.f;
    }
  }
  // W''[ci0 + ci][tap*Co + co0 + co]: runs of nco floats.
  if (b.wdx) {
    for (int t = threadIdx.x; t < nci * cc * nco; t += kBlock) {
      const int r = t / nco, co = t - r * nco;
      const int ci = r / cc, tap = r - ci * cc;
      b.wdx[(int64_t)(ci0 + ci) * cc * b.Co + (int64_t)tap * b.Co + co0 + co] = T[co * ld + ci * cc + tap];
    }
  }
}

// Small layers of other filter sizes (LeNet-5's 5x5 convolutions: a few thousand floats in all):
// one thread per destination float of W' and W'', no staging.  There the staged kernel runs as one or
// two blocks whose serial loops bound the copy; here every thread does one load and one store.
// Threads are numbered job by job: W' (Co x ldk, the zero columns included), then W'' if wanted.
constexpr int64_t kRepackDirectMax = 1 << 16;  // destination floats of all such layers
struct RepackDirectJob {
  const float* w;
  float* wrep;
  float* wdx;  // nullptr: no W''
  int Co, Ci, c, ldk;
  int start;  // first thread of the job
};
struct RepackDirectJobs {
  RepackDirectJob j[kMaxRepackJobs];
  int n, total;
};

__global__ __launch_bounds__(kBlock) void repack_conv_direct_kernel(RepackDirectJobs J) {
  const int t = (int)(blockIdx.x * kBlock + threadIdx.x);
  if (t >= J.total) return;
  int l = 0;
  while (l + 1 < J.n && J.j[l + 1].start <= t) ++l;
  const RepackDirectJob b = J.j[l];
  const int cc = b.c * b.c;
  int i = t - b.start;
  const int nrep = b.Co * b.ldk;
  if (i < nrep) {  // W'[co][tap*Ci + ci]
    const int co = i / b.ldk, k = i - co * b.ldk;
    float v = 0.f;
    if (k < cc * b.Ci) {
      const int tap = k / b.Ci, ci = k - tap * b.Ci;
      v = b.w[(co * b.Ci + ci) * cc + tap];
    }
    b.wrep[i] = v;
    return;
  }
  i -= nrep;  // W''[ci][tap*Co + co]
  const int r = i / b.Co, co = i - r * b.Co;
  const int ci = r / cc, tap = r - ci * cc;
  b.wdx[i] = b.w[(co * b.Ci + ci) * cc + tap];
}

// The same for 3x3 filters (every conv of the VGG networks) with the tile
// fixed at 32 output x 16 input channels: the index arithmetic is shifts and
// multiplications by constants, and the 18.5 KiB tile lets more blocks share
// a CU.  Threads past a partial tile's edge skip their element.  When Ci and
// Co are multiples of 4 and the pointers 16-byte aligned (vec), every global
// load and store moves a float4.
constexpr int kR3Co = 32, kR3Ci = 16, kR3Ld = kR3Ci * 9 + 1;
__global__ __launch_bounds__(kBlock) void repack_conv3x3_kernel(RepackJobs J) {
  __shared__ float T[kR3Co * kR3Ld];
  int l = 0;
  while (l + 1 < J.n && J.j[l + 1].block0 <= (int)blockIdx.x) ++l;
  const RepackJob b = J.j[l];
  const int bi = (int)blockIdx.x - b.block0;
  const int tco = bi / b.tiles_ci, tci = bi - tco * b.tiles_ci;
  const int co0 = tco * kR3Co, ci0 = tci * kR3Ci;
  const int nco = min(kR3Co, b.Co - co0), nci = min(kR3Ci, b.Ci - ci0);
  const int seg = nci * 9;
  if (b.vec) {
    // Whole float4s: nci, nco, seg, the source rows, ldk and every run start
    // are multiples of 4.
    for (int t = threadIdx.x; t < kR3Co * kR3Ci * 9 / 4; t += kBlock) {
      const int co = t / (kR3Ci * 9 / 4), r = 4 * (t - co * (kR3Ci * 9 / 4));
      if (co < nco && r < seg) {
        const float4 v = *reinterpret_cast<const float4*>(b.w + ((int64_t)(co0 + co) * b.Ci + ci0) * 9 + r);
        float* d = T + co * kR3Ld + r;
        d[0] = v.x;
        d[1] = v.y;
        d[2] = v.z;
        d[3] = v.w;
      }
    }
  } else {
    for (int t = threadIdx.x; t < kR3Co * kR3Ci * 9; t += kBlock) {
      const int co = t / (kR3Ci * 9), r = t - co * (kR3Ci * 9);
      if (co < nco && r < seg) T[co * kR3Ld + r] = b.w[((int64_t)(co0 + co) * b.Ci + ci0) * 9 + r];
    }
  }
  __syncthreads();
  if (b.vec) {
    for (int t = threadIdx.x; t < kR3Co * 9 * kR3Ci / 4; t += kBlock) {
      const int ci = 4 * (t & (kR3Ci / 4 - 1)), r = t / (kR3Ci / 4);
      const int co = r / 9, tap = r - co * 9;
      if (co < nco && ci < nci) {
        const float* src = T + co * kR3Ld + ci * 9 + tap;
        *reinterpret_cast<float4*>(b.wrep + (int64_t)(co0 + co) * b.ldk + tap * b.Ci + ci0 + ci) =
            make_float4(src[0], src[9], src[18], src[27]);
      }
    }
  } else {
    for (int t = threadIdx.x; t < kR3Co * 9 * kR3Ci; t += kBlock) {
      const int ci = t & (kR3Ci - 1), r = t / kR3Ci;
      const int co = r / 9, tap = r - co * 9;
      if (co < nco && ci < nci)
        b.wrep[(int64_t)(co0 + co) * b.ldk + tap * b.Ci + ci0 + ci] = T[co * kR3Ld + ci * 9 + tap];
    }
  }
  if (tci == b.tiles_ci - 1) {
    const int pad = b.ldk - 9 * b.Ci;
    for (int t = threadIdx.x; t < nco * pad; t += kBlock) {
      const int co = t / pad, q = t - co * pad;
      b.wrep[(int64_t)(co0 + co) * b.ldk + 9 * b.Ci + q] = 0.f;
    }
  }
  if (b.wdx && b.vec) {
    for (int t = threadIdx.x; t < kR3Ci * 9 * kR3Co / 4; t += kBlock) {
      const int co = 4 * (t & (kR3Co / 4 - 1)), r = t / (kR3Co / 4);
      const int ci = r / 9, tap = r - ci * 9;
      if (co < nco && ci < nci) {
        const float* src = T + co * kR3Ld + ci * 9 + tap;
        *reinterpret_cast<float4*>(b.wdx + (int64_t)(ci0 + ci) * 9 * b.Co + (int64_t)tap * b.Co + co0 + co) =
            make_float4(src[0], src[kR3Ld], src[2 * kR3Ld], src[3 * kR3Ld]);
      }
    }
  } else if (b.wdx) {
    for (int t = threadIdx.x; t < kR3Ci * 9 * kR3Co; t += kBlock) {
      const int co = t & (kR3Co - 1), r = t / kR3Co;
      const int ci = r / 9, tap = r - ci * 9;
      if (co < nco && ci < nci)
        b.wdx[(int64_t)(ci0 + ci) * 9 * b.Co + (int64_t)tap * b.Co + co0 + co] = T[co * kR3Ld + ci * 9 + tap];
    }
  }
}

// --------------------------------------------------------------- max pool ----
// p x p windows, stride p, over NHWC input.  The window is scanned row-major
// and a strict '>' keeps the first maximum; a NaN in the window makes the
// output NaN.  argmax stores the window-local index ky*p + kx.  The output
// (and argmax) is NHWC, or NCHW when out_nchw is set.
__global__ void maxpool_fwd_kernel(const float* __restrict__ x, float* __restrict__ y,
                                   uint8_t* __restrict__ argmax, int N, int C, int H, int W, int p, int out_nchw) {
  const int Ho = H / p, Wo = W / p;
  const int64_t total = (int64_t)N * Ho * Wo * C;
  GRID_STRIDE(i, total) {
    const int ch = (int)(i % C);
    const int64_t t = i / C;
    const int ox = (int)(t % Wo);
    const int64_t t2 = t / Wo;
    const int oy = (int)(t2 % Ho);
    const int n = (int)(t2 / Ho);
    const float* base = x + (((int64_t)n * H + oy * p) * W + ox * p) * C + ch;
    float best = base[0];
    int bi = 0;
    bool nan = false;
    for (int ky = 0; ky < p; ++ky)
      for (int kx = 0; kx < p; ++kx) {
        const float v = base[((int64_t)ky * W + kx) * C];
        if (v != v) nan = true;
        if (v > best) {
          best = v;
          bi = ky * p + kx;
        }
      }
    const int64_t o = out_nchw ? (((int64_t)n * C + ch) * Ho + oy) * Wo + ox : i;
    y[o] = nan ? __builtin_nanf("") : best;
    argmax[o] = (uint8_t)bi;
  }
}

// Gather form of the pooling backward pass: each input position takes the
// window's gradient if it is the window's argmax, else 0.  When `pooled` is
// given (the pool follows a ReLU) the result is also multiplied by the ReLU
// derivative, which at the argmax equals [pooled > 0].  dx is NHWC; dy,
// argmax and pooled use the forward output layout.
__global__ void maxpool_bwd_kernel(const float* __restrict__ dy, const uint8_t* __restrict__ argmax,
                                   const float* __restrict__ pooled, float* __restrict__ dx, int N, int C, int H,
                                   int W, int p, int out_nchw) {
  const int Ho = H / p, Wo = W / p;
  const int64_t total = (int64_t)N * H * W * C;
  GRID_STRIDE(i, total) {
    const int ch = (int)(i % C);
    const int64_t t = i / C;
    const int ix = (int)(t % W);
    const int64_t t2 = t / W;
    const int iy = (int)(t2 % H);
    const int n = (int)(t2 / H);
    const int oy = iy / p, ox = ix / p;
    const int local = (iy - oy * p) * p + (ix - ox * p);
    const int64_t o = out_nchw ? (((int64_t)n * C + ch) * Ho + oy) * Wo + ox
                               : (((int64_t)n * Ho + oy) * Wo + ox) * C + ch;
    float g = 0.f;
    if (argmax[o] == local) {
      g = dy[o];
      if (pooled && !(pooled[o] > 0.f)) g = 0.f;
    }
    dx[i] = g;
  }
}

// Four channels per thread (C % 4 == 0, NHWC in and out, 16-byte aligned,
// fewer than 2^31 quads): thread i owns output pixel i / (C/4), channels
// 4*(i % (C/4)) .. +3, so every load and store is a float4 (the argmax a
// uchar4).  Per channel the same comparisons as maxpool_fwd_kernel.
__global__ void maxpool_fwd_vec4(const float4* __restrict__ x, float4* __restrict__ y, uchar4* __restrict__ argmax,
                                 int N, int C4, int H, int W, int p) {
  const int Ho = H / p, Wo = W / p;
  const int total = N * Ho * Wo * C4;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    const int c4 = i % C4;
    int t = i / C4;
    const int ox = t % Wo;
    t /= Wo;
    const int oy = t % Ho;
    const int n = t / Ho;
    const float4* base = x + ((int64_t)(n * H + oy * p) * W + ox * p) * C4 + c4;
    float b[4], v0[4];
    int bi[4] = {0, 0, 0, 0};
    bool nan[4] = {false, false, false, false};
    {
      const float4 v = base[0];
      b[0] = v.x, b[1] = v.y, b[2] = v.z, b[3] = v.w;
    }
    for (int ky = 0; ky < p; ++ky)
      for (int kx = 0; kx < p; ++kx) {
        const float4 v = base[((int64_t)ky * W + kx) * C4];
        v0[0] = v.x, v0[1] = v.y, v0[2] = v.z, v0[3] = v.w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (v0[q] != v0[q]) nan[q] = true;
          if (v0[q] > b[q]) {
            b[q] = v0[q];
            bi[q] = ky * p + kx;
          }
        }
      }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (nan[q]) b[q] = __builtin_nanf("");
    y[i] = make_float4(b[0], b[1], b[2], b[3]);
    argmax[i] = make_uchar4((unsigned char)bi[0], (unsigned char)bi[1], (unsigned char)bi[2], (unsigned char)bi[3]);
  }
}

// The backward pass in the same layout: thread i reads its window's
// gradient, argmax (and pooled value) once and writes all p x p input
// positions of the window, so the only large stream is the float4 stores of
// dx.  Per channel the same rule as maxpool_bwd_kernel.
__global__ void maxpool_bwd_vec4(const float4* __restrict__ dy, const uchar4* __restrict__ argmax,
                                 const float4* __restrict__ pooled, float4* __restrict__ dx, int N, int C4, int H,
                                 int W, int p) {
  const int Ho = H / p, Wo = W / p;
  const int total = N * Ho * Wo * C4;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    const int c4 = i % C4;
    int t = i / C4;
    const int ox = t % Wo;
    t /= Wo;
    const int oy = t % Ho;
    const int n = t / Ho;
    const float4 d = dy[i];
    const uchar4 am = argmax[i];
    float g[4] = {d.x, d.y, d.z, d.w};
    const int a[4] = {am.x, am.y, am.z, am.w};
    if (pooled) {
      const float4 pv = pooled[i];
      const float pq[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (!(pq[q] > 0.f)) g[q] = 0.f;
    }
    float4* base = dx + ((int64_t)(n * H + oy * p) * W + ox * p) * C4 + c4;
    for (int ky = 0; ky < p; ++ky)
      for (int kx = 0; kx < p; ++kx) {
        const int l = ky * p + kx;
        base[((int64_t)ky * W + kx) * C4] =
            make_float4(a[0] == l ? g[0] : 0.f, a[1] == l ? g[1] : 0.f, a[2] == l ? g[2] : 0.f, a[3] == l ? g[3] : 0.f);
      }
  }
}

// ------------------------------------------------------ softmax + CE loss ----
// One wavefront per sample row.  lse = m + log(sum exp(z - m)), the row loss
// lse - z[y], and dz = scale * (exp(z - lse) - [j == y]).  Wavefront
// reductions use a fixed butterfly, so results are deterministic.
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// One row of softmax-CE on one wavefront: writes the row's logit gradient
// and returns its loss (every lane gets it).
__device__ __forceinline__ float softmax_ce_row(const float* __restrict__ z, const int32_t* __restrict__ y,
                                                float* __restrict__ dz, int row, int C, float scale, int lane) {
  const float* zr = z + (int64_t)row * C;
  float m = -INFINITY;
  bool nan = false;
  for (int j = lane; j < C; j += 64) {
    const float v = zr[j];
    nan |= (v != v);
    m = fmaxf(m, v);
  }
  m = wave_max(m);
  float se = 0.f;
  for (int j = lane; j < C; j += 64) se += expf(zr[j] - m);
  se = wave_sum(se);
  nan = __any(nan);
  const int lbl = y[row];
  // A label outside [0, C) is never used as an index: the row's loss and
  // logit gradient become NaN instead.
  const bool ok = (unsigned)lbl < (unsigned)C;
  const float lse = (nan || !ok) ? __builtin_nanf("") : m + logf(se);
  for (int j = lane; j < C; j += 64) dz[(int64_t)row * C + j] = scale * (expf(zr[j] - lse) - (j == lbl ? 1.f : 0.f));
  return lse - zr[ok ? lbl : 0];
}

__global__ void softmax_ce_kernel(const float* __restrict__ z, const int32_t* __restrict__ y,
                                  float* __restrict__ dz, float* __restrict__ row_loss, int N, int C, float scale) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (row >= N) return;
  const float l = softmax_ce_row(z, y, dz, row, C, scale, lane);
  if (lane == 0) row_loss[row] = l;
}

// Small batches (N <= kFusedRows): every row and the loss in one block of
// 1024 threads -- each wavefront takes rows w, w + 16, ..., then threads
// 0..kBlock-1 sum the row losses with loss_sum_kernel's reduction tree (one
// term per thread), so the loss is bitwise the same as the two-kernel path.
constexpr int kFusedRows = 64;
__global__ __launch_bounds__(1024) void softmax_ce_loss_kernel(const float* __restrict__ z,
                                                               const int32_t* __restrict__ y, float* __restrict__ dz,
                                                               float* __restrict__ row_loss, float* __restrict__ loss,
                                                               int N, int C, float scale, float lscale) {
  __shared__ float sh[kBlock];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x < kBlock) sh[threadIdx.x] = 0.f;
  __syncthreads();
  for (int row = wave; row < N; row += 16) {
    const float l = softmax_ce_row(z, y, dz, row, C, scale, lane);
    if (lane == 0) {
      row_loss[row] = l;
      sh[row] = l;
    }
  }
  __syncthreads();
  for (int o = kBlock / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = lscale * sh[0];
}

// loss = scale * sum of row losses, one block, fixed reduction tree.
__global__ void loss_sum_kernel(const float* __restrict__ row_loss, float* __restrict__ loss, int N, float scale) {
  __shared__ float sh[kBlock];
  float s = 0.f;
  for (int i = threadIdx.x; i < N; i += kBlock) s += row_loss[i];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int o = kBlock / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = scale * sh[0];
}

}  // namespace

int im2col(const float* x, bool x_nchw, float* col, int N, int Ci, int H, int W, int c, int P, int Ho, int Wo,
           int ldk, hipStream_t s) {
  const bool vec = !x_nchw && Ci % 4 == 0 && ldk == c * c * Ci;
  prof_begin("im2col", 0, 4.0 * ((double)N * Ho * Wo * ldk + (double)N * Ci * H * W), s);
  if (vec) {
    const int64_t total = (int64_t)N * Ho * Wo * c * c * (Ci / 4);
    hipLaunchKernelGGL(im2col_nhwc_vec4, dim3(grid_for(total)), dim3(kBlock), 0, s, x, col, N, Ci, H, W, c, P, Ho,
                       Wo, ldk);
  } else if (ldk % 4 == 0 && (reinterpret_cast<uintptr_t>(col) & 15) == 0 &&
             (int64_t)N * Ho * Wo * (ldk / 4) < ((int64_t)1 << 31)) {
    const int64_t quads = (int64_t)N * Ho * Wo * (ldk / 4);
    if (x_nchw)
      hipLaunchKernelGGL(im2col_quad<true>, dim3(grid_for(quads)), dim3(kBlock), 0, s, x,
                         reinterpret_cast<float4*>(col), N, Ci, H, W, c, P, Ho, Wo, ldk);
    else
      hipLaunchKernelGGL(im2col_quad<false>, dim3(grid_for(quads)), dim3(kBlock), 0, s, x,
                         reinterpret_cast<float4*>(col), N, Ci, H, W, c, P, Ho, Wo, ldk);
  } else {
    const int64_t total = (int64_t)N * Ho * Wo * ldk;
    if (x_nchw)
      hipLaunchKernelGGL(im2col_scalar<true>, dim3(grid_for(total)), dim3(kBlock), 0, s, x, col, N, Ci, H, W, c, P,
                         Ho, Wo, ldk);
    else
      hipLaunchKernelGGL(im2col_scalar<false>, dim3(grid_for(total)), dim3(kBlock), 0, s, x, col, N, Ci, H, W, c,
                         P, Ho, Wo, ldk);
  }
  prof_end(s);
  return check_launch("im2col");
}

int col2im(const float* dcol, const float* mask_act, float* dx, int N, int Ci, int H, int W, int c, int P, int Ho,
           int Wo, int ldk, hipStream_t s) {
  prof_begin("col2im", (double)N * Ho * Wo * c * c * Ci,
             4.0 * ((double)N * Ho * Wo * c * c * Ci + (mask_act ? 2.0 : 1.0) * N * H * W * Ci), s);
  if (Ci % 4 == 0 && ldk % 4 == 0) {
    const int64_t total = (int64_t)N * H * W * (Ci / 4);
    hipLaunchKernelGGL(col2im_nhwc_vec4, dim3(grid_for(total)), dim3(kBlock), 0, s, dcol, mask_act, dx, N, Ci, H,
                       W, c, P, Ho, Wo, ldk);
  } else {
    const int64_t total = (int64_t)N * H * W * Ci;
    hipLaunchKernelGGL(col2im_nhwc_scalar, dim3(grid_for(total)), dim3(kBlock), 0, s, dcol, mask_act, dx, N, Ci,
                       H, W, c, P, Ho, Wo, ldk);
  }
  prof_end(s);
  return check_launch("col2im");
}

int repack_conv_weights(const RepackLayer* layers, int n, hipStream_t s) {
  // Two launch tables: 3x3 filters (fixed tile) and everything else.
  for (int pass = 0; pass < 2; ++pass) {
    const bool three = pass == 0;
    RepackJobs J{};
    int blocks = 0;
    double bytes = 0.0;
    auto flush = [&]() -> int {
      if (J.n == 0) return 0;
      prof_begin("repack_weights", 0, bytes, s);
      if (three)
        hipLaunchKernelGGL(repack_conv3x3_kernel, dim3(blocks), dim3(kBlock), 0, s, J);
      else
        hipLaunchKernelGGL(repack_conv_weights_kernel, dim3(blocks), dim3(kBlock), 0, s, J);
      prof_end(s);
      J = RepackJobs{};
      blocks = 0;
      bytes = 0.0;
      return check_launch("repack_conv_weights");
    };
    if (!three) {
      // All of the other layers in one direct launch when they are small.
      RepackDirectJobs D{};
      int64_t total = 0;
      double dbytes = 0.0;
      for (int i = 0; i < n; ++i) {
        const RepackLayer& L = layers[i];
        if (L.c == 3) continue;
        const int64_t cc = (int64_t)L.c * L.c, wfl = (int64_t)L.Co * L.Ci * cc;
        if (D.n == kMaxRepackJobs) {
          total = kRepackDirectMax + 1;
          break;
        }
        D.j[D.n++] = {L.w, L.wrep, L.wdx, L.Co, L.Ci, L.c, L.ldk, (int)std::min<int64_t>(total, INT32_MAX)};
        total += (int64_t)L.Co * L.ldk + (L.wdx ? wfl : 0);
        dbytes += 4.0 * ((L.wdx ? 2.0 : 1.0) * wfl + (double)L.Co * L.ldk + (L.wdx ? wfl : 0.0));
      }
      if (D.n > 0 && total <= kRepackDirectMax) {
        D.total = (int)total;
        prof_begin("repack_weights", 0, dbytes, s);
        hipLaunchKernelGGL(repack_conv_direct_kernel, dim3((unsigned)ceil_div(total, kBlock)), dim3(kBlock), 0, s, D);
        prof_end(s);
        if (int e = check_launch("repack_conv_weights")) return e;
        continue;
      }
    }
    for (int i = 0; i < n; ++i) {
      const RepackLayer& L = layers[i];
      if ((L.c == 3) != three) continue;
      const int cc = L.c * L.c;
      if (cc + 1 > kRepackLds) {
        set_error("repack_conv_weights: filter too large for the staged repack");
        return SGD_EUNSUPPORTED;
      }
      // Largest tile with cot <= 32 and cit <= 16 whose staging fits.
      const int cit = three ? kR3Ci : std::max(1, std::min(16, (kRepackLds / 32 - 1) / cc));
      const int cot = three ? kR3Co : std::max(1, std::min(32, kRepackLds / (cit * cc + 1)));
      const int64_t tiles = ceil_div(L.Co, cot) * ceil_div(L.Ci, cit);
      if (J.n == kMaxRepackJobs || blocks + tiles > INT32_MAX / 2)
        if (int e = flush()) return e;
      RepackJob& b = J.j[J.n++];
      b.w = L.w;
      b.wrep = L.wrep;
      b.wdx = L.wdx;
      b.Co = L.Co;
      b.Ci = L.Ci;
      b.c = L.c;
      b.ldk = L.ldk;
      b.cot = cot;
      b.cit = cit;
      b.tiles_ci = (int)ceil_div(L.Ci, cit);
      b.block0 = blocks;
      b.vec = three && L.Ci % 4 == 0 && L.Co % 4 == 0 && L.ldk % 4 == 0 &&
              reinterpret_cast<uintptr_t>(L.w) % 16 == 0 && reinterpret_cast<uintptr_t>(L.wrep) % 16 == 0 &&
              (!L.wdx || reinterpret_cast<uintptr_t>(L.wdx) % 16 == 0);
      blocks += (int)tiles;
      const double wfl = (double)L.Co * L.Ci * cc;
      bytes += 4.0 * (wfl + (double)L.Co * L.ldk + (L.wdx ? wfl : 0.0));
    }
    if (int e = flush()) return e;
  }
  return 0;
}

namespace {
bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; }
// The float4 pooling kernels: NHWC output, whole channel quads, aligned
// pointers (the argmax as uchar4) and a quad count that fits their int math.
bool pool_vec4_ok(int C, int64_t outputs, bool out_nchw, const void* a, const void* b, const void* am) {
  return !out_nchw && C % 4 == 0 && outputs / 4 < ((int64_t)1 << 31) && aligned16(a) && aligned16(b) &&
         (reinterpret_cast<uintptr_t>(am) & 3) == 0;
}
}  // namespace

int maxpool_fwd(const float* x, float* y, uint8_t* argmax, int N, int C, int H, int W, int p, bool out_nchw,
                hipStream_t s) {
  const int64_t total = (int64_t)N * (H / p) * (W / p) * C;
  prof_begin("maxpool_fwd", (double)N * H * W * C, 4.0 * N * H * W * C + 5.0 * total, s);
  if (pool_vec4_ok(C, total, out_nchw, x, y, argmax))
    hipLaunchKernelGGL(maxpool_fwd_vec4, dim3(grid_for(total / 4)), dim3(kBlock), 0, s,
                       reinterpret_cast<const float4*>(x), reinterpret_cast<float4*>(y),
                       reinterpret_cast<uchar4*>(argmax), N, C / 4, H, W, p);
  else
    hipLaunchKernelGGL(maxpool_fwd_kernel, dim3(grid_for(total)), dim3(kBlock), 0, s, x, y, argmax, N, C, H, W, p,
                       (int)out_nchw);
  prof_end(s);
  return check_launch("maxpool_fwd");
}

int maxpool_bwd(const float* dy, const uint8_t* argmax, const float* pooled, float* dx, int N, int C, int H, int W,
                int p, bool out_nchw, hipStream_t s) {
  const int64_t total = (int64_t)N * H * W * C;
  const double pooled_n = (double)total / ((double)p * p);
  prof_begin("maxpool_bwd", 0, 4.0 * total + pooled_n * (pooled ? 9.0 : 5.0), s);
  const int64_t outs = total / ((int64_t)p * p);
  if (pool_vec4_ok(C, outs, out_nchw, dy, dx, argmax) && (!pooled || aligned16(pooled)))
    hipLaunchKernelGGL(maxpool_bwd_vec4, dim3(grid_for(outs / 4)), dim3(kBlock), 0, s,
                       reinterpret_cast<const float4*>(dy), reinterpret_cast<const uchar4*>(argmax),
                       reinterpret_cast<const float4*>(pooled), reinterpret_cast<float4*>(dx), N, C / 4, H, W, p);
  else
    hipLaunchKernelGGL(maxpool_bwd_kernel, dim3(grid_for(total)), dim3(kBlock), 0, s, dy, argmax, pooled, dx, N, C,
                       H, W, p, (int)out_nchw);
  prof_end(s);
  return check_launch("maxpool_bwd");
}

int softmax_ce(const float* z, const int32_t* y, float* dz, float* row_loss, float* loss, int N, int C,
               float scale, hipStream_t s) {
  static_assert(kFusedRows <= kBlock, "the fused kernel's sum keeps one row loss per thread of the tree");
  if (N <= kFusedRows) {
    prof_begin("softmax_ce", 7.0 * N * C, 4.0 * (2.0 * N * C + 2.0 * N + 1), s);
    hipLaunchKernelGGL(softmax_ce_loss_kernel, dim3(1), dim3(1024), 0, s, z, y, dz, row_loss, loss, N, C, scale,
                       scale);
    prof_end(s);
    return check_launch("softmax_ce");
  }
  const int rows_per_block = kBlock / 64;
  prof_begin("softmax_ce", 6.0 * N * C, 4.0 * (2.0 * N * C + 2.0 * N), s);
  hipLaunchKernelGGL(softmax_ce_kernel, dim3((int)ceil_div(N, rows_per_block)), dim3(kBlock), 0, s, z, y, dz,
                     row_loss, N, C, scale);
  prof_end(s);
  if (int e = check_launch("softmax_ce")) return e;
  prof_begin("loss_sum", N, 4.0 * (N + 1), s);
  hipLaunchKernelGGL(loss_sum_kernel, dim3(1), dim3(kBlock), 0, s, row_loss, loss, N, scale);
  prof_end(s);
  return check_launch("loss_sum");
}

}  // namespace sgd
