// Host launchers of the layer kernels (internal; see layers.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace sgd {

int im2col(const float* x, bool x_nchw, float* col, int N, int Ci, int H, int W, int c, int P, int Ho, int Wo,
           int ldk, hipStream_t s);
int col2im(const float* dcol, const float* mask_act, float* dx, int N, int Ci, int H, int W, int c, int P, int Ho,
           int Wo, int ldk, hipStream_t s);
// One conv layer's weights w[Co][Ci][c][c] and the repacked copies made of
// them: wrep[co][(ky*c + kx)*Ci + ci] in rows of ldk floats (zero padded) and,
// when wdx is set, wdx[ci][(ky*c + kx)*Co + co] (the gather-form dedx's B
// operand).  repack_conv_weights makes all of them in one launch.
struct RepackLayer {
  const float* w;
  float* wrep;
  float* wdx;
  int Co, Ci, c, ldk;
};
int repack_conv_weights(const RepackLayer* layers, int n, hipStream_t s);
int maxpool_fwd(const float* x, float* y, uint8_t* argmax, int N, int C, int H, int W, int p, bool out_nchw,
                hipStream_t s);
int maxpool_bwd(const float* dy, const uint8_t* argmax, const float* pooled, float* dx, int N, int C, int H, int W,
                int p, bool out_nchw, hipStream_t s);
int softmax_ce(const float* z, const int32_t* y, float* dz, float* row_loss, float* loss, int N, int C,
               float scale, hipStream_t s);

// update.hip
int accumulate(float* buf, const float* const* grads, int k, bool first_is_copy, int64_t n, hipStream_t s);
int apply_rule(float* W, float* state, const float* const* grads, int k, int64_t n, int rule, float eta, float mu,
               float eps, float decay, hipStream_t s);
int stream_ref(float* const* outs, int n_out, const float* const* ins, int n_in, int64_t n, int groups,
               hipStream_t s);

}  // namespace sgd
