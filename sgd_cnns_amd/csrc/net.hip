// Network planner, step orchestration and the C ABI of libsgdstep.
//
// sgd_create_net walks the layer list once on the host: it infers every
// shape (SPRINT report section 3.2 eq. (2), generalised to zero padding),
// lays out the flat parameter vector (eq. (3)), chooses the matrix-product
// split factors and assigns every intermediate tensor a fixed offset in the
// caller's workspace.  sgd_compute_gradient then only enqueues kernels: the
// forward pass layer by layer, softmax cross-entropy, and the backward pass
// in reverse layer order (the dependency order of backpropagation described
// in "Pipelined training with stale weights of deep CNNs", section 2), with
// each layer's dedw / dedb / dedx products as listed in the SPRINT report's
// section 3.3 SGEMM table.
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include <cmath>

#include "common.h"
#include "layers.h"

namespace sgd {

thread_local std::string g_error;

void set_error(const std::string& msg) { g_error = msg; }

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error(std::string(what) + ": " + hipGetErrorString(e));
    return SGD_EDEVICE;
  }
  return 0;
}

// ---------------------------------------------------------------- profiler
struct ProfRec {
  const char* kernel;
  int layer, phase;
  double flops, bytes;
  hipEvent_t beg, end;
  int m, n, k, product;
};

struct Profiler {
  bool on = false;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;  // events reused across recordings
  size_t used = 0;
  int layer = -1, phase = 0;
  int m = 0, n = 0, k = 0;  // shape of the product being launched (0: none)
  int product = -1;         // its index among this recording's products
  int products = 0;
  hipEvent_t get() {
    if (used == pool.size()) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
  ~Profiler() {
    for (hipEvent_t e : pool) (void)hipEventDestroy(e);
  }
};

thread_local Profiler* g_prof = nullptr;

// The stream the weight-gradient products run on, so each overlaps the next
// layer's input-gradient product on the caller's stream (and fills the
// partly occupied last round of each): created on first use per device,
// default priority, with one fork event per weighted layer and a join event.
struct SideStream {
  int dev = -1;
  hipStream_t s = nullptr;
  std::vector<hipEvent_t> ev;
  void release() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
    ev.clear();
    if (s) (void)hipStreamDestroy(s);
    s = nullptr;
    dev = -1;
  }
  // Ready on the current device with n fork events plus the join event.
  int ready(int n) {
    int d = -1;
    if (hipGetDevice(&d) != hipSuccess) return SGD_EDEVICE;
    if (s && d != dev) release();
    if (!s) {
      if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) {
        s = nullptr;
        return SGD_EDEVICE;
      }
      dev = d;
    }
    while ((int)ev.size() < n + 1) {
      hipEvent_t e = nullptr;
      if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return SGD_EDEVICE;
      ev.push_back(e);
    }
    return 0;
  }
  ~SideStream() { release(); }
};

void prof_set_layer(int layer, int phase) {
  if (g_prof) {
    g_prof->layer = layer;
    g_prof->phase = phase;
  }
}

void prof_set_shape(int m, int n, int k) {
  if (g_prof) {
    g_prof->m = m;
    g_prof->n = n;
    g_prof->k = k;
    g_prof->product = m > 0 ? g_prof->products++ : -1;
  }
}

void prof_begin(const char* kernel, double flops, double bytes, hipStream_t s) {
  if (!g_prof || !g_prof->on) return;
  ProfRec r{kernel, g_prof->layer, g_prof->phase, flops, bytes, g_prof->get(), g_prof->get(),
            g_prof->m, g_prof->n, g_prof->k, g_prof->product};
  if (!r.beg || !r.end) return;
  (void)hipEventRecord(r.beg, s);
  g_prof->recs.push_back(r);
}

void prof_end(hipStream_t s) {
  if (!g_prof || !g_prof->on || g_prof->recs.empty()) return;
  (void)hipEventRecord(g_prof->recs.back().end, s);
}

namespace {

struct Tensor {
  int64_t off = -1;  // byte offset in the workspace
  int64_t dims[4] = {0, 0, 0, 0};
  int layout = 0;
};

// One planned stage.  ReLU entries of the layer list are folded into the
// conv/fc stage they follow; an fc fed by a conv map without pooling gets a
// p = 1 "pool" stage that only reorders NHWC to NCHW (the (c, h, w) flatten).
struct Stage {
  int kind = 0;   // SGD_CONV, SGD_MAXPOOL, SGD_FC, SGD_SOFTMAX_CE
  int spec = -1;  // index in the caller's layer list (-1: inserted flatten)
  int input = -1; // producing stage, -1 = the images
  bool relu = false;
  bool first_weighted = false;
  int weighted_rank = -1;  // 0 for the first weighted layer, 1 for the next, ...
  // With the overlap on, this layer's dedw runs on the caller's stream after
  // its dedx (see run_backward), in the caller's-stream scratch, planned with
  // capacity dw_cap in both modes so its schedule does not change.
  bool dw_main = false;
  int64_t dw_cap = 0;
  int N = 0, Ci = 0, H = 0, W = 0;   // input shape (fc: Ci = input width, H = W = 1)
  int Co = 0, Ho = 0, Wo = 0;        // output shape (fc: Co = output width)
  int c = 0, P = 0, p = 1;           // conv filter / padding, pool window
  int K = 0, ldk = 0;                // conv: c*c*Ci and its padded row length
  bool out_nchw = false;             // pool: output written NCHW (feeds an fc)
  int64_t w_off = -1, b_off = -1;    // parameter offsets (elements)
  int split_fwd = 1, split_dw = 1, split_dx = 1;
  // conv: implicit GEMM.  `implicit`: the forward and dedw products gather
  // their im2col operand straight from the NHWC input (no Col in HBM; needs
  // Ci % 16 == 0 and an NHWC input).  `implicit_dx`: dedx is one gather-form
  // product over the output gradient (needs Co % 16 == 0), replacing the dCol
  // product and col2im.
  bool implicit = false, implicit_dx = false;
  Tensor out, dout, col, wrep, wdx, argmax;
};

}  // namespace
}  // namespace sgd

struct sgd_net {
  sgd_input input{};
  int reduction = SGD_REDUCE_MEAN;
  int classes = 0;
  std::vector<sgd_layer> spec;
  std::vector<sgd::Stage> stages;
  std::vector<int> spec_to_stage;  // layer-list index -> stage (ReLU -> its conv/fc)
  int64_t n_params = 0;
  std::vector<int64_t> w_offs, b_offs;
  int64_t ws_bytes = 0;
  sgd::Tensor row_loss;
  // Partial-tile scratch of the GEMMs: one region for the products on the
  // caller's stream, one for the weight-gradient products on the side
  // stream (they run concurrently).
  int64_t partial_off = 0, partial_floats = 0;
  int64_t partial_dw_off = 0, partial_dw_floats = 0;
  // dCol of the conv dedx products (dedw reads Col concurrently).
  int64_t dcol_off = 0;
  sgd::Profiler prof;
  sgd::SideStream side;
  // dedw products on the side stream: overlap_req is the caller's choice
  // (sgd_set_overlap; -1 = not set), overlap_auto the planned default
  int overlap_req = -1;
  bool overlap_auto = true;
  int64_t dw_flops = 0;  // the backward pass's weight-gradient products, 2 m n k summed
  bool implicit = true;  // implicit-GEMM convolutions where the shapes allow
  bool debug = false;    // validate labels on the host before launching
};

// The overlap in effect: the caller's setting, else the planned default.
inline bool overlap_on(const sgd_net* net) { return net->overlap_req >= 0 ? net->overlap_req != 0 : net->overlap_auto; }

namespace sgd {
namespace {
// The dedw products of the first kMainDw weighted layers run on the caller's
// stream after their layer's dedx (see run_backward).  Once the second
// weighted layer's dedx is issued, the caller's stream has nothing left but
// the first layer's dedw, while the side stream still works through the
// chain of the other layers' dedw products.  Measured on MI355X (ms/step
// with 1 / 2 / 3 such layers): MLP-5000 3.071 / 3.072 / 3.127, VGG-CIFAR
// 2.839 / 2.804 / 2.832, VGG-16 25.85 / 25.76 / 26.09, LeNet-5 (launched
// call by call) 0.239 / 0.166 / 0.203.
constexpr int kMainDw = 2;

struct Bump {
  int64_t top = 0;
  int64_t take(int64_t bytes) {
    const int64_t o = top;
    top += round_up(std::max<int64_t>(bytes, 1), 256);
    return o;
  }
};

// dims follow the SGD_LAYOUT_* conventions; a row-major matrix is
// {rows, cols, row stride, 1} and occupies rows * stride elements.
Tensor make_tensor(Bump& b, int64_t elem_bytes, int layout, int64_t d0, int64_t d1, int64_t d2, int64_t d3) {
  Tensor t;
  t.layout = layout;
  t.dims[0] = d0;
  t.dims[1] = d1;
  t.dims[2] = d2;
  t.dims[3] = d3;
  const int64_t elems = layout == SGD_LAYOUT_ROWS ? d0 * d2 : d0 * d1 * d2 * d3;
  t.off = b.take(elem_bytes * elems);
  return t;
}

int fail(int code, const std::string& msg) {
  set_error(msg);
  return code;
}

int plan(sgd_net* net) {
  const sgd_input in = net->input;
  if (in.batch <= 0 || in.channels <= 0 || in.height <= 0 || in.width <= 0)
    return fail(SGD_ESHAPE, "input sizes must be positive");
  auto& st = net->stages;
  st.clear();
  net->w_offs.clear();
  net->b_offs.clear();
  const int n_layers = (int)net->spec.size();
  net->spec_to_stage.assign(n_layers, -1);
  // current activation: producing stage (-1 = images), shape, whether flat
  int cur = -1, C = in.channels, H = in.height, W = in.width;
  bool flat = false;
  int64_t off = 0;
  bool seen_weighted = false;
  int n_weighted = 0;
  for (int i = 0; i < n_layers; ++i) {
    const sgd_layer& L = net->spec[i];
    if (L.kind == SGD_CONV) {
      if (flat) return fail(SGD_EUNSUPPORTED, "layer " + std::to_string(i) + ": conv after fc");
      if (L.out <= 0 || L.kernel <= 0 || L.pad < 0)
        return fail(SGD_ESHAPE, "layer " + std::to_string(i) + ": bad conv parameters");
      Stage s;
      s.kind = SGD_CONV;
      s.spec = i;
      s.input = cur;
      s.N = in.batch;
      s.Ci = C;
      s.H = H;
      s.W = W;
      s.c = L.kernel;
      s.P = L.pad;
      s.Co = L.out;
      s.Ho = H + 2 * L.pad - L.kernel + 1;
      s.Wo = W + 2 * L.pad - L.kernel + 1;
      if (s.Ho < 1 || s.Wo < 1) return fail(SGD_ESHAPE, "layer " + std::to_string(i) + ": conv output is empty");
      s.K = s.c * s.c * s.Ci;
      s.ldk = (int)round_up(s.K, 4);
      s.first_weighted = !seen_weighted;
      s.weighted_rank = n_weighted++;
      seen_weighted = true;
      s.w_off = off;
      off += (int64_t)s.Co * s.K;
      s.b_off = off;
      off += s.Co;
      st.push_back(s);
      cur = (int)st.size() - 1;
      C = s.Co;
      H = s.Ho;
      W = s.Wo;
      net->spec_to_stage[i] = cur;
    } else if (L.kind == SGD_RELU) {
      if (cur < 0 || (st[cur].kind != SGD_CONV && st[cur].kind != SGD_FC) || st[cur].relu ||
          net->spec_to_stage[i - 1] != cur)
        return fail(SGD_EUNSUPPORTED, "layer " + std::to_string(i) + ": ReLU must directly follow a conv or fc");
      st[cur].relu = true;
      net->spec_to_stage[i] = cur;
    } else if (L.kind == SGD_MAXPOOL) {
      if (flat || cur < 0) return fail(SGD_EUNSUPPORTED, "layer " + std::to_string(i) + ": pool needs a conv map");
      if (L.pool <= 0 || L.pool > 15 || H % L.pool || W % L.pool)
        return fail(SGD_ESHAPE, "layer " + std::to_string(i) + ": pool window must divide the feature map");
      Stage s;
      s.kind = SGD_MAXPOOL;
      s.spec = i;
      s.input = cur;
      s.N = in.batch;
      s.Ci = s.Co = C;
      s.H = H;
      s.W = W;
      s.p = L.pool;
      s.Ho = H / L.pool;
      s.Wo = W / L.pool;
      st.push_back(s);
      cur = (int)st.size() - 1;
      H = s.Ho;
      W = s.Wo;
      net->spec_to_stage[i] = cur;
    } else if (L.kind == SGD_FC) {
      if (L.out <= 0) return fail(SGD_ESHAPE, "layer " + std::to_string(i) + ": fc width must be positive");
      if (!flat && cur >= 0 && H * W > 1) {
        if (st[cur].kind == SGD_MAXPOOL) {
          st[cur].out_nchw = true;
        } else {  // conv map without pooling: insert the NHWC -> NCHW flatten
          Stage f;
          f.kind = SGD_MAXPOOL;
          f.input = cur;
          f.N = in.batch;
          f.Ci = f.Co = C;
          f.H = f.Ho = H;
          f.W = f.Wo = W;
          f.p = 1;
          f.out_nchw = true;
          st.push_back(f);
          cur = (int)st.size() - 1;
        }
      }
      Stage s;
      s.kind = SGD_FC;
      s.spec = i;
      s.input = cur;
      s.N = in.batch;
      s.Ci = flat ? C : C * H * W;
      s.H = s.W = 1;
      s.Co = L.out;
      s.Ho = s.Wo = 1;
      s.first_weighted = !seen_weighted;
      s.weighted_rank = n_weighted++;
      seen_weighted = true;
      s.w_off = off;
      off += (int64_t)s.Co * s.Ci;
      s.b_off = off;
      off += s.Co;
      st.push_back(s);
      cur = (int)st.size() - 1;
      C = s.Co;
      H = W = 1;
      flat = true;
      net->spec_to_stage[i] = cur;
    } else if (L.kind == SGD_SOFTMAX_CE) {
      if (i != n_layers - 1) return fail(SGD_ESHAPE, "softmax_ce must be the last layer");
      if (cur < 0 || st[cur].kind != SGD_FC || st[cur].relu || net->spec_to_stage[i - 1] != cur)
        return fail(SGD_EUNSUPPORTED, "softmax_ce must directly follow an fc layer without ReLU");
      Stage s;
      s.kind = SGD_SOFTMAX_CE;
      s.spec = i;
      s.input = cur;
      s.N = in.batch;
      s.Ci = s.Co = C;
      st.push_back(s);
      net->classes = C;
      net->spec_to_stage[i] = (int)st.size() - 1;
    } else {
      return fail(SGD_EINVAL, "layer " + std::to_string(i) + ": unknown kind " + std::to_string(L.kind));
    }
  }
  if (st.empty() || st.back().kind != SGD_SOFTMAX_CE) return fail(SGD_ESHAPE, "last layer must be softmax_ce");
  net->n_params = off;

  // Workspace layout and product split factors.
  Bump b;
  int64_t partial = 0, partial_dw = 0, dcol = 0;
  for (Stage& s : st) {
    const int64_t N = s.N;
    if (s.kind == SGD_CONV) {
      const int64_t P = N * s.Ho * s.Wo;
      const int64_t Pin = N * s.H * s.W;
      // pixel indices of the gathers stay below 2^22 (their float division)
      s.implicit = net->implicit && s.input >= 0 && s.Ci % 16 == 0 && P + 256 < (1 << 22);
      s.implicit_dx = net->implicit && !s.first_weighted && s.Co % 16 == 0 && Pin + 256 < (1 << 22);
      s.wrep = make_tensor(b, 4, SGD_LAYOUT_ROWS, s.Co, s.K, s.ldk, 1);
      if (!s.implicit) s.col = make_tensor(b, 4, SGD_LAYOUT_ROWS, P, s.K, s.ldk, 1);
      if (s.implicit_dx) s.wdx = make_tensor(b, 4, SGD_LAYOUT_ROWS, s.Ci, s.c * s.c * s.Co, s.c * s.c * s.Co, 1);
      s.out = make_tensor(b, 4, SGD_LAYOUT_NHWC, N, s.Ho, s.Wo, s.Co);
      s.dout = make_tensor(b, 4, SGD_LAYOUT_NHWC, N, s.Ho, s.Wo, s.Co);
      s.split_fwd = gemm_pick_splits((int)P, s.Co, s.ldk);
      s.split_dw = gemm_pick_splits(s.Co, s.ldk + 1, (int)P);
      s.split_dx = s.first_weighted ? 1 : gemm_pick_splits((int)P, s.ldk, s.Co);
      partial = std::max(partial, gemm_scratch_floats((int)P, s.Co, s.ldk, false, false, false, s.split_fwd));
      for (bool fused : {false, true}) {
        const int64_t need = gemm_scratch_floats(s.Co, s.ldk + 1, (int)P, true, true, fused, s.split_dw);
        partial_dw = std::max(partial_dw, need);
        s.dw_cap = std::max(s.dw_cap, need);
      }
      s.dw_main = s.weighted_rank < kMainDw;
      if (s.dw_main) partial = std::max(partial, s.dw_cap);
      if (s.implicit_dx) {
        partial = std::max(partial, gemm_scratch_floats((int)Pin, s.Ci, s.c * s.c * s.Co, false, false, false, 1));
      } else if (!s.first_weighted) {
        partial = std::max(partial, gemm_scratch_floats((int)P, s.ldk, s.Co, false, true, false, s.split_dx));
        dcol = std::max(dcol, P * s.ldk);
      }
    } else if (s.kind == SGD_MAXPOOL) {
      const int lay = s.out_nchw ? SGD_LAYOUT_NCHW : SGD_LAYOUT_NHWC;
      if (s.out_nchw) {
        s.out = make_tensor(b, 4, lay, N, s.Co, s.Ho, s.Wo);
        s.argmax = make_tensor(b, 1, lay, N, s.Co, s.Ho, s.Wo);
        s.dout = make_tensor(b, 4, lay, N, s.Co, s.Ho, s.Wo);
      } else {
        s.out = make_tensor(b, 4, lay, N, s.Ho, s.Wo, s.Co);
        s.argmax = make_tensor(b, 1, lay, N, s.Ho, s.Wo, s.Co);
        s.dout = make_tensor(b, 4, lay, N, s.Ho, s.Wo, s.Co);
      }
    } else if (s.kind == SGD_FC) {
      s.out = make_tensor(b, 4, SGD_LAYOUT_ROWS, N, s.Co, s.Co, 1);
      s.dout = make_tensor(b, 4, SGD_LAYOUT_ROWS, N, s.Co, s.Co, 1);
      s.split_fwd = gemm_pick_splits((int)N, s.Co, s.Ci);
      s.split_dw = gemm_pick_splits(s.Co, s.Ci + 1, (int)N);
      s.split_dx = s.first_weighted ? 1 : gemm_pick_splits((int)N, s.Ci, s.Co);
      partial = std::max(partial, gemm_scratch_floats((int)N, s.Co, s.Ci, false, false, false, s.split_fwd));
      for (bool fused : {false, true}) {
        const int64_t need = gemm_scratch_floats(s.Co, s.Ci + 1, (int)N, true, true, fused, s.split_dw);
        partial_dw = std::max(partial_dw, need);
        s.dw_cap = std::max(s.dw_cap, need);
      }
      s.dw_main = s.weighted_rank < kMainDw;
      if (s.dw_main) partial = std::max(partial, s.dw_cap);
      if (!s.first_weighted)
        partial = std::max(partial, gemm_scratch_floats((int)N, s.Ci, s.Co, false, true, false, s.split_dx));
    } else if (s.kind == SGD_SOFTMAX_CE) {
      // the logits' gradient lives in the last fc stage's dout
      net->row_loss = make_tensor(b, 4, SGD_LAYOUT_ROWS, N, 1, 1, 1);
      s.out = net->row_loss;
      s.dout = st[s.input].dout;
    }
  }
  // The side stream pays when the weight-gradient products are large enough
  // to leave partly filled rounds for the next dedx to fill; below about
  // 2^30 flops per step the fork and join cost more than they overlap
  // (LeNet-5 at batch 16: 0.183 ms per step launched call by call and 0.158
  // ms as a graph replay with it off, 0.213 and 0.201 with it on; the MLP
  // and the VGG nets, 10^11 flops and up, gain 5-12 % with it on).
  net->dw_flops = 0;
  for (const Stage& s : st) {
    if (s.kind == SGD_FC) net->dw_flops += 2 * (int64_t)s.Co * (s.Ci + 1) * s.N;
    if (s.kind == SGD_CONV) net->dw_flops += 2 * (int64_t)s.Co * (s.K + 1) * ((int64_t)s.N * s.Ho * s.Wo);
  }
  net->overlap_auto = net->dw_flops >= ((int64_t)1 << 30);
  net->partial_floats = partial;
  net->partial_off = b.take(4 * std::max<int64_t>(partial, 1));
  net->partial_dw_floats = partial_dw;
  net->partial_dw_off = b.take(4 * std::max<int64_t>(partial_dw, 1));
  net->dcol_off = b.take(4 * std::max<int64_t>(dcol, 1));
  net->ws_bytes = b.top;
  for (const Stage& s : st)
    if (s.kind == SGD_CONV || s.kind == SGD_FC) {
      net->w_offs.push_back(s.w_off);
      net->b_offs.push_back(s.b_off);
    }
  return SGD_OK;
}

// Fused training step: the dedw product applies `rule` to the layer's
// weights and bias (state at the same offsets) instead of storing gradients.
void set_update(GemmDesc& g, const sgd_rule* rule, float* state, const Stage& s) {
  if (!rule) return;
  g.urule = rule->rule;
  g.eta = rule->eta;
  g.mu = rule->mu;
  g.eps = rule->eps;
  g.decay = rule->decay;
  g.ustate = state ? state + s.w_off : nullptr;
  g.ustate_b = state ? state + s.b_off : nullptr;
}

template <typename T>
T* at(void* ws, const Tensor& t) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + t.off);
}

// Forward output of the stage feeding `s` (nullptr = the images).
const float* input_of(const sgd_net* net, const Stage& s, void* ws, const float* X) {
  return s.input < 0 ? X : at<float>(ws, net->stages[s.input].out);
}

// Gather over a source tensor (NHWC, sh x sw x sc per image) for a product
// whose gathered index runs over an rh x rw pixel grid.
ConvGather conv_gather(const float* src, int rh, int rw, int sh, int sw, int sc, int c, int P, bool flip) {
  ConvGather g{};
  g.src = src;
  g.RH = rh;
  g.RW = rw;
  g.SH = sh;
  g.SW = sw;
  g.SC = sc;
  g.c = c;
  g.P = P;
  g.flip = flip ? 1 : 0;
  g.inv_RW = 1.f / (float)rw;
  g.inv_RH = 1.f / (float)rh;
  return g;
}

int run_forward(sgd_net* net, const float* Wt, const float* X, const int32_t* y, float* loss, void* ws,
                hipStream_t st) {
  float* partial = reinterpret_cast<float*>(static_cast<char*>(ws) + net->partial_off);
  // Every conv layer's repacked weights, in one launch before the first
  // product.  The dedx operands are made from the same weights the forward
  // pass uses (the fused training step updates W during the backward pass).
  std::vector<RepackLayer> rep;
  for (const Stage& s : net->stages)
    if (s.kind == SGD_CONV)
      rep.push_back({Wt + s.w_off, at<float>(ws, s.wrep), s.implicit_dx ? at<float>(ws, s.wdx) : nullptr, s.Co, s.Ci,
                     s.c, s.ldk});
  if (!rep.empty()) {
    prof_set_layer(-1, 0);
    if (int e = repack_conv_weights(rep.data(), (int)rep.size(), st)) return e;
  }
  for (Stage& s : net->stages) {
    const float* xin = input_of(net, s, ws, X);
    int e = 0;
    prof_set_layer(s.spec, 0);
    if (s.kind == SGD_CONV) {
      float* wrep = at<float>(ws, s.wrep);
      GemmDesc g{};
      if (s.implicit) {
        g.gather = 1;
        g.cv = conv_gather(xin, s.Ho, s.Wo, s.H, s.W, s.Ci, s.c, s.P, false);
      } else {
        float* col = at<float>(ws, s.col);
        if ((e = im2col(xin, s.input < 0, col, s.N, s.Ci, s.H, s.W, s.c, s.P, s.Ho, s.Wo, s.ldk, st))) return e;
        g.A = col;
        g.lda = s.ldk;
      }
      g.B = wrep;
      g.ldb = s.ldk;
      g.C = at<float>(ws, s.out);
      g.ldc = s.Co;
      g.M = s.N * s.Ho * s.Wo;
      g.N = s.Co;
      g.K = s.ldk;
      g.flops = 2.0 * g.M * g.N * (double)s.K;
      g.epi = s.relu ? EPI_BIAS_RELU : EPI_BIAS;
      g.bias = Wt + s.b_off;
      g.splits = s.split_fwd;
      g.partial = partial;
      g.partial_floats = net->partial_floats;
      if ((e = gemm(g, st))) return e;
    } else if (s.kind == SGD_MAXPOOL) {
      if ((e = maxpool_fwd(xin, at<float>(ws, s.out), at<uint8_t>(ws, s.argmax), s.N, s.Ci, s.H, s.W, s.p,
                           s.out_nchw, st)))
        return e;
    } else if (s.kind == SGD_FC) {
      GemmDesc g{};
      g.A = xin;
      g.lda = s.Ci;
      g.B = Wt + s.w_off;
      g.ldb = s.Ci;
      g.C = at<float>(ws, s.out);
      g.ldc = s.Co;
      g.M = s.N;
      g.N = s.Co;
      g.K = s.Ci;
      g.epi = s.relu ? EPI_BIAS_RELU : EPI_BIAS;
      g.bias = Wt + s.b_off;
      g.skinny = true;
      g.splits = s.split_fwd;
      g.partial = partial;
      g.partial_floats = net->partial_floats;
      if ((e = gemm(g, st))) return e;
    } else if (s.kind == SGD_SOFTMAX_CE) {
      const float scale = net->reduction == SGD_REDUCE_SUM ? 1.f : 1.f / (float)s.N;
      if ((e = softmax_ce(xin, y, at<float>(ws, s.dout), at<float>(ws, s.out), loss, s.N, s.Ci, scale, st)))
        return e;
    }
  }
  return 0;
}

// accum: add the weight and bias gradients into `grad` instead of storing
// them (the GradBuf update of SPRINT Algorithm 1 for a non-empty buffer).
// rule (fused training step): `grad` is the weight vector itself and each
// layer's update is applied as soon as its gradient is final; an fc layer's
// dedx product, which reads that layer's weights, runs before its dedw (a
// conv layer's dedx reads the repacked copy W').
//
// Every dedw product but those of the first kMainDw weighted layers runs on
// the side stream, forked from the caller's stream once its inputs (the
// layer's output gradient, and the input activation or Col from the forward
// pass) are final and, for an fc layer, after the dedx product that reads W.
// The first kMainDw layers' dedw products run on the caller's stream after
// the layer's dedx (little else is left there by then), next to the side
// stream's tail.  Nothing on the caller's stream
// writes what a dedw product reads or reads what it writes, and the caller's
// stream joins the side stream at the end, so the step stays one stream-
// ordered operation for the caller.
int run_backward(sgd_net* net, const float* Wt, const float* X, float* grad, bool accum, const sgd_rule* rule,
                 float* state, float gscale, void* ws, hipStream_t st, bool overlap) {
  float* partial = reinterpret_cast<float*>(static_cast<char*>(ws) + net->partial_off);
  float* partial_dw = reinterpret_cast<float*>(static_cast<char*>(ws) + net->partial_dw_off);
  float* dcol = reinterpret_cast<float*>(static_cast<char*>(ws) + net->dcol_off);
  auto& stages = net->stages;
  int weighted = 0;
  for (const Stage& s : stages) weighted += (s.kind == SGD_FC || s.kind == SGD_CONV);
  if (overlap && net->side.ready(weighted)) return fail(SGD_EDEVICE, "backward: could not create the side stream");
  const hipStream_t side = overlap ? net->side.s : st;
  int fork_i = 0;
  auto fork = [&]() -> int {
    if (!overlap) return 0;
    hipEvent_t ev = net->side.ev[fork_i++];
    if (hipEventRecord(ev, st) != hipSuccess || hipStreamWaitEvent(side, ev, 0) != hipSuccess)
      return fail(SGD_EDEVICE, "backward: fork to the side stream failed");
    return 0;
  };
  // A dedw product on the side stream (forked once its inputs are final),
  // except those of the first kMainDw weighted layers, which run on the
  // caller's stream after the layer's dedx, concurrently with the side
  // stream's last ones.
  auto launch_dw = [&](GemmDesc& g, const Stage& s) -> int {
    if (s.dw_main) {
      g.partial = overlap ? partial : partial_dw;
      g.partial_floats = s.dw_cap;
      return gemm(g, st);
    }
    g.partial = partial_dw;
    g.partial_floats = net->partial_dw_floats;
    if (int e = fork()) return e;
    return gemm(g, side);
  };
  int e = 0;
  for (int si = (int)stages.size() - 1; si >= 0 && !e; --si) {
    Stage& s = stages[si];
    const float* xin = input_of(net, s, ws, X);
    prof_set_layer(s.spec, 1);
    if (s.kind == SGD_FC) {
      const float* dout = at<float>(ws, s.dout);
      if (!s.first_weighted) {
        const Stage& src = stages[s.input];
        GemmDesc d{};  // dedx_fc: d_input[N][in] = dout * W
        d.A = dout;
        d.lda = s.Co;
        d.B = Wt + s.w_off;
        d.ldb = s.Ci;
        d.b_t = true;
        d.C = at<float>(ws, src.dout);
        d.ldc = s.Ci;
        d.M = s.N;
        d.N = s.Ci;
        d.K = s.Co;
        const bool mask = src.relu && src.kind != SGD_MAXPOOL;
        d.epi = mask ? EPI_MASK : EPI_STORE;
        d.mask = mask ? at<float>(ws, src.out) : nullptr;
        d.ldm = s.Ci;
        d.skinny = true;
        d.beside_side = overlap;
        d.splits = s.split_dx;
        d.partial = partial;
        d.partial_floats = net->partial_floats;
        if ((e = gemm(d, st))) continue;
      }
      GemmDesc g{};  // dedw: dW[out][in] = dout^T * input; dedb via the ones column
      g.A = dout;
      g.lda = s.Co;
      g.a_t = true;
      g.B = xin;
      g.ldb = s.Ci;
      g.b_t = true;
      g.C = grad + s.w_off;
      g.ldc = s.Ci;
      g.M = s.Co;
      g.N = s.Ci;
      g.K = s.N;
      g.epi = EPI_STORE;
      g.splits = s.split_dw;
      g.ones_out = grad + s.b_off;
      g.accum = accum;
      g.gscale = gscale;
      set_update(g, rule, state, s);
      if ((e = launch_dw(g, s))) continue;
    } else if (s.kind == SGD_MAXPOOL) {
      const Stage& src = stages[s.input];
      const float* pooled = src.relu ? at<float>(ws, s.out) : nullptr;
      if ((e = maxpool_bwd(at<float>(ws, s.dout), at<uint8_t>(ws, s.argmax), pooled, at<float>(ws, src.dout), s.N,
                           s.Ci, s.H, s.W, s.p, s.out_nchw, st)))
        continue;
    } else if (s.kind == SGD_CONV) {
      const float* dout = at<float>(ws, s.dout);
      const int64_t P = (int64_t)s.N * s.Ho * s.Wo;
      GemmDesc g{};  // dedw: dW'[co][kk] = dout^T * col, stored permuted to [co][ci][ky][kx]; dedb via ones
      g.A = dout;
      g.lda = s.Co;
      g.a_t = true;
      if (s.implicit) {  // Col's rows gathered from the input activation
        g.gather = 2;
        g.cv = conv_gather(xin, s.Ho, s.Wo, s.H, s.W, s.Ci, s.c, s.P, false);
      } else {
        g.B = at<float>(ws, s.col);
        g.ldb = s.ldk;
      }
      g.b_t = true;
      g.C = grad + s.w_off;
      g.ldc = s.K;
      g.M = s.Co;
      g.N = s.ldk;
      g.K = (int)P;
      g.flops = 2.0 * s.Co * (double)s.K * (double)P;
      g.epi = EPI_STORE;
      g.splits = s.split_dw;
      g.perm_c = s.c;
      g.perm_ci = s.Ci;
      g.perm_k = s.K;
      g.ones_out = grad + s.b_off;
      g.accum = accum;
      g.gscale = gscale;
      set_update(g, rule, state, s);
      // a dedw on the caller's stream goes after the dedx, which the
      // remaining layers wait for (the dedx reads the repacked W'' or W')
      if (!s.dw_main && (e = launch_dw(g, s))) continue;
      if (s.implicit_dx) {
        // dedx_conv as one gather-form product: each input pixel gathers its
        // c*c taps of dout (flipped offsets) against W''; the ReLU mask of
        // the conv below is the epilogue
        const Stage& src = stages[s.input];
        const bool mask = src.relu && src.kind != SGD_MAXPOOL;
        GemmDesc d{};
        d.gather = 1;
        d.cv = conv_gather(dout, s.H, s.W, s.Ho, s.Wo, s.Co, s.c, s.P, true);
        d.B = at<float>(ws, s.wdx);
        d.ldb = (int64_t)s.c * s.c * s.Co;
        d.C = at<float>(ws, src.dout);
        d.ldc = s.Ci;
        d.M = s.N * s.H * s.W;
        d.N = s.Ci;
        d.K = s.c * s.c * s.Co;
        d.epi = mask ? EPI_MASK : EPI_STORE;
        d.mask = mask ? at<float>(ws, src.out) : nullptr;
        d.ldm = s.Ci;
        d.splits = 1;
        d.beside_side = overlap;
        d.partial = partial;
        d.partial_floats = net->partial_floats;
        if ((e = gemm(d, st))) continue;
      } else if (!s.first_weighted) {
        GemmDesc d{};  // dedx_conv: dcol[P][kk] = dout * W' (its own buffer: dedw reads Col meanwhile)
        d.A = dout;
        d.lda = s.Co;
        d.B = at<float>(ws, s.wrep);
        d.ldb = s.ldk;
        d.b_t = true;
        d.C = dcol;
        d.ldc = s.ldk;
        d.M = (int)P;
        d.N = s.ldk;
        d.K = s.Co;
        d.flops = 2.0 * (double)P * s.K * (double)s.Co;
        d.epi = EPI_STORE;
        d.splits = s.split_dx;
        d.beside_side = overlap;
        d.partial = partial;
        d.partial_floats = net->partial_floats;
        if ((e = gemm(d, st))) continue;
        const Stage& src = stages[s.input];
        const float* mask = (src.relu && src.kind != SGD_MAXPOOL) ? at<float>(ws, src.out) : nullptr;
        if ((e = col2im(dcol, mask, at<float>(ws, src.dout), s.N, s.Ci, s.H, s.W, s.c, s.P, s.Ho, s.Wo, s.ldk, st)))
          continue;
      }
      if (s.dw_main && (e = launch_dw(g, s))) continue;
    }
  }
  // Join even after an error, so nothing enqueued on the side stream is left
  // unordered with the caller's stream.
  if (!overlap) return e;
  hipEvent_t join = net->side.ev[weighted];
  if (hipEventRecord(join, side) != hipSuccess || hipStreamWaitEvent(st, join, 0) != hipSuccess)
    return e ? e : fail(SGD_EDEVICE, "backward: join of the side stream failed");
  return e;
}

}  // namespace
}  // namespace sgd

// ======================================================================= ABI
using sgd::fail;

extern "C" {

const char* sgd_last_error(void) { return sgd::g_error.c_str(); }

// plan() and the launch sequence allocate host vectors; a failed allocation
// becomes an error code here instead of an exception crossing the C ABI.
static int plan_guarded(sgd_net* net) {
  try {
    return sgd::plan(net);
  } catch (...) {
    return fail(SGD_EINVAL, "out of host memory while planning");
  }
}

int sgd_create_net(const sgd_input* input, const sgd_layer* layers, int n_layers, int reduction, sgd_net** out) {
  if (!input || !layers || !out) return fail(SGD_EINVAL, "sgd_create_net: null pointer");
  *out = nullptr;
  if (n_layers < 2) return fail(SGD_EINVAL, "sgd_create_net: need at least an fc and softmax_ce layer");
  if (reduction != SGD_REDUCE_MEAN && reduction != SGD_REDUCE_SUM)
    return fail(SGD_EINVAL, "sgd_create_net: bad reduction");
  sgd_net* net = new (std::nothrow) sgd_net();
  if (!net) return fail(SGD_EINVAL, "sgd_create_net: out of host memory");
  net->input = *input;
  net->reduction = reduction;
  try {
    net->spec.assign(layers, layers + n_layers);
  } catch (...) {
    delete net;
    return fail(SGD_EINVAL, "sgd_create_net: out of host memory");
  }
  const int rc = plan_guarded(net);
  if (rc != SGD_OK) {
    delete net;
    return rc;
  }
  *out = net;
  return SGD_OK;
}

void sgd_destroy_net(sgd_net* net) { delete net; }



int64_t sgd_param_count(const sgd_net* net) { return net ? net->n_params : -1; }

int sgd_param_offsets(const sgd_net* net, int64_t* w_off, int64_t* b_off, int max_layers) {
  if (!net) return fail(SGD_EINVAL, "sgd_param_offsets: null net");
  const int n = (int)net->w_offs.size();
  for (int i = 0; i < n && i < max_layers; ++i) {
    if (w_off) w_off[i] = net->w_offs[i];
    if (b_off) b_off[i] = net->b_offs[i];
  }
  return n;
}

size_t sgd_workspace_bytes(const sgd_net* net) { return net ? (size_t)net->ws_bytes : 0; }

int sgd_tensor_info(const sgd_net* net, int layer, int which, int64_t* byte_offset, int64_t dims[4], int* layout) {
  if (!net || !byte_offset || !dims || !layout) return fail(SGD_EINVAL, "sgd_tensor_info: null pointer");
  if (layer < 0 || layer >= (int)net->spec_to_stage.size()) return fail(SGD_EINVAL, "sgd_tensor_info: bad layer");
  const sgd::Stage& s = net->stages[net->spec_to_stage[layer]];
  const sgd::Tensor* t = nullptr;
  switch (which) {
    case SGD_T_OUT: t = &s.out; break;
    case SGD_T_DOUT: t = &s.dout; break;
    case SGD_T_COL: t = s.kind == SGD_CONV ? &s.col : nullptr; break;
    case SGD_T_WREP: t = s.kind == SGD_CONV ? &s.wrep : nullptr; break;
    case SGD_T_ARGMAX: t = s.kind == SGD_MAXPOOL ? &s.argmax : nullptr; break;
    default: break;
  }
  if (!t || t->off < 0) return fail(SGD_EINVAL, "sgd_tensor_info: layer has no such tensor");
  *byte_offset = t->off;
  for (int i = 0; i < 4; ++i) dims[i] = t->dims[i];
  *layout = t->layout;
  return SGD_OK;
}

// Debug mode: read the labels back (synchronously on `st`; null is the
// default stream) and reject any outside [0, classes) before anything is
// launched.
static int check_labels(const sgd_net* net, const int32_t* y, hipStream_t st, const char* who) {
  const int N = net->input.batch;
  std::vector<int32_t> h;
  try {
    h.resize((size_t)N);
  } catch (...) {
    return fail(SGD_EINVAL, std::string(who) + ": out of host memory");
  }
  if (hipMemcpyAsync(h.data(), y, (size_t)N * sizeof(int32_t), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return fail(SGD_EDEVICE, std::string(who) + ": reading the labels back failed");
  for (int i = 0; i < N; ++i)
    if (h[i] < 0 || h[i] >= net->classes)
      return fail(SGD_EINVAL, std::string(who) + ": label " + std::to_string(h[i]) + " at row " + std::to_string(i) +
                                  " is outside [0, " + std::to_string(net->classes) + ")");
  return SGD_OK;
}

static int step(sgd_net* net, const float* W, const float* X, const int32_t* y, float* grad, bool accum,
                const sgd_rule* rule, float* state, float* loss, void* ws, size_t ws_bytes, void* stream,
                const char* who, float gscale = 1.f, bool labels_checked = false, bool serial = false) {
  if (!net || !W || !X || !y || !grad || !loss || !ws) return fail(SGD_EINVAL, std::string(who) + ": null pointer");
  if ((int64_t)ws_bytes < net->ws_bytes)
    return fail(SGD_EWORKSPACE, std::string(who) + ": workspace has " + std::to_string(ws_bytes) + " bytes, needs " +
                                    std::to_string(net->ws_bytes));
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(SGD_EINVAL, std::string(who) + ": workspace not 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error from an unrelated earlier call
  if (net->debug && !labels_checked)
    if (int e = check_labels(net, y, st, who)) return e;
  sgd::g_prof = &net->prof;
  int e = SGD_OK;
  try {
    e = sgd::run_forward(net, W, X, y, loss, ws, st);
    if (!e) e = sgd::run_backward(net, W, X, grad, accum, rule, state, gscale, ws, st, overlap_on(net) && !serial);
  } catch (...) {
    e = fail(SGD_EINVAL, std::string(who) + ": out of host memory");
  }
  sgd::g_prof = nullptr;
  return e;
}

int sgd_compute_gradient(sgd_net* net, const float* W, const float* X, const int32_t* y, float* grad, float* loss,
                         void* ws, size_t ws_bytes, void* stream) {
  return step(net, W, X, y, grad, false, nullptr, nullptr, loss, ws, ws_bytes, stream, "sgd_compute_gradient");
}

int sgd_compute_gradient_into_scaled(sgd_net* net, const float* W, const float* X, const int32_t* y,
                                     sgd_gradbuf* gb, float scale, float* loss, void* ws, size_t ws_bytes,
                                     void* stream) {
  if (!std::isfinite(scale)) return fail(SGD_EINVAL, "sgd_compute_gradient_into_scaled: non-finite scale");
  if (!gb || !gb->data) return fail(SGD_EINVAL, "sgd_compute_gradient_into_scaled: null gradient buffer");
  if (net && gb->n != net->n_params)
    return fail(SGD_EINVAL, "sgd_compute_gradient_into_scaled: buffer length " + std::to_string(gb->n) +
                                " != parameter count " + std::to_string(net->n_params));
  const int e = step(net, W, X, y, gb->data, gb->empty == 0, nullptr, nullptr, loss, ws, ws_bytes, stream,
                     "sgd_compute_gradient_into_scaled", scale);
  if (!e) gb->empty = 0;
  return e;
}

int sgd_compute_gradient_into(sgd_net* net, const float* W, const float* X, const int32_t* y, sgd_gradbuf* gb,
                              float* loss, void* ws, size_t ws_bytes, void* stream) {
  if (!gb || !gb->data) return fail(SGD_EINVAL, "sgd_compute_gradient_into: null gradient buffer");
  if (net && gb->n != net->n_params)
    return fail(SGD_EINVAL, "sgd_compute_gradient_into: buffer length " + std::to_string(gb->n) + " != parameter count " +
                                std::to_string(net->n_params));
  const int e = step(net, W, X, y, gb->data, gb->empty == 0, nullptr, nullptr, loss, ws, ws_bytes, stream,
                     "sgd_compute_gradient_into");
  if (!e) gb->empty = 0;
  return e;
}

static int gemm_args_ok(const sgd_gemm_args* g) {
  if (!g) return fail(SGD_EINVAL, "sgd_gemm: null arguments");
  if (g->m < 1 || g->n < 1 || g->k < 1) return fail(SGD_EINVAL, "sgd_gemm: sizes must be positive");
  // Launch grids count output tiles (64 x 64 and larger) in 32-bit fields.
  if (((int64_t)g->m + 63) / 64 * (((int64_t)g->n + 63) / 64) >= ((int64_t)1 << 22))
    return fail(SGD_EINVAL, "sgd_gemm: more than 2^22 output tiles");
  const int64_t a_row = g->a_t ? g->m : g->k, b_row = g->b_t ? g->n : g->k;
  if (g->lda < a_row || g->ldb < b_row || g->ldc < g->n) return fail(SGD_EINVAL, "sgd_gemm: stride shorter than a row");
  return SGD_OK;
}

int sgd_gemm_plan(int m, int n, int k, int a_t, int b_t, int64_t* out, int nout) {
  if (m < 1 || n < 1 || k < 1 || !out || nout < 12) return fail(SGD_EINVAL, "sgd_gemm_plan: bad arguments");
  if (((int64_t)m + 63) / 64 * (((int64_t)n + 63) / 64) >= ((int64_t)1 << 22))
    return fail(SGD_EINVAL, "sgd_gemm_plan: more than 2^22 output tiles");
  const int form = a_t ? (b_t ? 1 : 3) : (b_t ? 2 : 0);
  return sgd::gemm_plan_query(m, n, k, form, out);
}

size_t sgd_gemm_workspace_bytes(const sgd_gemm_args* g) {
  if (gemm_args_ok(g)) return 0;
  const int splits = sgd::gemm_pick_splits(g->m, g->n, g->k);
  return (size_t)(4 * sgd::gemm_scratch_floats(g->m, g->n, g->k, g->a_t != 0, g->b_t != 0, false, splits));
}

int sgd_gemm(const sgd_gemm_args* g, void* ws, size_t ws_bytes, void* stream) {
  if (int e = gemm_args_ok(g)) return e;
  if (!g->A || !g->B || !g->C) return fail(SGD_EINVAL, "sgd_gemm: null matrix");
  const size_t need = sgd_gemm_workspace_bytes(g);
  if (ws_bytes < need || (need && !ws)) return fail(SGD_EWORKSPACE, "sgd_gemm: workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(SGD_EINVAL, "sgd_gemm: workspace not 256-byte aligned");
  sgd::GemmDesc d{};
  d.A = g->A;
  d.lda = g->lda;
  d.a_t = g->a_t != 0;
  d.B = g->B;
  d.ldb = g->ldb;
  d.b_t = g->b_t != 0;
  d.C = g->C;
  d.ldc = g->ldc;
  d.M = g->m;
  d.N = g->n;
  d.K = g->k;
  d.epi = sgd::EPI_STORE;
  d.skinny = true;
  d.splits = sgd::gemm_pick_splits(g->m, g->n, g->k);
  d.partial = static_cast<float*>(ws);
  d.partial_floats = (int64_t)(ws_bytes / 4);
  (void)hipGetLastError();
  return sgd::gemm(d, static_cast<hipStream_t>(stream));
}

int sgd_set_implicit_conv(sgd_net* net, int enable) {
  if (!net) return fail(SGD_EINVAL, "sgd_set_implicit_conv: null net");
  net->implicit = enable != 0;
  return plan_guarded(net);
}

int sgd_set_debug(sgd_net* net, int enable) {
  if (!net) return fail(SGD_EINVAL, "sgd_set_debug: null net");
  net->debug = enable != 0;
  return SGD_OK;
}

int sgd_set_overlap(sgd_net* net, int enable) {
  if (!net) return fail(SGD_EINVAL, "sgd_set_overlap: null net");
  net->overlap_req = enable < 0 ? -1 : enable != 0;
  return SGD_OK;
}

int sgd_get_overlap(const sgd_net* net, int* on) {
  if (!net || !on) return fail(SGD_EINVAL, "sgd_get_overlap: null net or output");
  *on = overlap_on(net) ? 1 : 0;
  return SGD_OK;
}

int sgd_profile(sgd_net* net, int enable) {
  if (!net) return fail(SGD_EINVAL, "sgd_profile: null net");
  if (enable) {
    net->prof.recs.clear();
    net->prof.used = 0;
    net->prof.products = 0;
  }
  net->prof.on = enable != 0;
  return SGD_OK;
}

int sgd_profile_read(sgd_net* net, sgd_kernel_time* out, int max_records) {
  if (!net) return fail(SGD_EINVAL, "sgd_profile_read: null net");
  const int n = (int)net->prof.recs.size();
  for (int i = 0; i < n && i < max_records && out; ++i) {
    const sgd::ProfRec& r = net->prof.recs[i];
    float ms = 0.f;
    if (hipEventSynchronize(r.end) != hipSuccess || hipEventElapsedTime(&ms, r.beg, r.end) != hipSuccess)
      return fail(SGD_EDEVICE, "sgd_profile_read: event query failed");
    out[i].kernel = r.kernel;
    out[i].layer = r.layer;
    out[i].phase = r.phase;
    out[i].ms = ms;
    out[i].flops = r.flops;
    out[i].bytes = r.bytes;
    out[i].m = r.m;
    out[i].n = r.n;
    out[i].k = r.k;
    out[i].product = r.product;
  }
  return n;
}

static int check_rule(const sgd_rule* rule, const float* state, const char* who);

int sgd_train_step(sgd_net* net, float* W, const float* X, const int32_t* y, float* state, const sgd_rule* rule,
                   float* loss, void* ws, size_t ws_bytes, void* stream) {
  if (int e = check_rule(rule, state, "sgd_train_step")) return e;
  return step(net, W, X, y, W, false, rule, state, loss, ws, ws_bytes, stream, "sgd_train_step");
}

// ---------------------------------------------- allocation-free step ----
// The device memory sgd_train_step_noalloc uses in place of a caller
// workspace: one static array per GPU the library runs on, held until the
// process ends.  Host code never passes `scratch` itself (in host code that
// name is a host-side stand-in, not a device address): it uses the address
// hipGetSymbolAddress reports for the current device, looked up once per
// device and kept in scratch_addr.
static __device__ __align__(256) unsigned char scratch[SGD_NOALLOC_SCRATCH_BYTES];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_addr[kMaxDevices] = {};

static int scratch_addr(void** out, const char* who) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(SGD_EDEVICE, std::string(who) + ": no current device");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(SGD_EDEVICE, std::string(who) + ": hipGetSymbolAddress of the static scratch failed: " +
                                   hipGetErrorString(e));
    }
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return SGD_OK;
}

int sgd_train_step_noalloc(sgd_net* net, float* W, const float* X, const int32_t* y, float* state,
                           const sgd_rule* rule, float* loss, void* stream) {
  const char* who = "sgd_train_step_noalloc";
  if (!net) return fail(SGD_EINVAL, std::string(who) + ": null net");
  if (int e = check_rule(rule, state, who)) return e;
  if (net->prof.on) return fail(SGD_EINVAL, std::string(who) + ": profiling is on (its events are created on demand)");
  if (net->ws_bytes > (int64_t)SGD_NOALLOC_SCRATCH_BYTES)
    return fail(SGD_EWORKSPACE, std::string(who) + ": the net needs " + std::to_string(net->ws_bytes) +
                                    " bytes of workspace; the static scratch holds " +
                                    std::to_string((long long)SGD_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if (int e = scratch_addr(&ws, who)) return e;
  // every dedw product on the caller's stream: no side stream or event is created
  return step(net, W, X, y, W, false, rule, state, loss, ws, SGD_NOALLOC_SCRATCH_BYTES, stream, who, 1.f, false,
              true);
}

struct sgd_step_graph {
  hipGraphExec_t exec = nullptr;
};

int sgd_train_step_graph(sgd_net* net, float* W, const float* X, const int32_t* y, float* state,
                         const sgd_rule* rule, float* loss, void* ws, size_t ws_bytes, sgd_step_graph** out) {
  const char* who = "sgd_train_step_graph";
  if (!out) return fail(SGD_EINVAL, std::string(who) + ": null output");
  *out = nullptr;
  if (!net) return fail(SGD_EINVAL, std::string(who) + ": null net");
  if (int e = check_rule(rule, state, who)) return e;
  if (net->prof.on) return fail(SGD_EINVAL, std::string(who) + ": profiling is on (its timing events cannot be captured)");
  // the dedw side stream and its fork/join events must exist before the capture starts
  if (overlap_on(net) && net->side.ready((int)net->w_offs.size()))
    return fail(SGD_EDEVICE, std::string(who) + ": could not create the side stream");
  // debug mode: the labels are checked once here, before the capture (a
  // captured stream cannot be synchronised)
  if (net->debug && y)
    if (int e = check_labels(net, y, nullptr, who)) return e;
  hipStream_t cs = nullptr;
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess)
    return fail(SGD_EDEVICE, std::string(who) + ": hipStreamCreate failed");
  int e = SGD_OK;
  if (hipStreamBeginCapture(cs, hipStreamCaptureModeRelaxed) != hipSuccess) {
    e = fail(SGD_EDEVICE, std::string(who) + ": hipStreamBeginCapture failed");
  } else {
    e = step(net, W, X, y, W, false, rule, state, loss, ws, ws_bytes, cs, who, 1.f, true);
    hipGraph_t g = nullptr;
    const hipError_t ce = hipStreamEndCapture(cs, &g);  // always ends the capture
    if (!e && ce != hipSuccess) e = fail(SGD_EDEVICE, std::string(who) + ": hipStreamEndCapture failed");
    if (!e) {
      hipGraphExec_t ex = nullptr;
      if (hipGraphInstantiate(&ex, g, nullptr, nullptr, 0) != hipSuccess) {
        e = fail(SGD_EDEVICE, std::string(who) + ": hipGraphInstantiate failed");
      } else {
        sgd_step_graph* sg = new (std::nothrow) sgd_step_graph();
        if (!sg) {
          (void)hipGraphExecDestroy(ex);
          e = fail(SGD_EINVAL, std::string(who) + ": out of host memory");
        } else {
          sg->exec = ex;
          *out = sg;
        }
      }
    }
    if (g) (void)hipGraphDestroy(g);
  }
  (void)hipStreamDestroy(cs);
  return e;
}

int sgd_step_graph_launch(sgd_step_graph* g, void* stream) {
  if (!g || !g->exec) return fail(SGD_EINVAL, "sgd_step_graph_launch: null graph");
  if (hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)) != hipSuccess)
    return fail(SGD_EDEVICE, "sgd_step_graph_launch: hipGraphLaunch failed");
  return SGD_OK;
}

void sgd_step_graph_destroy(sgd_step_graph* g) {
  if (!g) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  delete g;
}

int sgd_accumulate_grad(sgd_gradbuf* gb, const float* grad, void* stream) {
  if (!gb || !gb->data || !grad) return fail(SGD_EINVAL, "sgd_accumulate_grad: null pointer");
  if (gb->n <= 0) return fail(SGD_EINVAL, "sgd_accumulate_grad: n must be positive");
  const float* g[1] = {grad};
  const int e = sgd::accumulate(gb->data, g, 1, gb->empty != 0, gb->n, static_cast<hipStream_t>(stream));
  if (!e) gb->empty = 0;
  return e;
}

int sgd_accumulate_grads(sgd_gradbuf* gb, const float* const* grads, int k, void* stream) {
  if (!gb || !gb->data || !grads) return fail(SGD_EINVAL, "sgd_accumulate_grads: null pointer");
  if (gb->n <= 0) return fail(SGD_EINVAL, "sgd_accumulate_grads: n must be positive");
  if (k < 1 || k > 16) return fail(SGD_EINVAL, "sgd_accumulate_grads: k must be in 1..16");
  for (int j = 0; j < k; ++j)
    if (!grads[j]) return fail(SGD_EINVAL, "sgd_accumulate_grads: null gradient pointer");
  const int e = sgd::accumulate(gb->data, grads, k, gb->empty != 0, gb->n, static_cast<hipStream_t>(stream));
  if (!e) gb->empty = 0;
  return e;
}

static int check_rule(const sgd_rule* rule, const float* state, const char* who) {
  if (!rule) return fail(SGD_EINVAL, std::string(who) + ": null rule");
  if (rule->rule != SGD_PLAIN && rule->rule != SGD_MOMENTUM && rule->rule != SGD_ADAGRAD &&
      rule->rule != SGD_NESTEROV)
    return fail(SGD_EINVAL, std::string(who) + ": unknown rule");
  if (rule->rule != SGD_PLAIN && !state) return fail(SGD_EINVAL, std::string(who) + ": rule needs a state buffer");
  return SGD_OK;
}

int sgd_apply_update(float* W, sgd_gradbuf* gb, float* state, const sgd_rule* rule, void* stream) {
  if (!W || !gb || !gb->data) return fail(SGD_EINVAL, "sgd_apply_update: null pointer");
  if (gb->n <= 0) return fail(SGD_EINVAL, "sgd_apply_update: n must be positive");
  if (int e = check_rule(rule, state, "sgd_apply_update")) return e;
  int e = SGD_OK;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (gb->empty) {
    // zero gradient: without weight decay plain and Adagrad leave W (and A)
    // unchanged; the momentum rules still decay V (and move W)
    if (rule->rule == SGD_MOMENTUM || rule->rule == SGD_NESTEROV || rule->decay != 0.f)
      e = sgd::apply_rule(W, state, nullptr, 0, gb->n, rule->rule, rule->eta, rule->mu, rule->eps, rule->decay, st);
  } else {
    const float* g[1] = {gb->data};
    e = sgd::apply_rule(W, state, g, 1, gb->n, rule->rule, rule->eta, rule->mu, rule->eps, rule->decay, st);
  }
  if (!e) gb->empty = 1;
  return e;
}

int sgd_apply_fused(float* W, float* state, const float* const* grads, int k, int64_t n, const sgd_rule* rule,
                    void* stream) {
  if (!W || !grads) return fail(SGD_EINVAL, "sgd_apply_fused: null pointer");
  if (n <= 0) return fail(SGD_EINVAL, "sgd_apply_fused: n must be positive");
  if (k < 1 || k > 16) return fail(SGD_EINVAL, "sgd_apply_fused: k must be in 1..16");
  for (int j = 0; j < k; ++j)
    if (!grads[j]) return fail(SGD_EINVAL, "sgd_apply_fused: null gradient pointer");
  if (int e = check_rule(rule, state, "sgd_apply_fused")) return e;
  return sgd::apply_rule(W, state, grads, k, n, rule->rule, rule->eta, rule->mu, rule->eps, rule->decay,
                         static_cast<hipStream_t>(stream));
}

}  // extern "C"

extern "C" int sgd_stream_ref(float* const* outs, int n_out, const float* const* ins, int n_in, int64_t n,
                              int groups, void* stream) {
  if (!ins || (n_out > 0 && !outs)) return fail(SGD_EINVAL, "sgd_stream_ref: null pointer array");
  (void)hipGetLastError();
  return sgd::stream_ref(outs, n_out, ins, n_in, n, groups, static_cast<hipStream_t>(stream));
}

namespace sgd {
sgd_input net_input(const sgd_net* net) { return net->input; }

int clone_net(const sgd_net* src, sgd_net** out) {
  if (int e = sgd_create_net(&src->input, src->spec.data(), (int)src->spec.size(), src->reduction, out)) return e;
  (*out)->overlap_req = src->overlap_req;
  if ((*out)->implicit != src->implicit) {
    (*out)->implicit = src->implicit;
    if (int e = plan(*out)) {
      delete *out;
      *out = nullptr;
      return e;
    }
  }
  return SGD_OK;
}
}  // namespace sgd
