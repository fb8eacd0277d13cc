// TEST INFRASTRUCTURE ONLY.  Runs the host side of libsgdstep (the planner,
// the workspace and argument checks of every entry point) without a GPU,
// for a build whose host code is compiled with AddressSanitizer and
// UndefinedBehaviorSanitizer: an out-of-bounds access, overflow or undefined
// operation in that code aborts the run.  Every call below either succeeds
// on the host alone or must fail its argument checks before any device work.
// Built and run by tests/test_host_sanitize.py.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "sgdstep.h"

static int failures = 0;
#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      std::fprintf(stderr, "line %d: %s\n", __LINE__, #cond);     \
      ++failures;                                                 \
    }                                                             \
  } while (0)

static sgd_layer L(int kind, int out = 0, int kernel = 0, int pad = 0, int pool = 0) {
  sgd_layer l{};
  l.kind = kind;
  l.out = out;
  l.kernel = kernel;
  l.pad = pad;
  l.pool = pool;
  return l;
}

static std::vector<sgd_layer> vgg(const int* widths, const int* pool_after, int nconv, const int* fc, int nfc) {
  std::vector<sgd_layer> v;
  for (int i = 0; i < nconv; ++i) {
    v.push_back(L(SGD_CONV, widths[i], 3, 1));
    v.push_back(L(SGD_RELU));
    if (pool_after[i]) v.push_back(L(SGD_MAXPOOL, 0, 0, 0, 2));
  }
  for (int i = 0; i < nfc; ++i) {
    v.push_back(L(SGD_FC, fc[i]));
    if (i + 1 < nfc) v.push_back(L(SGD_RELU));
  }
  v.push_back(L(SGD_SOFTMAX_CE));
  return v;
}

// Plans the net, walks every query, toggles the settings that re-plan.
static void exercise(sgd_input in, const std::vector<sgd_layer>& layers, int64_t want_params) {
  sgd_net* net = nullptr;
  EXPECT(sgd_create_net(&in, layers.data(), (int)layers.size(), SGD_REDUCE_MEAN, &net) == SGD_OK && net);
  if (!net) return;
  if (sgd_param_count(net) != want_params)
    std::fprintf(stderr, "param count %lld, want %lld\n", (long long)sgd_param_count(net), (long long)want_params);
  EXPECT(sgd_param_count(net) == want_params);
  const int nw = sgd_param_offsets(net, nullptr, nullptr, 0);
  EXPECT(nw > 0);
  std::vector<int64_t> wo(nw), bo(nw);
  EXPECT(sgd_param_offsets(net, wo.data(), bo.data(), nw) == nw);
  for (int i = 1; i < nw; ++i) EXPECT(wo[i] > bo[i - 1]);
  for (int implicit = 1; implicit >= 0; --implicit) {
    EXPECT(sgd_set_implicit_conv(net, implicit) == SGD_OK);
    EXPECT(sgd_workspace_bytes(net) > 0);
    for (int li = -1; li <= (int)layers.size(); ++li)
      for (int which = -1; which <= 5; ++which) {
        int64_t off = -1, dims[4] = {0, 0, 0, 0};
        int layout = 0;
        const int rc = sgd_tensor_info(net, li, which, &off, dims, &layout);
        EXPECT(rc == SGD_OK || rc == SGD_EINVAL);
        if (rc == SGD_OK) EXPECT(off >= 0 && off < (int64_t)sgd_workspace_bytes(net));
      }
  }
  EXPECT(sgd_set_overlap(net, 0) == SGD_OK && sgd_set_overlap(net, 1) == SGD_OK);
  sgd_sprint_config cfg{4, 2, 1, 1, 1, 0};
  EXPECT(sgd_sprint_workspace_bytes(net, &cfg) > 0);
  cfg.workers = 17;
  EXPECT(sgd_sprint_workspace_bytes(net, &cfg) == 0);
  sgd_destroy_net(net);
}

int main() {
  // the four networks of the benchmark (parameter counts from eq. (3))
  {
    std::vector<sgd_layer> lenet = {L(SGD_CONV, 6, 5, 2), L(SGD_RELU), L(SGD_MAXPOOL, 0, 0, 0, 2),
                                    L(SGD_CONV, 16, 5, 0), L(SGD_RELU), L(SGD_MAXPOOL, 0, 0, 0, 2),
                                    L(SGD_FC, 120), L(SGD_RELU), L(SGD_FC, 84), L(SGD_RELU), L(SGD_FC, 10),
                                    L(SGD_SOFTMAX_CE)};
    exercise(sgd_input{16, 1, 28, 28}, lenet, 61706);
  }
  {
    std::vector<sgd_layer> mlp;
    for (int i = 0; i < 5; ++i) {
      mlp.push_back(L(SGD_FC, 5000));
      mlp.push_back(L(SGD_RELU));
    }
    mlp.push_back(L(SGD_FC, 10));
    mlp.push_back(L(SGD_SOFTMAX_CE));
    exercise(sgd_input{512, 3072, 1, 1}, mlp, 115435010);
  }
  const int widths[13] = {64, 64, 128, 128, 256, 256, 256, 512, 512, 512, 512, 512, 512};
  const int pools[13] = {0, 1, 0, 1, 0, 0, 1, 0, 0, 1, 0, 0, 1};
  {
    const int fc[2] = {512, 10};  // the 512-wide flatten, one hidden fc of 512, 10 classes
    exercise(sgd_input{128, 3, 32, 32}, vgg(widths, pools, 13, fc, 2), 14982474);
  }
  {
    const int fc[3] = {4096, 4096, 1000};
    exercise(sgd_input{32, 3, 224, 224}, vgg(widths, pools, 13, fc, 3), 138357544);
  }
  // a ragged net: odd maps, an unpooled conv into fc, 1x1 and 5x5 filters
  {
    std::vector<sgd_layer> odd = {L(SGD_CONV, 5, 1, 0), L(SGD_RELU), L(SGD_CONV, 7, 5, 2), L(SGD_MAXPOOL, 0, 0, 0, 3),
                                  L(SGD_FC, 9), L(SGD_SOFTMAX_CE)};
    const int64_t p1 = 5 * (3 + 1), p2 = 7 * (25 * 5 + 1), p3 = 9 * (7 * 3 * 3 + 1);
    exercise(sgd_input{3, 3, 9, 9}, odd, p1 + p2 + p3);
  }
  // nets the planner must reject
  {
    sgd_input in{2, 3, 8, 8};
    sgd_net* net = nullptr;
    std::vector<sgd_layer> bad_pool = {L(SGD_CONV, 4, 3, 1), L(SGD_MAXPOOL, 0, 0, 0, 3), L(SGD_FC, 3),
                                       L(SGD_SOFTMAX_CE)};
    EXPECT(sgd_create_net(&in, bad_pool.data(), (int)bad_pool.size(), SGD_REDUCE_MEAN, &net) == SGD_ESHAPE);
    std::vector<sgd_layer> relu_first = {L(SGD_RELU), L(SGD_FC, 3), L(SGD_SOFTMAX_CE)};
    EXPECT(sgd_create_net(&in, relu_first.data(), 3, SGD_REDUCE_MEAN, &net) == SGD_EUNSUPPORTED);
    std::vector<sgd_layer> too_big = {L(SGD_CONV, 4, 11, 0), L(SGD_FC, 3), L(SGD_SOFTMAX_CE)};
    EXPECT(sgd_create_net(&in, too_big.data(), 3, SGD_REDUCE_MEAN, &net) == SGD_ESHAPE);
    std::vector<sgd_layer> no_loss = {L(SGD_FC, 3), L(SGD_FC, 3)};
    EXPECT(sgd_create_net(&in, no_loss.data(), 2, SGD_REDUCE_MEAN, &net) == SGD_ESHAPE);
    EXPECT(sgd_create_net(&in, nullptr, 2, SGD_REDUCE_MEAN, &net) == SGD_EINVAL);
    EXPECT(sgd_create_net(&in, no_loss.data(), 2, 7, &net) == SGD_EINVAL);
    EXPECT(sgd_param_count(nullptr) == -1 && sgd_workspace_bytes(nullptr) == 0);
  }
  // the standalone product: workspace queries over shapes and forms, and
  // calls rejected by their argument checks
  for (int form = 0; form < 4; ++form)
    for (int m : {1, 7, 64, 513, 4096, 1 << 20})
      for (int n : {1, 3, 128, 1000})
        for (int k : {1, 5, 512, 30000}) {
          sgd_gemm_args g{};
          g.m = m, g.n = n, g.k = k, g.a_t = form & 1, g.b_t = (form >> 1) & 1;
          g.lda = g.a_t ? m : k, g.ldb = g.b_t ? n : k, g.ldc = n;
          (void)sgd_gemm_workspace_bytes(&g);
        }
  {
    sgd_gemm_args g{};
    g.m = 4, g.n = 4, g.k = 4, g.lda = 4, g.ldb = 4, g.ldc = 4;
    EXPECT(sgd_gemm(&g, nullptr, 0, nullptr) == SGD_EINVAL);      // null matrices
    EXPECT(sgd_gemm(nullptr, nullptr, 0, nullptr) == SGD_EINVAL);
    g.lda = 2;
    EXPECT(sgd_gemm_workspace_bytes(&g) == 0);                    // stride shorter than a row
    g.lda = 4;
    g.m = 1 << 30, g.n = 1 << 30;
    EXPECT(sgd_gemm_workspace_bytes(&g) == 0);                    // too many output tiles
  }
  // update entry points: argument checks only
  {
    sgd_rule r{SGD_MOMENTUM, 0.1f, 0.9f, 0.f, 0.f};
    sgd_gradbuf gb{nullptr, 10, 1};
    EXPECT(sgd_apply_update(nullptr, &gb, nullptr, &r, nullptr) == SGD_EINVAL);
    EXPECT(sgd_accumulate_grad(nullptr, nullptr, nullptr) == SGD_EINVAL);
    r.rule = 9;
    EXPECT(sgd_apply_fused(nullptr, nullptr, nullptr, 0, 10, &r, nullptr) == SGD_EINVAL);
  }
  EXPECT(sgd_last_error() != nullptr);
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("host sanitizer run: ok\n");
  return 0;
}
