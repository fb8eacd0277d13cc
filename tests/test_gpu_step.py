"""GPU parity of sgd_compute_gradient against the CPU oracle (end to end).

Loss to |dL| <= 1e-5 |L|; every layer's weight and bias gradient to
max|d| <= 1e-4 max|g| (fp32 products with fp32 accumulation on the GPU, the
oracle rounding to float after each layer with double sums).  Sizes are ones
the oracle finishes in seconds, chosen to span several GEMM tiles and leave
ragged tails (odd channel counts, widths not divisible by 4, 16, 64 or 128).
"""
import numpy as np
import pytest

import oracle as O
import workloads
from tests._util import LOSS_RTOL, per_tensor_grad_check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import sgd_cnns_amd as S  # noqa: E402


def run_gpu(chw, layers, X, y, W, reduce_sum=False, keep_ws=False):
    N = X.shape[0]
    net = S.Net((N,) + tuple(chw), layers, reduce_sum=reduce_sum)
    dev = torch.device("cuda")
    Wd = torch.from_numpy(W).to(dev)
    Xd = torch.from_numpy(np.ascontiguousarray(X)).to(dev)
    yd = torch.from_numpy(y).to(dev)
    grad = torch.full((net.param_count(),), float("nan"), device=dev)
    loss = torch.full((1,), float("nan"), device=dev)
    ws = net.workspace()
    net.compute_gradient(Wd, Xd, yd, grad, loss, ws)
    torch.cuda.synchronize()
    out = (float(loss.item()), grad.cpu().numpy())
    if keep_ws:
        return out + (net, ws)
    return out


def check(chw, layers, N, seed, classes, x_dist="uniform", reduce_sum=False, w_scale=None):
    print(f"[parity] chw={chw} N={N} seed={seed} layers={layers}", flush=True)
    shape = (N,) + tuple(chw)
    X = workloads.uniform01(seed, 0, shape) if x_dist == "uniform" else workloads.normal(seed, 0, shape)
    y = workloads.labels(seed, 1, N, classes)
    W = workloads.he_normal_params(seed, chw, layers)
    onet = O.OracleNet(chw, layers, reduce_sum=reduce_sum)
    assert onet.param_count() == W.size
    l_ref, g_ref = onet.gradient(W, X, y)
    l_gpu, g_gpu = run_gpu(chw, layers, X, y, W, reduce_sum)
    assert np.isfinite(g_gpu).all()
    assert abs(l_gpu - l_ref) <= LOSS_RTOL * abs(l_ref), (l_gpu, l_ref)
    wo = [onet.params[i][0] for i in sorted(onet.params)]
    bo = [onet.params[i][2] for i in sorted(onet.params)]
    worst = per_tensor_grad_check(g_gpu, g_ref, wo, bo, W.size)
    print(f"[parity] loss {l_gpu:.7f} vs {l_ref:.7f}; worst grad ratio {worst:.2e}", flush=True)


def test_lenet5_config():
    wl = workloads.WORKLOADS["lenet5"]
    check(wl.chw, wl.layers, wl.batch, wl.seed, wl.classes)


def test_tiny_cnn_ragged():
    layers = [("conv", 5, 3, 1), ("relu",), ("pool", 2), ("conv", 7, 3, 0), ("relu",), ("pool", 3),
              ("fc", 13), ("relu",), ("fc", 6), ("softmax_ce",)]
    check((3, 16, 16), layers, 3, 101, 6, x_dist="normal")


def test_cnn_unpooled_conv_into_fc_and_sum_reduction():
    layers = [("conv", 4, 3, 1), ("relu",), ("conv", 6, 5, 2), ("fc", 11), ("relu",), ("fc", 5), ("softmax_ce",)]
    check((2, 9, 7), layers, 5, 102, 5, x_dist="normal", reduce_sum=True)


def test_large_filter_conv_repack_tiles():
    # a 21x21 conv after a 16-channel one: the weight repack stages 28 output x 1 input channel per tile
    # (two output-channel tiles, 28 + 4), and the layer takes the gathered forward, dedw and dedx products
    layers = [("conv", 16, 3, 1), ("relu",), ("conv", 32, 21, 0), ("relu",), ("fc", 7), ("softmax_ce",)]
    check((3, 22, 22), layers, 2, 106, 7, x_dist="normal")


def test_conv3x3_repack_ragged_channel_tiles():
    # 3x3 weights are repacked in tiles of 32 output x 16 input channels: 20 and 40 input channels end
    # in a short input tile (4, 8), 40, 48 and 36 output channels in a short output tile (8, 16, 4);
    # the 48-channel layer also writes the dedx copy W'' (its dedx is the gathered product)
    layers = [("conv", 40, 3, 1), ("relu",), ("conv", 48, 3, 1), ("relu",), ("conv", 36, 3, 0), ("relu",),
              ("fc", 5), ("softmax_ce",)]
    check((20, 7, 7), layers, 3, 107, 5, x_dist="normal")


def test_conv3x3_repack_misaligned_weights():
    # two 1x1 convs (5 x (2+1) and 8 x (5+1) parameters) put the 3x3 layer's weights at float offset 63:
    # its channel counts are multiples of 4 but the repack must take the one-float path; the 1x1 layers go
    # to the generic repack kernel in a launch of their own
    layers = [("conv", 5, 1, 0), ("relu",), ("conv", 8, 1, 0), ("relu",), ("conv", 12, 3, 1), ("relu",),
              ("fc", 4), ("softmax_ce",)]
    offs = sorted(O.OracleNet((2, 6, 6), layers).params.items())
    assert offs[2][1][0] % 4 == 3, offs
    check((2, 6, 6), layers, 3, 108, 4, x_dist="normal")


def test_mlp_ragged_tiles():
    layers = [("fc", 300), ("relu",), ("fc", 129), ("relu",), ("fc", 10), ("softmax_ce",)]
    check((3072, 1, 1), layers, 70, 103, 10)


def test_conv_channels_multiple_of_4_vector_paths():
    # Ci % 4 == 0 takes the float4 im2col / col2im paths; 3 pools; 2 tiles in M
    layers = [("conv", 8, 3, 1), ("relu",), ("conv", 16, 3, 1), ("relu",), ("pool", 2),
              ("conv", 32, 3, 1), ("relu",), ("pool", 2), ("fc", 40), ("relu",), ("fc", 10), ("softmax_ce",)]
    check((4, 16, 16), layers, 6, 104, 10, x_dist="normal")


def test_vgg_cifar_reduced_batch():
    wl = workloads.WORKLOADS["vgg_cifar"]
    check(wl.chw, wl.layers, 2, 105, wl.classes, x_dist="normal")


def test_deterministic_bitwise():
    wl = workloads.WORKLOADS["lenet5"]
    X, y, W = workloads.make_inputs(wl)
    a = run_gpu(wl.chw, wl.layers, X, y, W)
    b = run_gpu(wl.chw, wl.layers, X, y, W)
    assert a[0] == b[0]
    np.testing.assert_array_equal(a[1], b[1])


def test_zero_weights_closed_form():
    # W = 0: loss = ln C; only the last bias has a gradient, 1/C - count(y=j)/N
    wl = workloads.WORKLOADS["lenet5"]
    X, y, W = workloads.make_inputs(wl)
    W[:] = 0
    l, g = run_gpu(wl.chw, wl.layers, X, y, W)
    assert l == pytest.approx(np.log(10), rel=1e-6)
    net = S.Net((wl.batch,) + wl.chw, wl.layers)
    wo, bo = net.param_offsets()
    expect = 1.0 / 10 - np.bincount(y, minlength=10) / wl.batch
    np.testing.assert_allclose(g[bo[-1]:], expect, atol=1e-7)
    assert np.all(g[:bo[-1]] == 0)


def test_nan_input_propagates_without_error():
    wl = workloads.WORKLOADS["lenet5"]
    X, y, W = workloads.make_inputs(wl)
    X[3, 0, 10, 10] = np.nan
    l, g = run_gpu(wl.chw, wl.layers, X, y, W)
    assert np.isnan(l)
    assert np.isnan(O.OracleNet(wl.chw, wl.layers).gradient(W, X, y)[0])


def test_compute_gradient_into_matches_compute_plus_accumulate():
    # empty buffer: bitwise the gradient; non-empty: bitwise g0 + gradient
    wl = workloads.WORKLOADS["lenet5"]
    X, y, W = workloads.make_inputs(wl)
    net = S.Net((wl.batch,) + wl.chw, wl.layers)
    n = net.param_count()
    dev = torch.device("cuda")
    Wd, Xd, yd = (torch.from_numpy(a).to(dev) for a in (W, X, y))
    ws = net.workspace()
    loss = torch.empty(1, device=dev)
    grad = torch.empty(n, device=dev)
    net.compute_gradient(Wd, Xd, yd, grad, loss, ws)
    gb = S.GradBuf(n)
    gb.data.fill_(7.0)
    net.compute_gradient_into(Wd, Xd, yd, gb, loss, ws)
    assert not gb.empty
    torch.cuda.synchronize()
    g = grad.cpu().numpy()
    np.testing.assert_array_equal(gb.data.cpu().numpy(), g)
    g0 = workloads.normal(7, 3, n, 1e-2)
    gb.data.copy_(torch.from_numpy(g0))
    net.compute_gradient_into(Wd, Xd, yd, gb, loss, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gb.data.cpu().numpy(), (g0 + g).astype(np.float32))
    bad = S.GradBuf(n - 1)
    with pytest.raises(ValueError):        # the binding's length check
        net.compute_gradient_into(Wd, Xd, yd, bad, loss, ws)
    bad = S.GradBuf(n - 1, data=torch.empty(n, device=dev))
    with pytest.raises(S.SgdError):        # the library's: the buffer's declared length is wrong
        net.compute_gradient_into(Wd, Xd, yd, bad, loss, ws)


def test_compute_gradient_into_vgg_split_k_paths():
    # conv dedw with split-K and permuted store, fc dedw direct store: both accumulate
    wl = workloads.WORKLOADS["vgg_cifar"]
    X, y, W = workloads.make_inputs(wl.with_batch(2))
    net = S.Net((2,) + wl.chw, wl.layers)
    n = net.param_count()
    dev = torch.device("cuda")
    Wd, Xd, yd = (torch.from_numpy(a).to(dev) for a in (W, X, y))
    ws = net.workspace()
    loss = torch.empty(1, device=dev)
    grad = torch.empty(n, device=dev)
    net.compute_gradient(Wd, Xd, yd, grad, loss, ws)
    g0 = workloads.normal(8, 3, n, 1e-3)
    gb = S.GradBuf(n)
    gb.data.copy_(torch.from_numpy(g0))
    gb.empty = False
    net.compute_gradient_into(Wd, Xd, yd, gb, loss, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gb.data.cpu().numpy(), (g0 + grad.cpu().numpy()).astype(np.float32))


@pytest.mark.parametrize("rule", ["plain", "momentum", "adagrad", "nesterov_wd"])
@pytest.mark.parametrize("case", ["lenet5", "vgg_cifar_b2", "mlp_ragged", "mlp5000", "mlp_k320", "mlp_b32"])
def test_train_step_equals_gradient_then_apply(rule, case):
    # the fused step (update applied in the dedw epilogues / split-K reduction)
    # must give bitwise the same W and optimizer state as gradient-into-GradBuf
    # followed by the separate apply
    if case == "lenet5":
        wl = workloads.WORKLOADS["lenet5"]
    elif case == "vgg_cifar_b2":
        wl = workloads.WORKLOADS["vgg_cifar"].with_batch(2)
    elif case == "mlp_ragged":
        wl = workloads.Workload("mlp_ragged", 31, 70, (3072, 1, 1),
                                [("fc", 300), ("relu",), ("fc", 129), ("relu",), ("fc", 10), ("softmax_ce",)])
    elif case == "mlp_b32":    # k = 32: the short-reduction weight-gradient kernel, one and two blocks per batch
        wl = workloads.Workload("mlp_b32", 35, 32, (3072, 1, 1),
                                [("fc", 4096), ("relu",), ("fc", 4096), ("relu",), ("fc", 10), ("softmax_ce",)])
    elif case == "mlp_k320":   # fc weight gradients with k = 320: whole tiles and a stream-K remainder
        wl = workloads.Workload("mlp_k320", 33, 320, (3072, 1, 1),
                                [("fc", 4096), ("relu",), ("fc", 4096), ("relu",), ("fc", 10), ("softmax_ce",)])
    else:
        wl = workloads.WORKLOADS["mlp5000"]
    print(f"[train_step] {case} {rule}", flush=True)
    X, y, W = workloads.make_inputs(wl)
    net = S.Net((wl.batch,) + tuple(wl.chw), wl.layers)
    n = net.param_count()
    dev = torch.device("cuda")
    Xd, yd = torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev)
    st0 = workloads.normal(9, 3, n, 1e-3)
    if rule == "adagrad":
        st0 = np.abs(st0) + np.float32(0.1)
    # nesterov_wd: Nesterov momentum with weight decay 5e-4 (PIPE appendix A)
    R = S.Rule("nesterov", 0.01, 0.9, 0.0, 5e-4) if rule == "nesterov_wd" else S.Rule(rule, 0.01, 0.9, 1e-8)
    ws = net.workspace()
    loss_a = torch.empty(1, device=dev)
    loss_b = torch.empty(1, device=dev)
    # reference: gradient into an empty GradBuf, then apply
    Wa = torch.from_numpy(W).to(dev)
    sa = torch.from_numpy(st0).to(dev)
    gb = S.GradBuf(n)
    net.compute_gradient_into(Wa, Xd, yd, gb, loss_a, ws)
    S.apply_update(Wa, gb, sa if rule != "plain" else None, R)
    # fused
    Wb = torch.from_numpy(W).to(dev)
    sb = torch.from_numpy(st0).to(dev)
    net.train_step(Wb, Xd, yd, sb if rule != "plain" else None, R, loss_b, ws)
    torch.cuda.synchronize()
    assert loss_a.item() == loss_b.item()
    assert torch.equal(Wa, Wb), f"max |dW| {(Wa - Wb).abs().max().item()}"
    if rule != "plain":
        assert torch.equal(sa, sb)
    assert not torch.equal(Wb, torch.from_numpy(W).to(dev))


@pytest.mark.parametrize("case", ["lenet5", "vgg_cifar_b2", "mlp_ragged"])
def test_overlap_on_and_off_bitwise_equal(case):
    # the dedw products run on a second stream by default; with overlap off
    # they run in order on the caller's stream: every output must be bitwise
    # the same (gradient, loss, and a fused momentum step's W and V)
    if case == "lenet5":
        wl = workloads.WORKLOADS["lenet5"]
    elif case == "vgg_cifar_b2":
        wl = workloads.WORKLOADS["vgg_cifar"].with_batch(2)
    else:
        wl = workloads.Workload("mlp_ragged", 31, 70, (3072, 1, 1),
                                [("fc", 300), ("relu",), ("fc", 129), ("relu",), ("fc", 10), ("softmax_ce",)])
    print(f"[overlap] {case}", flush=True)
    X, y, W = workloads.make_inputs(wl)
    net = S.Net((wl.batch,) + tuple(wl.chw), wl.layers)
    n = net.param_count()
    dev = torch.device("cuda")
    Xd, yd, Wd = torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev), torch.from_numpy(W).to(dev)
    ws = net.workspace()
    R = S.Rule("momentum", 0.01, 0.9, 1e-8)
    out = {}
    for ov in (True, False):
        net.set_overlap(ov)
        g = torch.empty(n, device=dev)
        loss = torch.empty(1, device=dev)
        net.compute_gradient(Wd, Xd, yd, g, loss, ws)
        Wt = Wd.clone()
        V = torch.zeros(n, device=dev)
        loss2 = torch.empty(1, device=dev)
        net.train_step(Wt, Xd, yd, V, R, loss2, ws)
        net.train_step(Wt, Xd, yd, V, R, loss2, ws)
        torch.cuda.synchronize()
        out[ov] = (g.cpu(), loss.item(), Wt.cpu(), V.cpu(), loss2.item())
    a, b = out[True], out[False]
    assert torch.equal(a[0], b[0]) and a[1] == b[1]
    assert torch.equal(a[2], b[2]) and torch.equal(a[3], b[3]) and a[4] == b[4]


@pytest.mark.parametrize("case", ["mlp_ragged", "vgg_cifar_b2"])
def test_prescaled_gradient(case):
    # SPRINT Algorithm 1: the worker stores Grad = -eta * grad.  The
    # scaled product rounds fl(scale * g) of the very g the unscaled path
    # stores, added into a non-empty buffer the same way; applied with
    # eta = -1 it gives the unscaled step's W and V bitwise; against the
    # oracle's gradient it is within the gradient tolerance.
    if case == "vgg_cifar_b2":
        wl = workloads.WORKLOADS["vgg_cifar"].with_batch(2)
    else:
        wl = workloads.Workload("mlp_ragged", 31, 70, (3072, 1, 1),
                                [("fc", 300), ("relu",), ("fc", 129), ("relu",), ("fc", 10), ("softmax_ce",)])
    print(f"[prescaled] {case}", flush=True)
    X, y, W = workloads.make_inputs(wl)
    net = S.Net((wl.batch,) + tuple(wl.chw), wl.layers)
    n = net.param_count()
    dev = torch.device("cuda")
    Xd, yd, Wd = torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev), torch.from_numpy(W).to(dev)
    ws = net.workspace()
    loss = torch.empty(1, device=dev)
    eta = np.float32(0.01)
    g = torch.empty(n, device=dev)
    net.compute_gradient(Wd, Xd, yd, g, loss, ws)
    gs = S.GradBuf(n)
    net.compute_gradient_into_scaled(Wd, Xd, yd, gs, float(-eta), loss, ws)
    torch.cuda.synchronize()
    g_np = g.cpu().numpy()
    np.testing.assert_array_equal(gs.data.cpu().numpy(), (np.float32(-eta) * g_np).astype(np.float32))
    # into a non-empty buffer: GradBuf + fl(scale * g)
    base = workloads.normal(14, 1, n, 1e-3)
    gb2 = S.GradBuf(n, data=torch.from_numpy(base).to(dev))
    gb2.empty = False
    net.compute_gradient_into_scaled(Wd, Xd, yd, gb2, float(-eta), loss, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gb2.data.cpu().numpy(), base + (np.float32(-eta) * g_np).astype(np.float32))
    # apply with eta = -1 == the unscaled step
    V0 = workloads.normal(14, 2, n, 1e-3)
    Wa, Va = Wd.clone(), torch.from_numpy(V0).to(dev)
    gu = S.GradBuf(n)
    net.compute_gradient_into(Wd, Xd, yd, gu, loss, ws)
    S.apply_update(Wa, gu, Va, S.Rule("momentum", float(eta), 0.9))
    Wb, Vb = Wd.clone(), torch.from_numpy(V0).to(dev)
    S.apply_update(Wb, gs, Vb, S.Rule("momentum", -1.0, 0.9))
    torch.cuda.synchronize()
    assert torch.equal(Wa, Wb) and torch.equal(Va, Vb)
    # against the oracle
    onet = O.OracleNet(wl.chw, wl.layers)
    _, g_ref = onet.gradient(W, X, y)
    wo = [onet.params[i][0] for i in sorted(onet.params)]
    bo = [onet.params[i][2] for i in sorted(onet.params)]
    per_tensor_grad_check((np.float32(-eta) * g_np).astype(np.float32), (np.float32(-eta) * g_ref).astype(np.float32),
                          wo, bo, n)


# ------------------------------------------------ implicit-GEMM convolution ----
# Conv layers after the first with Ci % 16 == 0 gather their im2col operand
# from the activation; those with Co % 16 == 0 compute dedx as one gathered
# product.  These nets cover odd map sizes (ragged tiles), 3x3 / 5x5 / 1x1
# filters, pad 0 / 1 / 2, a pool feeding the gathered dedx (no mask) and a
# ReLU'd conv feeding it (mask in the epilogue).
IMPLICIT_NET = [("conv", 16, 3, 1), ("relu",), ("conv", 32, 3, 1), ("relu",), ("pool", 2),
                ("conv", 16, 5, 2), ("relu",), ("conv", 48, 1, 0), ("relu",), ("conv", 32, 3, 0), ("relu",),
                ("fc", 10), ("softmax_ce",)]


def test_implicit_conv_net_matches_oracle():
    check((3, 10, 10), IMPLICIT_NET, 3, 41, 10)


def test_implicit_conv_net_odd_maps():
    check((3, 9, 7), [("conv", 16, 3, 1), ("relu",), ("conv", 16, 3, 1), ("relu",), ("conv", 32, 3, 0), ("relu",),
                      ("fc", 7), ("softmax_ce",)], 5, 42, 7, x_dist="normal")


def test_implicit_and_explicit_conv_agree():
    # forward and dedw take the same k order either way (bitwise); dedx is
    # summed in another order (gradient tolerance)
    chw, N = (3, 10, 10), 3
    X = workloads.normal(43, 0, (N,) + chw)
    y = workloads.labels(43, 1, N, 10)
    W = workloads.he_normal_params(43, chw, IMPLICIT_NET)
    dev = torch.device("cuda")
    out = {}
    for imp in (True, False):
        net = S.Net((N,) + chw, IMPLICIT_NET)
        net.set_implicit_conv(imp)
        ws = net.workspace()
        g = torch.empty(W.size, device=dev)
        loss = torch.empty(1, device=dev)
        net.compute_gradient(torch.from_numpy(W).to(dev), torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev),
                             g, loss, ws)
        torch.cuda.synchronize()
        outs = [net.view(ws, i, S.T_OUT).cpu().numpy() for i in (0, 2, 5, 7, 9)]
        out[imp] = (g.cpu().numpy(), loss.item(), outs, net)
    (ga, la, oa, neta), (gb, lb, ob, netb) = out[True], out[False]
    assert la == lb
    for a, b in zip(oa, ob):
        np.testing.assert_array_equal(a, b)
    onet = O.OracleNet(chw, IMPLICIT_NET)
    wo = [onet.params[i][0] for i in sorted(onet.params)]
    bo = [onet.params[i][2] for i in sorted(onet.params)]
    # the last conv's dedw reads only forward data: bitwise
    last = max(i for i, L in enumerate(IMPLICIT_NET) if L[0] == "conv")
    w0, _, b0, nb = onet.params[last]
    np.testing.assert_array_equal(ga[w0:b0 + nb], gb[w0:b0 + nb])
    per_tensor_grad_check(ga, gb.astype(np.float32), wo, bo, W.size)
    assert neta.workspace_bytes() < netb.workspace_bytes()


@pytest.mark.parametrize("rule", ["momentum", "adagrad"])
def test_train_step_explicit_conv_matches_unfused(rule):
    """With implicit convolution off, a conv layer's weight gradient is an ungathered product with the
    permuted [co][ci][ky][kx] store, with the update in its epilogue (VGG-CIFAR, batch 2).  Bitwise
    equal to gradient + apply, and the gradient itself against the oracle."""
    wl = workloads.WORKLOADS["vgg_cifar"].with_batch(2)
    print(f"[explicit-conv train_step] {rule}", flush=True)
    X, y, W = workloads.make_inputs(wl)
    net = S.Net((wl.batch,) + tuple(wl.chw), wl.layers)
    net.set_implicit_conv(False)
    n = net.param_count()
    dev = torch.device("cuda")
    Xd, yd = torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev)
    st0 = workloads.normal(9, 3, n, 1e-3)
    if rule == "adagrad":
        st0 = np.abs(st0) + np.float32(0.1)
    R = S.Rule(rule, 0.01, 0.9, 1e-8)
    ws = net.workspace()
    la, lb = torch.empty(1, device=dev), torch.empty(1, device=dev)
    Wa, sa = torch.from_numpy(W).to(dev), torch.from_numpy(st0).to(dev)
    gb = S.GradBuf(n)
    net.compute_gradient_into(Wa, Xd, yd, gb, la, ws)
    g = gb.data.clone()
    S.apply_update(Wa, gb, sa, R)
    Wb, sb = torch.from_numpy(W).to(dev), torch.from_numpy(st0).to(dev)
    net.train_step(Wb, Xd, yd, sb, R, lb, ws)
    torch.cuda.synchronize()
    assert la.item() == lb.item()
    assert torch.equal(Wa, Wb) and torch.equal(sa, sb)
    onet = O.OracleNet(wl.chw, wl.layers)
    _, g_ref = onet.gradient(W, X, y)
    wo = [onet.params[i][0] for i in sorted(onet.params)]
    bo = [onet.params[i][2] for i in sorted(onet.params)]
    per_tensor_grad_check(g.cpu().numpy(), g_ref, wo, bo, n)
