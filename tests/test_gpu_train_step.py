"""The timed path against the oracle directly.

sgd_train_step applies each layer's update rule in the epilogue of its dedw
product (the path the benchmark times, launched call by call or replayed as
a HIP graph).  Here its W, optimiser state and loss are compared with the
oracle's gradient followed by the oracle's update rule (SPRINT report eq. (1)
and Algorithm 2 for plain and momentum SGD; the DistBelief review's Adagrad;
the PIPE report's appendix A for Nesterov momentum and weight decay):

  * loss to |dL| <= 1e-5 |L|;
  * per parameter tensor, W and the state within the distance a gradient
    inside the gradient contract (max|dg| <= 1e-4 max|g|) can move them
    through the rule, plus a few ulps of the rounded statements
    (tests/_util.update_tolerance).

Two steps per case: the second starts from the GPU's own W and state after
the first (the oracle's gradient is taken there), so errors do not compound
and the momentum and Adagrad states are non-trivial.  Config 2 (the MLP at
its full batch of 512, momentum mu = 0.9, eta = 0.01, V0 = 0) is compared
over all 115,435,010 parameters.
"""
import numpy as np
import pytest

import oracle as O
import workloads
from tests._util import LOSS_RTOL, check_update, tensor_bounds

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import sgd_cnns_amd as S  # noqa: E402

IMPLICIT_NET = [("conv", 16, 3, 1), ("relu",), ("conv", 32, 3, 1), ("relu",), ("pool", 2),
                ("conv", 16, 5, 2), ("relu",), ("conv", 48, 1, 0), ("relu",), ("conv", 32, 3, 0), ("relu",),
                ("fc", 10), ("softmax_ce",)]

NETS = {
    "lenet5": workloads.WORKLOADS["lenet5"],
    "mlp_ragged": workloads.Workload("mlp_ragged", 31, 70, (3072, 1, 1),
                                     [("fc", 300), ("relu",), ("fc", 129), ("relu",), ("fc", 10), ("softmax_ce",)]),
    "vgg_cifar_b2": workloads.WORKLOADS["vgg_cifar"].with_batch(2),
    "implicit_conv": workloads.Workload("implicit_conv", 41, 3, (3, 10, 10), IMPLICIT_NET),
    # k = 32: every fc weight gradient on the short-reduction kernel, 4096 x 4096 with two column blocks per
    # batch of loads (plain SGD), the others one
    "mlp_b32": workloads.Workload("mlp_b32", 35, 32, (3072, 1, 1),
                                  [("fc", 4096), ("relu",), ("fc", 4096), ("relu",), ("fc", 10), ("softmax_ce",)]),
}

# (rule, eta, mu, eps, decay)
RULES = {
    "plain": ("plain", 0.01, 0.0, 0.0, 0.0),
    "plain_wd": ("plain", 0.01, 0.0, 0.0, 5e-4),
    "momentum": ("momentum", 0.01, 0.9, 0.0, 0.0),
    "nesterov_wd": ("nesterov", 0.01, 0.9, 0.0, 5e-4),
    "adagrad": ("adagrad", 0.01, 0.0, 1e-8, 0.0),
}


def initial_state(rule, n, seed):
    if rule == "plain":
        return None
    if rule == "adagrad":
        return np.abs(workloads.normal(seed, 3, n)) + np.float32(0.1)
    return workloads.normal(seed, 3, n, 1e-3)


def compare_step(onet, w_offs, b_offs, X, y, W_prev, st_prev, W_gpu, st_gpu, l_gpu, spec, label):
    rule, eta, mu, eps, decay = spec
    l_ref, g_ref = onet.gradient(W_prev, X, y)
    assert abs(l_gpu - l_ref) <= LOSS_RTOL * abs(l_ref), (label, l_gpu, l_ref)
    W_ref = W_prev.copy()
    st_ref = None if st_prev is None else st_prev.copy()
    O.apply_rule(rule, W_ref, st_ref, g_ref, eta, mu, eps, decay)
    worst = 0.0
    for name, a, b in tensor_bounds(w_offs, b_offs, W_prev.size):
        sl = slice(a, b)
        worst = max(worst, check_update(f"{label} {name}", rule, g_ref[sl], W_prev[sl],
                                        None if st_prev is None else st_prev[sl], W_ref[sl],
                                        None if st_ref is None else st_ref[sl], W_gpu[sl],
                                        None if st_gpu is None else st_gpu[sl], eta, mu, decay))
    return l_ref, worst


@pytest.mark.parametrize("rname", list(RULES))
@pytest.mark.parametrize("case", list(NETS))
def test_train_step_matches_oracle(case, rname):
    wl = NETS[case]
    spec = RULES[rname]
    print(f"[train_step-vs-oracle] {case} {rname}", flush=True)
    X, y, W0 = workloads.make_inputs(wl)
    net = S.Net((wl.batch,) + tuple(wl.chw), wl.layers)
    onet = O.OracleNet(wl.chw, wl.layers)
    n = net.param_count()
    assert n == onet.param_count()
    w_offs, b_offs = net.param_offsets()
    st0 = initial_state(spec[0], n, 50 + len(case))
    dev = torch.device("cuda")
    Wd = torch.from_numpy(W0).to(dev)
    sd = None if st0 is None else torch.from_numpy(st0).to(dev)
    Xd, yd = torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev)
    loss = torch.empty(1, device=dev)
    ws = net.workspace()
    rule = S.Rule(*spec)
    W_prev, st_prev = W0, st0
    for step in range(2):
        net.train_step(Wd, Xd, yd, sd, rule, loss, ws)
        torch.cuda.synchronize()
        W_gpu = Wd.cpu().numpy()
        st_gpu = None if sd is None else sd.cpu().numpy()
        l_ref, worst = compare_step(onet, w_offs, b_offs, X, y, W_prev, st_prev, W_gpu, st_gpu, float(loss.item()),
                                    spec, f"{case}/{rname} step {step + 1}")
        print(f"[train_step-vs-oracle] step {step + 1}: loss {loss.item():.7f} (oracle {l_ref:.7f}); "
              f"worst |d|/bound {worst:.3f}", flush=True)
        W_prev, st_prev = W_gpu, st_gpu


@pytest.mark.parametrize("case,rname", [("lenet5", "plain"), ("vgg_cifar_b2", "momentum"), ("mlp_ragged", "adagrad")])
def test_graph_replays_match_oracle(case, rname):
    """The step recorded once as a HIP graph (the form the benchmark times when it is faster), replayed
    three times with the caller's own device work in between, each replay against the oracle."""
    wl = NETS[case]
    spec = RULES[rname]
    print(f"[graph-vs-oracle] {case} {rname}", flush=True)
    X, y, W0 = workloads.make_inputs(wl)
    net = S.Net((wl.batch,) + tuple(wl.chw), wl.layers)
    onet = O.OracleNet(wl.chw, wl.layers)
    n = net.param_count()
    w_offs, b_offs = net.param_offsets()
    st0 = initial_state(spec[0], n, 61)
    dev = torch.device("cuda")
    Wd = torch.from_numpy(W0).to(dev)
    sd = None if st0 is None else torch.from_numpy(st0).to(dev)
    Xd, yd = torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev)
    loss = torch.empty(1, device=dev)
    ws = net.workspace()
    graph = S.StepGraph(net, Wd, Xd, yd, sd, S.Rule(*spec), loss, ws)
    W_prev, st_prev = W0, st0
    for rep in range(3):
        graph.launch()
        torch.cuda.synchronize()
        W_gpu = Wd.cpu().numpy()
        st_gpu = None if sd is None else sd.cpu().numpy()
        compare_step(onet, w_offs, b_offs, X, y, W_prev, st_prev, W_gpu, st_gpu, float(loss.item()), spec,
                     f"{case}/{rname} replay {rep + 1}")
        W_prev, st_prev = W_gpu, st_gpu
        ws.zero_()   # the caller's own work between replays: the step must not depend on the old workspace


def _mlp_chain(onet, net, ws, W, X, y, layers):
    """For an fc/ReLU network: the GPU's forward activations (from the workspace after the step), the
    pure oracle's forward activations and loss, and the oracle's whole backward pass -- softmax-CE,
    then each layer's dedw, dedb and dedx_fc products and ReLU backward (SPRINT report section 3.3's
    table; the PIPE report's section 2 order), every upstream gradient the oracle's own from the layer
    above -- with each layer's product taken on the GPU's forward activation of its input.

    Taking the GPU's activations keeps both sides on the same side of every ReLU kink: at this size a
    handful of activations lie within rounding of zero, and an oracle that recomputes them may mask
    one the GPU passes (or the reverse), which moves one sample's whole contribution to the gradient
    of every layer below.  The forward activations themselves are checked layer by layer against the
    oracle in tests/test_gpu_fullsize.py; here the mask disagreements are counted."""
    fc = [i for i, L in enumerate(layers) if L[0] == "fc"]
    N = X.shape[0]
    outs = {}
    for i in fc:
        v = net.view(ws, i, S.T_OUT).cpu().numpy()
        outs[i] = np.ascontiguousarray(v[:, :net.tensor_info(i, S.T_OUT)[1][1]])
    # the pure oracle's forward pass (its own activations) and loss
    a = X.reshape(N, -1)
    flips = []
    for j, i in enumerate(fc):
        w, b = onet.weight(W, i)
        z = O.fc_fwd(a, w, b)
        if i + 1 < len(layers) and layers[i + 1][0] == "relu":
            z = O.relu_fwd(z)
            flips.append(int(np.count_nonzero((z > 0) != (outs[i] > 0))))
        a = z
    l_pure, _ = O.softmax_ce(a, y)
    # the backward chain on the GPU's activations
    _, d = O.softmax_ce(outs[fc[-1]], y)
    g = np.zeros(W.size, np.float32)
    for j in range(len(fc) - 1, -1, -1):
        i = fc[j]
        a_in = X.reshape(N, -1) if j == 0 else outs[fc[j - 1]]
        w, _ = onet.weight(W, i)
        wo, _, bo, nb = onet.params[i]
        dw, db, da = O.fc_bwd(a_in, w, d, need_da=j > 0)
        g[wo:wo + dw.size] = dw.ravel()
        g[bo:bo + nb] = db
        if j > 0:
            d = O.relu_bwd(a_in, da)
    return l_pure, g, flips


def test_mlp5000_config_full_batch_matches_oracle():
    """Config 2: fc 3072-5000x5-10 with ReLU and softmax-CE, batch 512 U[0,1) images, He-normal
    weights, one gradient step plus the momentum update (mu = 0.9, eta = 0.01, V0 = 0), through the
    call the benchmark times; then a second step from the GPU's W1, V1 (mu V != 0).  Per step: the
    loss against the pure oracle's (end to end); all 115,435,010 weights and momenta per tensor
    against the oracle's backward chain (see _mlp_chain) followed by the oracle's momentum rule.  A
    graph replay of the first step from the same W0, V0 must give the eager step's W1, V1 and loss
    bitwise."""
    wl = workloads.WORKLOADS["mlp5000"]
    spec = (wl.rule, wl.eta, wl.mu, wl.eps, 0.0)
    X, y, W0 = workloads.make_inputs(wl)
    net = S.Net((wl.batch,) + tuple(wl.chw), wl.layers)
    onet = O.OracleNet(wl.chw, wl.layers)
    n = net.param_count()
    assert n == 115_435_010
    w_offs, b_offs = net.param_offsets()
    V0 = np.zeros(n, np.float32)
    dev = torch.device("cuda")
    Wd, Vd = torch.from_numpy(W0).to(dev), torch.from_numpy(V0).to(dev)
    Xd, yd = torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev)
    loss = torch.empty(1, device=dev)
    ws = net.workspace()
    ws_g = net.workspace()
    rule = S.Rule(*spec)
    # the graph form of the first step, from the same start, in its own workspace
    Wg, Vg = torch.from_numpy(W0).to(dev), torch.from_numpy(V0).to(dev)
    lg = torch.empty(1, device=dev)
    graph = S.StepGraph(net, Wg, Xd, yd, Vg, rule, lg, ws_g)
    graph.launch()
    net.train_step(Wd, Xd, yd, Vd, rule, loss, ws)
    torch.cuda.synchronize()
    assert lg.item() == loss.item()
    assert torch.equal(Wg, Wd) and torch.equal(Vg, Vd)
    del graph, Wg, Vg, ws_g
    W_prev, V_prev = W0, V0
    for step in range(2):
        if step == 1:
            net.train_step(Wd, Xd, yd, Vd, rule, loss, ws)
            torch.cuda.synchronize()
        W_gpu, V_gpu, l_gpu = Wd.cpu().numpy(), Vd.cpu().numpy(), float(loss.item())
        print(f"[config2] step {step + 1}: oracle", flush=True)
        l_pure, g_ref, flips = _mlp_chain(onet, net, ws, W_prev, X, y, wl.layers)
        assert abs(l_gpu - l_pure) <= LOSS_RTOL * abs(l_pure), (l_gpu, l_pure)
        W_ref, V_ref = W_prev.copy(), V_prev.copy()
        O.apply_rule(*spec[:1], W_ref, V_ref, g_ref, *spec[1:])
        worst = 0.0
        for name, a, b in tensor_bounds(w_offs, b_offs, n):
            sl = slice(a, b)
            worst = max(worst, check_update(f"config2 step {step + 1} {name}", spec[0], g_ref[sl], W_prev[sl],
                                            V_prev[sl], W_ref[sl], V_ref[sl], W_gpu[sl], V_gpu[sl], spec[1],
                                            spec[2]))
        print(f"[config2] step {step + 1}: loss {l_gpu:.7f} (oracle {l_pure:.7f}); worst |d|/bound {worst:.3f}; "
              f"ReLU masks where the pure oracle's forward pass disagrees, per layer: {flips}", flush=True)
        W_prev, V_prev = W_gpu, V_gpu


# An fc net whose weight gradients have k = 320 (20 slices of 16): 4096 x 4097 and 4096 x 3073
# products with the update in their epilogue, more tiles than resident blocks, so whole tiles and a
# stream-K remainder (partial sums reduced by the fix-up kernel, which applies the rule) both occur.
MLP_K320 = workloads.Workload("mlp_k320", 33, 320, (3072, 1, 1),
                            [("fc", 4096), ("relu",), ("fc", 4096), ("relu",), ("fc", 10), ("softmax_ce",)])


@pytest.mark.parametrize("rname", ["momentum", "adagrad", "nesterov_wd"])
def test_fc_update_k320_matches_oracle(rname):
    """Two training steps of MLP_K320 against the oracle's backward chain on the GPU's activations (the
    batch is large enough for ReLU-kink flips, see _mlp_chain) followed by the oracle's rule."""
    wl = MLP_K320
    spec = RULES[rname]
    print(f"[mlp_k320] {rname}", flush=True)
    X, y, W0 = workloads.make_inputs(wl)
    net = S.Net((wl.batch,) + tuple(wl.chw), wl.layers)
    onet = O.OracleNet(wl.chw, wl.layers)
    n = net.param_count()
    w_offs, b_offs = net.param_offsets()
    st0 = initial_state(spec[0], n, 77)
    dev = torch.device("cuda")
    Wd = torch.from_numpy(W0).to(dev)
    sd = None if st0 is None else torch.from_numpy(st0).to(dev)
    Xd, yd = torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev)
    loss = torch.empty(1, device=dev)
    ws = net.workspace()
    rule = S.Rule(*spec)
    W_prev, st_prev = W0, st0
    for step in range(2):
        net.train_step(Wd, Xd, yd, sd, rule, loss, ws)
        torch.cuda.synchronize()
        W_gpu, st_gpu, l_gpu = Wd.cpu().numpy(), sd.cpu().numpy(), float(loss.item())
        l_pure, g_ref, flips = _mlp_chain(onet, net, ws, W_prev, X, y, wl.layers)
        assert abs(l_gpu - l_pure) <= LOSS_RTOL * abs(l_pure), (l_gpu, l_pure)
        W_ref, st_ref = W_prev.copy(), st_prev.copy()
        O.apply_rule(spec[0], W_ref, st_ref, g_ref, *spec[1:])
        worst = 0.0
        for name, a, b in tensor_bounds(w_offs, b_offs, n):
            sl = slice(a, b)
            worst = max(worst, check_update(f"mlp_k320 {rname} step {step + 1} {name}", spec[0], g_ref[sl],
                                            W_prev[sl], st_prev[sl], W_ref[sl], st_ref[sl], W_gpu[sl], st_gpu[sl],
                                            spec[1], spec[2], spec[4]))
        print(f"[mlp_k320] step {step + 1}: worst |d|/bound {worst:.3f}; mask flips {flips}", flush=True)
        W_prev, st_prev = W_gpu, st_gpu


def test_debug_mode_rejects_bad_labels_before_launch():
    """A host-built out-of-range label: in debug mode the call returns SGD_EINVAL and launches nothing
    (W untouched); in normal mode the softmax kernel never indexes with it and the loss is NaN."""
    wl = NETS["lenet5"]
    X, y, W0 = workloads.make_inputs(wl)
    y = y.copy()
    y[5] = wl.classes          # one past the last class
    net = S.Net((wl.batch,) + tuple(wl.chw), wl.layers)
    dev = torch.device("cuda")
    Wd = torch.from_numpy(W0).to(dev)
    Xd, yd = torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev)
    loss = torch.full((1,), 7.0, device=dev)
    ws = net.workspace()
    grad = torch.zeros(net.param_count(), device=dev)
    net.set_debug(True)
    with pytest.raises(S.SgdError) as e:
        net.train_step(Wd, Xd, yd, None, S.Rule("plain", 0.01), loss, ws)
    assert e.value.code == S.EINVAL and "row 5" in str(e.value)
    with pytest.raises(S.SgdError):
        net.compute_gradient(Wd, Xd, yd, grad, loss, ws)
    with pytest.raises(S.SgdError):
        S.StepGraph(net, Wd, Xd, yd, None, S.Rule("plain", 0.01), loss, ws)
    torch.cuda.synchronize()
    assert loss.item() == 7.0 and torch.equal(Wd.cpu(), torch.from_numpy(W0))
    y[5] = -3
    yd.copy_(torch.from_numpy(y))
    with pytest.raises(S.SgdError):
        net.compute_gradient(Wd, Xd, yd, grad, loss, ws)
    # normal mode: no check, no out-of-range read; the bad row makes the loss NaN
    net.set_debug(False)
    net.compute_gradient(Wd, Xd, yd, grad, loss, ws)
    torch.cuda.synchronize()
    assert np.isnan(loss.item())
    # debug mode with valid labels runs normally and gives the same result as without it
    y[5] = 3
    yd.copy_(torch.from_numpy(y))
    net.set_debug(True)
    net.compute_gradient(Wd, Xd, yd, grad, loss, ws)
    g_dbg, l_dbg = grad.clone(), loss.item()
    net.set_debug(False)
    net.compute_gradient(Wd, Xd, yd, grad, loss, ws)
    torch.cuda.synchronize()
    assert l_dbg == loss.item() and torch.equal(g_dbg, grad)
