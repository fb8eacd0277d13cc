"""Whole-network pins for the CPU oracle (CPU only).

* central finite differences of the double-storage oracle's loss agree with
  its backpropagated gradient on tiny nets (the mathematics of backprop);
* torch's float64 CPU autograd of the same network agrees (a library routine);
* all-zero weights give loss = ln C exactly and a closed-form last-bias
  gradient (every other gradient is zero);
* the gradient is additive over a split batch (SUM reduction) and a weighted
  mean (MEAN reduction), the identity the Chainer data-parallel step relies on
  when it sums two half-batch gradients and halves the learning rate.
"""
import math

import numpy as np
import pytest

import oracle as O

TINY_CNN = [("conv", 3, 3, 1), ("relu",), ("pool", 2), ("conv", 4, 3, 0), ("relu",),
            ("fc", 6), ("relu",), ("fc", 5), ("softmax_ce",)]
TINY_MLP = [("fc", 7), ("relu",), ("fc", 6), ("relu",), ("fc", 4), ("softmax_ce",)]


def _setup(chw, layers, N, seed, classes):
    r = np.random.default_rng(seed)
    net = O.OracleNet(chw, layers, dtype=np.float64)
    W = r.standard_normal(net.param_count()) * 0.5
    X = r.standard_normal((N,) + tuple(chw))
    y = r.integers(0, classes, N).astype(np.int32)
    return net, W, X, y


def _kinks(net, W, X):
    """Pre-ReLU values and pool windows, to skip coordinates that cross a kink."""
    out = []
    a = X
    for i, L in enumerate(net.layers):
        if L[0] == "conv":
            w, b = net.weight(W, i)
            a = O.conv_fwd(a, w, b, L[3], np.float64)
            out.append(a.ravel())
        elif L[0] == "relu":
            a = O.relu_fwd(a, np.float64)
        elif L[0] == "pool":
            a, _ = O.maxpool_fwd(a, L[1], np.float64)
        elif L[0] == "fc":
            w, b = net.weight(W, i)
            a = O.fc_fwd(a.reshape(a.shape[0], -1), w, b, np.float64)
            out.append(a.ravel())
    return out


@pytest.mark.parametrize("chw,layers,N,classes", [((2, 6, 6), TINY_CNN, 3, 5), ((9, 1, 1), TINY_MLP, 4, 4)])
def test_gradient_matches_central_differences(chw, layers, N, classes):
    net, W, X, y = _setup(chw, layers, N, 11, classes)
    loss, g = net.gradient(W, X, y)
    h = 1e-5
    r = np.random.default_rng(12)
    idx = r.choice(W.size, size=min(W.size, 120), replace=False)
    checked = 0
    for i in idx:
        Wp, Wm = W.copy(), W.copy()
        Wp[i] += h
        Wm[i] -= h
        # skip coordinates whose +-h step moves a ReLU input or a pool argmax across a kink
        kp, km = _kinks(net, Wp, X), _kinks(net, Wm, X)
        if any(np.any(np.sign(a) != np.sign(b)) for a, b in zip(kp, km)):
            continue
        fd = (net.loss(Wp, X, y) - net.loss(Wm, X, y)) / (2 * h)
        assert fd == pytest.approx(g[i], rel=1e-6, abs=1e-8), (i, fd, g[i])
        checked += 1
    assert checked > 60


def test_whole_net_vs_torch_autograd():
    torch = pytest.importorskip("torch")
    net, W, X, y = _setup((2, 6, 6), TINY_CNN, 3, 13, 5)
    loss, g = net.gradient(W, X, y)
    tW = torch.tensor(W, requires_grad=True)
    a = torch.tensor(X)
    for i, L in enumerate(net.layers):
        if L[0] in ("conv", "fc"):
            wo, shape, bo, nb = net.params[i]
            w = tW[wo:wo + int(np.prod(shape))].reshape(shape)
            b = tW[bo:bo + nb]
            if L[0] == "conv":
                a = torch.nn.functional.conv2d(a, w, b, padding=L[3])
            else:
                a = torch.nn.functional.linear(a.reshape(a.shape[0], -1), w, b)
        elif L[0] == "relu":
            a = torch.relu(a)
        elif L[0] == "pool":
            a = torch.nn.functional.max_pool2d(a, L[1])
        elif L[0] == "softmax_ce":
            tl = torch.nn.functional.cross_entropy(a, torch.tensor(y, dtype=torch.long))
    tl.backward()
    assert loss == pytest.approx(tl.item(), rel=1e-13)
    np.testing.assert_allclose(g, tW.grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("chw,layers,C", [((1, 12, 12), [("conv", 3, 5, 2), ("relu",), ("pool", 2), ("fc", 8),
                                                          ("relu",), ("fc", 10), ("softmax_ce",)], 10),
                                          ((20, 1, 1), [("fc", 16), ("relu",), ("fc", 1000), ("softmax_ce",)], 1000)])
def test_zero_weights_closed_form(chw, layers, C):
    # W = 0, b = 0: every logit is 0, so loss = ln C exactly; only the last
    # bias has a gradient, 1/C - (number of samples with label j)/N.
    net = O.OracleNet(chw, layers)
    N = 7
    r = np.random.default_rng(14)
    X = r.random((N,) + chw).astype(np.float32)
    y = r.integers(0, C, N).astype(np.int32)
    loss, g = net.gradient(np.zeros(net.param_count(), np.float32), X, y)
    assert loss == pytest.approx(math.log(C), rel=1e-15)
    last = max(net.params)
    wo, shape, bo, nb = net.params[last]
    expect = np.full(C, 1.0 / C) - np.bincount(y, minlength=C) / N
    np.testing.assert_allclose(g[bo:bo + nb], expect, rtol=1e-6, atol=1e-9)
    rest = np.ones(g.size, bool)
    rest[bo:bo + nb] = False
    assert np.all(g[rest] == 0)


def test_batch_additivity_sum_and_mean():
    r = np.random.default_rng(15)
    chw, layers = (2, 6, 6), TINY_CNN
    for reduce_sum in (True, False):
        net = O.OracleNet(chw, layers, reduce_sum=reduce_sum, dtype=np.float64)
        W = r.standard_normal(net.param_count()) * 0.5
        X = r.standard_normal((5,) + chw)
        y = r.integers(0, 5, 5).astype(np.int32)
        l_all, g_all = net.gradient(W, X, y)
        l1, g1 = net.gradient(W, X[:2], y[:2])
        l2, g2 = net.gradient(W, X[2:], y[2:])
        if reduce_sum:
            np.testing.assert_allclose(g_all, g1 + g2, rtol=1e-12, atol=1e-13)
            assert l_all == pytest.approx(l1 + l2, rel=1e-13)
        else:
            np.testing.assert_allclose(g_all, (2 * g1 + 3 * g2) / 5, rtol=1e-12, atol=1e-13)
            assert l_all == pytest.approx((2 * l1 + 3 * l2) / 5, rel=1e-13)
