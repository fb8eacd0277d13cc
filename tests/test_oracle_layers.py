"""Pins for the CPU oracle's layer functions (CPU only).

Each oracle layer function is checked against something other than itself:
library routines that compute the same definition (scipy's 2-D correlation,
numpy matrix products, scipy's logsumexp, torch's float64 CPU convolution and
autograd), closed forms (equal logits, all-zero weights) and invariants (a conv
whose filter covers the whole input is an fc layer; a 1x1 conv is a per-pixel
matrix product).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.signal
import scipy.special

import oracle as O
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- shapes ----

@pytest.mark.parametrize("name", ["lenet5", "mlp5000", "vgg_cifar", "vgg16"])
def test_param_count_eq3(name):
    # SPRINT report sec. 3.2 eq. (3), values worked by hand (tests/golden).
    golden = json.load(open(os.path.join(GOLDEN, "param_counts.json")))
    wl = workloads.WORKLOADS[name]
    assert O.OracleNet(wl.chw, wl.layers).param_count() == golden[name]["value"]


def test_fc_input_sizes_fix_padding():
    # The configs' first fc widths (400, 512, 25088) pin the padded-shape rule.
    for name, fan in [("lenet5", 400), ("vgg_cifar", 512), ("vgg16", 25088)]:
        wl = workloads.WORKLOADS[name]
        net = O.OracleNet(wl.chw, wl.layers)
        first_fc = min(i for i, L in enumerate(wl.layers) if L[0] == "fc")
        assert net.params[first_fc][1][1] == fan


def test_pool_must_divide():
    with pytest.raises(ValueError):
        O.OracleNet((1, 5, 5), [("pool", 2), ("fc", 3), ("softmax_ce",)])


# ------------------------------------------------------------ convolution ----

@pytest.mark.parametrize("dtype,tol", [(np.float64, 1e-12), (np.float32, 2e-6)])
@pytest.mark.parametrize("N,Ci,H,W,Co,c,P", [(2, 3, 7, 6, 4, 3, 1), (1, 2, 9, 9, 3, 5, 2), (2, 1, 6, 8, 2, 5, 0)])
def test_conv_fwd_vs_scipy_correlate(dtype, tol, N, Ci, H, W, Co, c, P):
    r = _rng(1)
    x = r.standard_normal((N, Ci, H, W)).astype(dtype)
    w = r.standard_normal((Co, Ci, c, c)).astype(dtype)
    b = r.standard_normal(Co).astype(dtype)
    y = O.conv_fwd(x, w, b, P, dtype)
    xp = np.pad(x.astype(np.float64), ((0, 0), (0, 0), (P, P), (P, P)))
    ref = np.zeros(y.shape)
    for n in range(N):
        for co in range(Co):
            ref[n, co] = b[co] + sum(scipy.signal.correlate2d(xp[n, ci], w[co, ci].astype(np.float64), "valid")
                                     for ci in range(Ci))
    np.testing.assert_allclose(y, ref, rtol=tol, atol=tol * np.abs(ref).max())


def test_conv_fwd_and_bwd_vs_torch_autograd():
    torch = pytest.importorskip("torch")
    r = _rng(2)
    N, Ci, H, W, Co, c, P = 2, 3, 8, 7, 5, 3, 1
    x = r.standard_normal((N, Ci, H, W))
    w = r.standard_normal((Co, Ci, c, c))
    b = r.standard_normal(Co)
    dy = r.standard_normal((N, Co, H + 2 * P - c + 1, W + 2 * P - c + 1))
    y = O.conv_fwd(x, w, b, P, np.float64)
    dw, db, dx = O.conv_bwd(x, w, dy, P, True, np.float64)
    tx = torch.tensor(x, requires_grad=True)
    tw = torch.tensor(w, requires_grad=True)
    tb = torch.tensor(b, requires_grad=True)
    ty = torch.nn.functional.conv2d(tx, tw, tb, padding=P)
    ty.backward(torch.tensor(dy))
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=1e-12, atol=1e-11)
    np.testing.assert_allclose(db, tb.grad.numpy(), rtol=1e-12, atol=1e-11)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-12, atol=1e-11)


def test_conv_point_functions_match_torch():
    torch = pytest.importorskip("torch")
    r = _rng(3)
    N, Ci, H, W, Co, c, P = 2, 4, 9, 7, 3, 3, 1
    x = r.standard_normal((N, Ci, H, W)).astype(np.float32)
    w = r.standard_normal((Co, Ci, c, c)).astype(np.float32)
    b = r.standard_normal(Co).astype(np.float32)
    dy = r.standard_normal((N, Co, H, W)).astype(np.float32)
    tx = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    tw = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    ty = torch.nn.functional.conv2d(tx, tw, torch.tensor(b, dtype=torch.float64), padding=P)
    ty.backward(torch.tensor(dy, dtype=torch.float64))
    for (n, co, oy, ox) in [(0, 0, 0, 0), (1, 2, 8, 6), (0, 1, 4, 3), (1, 0, 0, 6)]:
        assert O.conv_fwd_point(x, w, b, P, n, co, oy, ox) == pytest.approx(ty[n, co, oy, ox].item(), abs=1e-12)
    for (co, ci, ky, kx) in [(0, 0, 0, 0), (2, 3, 2, 2), (1, 2, 1, 0)]:
        assert O.conv_dw_point(x, dy, c, P, co, ci, ky, kx) == pytest.approx(tw.grad[co, ci, ky, kx].item(),
                                                                           abs=1e-10)
    for (n, ci, iy, ix) in [(0, 0, 0, 0), (1, 3, 8, 6), (0, 2, 5, 1)]:
        assert O.conv_dx_point(w, dy, (H, W), P, n, ci, iy, ix) == pytest.approx(tx.grad[n, ci, iy, ix].item(),
                                                                                abs=1e-10)
    for co in range(Co):
        assert O.conv_db_point(dy, co) == pytest.approx(float(dy[:, co].astype(np.float64).sum()), abs=1e-10)


def test_one_by_one_conv_is_per_pixel_matmul():
    r = _rng(4)
    x = r.standard_normal((3, 5, 4, 6))
    w = r.standard_normal((7, 5, 1, 1))
    b = r.standard_normal(7)
    y = O.conv_fwd(x, w, b, 0, np.float64)
    ref = np.matmul(w[:, :, 0, 0], x.reshape(3, 5, 24)).reshape(3, 7, 4, 6) + b[None, :, None, None]
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_full_width_conv_equals_fc_both_directions():
    # eq. (3) counts an fc layer as a conv whose filter spans its whole input.
    r = _rng(5)
    N, Ci, S, Co = 3, 4, 5, 6
    x = r.standard_normal((N, Ci, S, S))
    w = r.standard_normal((Co, Ci, S, S))
    b = r.standard_normal(Co)
    dy = r.standard_normal((N, Co, 1, 1))
    yc = O.conv_fwd(x, w, b, 0, np.float64)
    yf = O.fc_fwd(x.reshape(N, -1), w.reshape(Co, -1), b, np.float64)
    np.testing.assert_array_equal(yc.reshape(N, Co), yf)
    dwc, dbc, dxc = O.conv_bwd(x, w, dy, 0, True, np.float64)
    dwf, dbf, dxf = O.fc_bwd(x.reshape(N, -1), w.reshape(Co, -1), dy.reshape(N, Co), True, np.float64)
    np.testing.assert_allclose(dwc.reshape(Co, -1), dwf, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dbc, dbf, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dxc.reshape(N, -1), dxf, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------- fc layer ----

def test_fc_vs_numpy():
    r = _rng(6)
    a = r.standard_normal((5, 13))
    w = r.standard_normal((7, 13))
    b = r.standard_normal(7)
    dz = r.standard_normal((5, 7))
    np.testing.assert_allclose(O.fc_fwd(a, w, b, np.float64), a @ w.T + b, rtol=1e-13, atol=1e-13)
    dw, db, da = O.fc_bwd(a, w, dz, True, np.float64)
    np.testing.assert_allclose(dw, dz.T @ a, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(db, dz.sum(0), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(da, dz @ w, rtol=1e-13, atol=1e-13)


def test_fc_float32_rounds_once_from_double_sum():
    r = _rng(7)
    a = r.standard_normal((4, 300)).astype(np.float32)
    w = r.standard_normal((3, 300)).astype(np.float32)
    b = r.standard_normal(3).astype(np.float32)
    z = O.fc_fwd(a, w, b, np.float32)
    ref = (a.astype(np.float64) @ w.astype(np.float64).T + b).astype(np.float32)
    # A double sum of 300 products rounds to the same float as the exact sum
    # unless the exact value sits within ~1e-13 relative of a rounding boundary.
    assert np.mean(z == ref) == 1.0


# ------------------------------------------------------------ relu / pool ----

def test_relu():
    y = np.array([-1.0, 0.0, 2.5, -0.0, 3.0], np.float32)
    a = O.relu_fwd(y)
    np.testing.assert_array_equal(a, [0, 0, 2.5, 0, 3.0])
    assert np.isnan(O.relu_fwd(np.array([np.nan], np.float32))[0])   # NaN passes through
    dy = O.relu_bwd(a, np.ones(5, np.float32))
    np.testing.assert_array_equal(dy, [0, 0, 1, 0, 1])   # derivative 0 at 0


def test_maxpool_vs_numpy_and_first_max_ties():
    r = _rng(8)
    x = r.standard_normal((2, 3, 6, 8)).astype(np.float32)
    y, am = O.maxpool_fwd(x, 2)
    ref = x.reshape(2, 3, 3, 2, 4, 2).max(axis=(3, 5))
    np.testing.assert_array_equal(y, ref)
    # hand-built ties: first maximum in row-major window order wins
    t = np.array([[[[1, 3, 0, 0], [3, 2, 0, 0], [5, 5, -1, -2], [5, 5, -3, -1]]]], np.float32)
    yt, amt = O.maxpool_fwd(t, 2)
    np.testing.assert_array_equal(yt[0, 0], [[3, 0], [5, -1]])
    np.testing.assert_array_equal(amt[0, 0], [[1, 0], [0, 0]])
    dx = O.maxpool_bwd(np.ones((1, 1, 2, 2), np.float32), amt, t.shape, 2)
    np.testing.assert_array_equal(dx[0, 0], [[0, 1, 1, 0], [0, 0, 0, 0], [1, 0, 1, 0], [0, 0, 0, 0]])


def test_maxpool_nan_propagates():
    x = np.zeros((1, 1, 2, 2), np.float32)
    x[0, 0, 1, 1] = np.nan
    y, _ = O.maxpool_fwd(x, 2)
    assert np.isnan(y).all()


def test_maxpool_bwd_vs_torch():
    torch = pytest.importorskip("torch")
    r = _rng(9)
    x = r.standard_normal((2, 3, 6, 4))
    dy = r.standard_normal((2, 3, 3, 2))
    y, am = O.maxpool_fwd(x, 2, np.float64)
    dx = O.maxpool_bwd(dy, am, x.shape, 2, np.float64)
    tx = torch.tensor(x, requires_grad=True)
    ty = torch.nn.functional.max_pool2d(tx, 2)
    ty.backward(torch.tensor(dy))
    np.testing.assert_array_equal(y, ty.detach().numpy())
    np.testing.assert_array_equal(dx, tx.grad.numpy())


# ------------------------------------------------------------- softmax-CE ----

def test_softmax_ce_vs_scipy_logsumexp():
    r = _rng(10)
    z = (r.standard_normal((6, 11)) * 5).astype(np.float64)
    y = r.integers(0, 11, 6).astype(np.int32)
    for rs in (False, True):
        loss, dz = O.softmax_ce(z, y, rs, np.float64)
        lse = scipy.special.logsumexp(z, axis=1)
        s = 1.0 if rs else 1.0 / 6
        assert loss == pytest.approx(s * float(np.sum(lse - z[np.arange(6), y])), rel=1e-14)
        ref = scipy.special.softmax(z, axis=1)
        ref[np.arange(6), y] -= 1
        np.testing.assert_allclose(dz, s * ref, rtol=1e-12, atol=1e-15)


def test_softmax_ce_equal_logits_closed_form():
    for C in (10, 1000):
        z = np.full((4, C), 3.25, np.float32)
        y = np.array([0, 1, C - 1, 1], np.int32)
        loss, dz = O.softmax_ce(z, y)
        assert loss == pytest.approx(math.log(C), rel=1e-15)
        expect = np.full((4, C), 1.0 / C)
        expect[np.arange(4), y] -= 1
        np.testing.assert_allclose(dz, expect / 4, rtol=2e-7, atol=0)


def test_softmax_ce_rejects_bad_label():
    with pytest.raises(ValueError):
        O.softmax_ce(np.zeros((2, 3), np.float32), np.array([0, 3], np.int32))
