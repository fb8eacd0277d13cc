"""Full-size GPU parity, layer by layer, at the workloads' real shapes.

The oracle cannot run the VGG steps end to end in seconds, so each layer is
checked locally: the GPU's own input activation and upstream gradient (read
from the workspace) are fed to the oracle's definitions (the direct
convolution sums, the naive fc loops), and the GPU's outputs are compared to
max|d| <= 1e-4 max|ref| with the scale taken from the oracle's values only:

  * fc layers (forward, dW, db, dX): whole tensors;
  * conv layers: whole output maps of a subset of output channels (forward),
    whole dW rows [co][ci][ky][kx] and db of a subset of output channels (the
    whole dW and db where the oracle's cost allows), whole input-gradient maps
    of a subset of input channels (dedx_conv + col2im or the gathered dedx,
    with the ReLU mask);
  * max-pooling forward (values and argmax) and backward (routing and the
    ReLU mask): exactly, over whole tensors;
  * loss to 1e-5 relative, and the logits' gradient over the whole tensor.

The timed path, sgd_train_step with the workload's rule in the dedw
epilogues, is run from the same weights: its updated weights (and momentum)
are compared with the oracle's rule applied to the oracle's dW and db, for
every fc tensor and every checked conv row (tests/_util.update_tolerance).
"""
import numpy as np
import pytest

import oracle as O
import workloads
from tests._util import GRAD_RTOL, LOSS_RTOL, check_update, nhwc_to_nchw

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import sgd_cnns_amd as S  # noqa: E402


def _to_nchw(t, layout):
    a = t.cpu().numpy()
    if layout == S.LAYOUT_NHWC:
        return nhwc_to_nchw(a)
    return np.ascontiguousarray(a)


def _close(name, got, ref):
    """max|got - ref| <= 1e-4 max|ref|, the scale from the oracle's values alone."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite GPU values"
    err = np.abs(got - ref).max() if got.size else 0.0
    scale = np.abs(ref).max() if ref.size else 0.0
    assert err <= GRAD_RTOL * scale + 1e-30, f"{name}: max|d| {err:.3e} > {GRAD_RTOL} * {scale:.3e}"
    return err / scale if scale else 0.0


class Step:
    """One compute_gradient on the GPU with every workspace tensor readable, and the fused training
    step (the benchmark's call) from the same weights."""

    def __init__(self, wl):
        self.wl = wl
        X, y, W = workloads.make_inputs(wl)
        self.X, self.y, self.W = X, y, W
        self.net = S.Net((wl.batch,) + tuple(wl.chw), wl.layers)
        self.onet = O.OracleNet(wl.chw, wl.layers)
        assert self.net.param_count() == self.onet.param_count() == W.size
        wo, bo = self.net.param_offsets()
        assert wo == [self.onet.params[i][0] for i in sorted(self.onet.params)]
        assert bo == [self.onet.params[i][2] for i in sorted(self.onet.params)]
        dev = torch.device("cuda")
        self.ws = self.net.workspace()
        Xd, yd = torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev)
        # the timed call first: W1 (and V1) after one step with the workload's rule, state zero
        self.rule = (wl.rule, wl.eta, wl.mu, wl.eps, 0.0)
        W1 = torch.from_numpy(W).to(dev)
        self.st0 = None if wl.rule == "plain" else np.zeros(W.size, np.float32) if wl.rule != "adagrad" else \
            np.full(W.size, 0.1, np.float32)
        st = None if self.st0 is None else torch.from_numpy(self.st0).to(dev)
        loss1 = torch.empty(1, device=dev)
        self.net.train_step(W1, Xd, yd, st, S.Rule(*self.rule), loss1, self.ws)
        torch.cuda.synchronize()
        self.W1 = W1.cpu().numpy()
        self.st1 = None if st is None else st.cpu().numpy()
        self.loss1 = float(loss1.item())
        del W1, st
        # then the gradient, whose workspace tensors are inspected
        grad = torch.empty(W.size, device=dev)
        loss = torch.empty(1, device=dev)
        self.net.compute_gradient(torch.from_numpy(W).to(dev), Xd, yd, grad, loss, self.ws)
        torch.cuda.synchronize()
        self.grad = grad.cpu().numpy()
        self.loss = float(loss.item())

    def t(self, i, which):
        v = self.net.view(self.ws, i, which)
        lay = self.net.tensor_info(i, which)[2]
        return v, lay

    def out_nchw(self, i):
        """Forward output of layer i as NCHW (or [N, F] for fc)."""
        v, lay = self.t(i, S.T_OUT)
        if lay == S.LAYOUT_ROWS:
            return v.cpu().numpy()
        return _to_nchw(v, lay)

    def dout_nchw(self, i):
        v, lay = self.t(i, S.T_DOUT)
        if lay == S.LAYOUT_ROWS:
            return v.cpu().numpy()
        return _to_nchw(v, lay)

    def input_of(self, i):
        """Activation entering layer i (the previous layer's output), and that layer's index."""
        if i == 0:
            return self.X, -1
        j = i - 1
        while self.wl.layers[j][0] == "relu":
            j -= 1
        return self.out_nchw(j), j

    def check_update_rows(self, name, off, rows, g_ref_rows):
        """The fused step's W (and state) at parameter rows `rows` of a tensor starting at `off`
        (rows of length g_ref_rows.shape[1]) against the oracle's rule on the oracle's gradient."""
        rule, eta, mu, eps, decay = self.rule
        L = g_ref_rows.shape[1]
        idx = (off + np.asarray(rows)[:, None] * L + np.arange(L)[None, :]).ravel()
        g = np.ascontiguousarray(g_ref_rows, np.float32).ravel()
        W0 = self.W[idx]
        st0 = None if self.st0 is None else self.st0[idx]
        W_ref = W0.copy()
        st_ref = None if st0 is None else st0.copy()
        O.apply_rule(rule, W_ref, st_ref, g, eta, mu, eps, decay)
        return check_update(name, rule, g, W0, st0, W_ref, st_ref, self.W1[idx],
                            None if self.st1 is None else self.st1[idx], eta, mu, decay)


def _pick(r, n, count, always=()):
    """`count` distinct indices in [0, n): the given ones (edges) first, then seeded random ones."""
    if count == "all" or count >= n:
        return list(range(n))
    out = [a % n for a in always]
    for v in r.permutation(n):
        if len(set(out)) >= count:
            break
        out.append(int(v))
    return sorted(set(out))


def check_step(wl, fwd_ch=4, dw_ch=4, dx_ch=2, seed=0):
    st = Step(wl)
    r = np.random.default_rng(seed)
    layers = wl.layers
    first_w = min(i for i, L in enumerate(layers) if L[0] in ("conv", "fc"))
    report = {}
    # ---- loss and logits' gradient from the GPU logits
    last_fc = max(i for i, L in enumerate(layers) if L[0] == "fc")
    logits = st.out_nchw(last_fc)
    l_ref, dz_ref = O.softmax_ce(logits, st.y)
    assert abs(st.loss - l_ref) <= LOSS_RTOL * abs(l_ref), (st.loss, l_ref)
    assert st.loss1 == st.loss, "the fused step's forward pass differs from the gradient call's"
    report["dlogits"] = _close("dlogits", st.dout_nchw(last_fc), dz_ref)
    for i, L in enumerate(layers):
        kind = L[0]
        if kind in ("relu", "softmax_ce"):
            continue
        relu_after = i + 1 < len(layers) and layers[i + 1][0] == "relu"
        x_in, src = st.input_of(i)
        src_masks = src >= 0 and layers[src][0] in ("conv", "fc") and src + 1 < len(layers) and \
            layers[src + 1][0] == "relu"
        print(f"[fullsize] {wl.name} layer {i} {L}", flush=True)
        if kind == "conv":
            co_n, c, P = L[1], L[2], L[3]
            w, b = st.onet.weight(st.W, i)
            wo, _, bo, _ = st.onet.params[i]
            y_gpu = st.out_nchw(i)
            dy = st.dout_nchw(i)
            N, Ci, H, Wd = x_in.shape
            xin = np.ascontiguousarray(x_in, np.float32)
            # forward: whole output maps of a channel subset
            cos = _pick(r, co_n, fwd_ch, (0, -1))
            y_ref = O.conv_fwd(xin, w[cos], b[cos], P)
            if relu_after:
                y_ref = np.maximum(y_ref, 0)
            report[f"{i}.fwd"] = _close(f"layer {i} conv fwd (out channels {cos})", y_gpu[:, cos], y_ref)
            # dedw rows and dedb of a channel subset (all channels where affordable)
            cos = _pick(r, co_n, dw_ch, (0, -1))
            dw_ref, db_ref, _ = O.conv_bwd(xin, np.ascontiguousarray(w[cos]), np.ascontiguousarray(dy[:, cos]), P,
                                           need_dx=False)
            g_w = st.grad[wo:wo + w.size].reshape(w.shape)
            g_b = st.grad[bo:bo + co_n]
            report[f"{i}.dw"] = _close(f"layer {i} conv dw (rows {len(cos)})", g_w[cos], dw_ref)
            report[f"{i}.db"] = _close(f"layer {i} conv db", g_b[cos], db_ref)
            # the fused step's update of those rows
            report[f"{i}.upd_w"] = st.check_update_rows(f"layer {i} conv W1", wo, cos, dw_ref.reshape(len(cos), -1))
            report[f"{i}.upd_b"] = st.check_update_rows(f"layer {i} conv b1", bo, cos, db_ref.reshape(len(cos), 1))
            # dedx_conv (+ col2im) over whole maps of an input-channel subset, ReLU mask of the layer below
            if i > first_w:
                dx_gpu = st.dout_nchw(src)
                cis = _pick(r, Ci, dx_ch, (0, -1))
                _, _, dx_ref = O.conv_bwd(np.ascontiguousarray(xin[:, cis]), np.ascontiguousarray(w[:, cis]), dy, P)
                if src_masks:
                    dx_ref = np.where(xin[:, cis] > 0, dx_ref, 0)
                report[f"{i}.dx"] = _close(f"layer {i} conv dx (in channels {cis})", dx_gpu[:, cis], dx_ref)
        elif kind == "pool":
            p = L[1]
            pooled = st.out_nchw(i)
            am_gpu, lay = st.t(i, S.T_ARGMAX)
            am_gpu = _to_nchw(am_gpu, lay).astype(np.int32)
            y_ref, am_ref = O.maxpool_fwd(x_in, p)
            np.testing.assert_array_equal(pooled, y_ref)
            np.testing.assert_array_equal(am_gpu, am_ref)
            # backward: route the pooled gradient to the argmax, then the ReLU mask of the conv below
            dpool = st.dout_nchw(i).reshape(pooled.shape)
            dx = O.maxpool_bwd(dpool, am_ref, x_in.shape, p)
            if src_masks:
                dx = O.relu_bwd(x_in, dx)
            np.testing.assert_array_equal(st.dout_nchw(src), dx)
            report[f"{i}.pool"] = 0.0
        elif kind == "fc":
            out_n = L[1]
            w, b = st.onet.weight(st.W, i)
            wo, _, bo, _ = st.onet.params[i]
            a = np.ascontiguousarray(x_in.reshape(x_in.shape[0], -1), np.float32)
            z_gpu = st.out_nchw(i)
            dz = st.dout_nchw(i)
            N = a.shape[0]
            z_ref = O.fc_fwd(a, w, b)
            if relu_after:
                z_ref = np.maximum(z_ref, 0)
            report[f"{i}.fwd"] = _close(f"layer {i} fc fwd", z_gpu, z_ref)
            dw_ref, db_ref, da = O.fc_bwd(a, w, np.ascontiguousarray(dz), i > first_w)
            g_w = st.grad[wo:wo + w.size].reshape(w.shape)
            g_b = st.grad[bo:bo + out_n]
            report[f"{i}.dw"] = _close(f"layer {i} fc dw", g_w, dw_ref)
            report[f"{i}.db"] = _close(f"layer {i} fc db", g_b, db_ref)
            report[f"{i}.upd_w"] = st.check_update_rows(f"layer {i} fc W1", wo, np.arange(out_n), dw_ref)
            report[f"{i}.upd_b"] = st.check_update_rows(f"layer {i} fc b1", bo, np.arange(out_n),
                                                        db_ref.reshape(out_n, 1))
            if i > first_w:
                if src_masks:
                    da = np.where(a > 0, da, 0)
                dx_gpu = st.dout_nchw(src).reshape(N, -1)
                report[f"{i}.dx"] = _close(f"layer {i} fc dx", dx_gpu, da)
    worst = max(v for k, v in report.items() if not k.endswith(("upd_w", "upd_b")))
    worst_u = max(v for k, v in report.items() if k.endswith(("upd_w", "upd_b")))
    print(f"[fullsize] {wl.name}: loss {st.loss:.6f} (oracle from GPU logits {l_ref:.6f}); worst |d|/max|ref| "
          f"{worst:.2e}; fused-step update worst |d|/bound {worst_u:.3f}", flush=True)
    return report


def test_mlp5000_full_batch():
    check_step(workloads.WORKLOADS["mlp5000"])


def test_vgg_cifar_full_batch():
    # every conv layer's whole dW and db
    check_step(workloads.WORKLOADS["vgg_cifar"], fwd_ch=8, dw_ch="all", dx_ch=4)


def test_vgg16_full_batch():
    check_step(workloads.WORKLOADS["vgg16"], fwd_ch=4, dw_ch=4, dx_ch=2)


def test_lenet5_layerwise():
    check_step(workloads.WORKLOADS["lenet5"], fwd_ch="all", dw_ch="all", dx_ch="all")
