"""Full-size GPU parity, layer by layer, at the workloads' real shapes.

The oracle cannot run these steps end to end in seconds, so each layer is
checked locally: the GPU's own input activation and upstream gradient (read
from the workspace) are fed to the oracle's definitions, and the GPU's
outputs are compared
  * at sampled points for convolution / fc forward, dedw, dedb, dedx (the
    oracle's single-output sums, or the fc loops on a row / column subset),
    to max|d| <= 1e-4 max|ref| per layer;
  * exactly over whole tensors for max-pooling forward (values and argmax)
    and backward (routing and the ReLU mask), which involve no rounding;
  * loss to 1e-5 relative and the logits' gradient from the GPU logits.
Together these cover every step of the forward and backward pass at the
sizes and launch configurations the benchmark times.
"""
import numpy as np
import pytest

import oracle as O
import workloads
from tests._util import LOSS_RTOL, nhwc_to_nchw

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import sgd_cnns_amd as S  # noqa: E402

RTOL = 1e-4


def _to_nchw(t, layout):
    a = t.cpu().numpy()
    if layout == S.LAYOUT_NHWC:
        return nhwc_to_nchw(a)
    return np.ascontiguousarray(a)


def _close(name, got, ref, scale):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref).max() if got.size else 0.0
    scale = max(scale, np.abs(ref).max() if ref.size else 0.0)
    assert err <= RTOL * scale + 1e-30, f"{name}: max|d| {err:.3e} > {RTOL} * {scale:.3e}"
    return err / scale if scale else 0.0


class Step:
    """One compute_gradient on the GPU with every workspace tensor readable."""

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
        grad = torch.empty(W.size, device=dev)
        loss = torch.empty(1, device=dev)
        self.net.compute_gradient(torch.from_numpy(W).to(dev), torch.from_numpy(X).to(dev),
                                  torch.from_numpy(y).to(dev), grad, loss, self.ws)
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


def check_step(wl, samples=24, seed=0):
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
    report["loss"] = _close("dlogits", st.dout_nchw(last_fc), dz_ref, 0.0)
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
            Ho, Wo = y_gpu.shape[2:]
            xin = np.ascontiguousarray(x_in, np.float32)
            # forward
            pts = [(r.integers(N), r.integers(co_n), r.integers(Ho), r.integers(Wo)) for _ in range(samples)]
            pts += [(0, 0, 0, 0), (N - 1, co_n - 1, Ho - 1, Wo - 1)]
            ref = [O.conv_fwd_point(xin, w, b, P, *p) for p in pts]
            if relu_after:
                ref = [max(v, 0.0) for v in ref]
            report[f"{i}.fwd"] = _close(f"layer {i} conv fwd", [y_gpu[p] for p in pts], ref, np.abs(y_gpu).max())
            # dedw and dedb
            g_w = st.grad[wo:wo + w.size].reshape(w.shape)
            g_b = st.grad[bo:bo + co_n]
            qs = [(r.integers(co_n), r.integers(Ci), r.integers(c), r.integers(c)) for _ in range(samples)]
            qs += [(0, 0, 0, 0), (co_n - 1, Ci - 1, c - 1, c - 1)]
            ref = [O.conv_dw_point(np.ascontiguousarray(xin[:, q[1]:q[1] + 1]),
                                   np.ascontiguousarray(dy[:, q[0]:q[0] + 1]), c, P, 0, 0, q[2], q[3]) for q in qs]
            report[f"{i}.dw"] = _close(f"layer {i} conv dw", [g_w[q] for q in qs], ref, np.abs(g_w).max())
            cos = sorted(set([0, co_n - 1] + list(r.integers(0, co_n, 8))))
            ref = [O.conv_db_point(np.ascontiguousarray(dy[:, co:co + 1]), 0) for co in cos]
            report[f"{i}.db"] = _close(f"layer {i} conv db", g_b[cos], ref, np.abs(g_b).max())
            # dedx_conv + col2im (the gradient entering the previous stage)
            if i > first_w:
                dx_gpu = st.dout_nchw(src)
                pts = [(r.integers(N), r.integers(Ci), r.integers(H), r.integers(Wd)) for _ in range(samples)]
                pts += [(0, 0, 0, 0), (N - 1, Ci - 1, H - 1, Wd - 1)]
                ref = []
                for (n, ci, iy, ix) in pts:
                    v = O.conv_dx_point(np.ascontiguousarray(w[:, ci:ci + 1]), np.ascontiguousarray(dy[n:n + 1]),
                                        (H, Wd), P, 0, 0, iy, ix)
                    if src_masks and not x_in[n, ci, iy, ix] > 0:
                        v = 0.0
                    ref.append(v)
                report[f"{i}.dx"] = _close(f"layer {i} conv dx", [dx_gpu[p] for p in pts], ref, np.abs(dx_gpu).max())
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
            rows = sorted(set([0, N - 1] + list(r.integers(0, N, 6))))
            z_ref = O.fc_fwd(a[rows], w, b)
            if relu_after:
                z_ref = np.maximum(z_ref, 0)
            report[f"{i}.fwd"] = _close(f"layer {i} fc fwd", z_gpu[rows], z_ref, np.abs(z_gpu).max())
            cols = sorted(set([0, out_n - 1] + list(r.integers(0, out_n, 6))))
            dw_ref, db_ref, _ = O.fc_bwd(a, np.ascontiguousarray(w[cols]), np.ascontiguousarray(dz[:, cols]), False)
            g_w = st.grad[wo:wo + w.size].reshape(w.shape)
            g_b = st.grad[bo:bo + out_n]
            report[f"{i}.dw"] = _close(f"layer {i} fc dw", g_w[cols], dw_ref, np.abs(g_w).max())
            report[f"{i}.db"] = _close(f"layer {i} fc db", g_b[cols], db_ref, np.abs(g_b).max())
            if i > first_w:
                _, _, da = O.fc_bwd(a[rows], w, np.ascontiguousarray(dz[rows]), True)
                if src_masks:
                    da = np.where(a[rows] > 0, da, 0)
                dx_gpu = st.dout_nchw(src).reshape(N, -1)
                report[f"{i}.dx"] = _close(f"layer {i} fc dx", dx_gpu[rows], da, np.abs(dx_gpu).max())
    worst = max(report.values())
    print(f"[fullsize] {wl.name}: loss {st.loss:.6f} (oracle from GPU logits {l_ref:.6f}); worst ratio {worst:.2e}",
          flush=True)
    return report


def test_mlp5000_full_batch():
    check_step(workloads.WORKLOADS["mlp5000"])


def test_vgg_cifar_full_batch():
    check_step(workloads.WORKLOADS["vgg_cifar"])


def test_vgg16_full_batch():
    check_step(workloads.WORKLOADS["vgg16"], samples=16)


def test_lenet5_layerwise():
    check_step(workloads.WORKLOADS["lenet5"])
