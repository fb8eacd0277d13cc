"""Shared test helpers: tolerance checks and NHWC <-> NCHW views (no method arithmetic)."""
import numpy as np

LOSS_RTOL = 1e-5      # loss: |dL| <= 1e-5 |L|
GRAD_RTOL = 1e-4      # gradients: max|dg| <= 1e-4 max|g|, per parameter tensor


def tensor_bounds(w_offs, b_offs, n_params):
    """[(name, start, end)] of every weight and bias tensor in the flat parameter vector."""
    out = []
    for j, (wo, bo) in enumerate(zip(w_offs, b_offs)):
        end = w_offs[j + 1] if j + 1 < len(w_offs) else n_params
        out.append(("w%d" % j, wo, bo))
        out.append(("b%d" % j, bo, end))
    return out


def per_tensor_grad_check(g_gpu, g_ref, w_offs, b_offs, n_params, rtol=GRAD_RTOL):
    """Compare each layer's weight and bias gradient; return the worst ratio max|d|/max|g|."""
    worst = 0.0
    for name, a, b in tensor_bounds(w_offs, b_offs, n_params):
        ref = g_ref[a:b].astype(np.float64)
        got = g_gpu[a:b].astype(np.float64)
        scale = np.abs(ref).max()
        err = np.abs(got - ref).max()
        if scale == 0:
            assert err <= 1e-30, (name, err)
            continue
        ratio = err / scale
        worst = max(worst, ratio)
        assert ratio <= rtol, f"{name}: max|d| {err:.3e} > {rtol} * max|g| {scale:.3e}"
    return worst


def _sp(x):
    """Spacing of float32 numbers at |x| (one unit in the last place), as float64."""
    return np.spacing(np.abs(np.asarray(x, np.float64)).astype(np.float32)).astype(np.float64)


def update_tolerance(rule, g_ref, W0, st0, W_ref, st_ref, tau, eta, mu=0.0, decay=0.0):
    """Elementwise bounds on |W_gpu - W_ref| and |state_gpu - state_ref| after one update from
    (W0, st0), where W_ref, st_ref are the oracle's rule applied to the oracle's gradient g_ref and
    the GPU's gradient may differ from g_ref by up to tau (the gradient contract for the tensor).

    The rules are Lipschitz in the gradient with these constants:
      plain     W = W0 - eta g                      |dW| <= eta tau
      momentum  V = mu V0 - eta g,  W = W0 + V      |dV| <= eta tau, |dW| <= |dV|
      nesterov  V as momentum, W = W0 + mu V - eta g  |dW| <= (1 + mu) eta tau
      adagrad   A = A0 + g^2,  W = W0 - eta g / (sqrt(A) + eps)
                |dA| <= (2|g| + tau) tau;  d/dg [g / sqrt(A0 + g^2)] = A0 / (A0 + g^2)^1.5 <= 1 / sqrt(A0),
                so |dW| <= eta tau / sqrt(A0)
    Weight decay adds decay * W0 to both gradients alike.  Every statement rounds once, so a few
    units in the last place of the intermediate and final values are added."""
    g = np.abs(g_ref.astype(np.float64) + decay * W0.astype(np.float64))
    G = g.max() if g.size else 0.0
    step = eta * G
    if rule == "plain":
        return eta * tau + 2 * _sp(step) + 2 * _sp(W_ref), None
    if rule in ("momentum", "nesterov"):
        tolS = eta * tau + 2 * _sp(step) + 2 * _sp(st_ref) + 2 * _sp(mu * np.abs(st0))
        if rule == "momentum":
            return tolS + 2 * _sp(W_ref), tolS
        return (1 + mu) * eta * tau + 4 * _sp(step) + 4 * _sp(mu * np.abs(st_ref)) + 2 * _sp(W_ref), tolS
    if rule == "adagrad":
        a0 = np.sqrt(st0.astype(np.float64))
        tolS = (2 * g + tau) * tau + 2 * _sp(st_ref)
        tolW = eta * tau / a0 + 8 * _sp(eta * g / a0) + 2 * _sp(W_ref)
        return tolW, tolS
    raise ValueError(rule)


def check_update(name, rule, g_ref, W0, st0, W_ref, st_ref, W_gpu, st_gpu, eta, mu=0.0, decay=0.0, tau_scale=None,
                 rtol=GRAD_RTOL):
    """Assert the GPU's updated W (and state) lie within update_tolerance of the oracle's; tau is
    rtol times max|g_ref| over the tensor (or over tau_scale when given).  Returns the worst ratio
    |d| / tolerance."""
    gmax = np.abs(g_ref if tau_scale is None else tau_scale).max() if g_ref.size else 0.0
    tau = rtol * float(gmax)
    tolW, tolS = update_tolerance(rule, g_ref, W0, st0, W_ref, st_ref, tau, eta, mu, decay)
    worst = 0.0
    for what, got, ref, tol in (("W", W_gpu, W_ref, tolW), ("state", st_gpu, st_ref, tolS)):
        if tol is None:
            continue
        d = np.abs(got.astype(np.float64) - ref.astype(np.float64))
        assert np.isfinite(got).all(), f"{name} {what}: non-finite values"
        bad = d > tol
        if bad.any():
            i = int(np.argmax(d - tol))
            raise AssertionError(f"{name} {what}: {int(bad.sum())} elements outside the bound; worst at {i}: "
                                 f"gpu {got.flat[i]!r} oracle {ref.flat[i]!r} |d| {d.flat[i]:.3e} > "
                                 f"{np.broadcast_to(tol, d.shape).flat[i]:.3e} (tau {tau:.3e})")
        with np.errstate(divide="ignore", invalid="ignore"):
            r = np.where(tol > 0, d / tol, 0.0)
        worst = max(worst, float(r.max()) if r.size else 0.0)
    return worst


def nhwc_to_nchw(a):
    return np.ascontiguousarray(np.transpose(a, (0, 3, 1, 2)))
