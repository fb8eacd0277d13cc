"""Shared test helpers: tolerance checks and NHWC <-> NCHW views (no method arithmetic)."""
import numpy as np

LOSS_RTOL = 1e-5      # loss: |dL| <= 1e-5 |L|
GRAD_RTOL = 1e-4      # gradients: max|dg| <= 1e-4 max|g|, per parameter tensor


def per_tensor_grad_check(g_gpu, g_ref, w_offs, b_offs, n_params, rtol=GRAD_RTOL):
    """Compare each layer's weight and bias gradient; return the worst ratio max|d|/max|g|."""
    bounds = []
    for j, (wo, bo) in enumerate(zip(w_offs, b_offs)):
        end = w_offs[j + 1] if j + 1 < len(w_offs) else n_params
        bounds.append(("w%d" % j, wo, bo))
        bounds.append(("b%d" % j, bo, end))
    worst = 0.0
    for name, a, b in bounds:
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


def nhwc_to_nchw(a):
    return np.ascontiguousarray(np.transpose(a, (0, 3, 1, 2)))
