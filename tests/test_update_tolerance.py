"""CPU checks of the update tolerance used by the GPU parity tests (tests/_util.update_tolerance).

The bound claims: if a gradient differs from the oracle's by at most tau per element, the rule's
results differ by at most the returned tolerance.  Planted in the oracle on the CPU: gradients
perturbed by up to tau must stay inside the bound for every rule; perturbations of 20 tau must be
caught.  No GPU is involved."""
import numpy as np
import pytest

import oracle as O
import workloads
from tests._util import check_update

RULES = [("plain", 0.0), ("plain", 5e-4), ("momentum", 0.0), ("momentum", 5e-4), ("nesterov", 5e-4),
         ("adagrad", 0.0), ("adagrad", 5e-4)]


def _state(rule, n, seed):
    if rule == "plain":
        return None
    if rule == "adagrad":
        return np.abs(workloads.normal(seed, 3, n)) + np.float32(0.1)
    return workloads.normal(seed, 3, n, 1e-3)


def _apply(rule, W0, st0, g, eta, mu, eps, decay):
    W = W0.copy()
    st = None if st0 is None else st0.copy()
    O.apply_rule(rule, W, st, g, eta, mu, eps, decay)
    return W, st


@pytest.mark.parametrize("rule,decay", RULES)
def test_perturbation_inside_contract_passes(rule, decay):
    n = 200_003
    eta, mu, eps = 0.01, 0.9, 1e-8
    W0 = workloads.normal(21, 2, n)
    st0 = _state(rule, n, 21)
    g = workloads.normal(21, 100, n, 1e-2)
    tau = 1e-4 * np.abs(g).max()
    r = np.random.default_rng(5)
    for kind in ("uniform", "edges"):
        d = r.uniform(-tau, tau, n) if kind == "uniform" else tau * np.where(r.random(n) < 0.5, -1.0, 1.0)
        g_gpu = (g.astype(np.float64) + d).astype(np.float32)
        # the float32 rounding of the perturbed gradient may push it a half ulp past tau: scale down
        over = np.abs(g_gpu.astype(np.float64) - g) > tau
        g_gpu[over] = g[over]
        W_ref, st_ref = _apply(rule, W0, st0, g, eta, mu, eps, decay)
        W_gpu, st_gpu = _apply(rule, W0, st0, g_gpu, eta, mu, eps, decay)
        worst = check_update("planted", rule, g, W0, st0, W_ref, st_ref, W_gpu, st_gpu, eta, mu, decay)
        assert worst <= 1.0


@pytest.mark.parametrize("rule,decay", RULES)
def test_perturbation_outside_contract_fails(rule, decay):
    n = 50_001
    eta, mu, eps = 0.01, 0.9, 1e-8
    W0 = workloads.normal(22, 2, n)
    st0 = _state(rule, n, 22)
    g = workloads.normal(22, 100, n, 1e-2)
    tau = 1e-4 * np.abs(g).max()
    g_gpu = (g.astype(np.float64) + 20 * tau).astype(np.float32)
    W_ref, st_ref = _apply(rule, W0, st0, g, eta, mu, eps, decay)
    W_gpu, st_gpu = _apply(rule, W0, st0, g_gpu, eta, mu, eps, decay)
    with pytest.raises(AssertionError):
        check_update("planted", rule, g, W0, st0, W_ref, st_ref, W_gpu, st_gpu, eta, mu, decay)


def test_wrong_rule_state_is_caught():
    # a momentum step whose V forgot mu*V0 (a plausible epilogue mistake) fails the bound
    n = 10_007
    W0 = workloads.normal(23, 2, n)
    V0 = workloads.normal(23, 3, n, 1e-2)
    g = workloads.normal(23, 100, n, 1e-2)
    W_ref, V_ref = _apply("momentum", W0, V0, g, 0.01, 0.9, 0.0, 0.0)
    W_bad, V_bad = _apply("momentum", W0, np.zeros_like(V0), g, 0.01, 0.9, 0.0, 0.0)
    with pytest.raises(AssertionError):
        check_update("planted", "momentum", g, W0, V0, W_ref, V_ref, W_bad, V_bad, 0.01, 0.9)
