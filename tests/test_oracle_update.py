"""Pins for the oracle's GradBuf accumulation and update rules (CPU only).

The reference values come from exact rational arithmetic with explicit
round-to-nearest-even to binary32 after every statement (an independent model
of IEEE single precision, not the oracle's C code), plus a few constants worked
by hand.  Sources: SPRINT report eq. (1) (plain SGD) and Algorithms 1-2
(GradBuf empty/add rule, momentum with nu times the previous weight change);
DistBelief review (server-side Adagrad, commutative additive gradients).
"""
import itertools
import math
import struct
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle as O


def rne32(x: Fr) -> Fr:
    """Round an exact rational to the nearest binary32 value, ties to even."""
    if x == 0:
        return Fr(0)
    s = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # find e with 2^23 <= a / 2^e < 2^24 (clamped at the subnormal exponent)
    while a / Fr(2) ** e >= 2 ** 24:
        e += 1
    while a / Fr(2) ** e < 2 ** 23:
        e -= 1
    e = max(e, -149)
    m = a / Fr(2) ** e
    q, r = divmod(m.numerator, m.denominator)
    rem = Fr(r, m.denominator)
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and q % 2 == 1):
        q += 1
    return s * Fr(q) * Fr(2) ** e


def sqrt32(x: Fr) -> Fr:
    """Correctly rounded binary32 square root of a non-negative rational."""
    if x == 0:
        return Fr(0)
    e = 0
    while math.sqrt(float(x)) / 2.0 ** e >= 2 ** 24:
        e += 1
    while math.sqrt(float(x)) / 2.0 ** e < 2 ** 23:
        e -= 1
    t = x / Fr(4) ** e           # want round(sqrt(t)) as an integer mantissa
    q = math.isqrt(t.numerator // t.denominator)
    mid = Fr(2 * q + 1, 2)
    if mid * mid < t or (mid * mid == t and q % 2 == 1):
        q += 1
    return rne32(Fr(q) * Fr(2) ** e)


def f32(v) -> Fr:
    return Fr(float(np.float32(v)))


def bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


# ----------------------------------------------------------- closed forms ----

def test_plain_closed_form():
    W = np.array([0.5], np.float32)
    O.apply_plain(W, np.array([0.25], np.float32), 0.01)
    # 0.01f * 0.25 = 0.0025f (exact scaling by 2^-2); 0.5 - 0.0025f rounds to 0.4975f
    assert W[0] == np.float32(0.4975)
    assert Fr(float(W[0])) == rne32(Fr(1, 2) - rne32(f32(0.01) / 4))


def test_momentum_two_steps_closed_form():
    W = np.array([1.0], np.float32)
    V = np.array([0.0], np.float32)
    g = np.array([1.0], np.float32)
    O.apply_momentum(W, V, g, 0.9, 0.01)
    assert V[0] == np.float32(-0.01) and W[0] == np.float32(0.99)
    O.apply_momentum(W, V, g, 0.9, 0.01)
    assert V[0] == np.float32(-0.019) and W[0] == np.float32(0.971)


def test_adagrad_two_steps_closed_form():
    W = np.array([0.0], np.float32)
    A = np.array([0.1], np.float32)
    g = np.array([1.0], np.float32)
    O.apply_adagrad(W, A, g, 0.01, 1e-8)
    assert A[0] == np.float32(1.1)
    assert bits(float(W[0])) == 0xBC1C371F          # -0.009534626f
    O.apply_adagrad(W, A, g, 0.01, 1e-8)
    assert A[0] == np.float32(2.1)
    # exact double closed form: -0.01/sqrt(1.1) - 0.01/sqrt(2.1); the float
    # chain stays within a few ulp of it
    exact = -0.01 / math.sqrt(1.1) - 0.01 / math.sqrt(2.1)
    assert abs(float(W[0]) - exact) < 4 * abs(float(np.spacing(np.float32(exact))))
    assert W[0] == np.float32(-0.016435282)


# ---------------------------------------- elementwise vs exact-rounding model ----

def _rand(n, seed, scale=1.0):
    r = np.random.default_rng(seed)
    return (r.standard_normal(n) * scale).astype(np.float32)


def test_rules_match_exact_rounding_model():
    n = 300
    W0, g, V0 = _rand(n, 1), _rand(n, 2, 1e-2), _rand(n, 3, 1e-3)
    A0 = np.abs(_rand(n, 4)) + np.float32(0.1)
    eta, mu, eps = np.float32(0.01), np.float32(0.9), np.float32(1e-8)
    Wp = W0.copy(); O.apply_plain(Wp, g, eta)
    Wm, Vm = W0.copy(), V0.copy(); O.apply_momentum(Wm, Vm, g, mu, eta)
    Wa, Aa = W0.copy(), A0.copy(); O.apply_adagrad(Wa, Aa, g, eta, eps)
    E, M, P = Fr(float(eta)), Fr(float(mu)), Fr(float(eps))
    for i in range(n):
        w, gi, v, a = Fr(float(W0[i])), Fr(float(g[i])), Fr(float(V0[i])), Fr(float(A0[i]))
        # plain: t = eta*g; W = W - t
        assert Fr(float(Wp[i])) == rne32(w - rne32(E * gi))
        # momentum: t1 = mu*V; t2 = eta*g; V = t1 - t2; W = W + V
        vn = rne32(rne32(M * v) - rne32(E * gi))
        assert Fr(float(Vm[i])) == vn and Fr(float(Wm[i])) == rne32(w + vn)
        # adagrad: A = A + g*g; d = sqrt(A) + eps; r = eta/d; W = W - r*g
        an = rne32(a + rne32(gi * gi))
        d = rne32(sqrt32(an) + P)
        r = rne32(E / d)
        assert Fr(float(Aa[i])) == an
        assert Fr(float(Wa[i])) == rne32(w - rne32(r * gi))


def test_empty_gradbuf_is_zero_gradient_update():
    W0, V0, A0 = _rand(50, 5), _rand(50, 6), np.abs(_rand(50, 7)) + 0.1
    W = W0.copy(); O.apply_rule("plain", W, None, None, 0.01)
    np.testing.assert_array_equal(W, W0)
    W, V = W0.copy(), V0.copy(); O.apply_rule("momentum", W, V, None, 0.01, mu=0.9)
    np.testing.assert_array_equal(V, (np.float32(0.9) * V0))
    np.testing.assert_array_equal(W, W0 + V)
    W, A = W0.copy(), A0.copy(); O.apply_rule("adagrad", W, A, None, 0.01, eps=1e-8)
    np.testing.assert_array_equal(W, W0)
    np.testing.assert_array_equal(A, A0)


# ---------------------------------------------------------- accumulation ----

def test_gradbuf_empty_copies_then_adds():
    g1, g2 = _rand(100, 8), _rand(100, 9)
    gb = O.GradBuf(100)
    gb.data[:] = 123.0         # stale contents are ignored while empty
    gb.accumulate(g1)
    assert not gb.empty
    np.testing.assert_array_equal(gb.data, g1)
    gb.accumulate(g2)
    np.testing.assert_array_equal(gb.data, g1 + g2)


def test_dyadic_accumulation_is_order_free():
    # integers times 2^-20, small enough that every partial sum is exact in
    # float32, so every order of the K buffers gives bitwise the same sum
    r = np.random.default_rng(10)
    K, n = 5, 1000
    gs = [(r.integers(-2 ** 12, 2 ** 12, n) * 2.0 ** -20).astype(np.float32) for _ in range(K)]
    ref = None
    for perm in itertools.permutations(range(K)):
        gb = O.GradBuf(n)
        for j in perm:
            gb.accumulate(gs[j])
        if ref is None:
            ref = gb.data.copy()
        np.testing.assert_array_equal(gb.data, ref)
    np.testing.assert_array_equal(ref, np.sum(np.stack(gs).astype(np.float64), 0).astype(np.float32))


def test_left_fold_order_is_the_fixed_order():
    r = np.random.default_rng(11)
    gs = [(r.standard_normal(2000) * 1e-3).astype(np.float32) for _ in range(8)]
    gb = O.GradBuf(2000)
    for g in gs:
        gb.accumulate(g)
    acc = gs[0].copy()
    for g in gs[1:]:
        acc = (acc + g).astype(np.float32)
    np.testing.assert_array_equal(gb.data, acc)
    # other orders agree within the fp32 bound (K-1) u sum|g|
    rev = gs[-1].copy()
    for g in gs[-2::-1]:
        rev = (rev + g).astype(np.float32)
    bound = 7 * 2.0 ** -24 * np.sum(np.abs(np.stack(gs)), 0)
    assert np.all(np.abs(rev.astype(np.float64) - acc) <= bound)


def test_adagrad_eps_is_outside_the_root():
    # A0 = 0, g = 1e-4, eps = 1e-4: sqrt(A) + eps = 2e-4, so W = -0.01/2e-4 * 1e-4 = -0.005
    # (eps inside the root would give about -1e-4 instead).
    W = np.array([0.0], np.float32)
    A = np.array([0.0], np.float32)
    O.apply_adagrad(W, A, np.array([1e-4], np.float32), 0.01, 1e-4)
    assert W[0] == pytest.approx(-0.005, rel=1e-6)


def test_relu_of_negative_zero_is_positive_zero():
    a = O.relu_fwd(np.array([-0.0, -1e-30], np.float32))
    assert not np.signbit(a).any()


# ------------------------------------------------ rule variants (NEXT f4) ----
# The PIPE report's appendix A trains with weight decay (5e-4) and Nesterov
# momentum and SPRINT Algorithm 1 has the worker scale its gradient by
# -eta; the pages give no formulas, so these pin the readings the oracle
# implements: decay adds decay*W to the gradient before any rule, Nesterov
# moves W by mu times the new change plus the gradient step.

def test_nesterov_two_steps_closed_form():
    W = np.array([1.0], np.float32)
    V = np.array([0.0], np.float32)
    g = np.array([1.0], np.float32)
    O.apply_nesterov(W, V, g, 0.9, 0.01)
    # V = -0.01, W = 1 + (0.9 * -0.01 - 0.01) = 0.981
    assert V[0] == np.float32(-0.01)
    assert abs(float(W[0]) - 0.981) <= float(np.spacing(np.float32(0.981)))
    O.apply_nesterov(W, V, g, 0.9, 0.01)
    # V = 0.9 * -0.01 - 0.01 = -0.019, W = 0.981 + (0.9 * -0.019 - 0.01) = 0.9539
    assert V[0] == np.float32(-0.019)
    assert abs(float(W[0]) - 0.9539) <= 2 * float(np.spacing(np.float32(0.9539)))


def test_nesterov_with_zero_momentum_is_plain_sgd_bitwise():
    W0, g, V0 = _rand(400, 11), _rand(400, 12, 1e-2), _rand(400, 13, 1e-3)
    Wn, Vn = W0.copy(), V0.copy()
    O.apply_nesterov(Wn, Vn, g, 0.0, 0.01)
    Wp = W0.copy()
    O.apply_plain(Wp, g, 0.01)
    np.testing.assert_array_equal(Wn, Wp)


def test_nesterov_matches_the_two_history_form_in_double():
    # the same step written as W -= (1 + mu) H_new - mu H_old with the
    # history H = mu H + eta g (H = -V): equal in exact arithmetic
    n = 500
    W0 = _rand(n, 14).astype(np.float64)
    g = _rand(n, 15, 1e-2).astype(np.float64)
    V0 = _rand(n, 16, 1e-3).astype(np.float64)
    mu, eta = 0.9, 0.01
    W, V = W0.copy(), V0.copy()
    O.apply_nesterov(W, V, g, mu, eta)
    h_old = -V0
    h_new = mu * h_old + eta * g
    ref = W0 - ((1 + mu) * h_new - mu * h_old)
    np.testing.assert_allclose(V, -h_new, rtol=0, atol=1e-15)
    np.testing.assert_allclose(W, ref, rtol=0, atol=1e-14)


def test_weight_decay_closed_form():
    W = np.array([0.5], np.float32)
    O.apply_plain(W, np.array([0.25], np.float32), 0.01, 5e-4)
    # g' = 0.25 + 5e-4 * 0.5 = 0.25025;  W = 0.5 - 0.01 * 0.25025 = 0.4974975
    lam, E = f32(5e-4), f32(0.01)
    gp = rne32(Fr(1, 4) + rne32(lam * Fr(1, 2)))
    assert Fr(float(W[0])) == rne32(Fr(1, 2) - rne32(E * gp))
    assert abs(float(W[0]) - 0.4974975) <= float(np.spacing(np.float32(0.4974975)))


def test_decayed_rules_match_exact_rounding_model():
    n = 300
    W0, g, V0 = _rand(n, 17), _rand(n, 18, 1e-2), _rand(n, 19, 1e-3)
    A0 = np.abs(_rand(n, 20)) + np.float32(0.1)
    eta, mu, eps, lam = np.float32(0.01), np.float32(0.9), np.float32(1e-8), np.float32(5e-4)
    Wp = W0.copy(); O.apply_plain(Wp, g, eta, lam)
    Wm, Vm = W0.copy(), V0.copy(); O.apply_momentum(Wm, Vm, g, mu, eta, lam)
    Wn, Vn = W0.copy(), V0.copy(); O.apply_nesterov(Wn, Vn, g, mu, eta, lam)
    Wa, Aa = W0.copy(), A0.copy(); O.apply_adagrad(Wa, Aa, g, eta, eps, lam)
    E, M, P, L = Fr(float(eta)), Fr(float(mu)), Fr(float(eps)), Fr(float(lam))
    for i in range(n):
        w, v, a = Fr(float(W0[i])), Fr(float(V0[i])), Fr(float(A0[i]))
        gi = rne32(Fr(float(g[i])) + rne32(L * w))          # wd = decay*W; g = g + wd
        assert Fr(float(Wp[i])) == rne32(w - rne32(E * gi))
        t2 = rne32(E * gi)
        vn = rne32(rne32(M * v) - t2)
        assert Fr(float(Vm[i])) == vn and Fr(float(Wm[i])) == rne32(w + vn)
        assert Fr(float(Vn[i])) == vn
        assert Fr(float(Wn[i])) == rne32(w + rne32(rne32(M * vn) - t2))
        an = rne32(a + rne32(gi * gi))
        r = rne32(E / rne32(sqrt32(an) + P))
        assert Fr(float(Aa[i])) == an and Fr(float(Wa[i])) == rne32(w - rne32(r * gi))


def test_empty_gradbuf_with_decay_still_decays():
    W0 = _rand(64, 21)
    W = W0.copy()
    O.apply_rule("plain", W, None, None, 0.01, decay=5e-4)
    E, L = Fr(float(np.float32(0.01))), Fr(float(np.float32(5e-4)))
    for i in range(64):
        w = Fr(float(W0[i]))
        assert Fr(float(W[i])) == rne32(w - rne32(E * rne32(L * w)))


def test_prescaled_gradient_applied_with_minus_one_is_bitwise_the_unscaled_step():
    # the SPRINT Algorithm 1 worker stores Grad = -eta * grad; applying that
    # buffer with eta = -1 rounds exactly like applying grad with eta
    # (-1 * fl(-eta g) = fl(eta g), negation is exact)
    W0, g, V0 = _rand(300, 22), _rand(300, 23, 1e-2), _rand(300, 24, 1e-3)
    eta = np.float32(0.01)
    G = (np.float32(-eta) * g).astype(np.float32)
    for rule in ("plain", "momentum", "nesterov"):
        Wa, Va = W0.copy(), V0.copy()
        O.apply_rule(rule, Wa, Va, g, eta, mu=0.9)
        Wb, Vb = W0.copy(), V0.copy()
        O.apply_rule(rule, Wb, Vb, G, -1.0, mu=0.9)
        np.testing.assert_array_equal(Wa, Wb)
        np.testing.assert_array_equal(Va, Vb)
