"""Pins of the oracle's SPRINT replay (SPRINT report section 3.4, Algorithms 1 and 2).

Each schedule below is small enough to write out by hand: the expected
weights are built from explicit gradient calls and rule steps in the order
the algorithms fix, so a replay that takes a step's gradient at the wrong
weight version, folds a push into the wrong update, or drops a worker's
buffer fails.  The gradient and the rules themselves are pinned by the
finite-difference and closed-form tests.
"""
import numpy as np
import pytest

import oracle as O
import workloads

LAYERS = [("conv", 3, 3, 1), ("relu",), ("pool", 2), ("fc", 5), ("softmax_ce",)]
CHW = (2, 6, 6)
N = 3


def setup(n_batches=6, seed=71):
    net = O.OracleNet(CHW, LAYERS, dtype=np.float64)
    W0 = workloads.he_normal_params(seed, CHW, LAYERS).astype(np.float64)
    X = workloads.uniform01(seed, 0, (n_batches * N,) + CHW).astype(np.float64)
    y = workloads.labels(seed, 1, n_batches * N, 5)
    batches = [(X[b * N:(b + 1) * N], y[b * N:(b + 1) * N]) for b in range(n_batches)]
    return net, W0, batches


def g(net, W, batch):
    return net.gradient(W, *batch)[1]


def test_sequential_schedule_is_plain_sgd():
    net, W0, B = setup()
    eta = 0.05
    log = [(0, i, i, i, i, i) for i in range(4)]   # one worker, each step its own update
    W, _, vers = O.sprint_replay(net, W0, None, "plain", B, log, eta)
    ref = W0.copy()
    for i in range(4):
        ref = ref - eta * g(net, ref, B[i])
        assert np.allclose(vers[i + 1], ref, rtol=0, atol=1e-12)
    assert np.allclose(W, ref, rtol=0, atol=1e-12)


def test_stale_gradients_use_the_version_they_were_taken_at():
    net, W0, B = setup()
    eta = 0.05
    # worker 1 fetches every second step (n_fetch = 2): its step 1 still uses version 0
    log = [(0, 0, 0, 0, 0, 0), (1, 0, 0, 1, 0, 0),
           (0, 1, 1, 2, 1, 1), (1, 1, 1, 3, 0, 1)]
    W, _, _ = O.sprint_replay(net, W0, None, "plain", B, log, eta)
    W1 = W0 - eta * (g(net, W0, B[0]) + g(net, W0, B[1]))
    W2 = W1 - eta * (g(net, W1, B[2]) + g(net, W0, B[3]))
    assert np.allclose(W, W2, rtol=0, atol=1e-12)
    assert not np.allclose(W, W1 - eta * (g(net, W1, B[2]) + g(net, W1, B[3])), rtol=0, atol=1e-9)


def test_push_interval_and_uneven_updates_with_momentum():
    net, W0, B = setup()
    eta, mu = 0.05, 0.9
    # worker 0 pushes every 2 steps; update 0 takes only worker 1's first push,
    # update 1 takes worker 0's push (2 steps) and worker 1's second push
    log = [(0, 0, 0, 0, 0, 1), (0, 1, 0, 1, 0, 1),
           (1, 0, 0, 2, 0, 0), (1, 1, 1, 3, 1, 1)]
    V0 = np.zeros_like(W0)
    W, V, _ = O.sprint_replay(net, W0, V0, "momentum", B, log, eta, mu=mu)
    Va = mu * V0 - eta * g(net, W0, B[2])
    W1 = W0 + Va
    Vb = mu * Va - eta * ((g(net, W0, B[0]) + g(net, W0, B[1])) + g(net, W1, B[3]))
    W2 = W1 + Vb
    assert np.allclose(V, Vb, rtol=0, atol=1e-12)
    assert np.allclose(W, W2, rtol=0, atol=1e-12)


def test_two_pushes_in_one_buffer_are_both_applied():
    net, W0, B = setup()
    eta = 0.05
    # worker 0 pushed twice before the updater took its buffer
    log = [(0, 0, 0, 4, 0, 0), (0, 1, 1, 5, 0, 0)]
    W, _, vers = O.sprint_replay(net, W0, None, "plain", B, log, eta)
    assert len(vers) == 2
    assert np.allclose(W, W0 - eta * (g(net, W0, B[4]) + g(net, W0, B[5])), rtol=0, atol=1e-12)


def test_inconsistent_schedules_are_rejected():
    net, W0, B = setup()
    with pytest.raises(ValueError):
        O.sprint_replay(net, W0, None, "plain", B, [(0, 0, 0, 0, 1, 0)], 0.1)   # version after its update
    with pytest.raises(ValueError):
        O.sprint_replay(net, W0, None, "plain", B, [(0, 0, 0, 0, 0, -1)], 0.1)  # never applied
