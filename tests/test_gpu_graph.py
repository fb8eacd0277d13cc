"""The training step recorded as a HIP graph (sgd_train_step_graph) against the eager step.

Replays run the same kernels on the same buffers, so every replay must give
bitwise the eager step's weights, rule state and loss.  Each replay is
followed by unrelated eager device work and a synchronisation before it is
checked, and several replays run back to back, as graph replays must stay
correct after the first.
"""
import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import sgd_cnns_amd as S  # noqa: E402

NETS = {
    "lenet5": (workloads.WORKLOADS["lenet5"].chw, workloads.WORKLOADS["lenet5"].layers, 16, 10),
    "cnn_implicit": ((16, 12, 12), [("conv", 32, 3, 1), ("relu",), ("pool", 2), ("conv", 32, 3, 1), ("relu",),
                                    ("fc", 20), ("relu",), ("fc", 9), ("softmax_ce",)], 6, 9),
    "mlp": ((300, 1, 1), [("fc", 260), ("relu",), ("fc", 130), ("relu",), ("fc", 10), ("softmax_ce",)], 40, 10),
}


@pytest.mark.parametrize("rule", ["momentum", "adagrad", "plain"])
@pytest.mark.parametrize("name", sorted(NETS))
def test_graph_replays_match_eager_steps(name, rule):
    chw, layers, N, classes = NETS[name]
    print(f"[graph] {name} rule={rule}", flush=True)
    seed = 90 + len(name)
    X = workloads.uniform01(seed, 0, (N,) + tuple(chw))
    y = workloads.labels(seed, 1, N, classes)
    W0 = workloads.he_normal_params(seed, chw, layers)
    dev = torch.device("cuda")
    Xd, yd = torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev)
    net = S.Net((N,) + tuple(chw), layers)
    n = net.param_count()
    r = S.Rule(rule, 0.02, 0.9, 1e-8)
    s0 = torch.full((n,), 0.1, device=dev) if rule == "adagrad" else torch.zeros(n, device=dev)

    # eager reference
    We, Se, le = torch.from_numpy(W0).to(dev), s0.clone(), torch.empty(1, device=dev)
    wse = net.workspace(dev)
    ref = []
    for _ in range(4):
        net.train_step(We, Xd, yd, Se if rule != "plain" else None, r, le, wse)
        torch.cuda.synchronize()
        ref.append((We.cpu().numpy().copy(), Se.cpu().numpy().copy(), le.cpu().numpy().copy()))

    Wg, Sg, lg = torch.from_numpy(W0).to(dev), s0.clone(), torch.full((1,), float("nan"), device=dev)
    wsg = net.workspace(dev)
    g = S.StepGraph(net, Wg, Xd, yd, Sg if rule != "plain" else None, r, lg, wsg)
    torch.cuda.synchronize()
    assert np.array_equal(Wg.cpu().numpy(), W0), "recording must not run the step"
    other = torch.randn(1 << 16, device=dev)
    for k in range(4):
        g.launch()
        other.mul_(1.0001).add_(0.5)   # unrelated eager work between replays
        torch.cuda.synchronize()
        W_ref, S_ref, l_ref = ref[k]
        assert np.array_equal(Wg.cpu().numpy(), W_ref), f"replay {k}: weights differ"
        assert np.array_equal(Sg.cpu().numpy(), S_ref), f"replay {k}: rule state differs"
        assert np.array_equal(lg.cpu().numpy(), l_ref), f"replay {k}: loss differs"


def test_graph_refuses_capture_while_profiling():
    chw, layers, N, classes = NETS["mlp"]
    dev = torch.device("cuda")
    net = S.Net((N,) + tuple(chw), layers)
    W = torch.zeros(net.param_count(), device=dev)
    X = torch.zeros((N,) + tuple(chw), device=dev)
    y = torch.zeros(N, dtype=torch.int32, device=dev)
    net.profile(True)
    with pytest.raises(S.SgdError):
        S.StepGraph(net, W, X, y, None, S.Rule("plain", 0.1), torch.empty(1, device=dev), net.workspace(dev))
    net.profile(False)
