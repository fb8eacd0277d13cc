"""SPRINT's workers and updater on the GPU (sgd_sprint_run) against the oracle's replay.

The schedule of an asynchronous run depends on timing, so the test takes
the run's own log (which weight version each step used, which sub-batch,
which push and which update applied it), checks that it is a schedule
Algorithms 1 and 2 can produce, and replays it in the oracle in fp64
(SPRINT report section 3.4).  The final weights and rule state must match
per parameter tensor to 1e-4 of the change the run made, plus the fp32
rounding of the stored weights (2^-23 of their size per update).
"""
import numpy as np
import pytest

import oracle as O
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import sgd_cnns_amd as S  # noqa: E402

LAYERS = [("conv", 8, 3, 1), ("relu",), ("pool", 2), ("fc", 24), ("relu",), ("fc", 7), ("softmax_ce",)]
CHW = (3, 10, 10)
N = 5
CLASSES = 7


def inputs(n_batches, seed):
    X = workloads.uniform01(seed, 0, (n_batches * N,) + CHW)
    y = workloads.labels(seed, 1, n_batches * N, CLASSES)
    W0 = workloads.he_normal_params(seed, CHW, LAYERS)
    return X, y, W0


def run(cfg, rule, eta, mu, n_batches, seed):
    X, y, W0 = inputs(n_batches, seed)
    net = S.Net((N,) + CHW, LAYERS)
    dev = torch.device("cuda")
    Wd = torch.from_numpy(W0.copy()).to(dev)
    Vd = torch.zeros_like(Wd)
    ws = torch.empty(S.sprint_workspace_bytes(net, cfg), dtype=torch.uint8, device=dev)
    stats, log = S.sprint_run(net, cfg, Wd, Vd, S.Rule(rule, eta, mu), torch.from_numpy(X).to(dev),
                              torch.from_numpy(y).to(dev), n_batches, ws)
    torch.cuda.synchronize()
    return stats, log, (X, y, W0), Wd.cpu().numpy(), Vd.cpu().numpy()


def check_schedule(log, cfg, n_batches):
    """Properties every schedule of Algorithms 1 and 2 has."""
    assert len(log) == cfg.workers * cfg.iters
    assert [(e[0], e[1]) for e in log] == [(t, i) for t in range(cfg.workers) for i in range(cfg.iters)]
    U = max(e[5] for e in log) + 1
    assert sorted({e[5] for e in log}) == list(range(U)), "every update applies at least one step"
    assert sorted(e[3] for e in log) == sorted(i % n_batches for i in range(len(log))), "shared batch counter"
    for t in range(cfg.workers):
        mine = log[t * cfg.iters:(t + 1) * cfg.iters]
        for i, e in enumerate(mine):
            assert 0 <= e[4] <= e[5], e
            assert e[2] == i // cfg.n_push, e                     # push interval
            if i % cfg.n_fetch:
                assert e[4] == mine[i - 1][4], e                  # no fetch between fetch points
            if i:
                assert e[4] >= mine[i - 1][4] and e[5] >= mine[i - 1][5], e
        for p in {e[2] for e in mine}:
            assert len({e[5] for e in mine if e[2] == p}) == 1, "a push is applied by one update"
    return U


def close(got, ref, base, U, what):
    scale = np.abs(ref - base).max()
    tol = 1e-4 * scale + U * 2.0 ** -23 * np.abs(ref).max()
    err = np.abs(got.astype(np.float64) - ref).max()
    assert err <= tol, f"{what}: max|d| {err:.3e} > {tol:.3e} (change {scale:.3e})"


def compare(log, data, W, V, rule, eta, mu):
    X, y, W0 = data
    onet = O.OracleNet(CHW, LAYERS, dtype=np.float64)
    n_batches = X.shape[0] // N
    batches = [(X[b * N:(b + 1) * N], y[b * N:(b + 1) * N]) for b in range(n_batches)]
    Wr, Vr, vers = O.sprint_replay(onet, W0.astype(np.float64), np.zeros(W0.size), rule, batches, log, eta, mu=mu)
    U = len(vers) - 1
    for i in sorted(onet.params):
        wo, shape, bo, nb = onet.params[i]
        for a, b in ((wo, wo + int(np.prod(shape))), (bo, bo + nb)):
            close(W[a:b], Wr[a:b], W0[a:b].astype(np.float64), U, f"W[{a}:{b}]")
            close(V[a:b], Vr[a:b], np.zeros(b - a), U, f"V[{a}:{b}]")


def test_bulk_synchronous_run_matches_replay():
    cfg = S.SprintConfig(workers=3, iters=3, min_bufs=3, sync=True)
    print("[sprint] sync 3 workers x 3 steps, momentum", flush=True)
    stats, log, data, W, V = run(cfg, "momentum", 0.05, 0.9, 9, 81)
    U = check_schedule(log, cfg, 9)
    assert U == 3 and stats["updates"] == 3
    for u in range(3):
        assert sorted((e[0], e[4]) for e in log if e[5] == u) == [(0, u), (1, u), (2, u)]
    assert stats["staleness_max"] == 0 and stats["n_minibatch_avg"] == 3 * N
    assert stats["steps"] == 9 and stats["fetches"] == 9
    compare(log, data, W, V, "momentum", 0.05, 0.9)


@pytest.mark.parametrize("workers,iters,n_fetch,n_push", [(4, 6, 1, 1), (3, 7, 2, 2), (1, 5, 1, 1)])
def test_asynchronous_run_matches_replay(workers, iters, n_fetch, n_push):
    cfg = S.SprintConfig(workers=workers, iters=iters, n_fetch=n_fetch, n_push=n_push)
    print(f"[sprint] async {workers} workers x {iters} steps, fetch {n_fetch}, push {n_push}", flush=True)
    stats, log, data, W, V = run(cfg, "momentum", 0.05, 0.5, 8, 82 + workers)
    U = check_schedule(log, cfg, 8)
    assert stats["updates"] == U and stats["steps"] == workers * iters
    stale = [e[5] - e[4] for e in log]
    assert stats["staleness_max"] == max(stale)
    assert stats["staleness_mean"] == pytest.approx(np.mean(stale))
    assert stats["n_minibatch_avg"] == pytest.approx(workers * iters * N / U)
    assert stats["t_gpu_ms"] > 0 and stats["wall_ms"] > 0
    compare(log, data, W, V, "momentum", 0.05, 0.5)


def test_bad_configs_are_rejected_on_the_host():
    net = S.Net((N,) + CHW, LAYERS)
    X, y, W0 = inputs(2, 1)
    dev = torch.device("cuda")
    Wd = torch.from_numpy(W0).to(dev)
    Xd, yd = torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev)
    good = S.SprintConfig(workers=2, iters=1)
    ws = torch.empty(S.sprint_workspace_bytes(net, good), dtype=torch.uint8, device=dev)
    for bad in (S.SprintConfig(0, 1), S.SprintConfig(17, 1), S.SprintConfig(2, 0), S.SprintConfig(2, 1, n_fetch=0),
                S.SprintConfig(2, 1, min_bufs=3)):
        assert S.sprint_workspace_bytes(net, bad) == 0
        with pytest.raises(S.SgdError):
            S.sprint_run(net, bad, Wd, Wd.clone(), S.Rule("plain", 0.1), Xd, yd, 2, ws)
    with pytest.raises(S.SgdError):                      # no sub-batches
        S.sprint_run(net, good, Wd, Wd.clone(), S.Rule("plain", 0.1), Xd, yd, 0, ws)
    with pytest.raises(S.SgdError):                      # momentum without its state
        S.sprint_run(net, good, Wd, None, S.Rule("momentum", 0.1, 0.9), Xd, yd, 2, ws)
    with pytest.raises(S.SgdError):                      # workspace too small
        S.sprint_run(net, good, Wd, Wd.clone(), S.Rule("plain", 0.1), Xd, yd, 2, ws[: ws.numel() // 2])


def library_replay(net, log, W0, S0, rule, Xd, yd, N, dev):
    """The run's schedule replayed on one stream with the library's own sequential calls:
    sgd_compute_gradient_into for each step's push sum, sgd_accumulate_grad into the worker's
    buffer, sgd_apply_fused over an update's buffers in worker order.  Deterministic kernels
    make this bitwise equal to a correct concurrent run: a missing or misplaced wait between
    the worker and update streams would show up as a difference."""
    n = net.param_count()
    W = torch.from_numpy(W0.copy()).to(dev)
    St = torch.from_numpy(S0.copy()).to(dev)
    versions = [W.clone()]
    ws = net.workspace(dev)
    loss = torch.empty(1, device=dev)
    U = max(e[5] for e in log) + 1
    for u in range(U):
        steps = [e for e in log if e[5] == u]
        bufs = []
        for t in sorted({e[0] for e in steps}):
            buf = S.GradBuf(n, device=dev)
            mine = [e for e in steps if e[0] == t]
            for p in sorted({e[2] for e in mine}):
                push = S.GradBuf(n, device=dev)
                for e in sorted((e for e in mine if e[2] == p), key=lambda e: e[1]):
                    b = e[3]
                    net.compute_gradient_into(versions[e[4]], Xd[b * N:(b + 1) * N], yd[b * N:(b + 1) * N], push,
                                              loss, ws)
                S.accumulate_grad(buf, push.data)
            bufs.append(buf.data)
        S.apply_fused(W, St, bufs, rule)
        versions.append(W.clone())
    torch.cuda.synchronize()
    return W.cpu().numpy(), St.cpu().numpy()


@pytest.mark.parametrize("workers,iters,n_fetch,n_push,min_bufs", [(4, 6, 1, 1, 1), (3, 6, 2, 3, 2)])
def test_run_is_bitwise_its_own_sequential_replay(workers, iters, n_fetch, n_push, min_bufs):
    cfg = S.SprintConfig(workers=workers, iters=iters, n_fetch=n_fetch, n_push=n_push, min_bufs=min_bufs)
    print(f"[sprint] replay {workers} workers x {iters}, fetch {n_fetch}, push {n_push}, min_bufs {min_bufs}",
          flush=True)
    stats, log, (X, y, W0), W, V = run(cfg, "momentum", 0.05, 0.9, 7, 90 + workers)
    check_schedule(log, cfg, 7)
    dev = torch.device("cuda")
    net = S.Net((N,) + CHW, LAYERS)
    Wr, Vr = library_replay(net, log, W0, np.zeros_like(W0), S.Rule("momentum", 0.05, 0.9),
                            torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev), N, dev)
    assert np.array_equal(W, Wr) and np.array_equal(V, Vr)


def test_full_size_mlp_run_is_bitwise_its_own_sequential_replay():
    """The MLP-5000 network at full width (115,435,010 parameters), sub-batch 128, four workers:
    the schedule must be valid and the result bitwise its sequential replay."""
    wl = workloads.WORKLOADS["mlp5000"].with_batch(128)
    n_batches = 6
    X = workloads.uniform01(wl.seed, 0, (n_batches * wl.batch,) + tuple(wl.chw))
    y = workloads.labels(wl.seed, 1, n_batches * wl.batch, wl.classes)
    W0 = workloads.he_normal_params(wl.seed, wl.chw, wl.layers)
    dev = torch.device("cuda")
    net = S.Net((wl.batch,) + tuple(wl.chw), wl.layers)
    cfg = S.SprintConfig(workers=4, iters=3)
    print("[sprint] full-size MLP, 4 workers x 3 steps", flush=True)
    Wd = torch.from_numpy(W0.copy()).to(dev)
    Vd = torch.zeros_like(Wd)
    Xd, yd = torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev)
    rule = S.Rule("momentum", 1e-3, 0.9)
    ws = torch.empty(S.sprint_workspace_bytes(net, cfg), dtype=torch.uint8, device=dev)
    stats, log = S.sprint_run(net, cfg, Wd, Vd, rule, Xd, yd, n_batches, ws)
    torch.cuda.synchronize()
    del ws
    check_schedule(log, cfg, n_batches)
    assert stats["steps"] == 12 and stats["updates"] == max(e[5] for e in log) + 1
    W, V = Wd.cpu().numpy(), Vd.cpu().numpy()
    assert np.isfinite(W).all() and not np.array_equal(W, W0)
    Wr, Vr = library_replay(net, log, W0, np.zeros_like(W0), rule, Xd, yd, wl.batch, dev)
    assert np.array_equal(W, Wr) and np.array_equal(V, Vr)


@pytest.mark.parametrize("where", ["w1:2", "w0:0", "u:1", "u:0"])
def test_a_failing_thread_stops_the_run_and_leaves_the_library_usable(where, monkeypatch):
    """A failure forced from the host (SGD_SPRINT_INJECT_FAILURE) in a worker while it holds its buffer
    lock, or in the updater while it holds the weights lock: the run returns that error (no thread
    is left waiting), and the next run on the same buffers succeeds."""
    cfg = S.SprintConfig(workers=3, iters=4)
    print(f"[sprint] injected failure at {where}", flush=True)
    monkeypatch.setenv("SGD_SPRINT_INJECT_FAILURE", where)
    with pytest.raises(S.SgdError, match="injected failure"):
        run(cfg, "momentum", 0.05, 0.9, 6, 70)
    monkeypatch.delenv("SGD_SPRINT_INJECT_FAILURE")
    stats, log, data, W, V = run(cfg, "momentum", 0.05, 0.9, 6, 70)
    check_schedule(log, cfg, 6)
    assert np.isfinite(W).all()
