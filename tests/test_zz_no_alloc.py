"""sgd_train_step_noalloc (the training step with the library's static scratch as its workspace)
against sgd_train_step with a caller workspace, through the C ABI: bitwise the same W, optimiser
state and loss, on two calls in a row -- LeNet-5 at batch 16, then at batch 4 (a smaller input whose
workspace is a prefix of what the first used) -- so the second call must not depend on what the
first left in the scratch.  Also: a net whose workspace exceeds the scratch is rejected before any
launch, and profiling must be off."""
import ctypes as C

import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import sgd_cnns_amd as S  # noqa: E402


def _run_pair(wl, rule_spec, seed):
    X, y, W0 = workloads.make_inputs(wl)
    net = S.Net((wl.batch,) + tuple(wl.chw), wl.layers)
    n = net.param_count()
    assert net.workspace_bytes() <= S.NOALLOC_SCRATCH_BYTES
    if rule_spec[0] == "adagrad":
        st0 = np.abs(workloads.normal(seed, 3, n)) + np.float32(0.1)   # an accumulator is positive
    elif rule_spec[0] != "plain":
        st0 = workloads.normal(seed, 3, n, 1e-3)
    else:
        st0 = None
    dev = torch.device("cuda")
    Xd, yd = torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev)
    rule = S.Rule(*rule_spec)
    out = []
    for noalloc in (False, True):
        Wd = torch.from_numpy(W0).to(dev)
        sd = None if st0 is None else torch.from_numpy(st0).to(dev)
        loss = torch.full((1,), float("nan"), device=dev)
        for _ in range(2):
            if noalloc:
                L = S.lib()
                rc = L.sgd_train_step_noalloc(net._h, C.c_void_p(Wd.data_ptr()), C.c_void_p(Xd.data_ptr()),
                                              C.c_void_p(yd.data_ptr()),
                                              None if sd is None else C.c_void_p(sd.data_ptr()), C.byref(rule),
                                              C.c_void_p(loss.data_ptr()),
                                              C.c_void_p(torch.cuda.current_stream().cuda_stream))
                assert rc == S.OK, L.sgd_last_error()
            else:
                ws = net.workspace()
                net.train_step(Wd, Xd, yd, sd, rule, loss, ws)
        torch.cuda.synchronize()
        out.append((Wd.cpu().numpy(), None if sd is None else sd.cpu().numpy(), float(loss.item())))
    (Wa, sa, la), (Wb, sb, lb) = out
    assert np.isfinite(la) and la == lb
    np.testing.assert_array_equal(Wa, Wb)
    if sa is not None:
        np.testing.assert_array_equal(sa, sb)
    assert not np.array_equal(Wa, W0)


def test_noalloc_step_matches_workspace_step_two_calls():
    wl = workloads.WORKLOADS["lenet5"]
    print("[noalloc] lenet5 batch 16, momentum", flush=True)
    _run_pair(wl, ("momentum", 0.01, 0.9, 0.0, 0.0), 71)
    print("[noalloc] lenet5 batch 4, adagrad (smaller input after the larger one)", flush=True)
    small = wl.with_batch(4)
    assert S.Net((4,) + wl.chw, wl.layers).workspace_bytes() < S.Net((16,) + wl.chw, wl.layers).workspace_bytes()
    _run_pair(small, ("adagrad", 0.01, 0.0, 1e-8, 0.0), 72)


def test_noalloc_rejects_large_nets_and_profiling():
    wl = workloads.WORKLOADS["vgg_cifar"]
    net = S.Net((wl.batch,) + wl.chw, wl.layers)
    assert net.workspace_bytes() > S.NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda")
    n = net.param_count()
    W = torch.zeros(n, device=dev)
    X = torch.zeros((wl.batch,) + wl.chw, device=dev)
    y = torch.zeros(wl.batch, dtype=torch.int32, device=dev)
    loss = torch.zeros(1, device=dev)
    with pytest.raises(S.SgdError) as e:
        net.train_step_noalloc(W, X, y, None, S.Rule("plain", 0.01), loss)
    assert e.value.code == S.EWORKSPACE
    small = workloads.WORKLOADS["lenet5"]
    net2 = S.Net((small.batch,) + small.chw, small.layers)
    net2.profile(True)
    with pytest.raises(S.SgdError) as e:
        net2.train_step_noalloc(torch.zeros(net2.param_count(), device=dev),
                                torch.zeros((small.batch,) + small.chw, device=dev),
                                torch.zeros(small.batch, dtype=torch.int32, device=dev), None,
                                S.Rule("plain", 0.01), loss)
    assert e.value.code == S.EINVAL
    net2.profile(False)
    torch.cuda.synchronize()
    assert torch.count_nonzero(W).item() == 0
