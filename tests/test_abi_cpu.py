"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, plans the workloads (eq. (3) parameter counts, offsets,
workspace) and rejects malformed requests with the documented status codes.
No compute call is made here."""
import ctypes as C
import json
import os
import re

import pytest

import sgd_cnns_amd as S
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", fn)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names |= set(re.findall(r"\b(sgd_\w+)\s*\(", txt))
    return names


def test_library_exports_every_declared_symbol():
    L = S.lib()
    declared = _declared()
    assert declared >= set(S.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_header_constants_match_binding():
    txt = open(os.path.join(ROOT, "include", "sgdstep.h")).read()
    consts = dict(re.findall(r"#define (SGD_\w+) \(?(-?\d+)\)?", txt))
    for name, val in consts.items():
        assert getattr(S, name[4:]) == int(val), name


@pytest.mark.parametrize("name", ["lenet5", "mlp5000", "vgg_cifar", "vgg16"])
def test_param_count_and_offsets(name):
    golden = json.load(open(os.path.join(ROOT, "tests", "golden", "param_counts.json")))
    wl = workloads.WORKLOADS[name]
    net = S.Net((wl.batch,) + wl.chw, wl.layers)
    assert net.param_count() == golden[name]["value"]
    w, b = net.param_offsets()
    assert w[0] == 0 and all(b[j] > w[j] for j in range(len(w)))
    assert all(w[j + 1] > b[j] for j in range(len(w) - 1))
    assert net.workspace_bytes() > 0


def test_lenet_shapes_from_tensor_info():
    wl = workloads.WORKLOADS["lenet5"]
    net = S.Net((16,) + wl.chw, wl.layers)
    assert net.tensor_info(0, S.T_OUT)[1:] == ((16, 28, 28, 6), S.LAYOUT_NHWC)
    assert net.tensor_info(1, S.T_OUT) == net.tensor_info(0, S.T_OUT)      # ReLU reports its conv
    assert net.tensor_info(2, S.T_OUT)[1:] == ((16, 14, 14, 6), S.LAYOUT_NHWC)
    assert net.tensor_info(3, S.T_COL)[1][:3] == (16 * 10 * 10, 150, 152)
    assert net.tensor_info(5, S.T_OUT)[1:] == ((16, 16, 5, 5), S.LAYOUT_NCHW)  # feeds fc: (c,h,w)
    assert net.tensor_info(6, S.T_OUT)[1][:2] == (16, 120)
    with pytest.raises(S.SgdError):
        net.tensor_info(6, S.T_COL)


@pytest.mark.parametrize("layers,code", [
    ([("fc", 10), ("relu",), ("softmax_ce",)], S.EUNSUPPORTED),        # softmax after ReLU
    ([("relu",), ("fc", 10), ("softmax_ce",)], S.EUNSUPPORTED),        # ReLU first
    ([("fc", 10), ("conv", 3, 3, 1), ("fc", 2), ("softmax_ce",)], S.EUNSUPPORTED),
    ([("conv", 3, 3, 0), ("pool", 4), ("fc", 2), ("softmax_ce",)], S.ESHAPE),  # 6 % 4 != 0
    ([("conv", 3, 9, 0), ("fc", 2), ("softmax_ce",)], S.ESHAPE),        # empty conv output
    ([("fc", 10), ("fc", 3)], S.ESHAPE),                                # no softmax
    ([("fc", 10), ("softmax_ce",), ("fc", 3)], S.ESHAPE),               # softmax not last
])
def test_create_net_rejects(layers, code):
    with pytest.raises(S.SgdError) as e:
        S.Net((2, 3, 8, 8), layers)
    assert e.value.code == code


def test_flatten_inserted_for_unpooled_conv_before_fc():
    net = S.Net((2, 3, 6, 6), [("conv", 4, 3, 1), ("relu",), ("fc", 5), ("softmax_ce",)])
    assert net.param_count() == 4 * (27 + 1) + 5 * (4 * 36 + 1)


def test_host_side_argument_errors():
    L = S.lib()
    wl = workloads.WORKLOADS["lenet5"]
    net = S.Net((16,) + wl.chw, wl.layers)
    dummy = C.c_void_p(256)
    # workspace too small: rejected before any device work
    rc = L.sgd_compute_gradient(net._h, dummy, dummy, dummy, dummy, dummy, dummy, 16, None)
    assert rc == S.EWORKSPACE and b"needs" in L.sgd_last_error()
    rc = L.sgd_compute_gradient(net._h, None, dummy, dummy, dummy, dummy, dummy, 1 << 40, None)
    assert rc == S.EINVAL
    gb = S.SgdGradBuf(256, 10, 1)
    arr = (C.c_void_p * 17)(*([256] * 17))
    assert L.sgd_accumulate_grads(C.byref(gb), arr, 17, None) == S.EINVAL
    assert L.sgd_accumulate_grads(C.byref(gb), arr, 0, None) == S.EINVAL
    bad = S.SgdRule(7, 0.1, 0.0, 0.0)
    assert L.sgd_apply_update(dummy, C.byref(gb), dummy, C.byref(bad), None) == S.EINVAL
    mom = S.SgdRule(S.MOMENTUM, 0.1, 0.9, 0.0)
    assert L.sgd_apply_update(dummy, C.byref(gb), None, C.byref(mom), None) == S.EINVAL   # needs V
    assert L.sgd_apply_fused(dummy, dummy, arr, 3, 0, C.byref(mom), None) == S.EINVAL      # n = 0
    assert L.sgd_param_count(None) == -1
    assert L.sgd_workspace_bytes(None) == 0


def test_empty_batch_and_sizes_rejected():
    for nchw in ((0, 1, 28, 28), (16, 0, 28, 28), (16, 1, 0, 28)):
        with pytest.raises(S.SgdError) as e:
            S.Net(nchw, workloads.LENET5)
        assert e.value.code == S.ESHAPE


def test_set_debug_flag():
    L = S.lib()
    assert L.sgd_set_debug(None, 1) == S.EINVAL
    wl = workloads.WORKLOADS["lenet5"]
    net = S.Net((16,) + wl.chw, wl.layers)
    net.set_debug(True)
    net.set_debug(False)


@pytest.mark.parametrize("name,default", [("lenet5", False), ("mlp5000", True), ("vgg_cifar", True), ("vgg16", True)])
def test_overlap_default_and_setting(name, default):
    """The dedw side stream is on by default only for nets whose weight-gradient products total at least
    2^30 flops per step (LeNet-5 at batch 16: about 10^7); an explicit setting wins and -1 restores the
    default, also after a re-plan."""
    L = S.lib()
    assert L.sgd_set_overlap(None, 1) == S.EINVAL
    assert L.sgd_get_overlap(None, C.byref(C.c_int())) == S.EINVAL
    wl = workloads.WORKLOADS[name]
    net = S.Net((wl.batch,) + wl.chw, wl.layers)
    assert net.overlap is default
    net.set_overlap(not default)
    assert net.overlap is (not default)
    net.set_implicit_conv(False)
    assert net.overlap is (not default)
    net.set_overlap(None)
    assert net.overlap is default


def test_binding_rejects_wrong_dtypes_and_lengths():
    # argument marshalling checks, on host tensors (no compute call is made)
    torch = pytest.importorskip("torch")
    wl = workloads.WORKLOADS["lenet5"]
    net = S.Net((16,) + wl.chw, wl.layers)
    n = net.param_count()
    W = torch.zeros(n)
    X = torch.zeros(16, 1, 28, 28)
    y = torch.zeros(16, dtype=torch.int32)
    loss = torch.zeros(1)
    ws = torch.zeros(16, dtype=torch.uint8)
    net._check_step(W, X, y, loss, ws)                       # well-formed: passes
    bad = [
        dict(y=torch.zeros(16, dtype=torch.int64)),          # torch.randint's default dtype
        dict(y=torch.zeros(15, dtype=torch.int32)),
        dict(W=torch.zeros(n - 1)),
        dict(W=torch.zeros(n, dtype=torch.float64)),
        dict(X=torch.zeros(16, 1, 28, 27)),
        dict(loss=torch.zeros(0)),
        dict(ws=torch.zeros(4)),
    ]
    for b in bad:
        args = dict(W=W, X=X, y=y, loss=loss, ws=ws)
        args.update(b)
        with pytest.raises(ValueError):
            net._check_step(args["W"], args["X"], args["y"], args["loss"], args["ws"])
    with pytest.raises(ValueError):
        net._check_step(W, X, y, loss, ws, state=torch.zeros(n - 4))
    with pytest.raises(ValueError):
        net._check_step(W, X, y, loss, ws, grad=torch.zeros(n + 1))
    with pytest.raises(ValueError):
        net._check_step(W, X, y, loss, ws, need_state=True)
