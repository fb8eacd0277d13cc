"""Python binding of libsgdstep (include/sgdstep.h): argument marshalling only.

Every step of the SGD step runs in the HIP library; this module converts
torch device tensors to raw pointers and calls the C ABI through ctypes.
PyTorch provides device memory and streams only.  If the library is not
built, or no GPU is present, the compute entry points raise: there is no CPU
fallback.

    import sgd_cnns_amd as S
    net = S.Net((N, C, H, W), layers)           # layers as in workloads/
    ws = net.workspace()                        # torch.uint8 device buffer
    net.compute_gradient(W, X, y, grad, loss, ws)
    gb = S.GradBuf(grad.numel(), device="cuda")
    S.accumulate_grad(gb, grad)
    S.apply_update(W, gb, state, S.Rule("momentum", eta=0.01, mu=0.9))
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsgdstep.so")

# Constants of include/sgdstep.h
OK, EINVAL, ESHAPE, EWORKSPACE, EDEVICE, EUNSUPPORTED = 0, -1, -2, -3, -4, -5
CONV, RELU, MAXPOOL, FC, SOFTMAX_CE = 1, 2, 3, 4, 5
REDUCE_MEAN, REDUCE_SUM = 0, 1
PLAIN, MOMENTUM, ADAGRAD, NESTEROV = 0, 1, 2, 3
T_OUT, T_DOUT, T_COL, T_WREP, T_ARGMAX = 0, 1, 2, 3, 4
LAYOUT_NHWC, LAYOUT_NCHW, LAYOUT_ROWS = 1, 2, 3

EXPORTS = ["sgd_create_net", "sgd_destroy_net", "sgd_param_count", "sgd_param_offsets", "sgd_workspace_bytes",
           "sgd_tensor_info", "sgd_compute_gradient", "sgd_compute_gradient_into", "sgd_compute_gradient_into_scaled", "sgd_accumulate_grad",
           "sgd_accumulate_grads",
           "sgd_apply_update", "sgd_apply_fused", "sgd_train_step", "sgd_set_debug", "sgd_set_overlap", "sgd_get_overlap", "sgd_set_implicit_conv", "sgd_gemm", "sgd_gemm_workspace_bytes", "sgd_gemm_plan", "sgd_profile", "sgd_profile_read",
           "sgd_sprint_workspace_bytes", "sgd_sprint_run", "sgd_train_step_graph", "sgd_step_graph_launch",
           "sgd_step_graph_destroy", "sgd_stream_ref", "sgd_train_step_noalloc", "sgd_last_error"]
NOALLOC_SCRATCH_BYTES = 64 << 20


class SgdLayer(C.Structure):
    _fields_ = [("kind", C.c_int), ("out", C.c_int), ("kernel", C.c_int), ("pad", C.c_int), ("pool", C.c_int)]


class SgdInput(C.Structure):
    _fields_ = [("batch", C.c_int), ("channels", C.c_int), ("height", C.c_int), ("width", C.c_int)]


class SgdGradBuf(C.Structure):
    _fields_ = [("data", C.c_void_p), ("n", C.c_int64), ("empty", C.c_int)]


class SgdGemmArgs(C.Structure):
    _fields_ = [("m", C.c_int), ("n", C.c_int), ("k", C.c_int), ("a_t", C.c_int), ("b_t", C.c_int),
                ("A", C.c_void_p), ("lda", C.c_int64), ("B", C.c_void_p), ("ldb", C.c_int64),
                ("C", C.c_void_p), ("ldc", C.c_int64)]


class SgdRule(C.Structure):
    _fields_ = [("rule", C.c_int), ("eta", C.c_float), ("mu", C.c_float), ("eps", C.c_float), ("decay", C.c_float)]


class SgdKernelTime(C.Structure):
    _fields_ = [("kernel", C.c_char_p), ("layer", C.c_int), ("phase", C.c_int), ("ms", C.c_double),
                ("flops", C.c_double), ("bytes", C.c_double), ("m", C.c_int), ("n", C.c_int), ("k", C.c_int),
                ("product", C.c_int)]


class SgdSprintConfig(C.Structure):
    _fields_ = [("workers", C.c_int), ("iters", C.c_int), ("n_fetch", C.c_int), ("n_push", C.c_int),
                ("min_bufs", C.c_int), ("sync", C.c_int)]


class SgdSprintContrib(C.Structure):
    _fields_ = [("worker", C.c_int), ("iter", C.c_int), ("push", C.c_int), ("batch", C.c_int64),
                ("version", C.c_int64), ("update", C.c_int64)]


class SgdSprintStats(C.Structure):
    _fields_ = [("updates", C.c_int64), ("steps", C.c_int64), ("fetches", C.c_int64), ("wall_ms", C.c_double),
                ("t_gpu_ms", C.c_double), ("t_update_ms", C.c_double), ("n_minibatch_avg", C.c_double),
                ("n_minibatch_eq9", C.c_double), ("staleness_mean", C.c_double), ("staleness_max", C.c_int64)]


class SgdError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (status {code})")
        self.code = code


_lib = None


def lib():
    """Load libsgdstep.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() or sgd_cnns_amd/build.py")
        L = C.CDLL(LIB_PATH)
        P, i, i64, sz = C.c_void_p, C.c_int, C.c_int64, C.c_size_t
        sig = {
            "sgd_create_net": (i, [C.POINTER(SgdInput), C.POINTER(SgdLayer), i, i, C.POINTER(P)]),
            "sgd_destroy_net": (None, [P]),
            "sgd_param_count": (i64, [P]),
            "sgd_param_offsets": (i, [P, C.POINTER(i64), C.POINTER(i64), i]),
            "sgd_workspace_bytes": (sz, [P]),
            "sgd_tensor_info": (i, [P, i, i, C.POINTER(i64), C.POINTER(i64), C.POINTER(i)]),
            "sgd_compute_gradient": (i, [P, P, P, P, P, P, P, sz, P]),
            "sgd_compute_gradient_into": (i, [P, P, P, P, C.POINTER(SgdGradBuf), P, P, sz, P]),
            "sgd_compute_gradient_into_scaled": (i, [P, P, P, P, C.POINTER(SgdGradBuf), C.c_float, P, P, sz, P]),
            "sgd_accumulate_grad": (i, [C.POINTER(SgdGradBuf), P, P]),
            "sgd_accumulate_grads": (i, [C.POINTER(SgdGradBuf), C.POINTER(P), i, P]),
            "sgd_apply_update": (i, [P, C.POINTER(SgdGradBuf), P, C.POINTER(SgdRule), P]),
            "sgd_apply_fused": (i, [P, P, C.POINTER(P), i, i64, C.POINTER(SgdRule), P]),
            "sgd_train_step": (i, [P, P, P, P, P, C.POINTER(SgdRule), P, P, sz, P]),
            "sgd_profile": (i, [P, i]),
            "sgd_set_overlap": (i, [P, i]),
            "sgd_get_overlap": (i, [P, C.POINTER(C.c_int)]),
            "sgd_set_debug": (i, [P, i]),
            "sgd_set_implicit_conv": (i, [P, i]),
            "sgd_gemm_workspace_bytes": (sz, [C.POINTER(SgdGemmArgs)]),
            "sgd_gemm": (i, [C.POINTER(SgdGemmArgs), P, sz, P]),
            "sgd_gemm_plan": (i, [i, i, i, i, i, C.POINTER(i64), i]),
            "sgd_profile_read": (i, [P, C.POINTER(SgdKernelTime), i]),
            "sgd_sprint_workspace_bytes": (sz, [P, C.POINTER(SgdSprintConfig)]),
            "sgd_sprint_run": (i, [P, C.POINTER(SgdSprintConfig), P, P, C.POINTER(SgdRule), P, P, i64, P, sz, P,
                                   C.POINTER(SgdSprintStats), C.POINTER(SgdSprintContrib), i64]),
            "sgd_train_step_graph": (i, [P, P, P, P, P, C.POINTER(SgdRule), P, P, sz, C.POINTER(P)]),
            "sgd_step_graph_launch": (i, [P, P]),
            "sgd_step_graph_destroy": (None, [P]),
            "sgd_stream_ref": (i, [C.POINTER(P), i, C.POINTER(P), i, i64, i, P]),
            "sgd_train_step_noalloc": (i, [P, P, P, P, P, C.POINTER(SgdRule), P, P]),
            "sgd_last_error": (C.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(rc):
    if rc != OK:
        raise SgdError(rc, lib().sgd_last_error().decode())
    return rc


def _require_cuda(*tensors, rows=False):
    """Device tensors, contiguous (rows=True: 2-D with unit column stride, any row stride)."""
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("sgd_cnns_amd compute calls need a ROCm GPU (no CPU fallback)")
    for t in tensors:
        if t is None:
            continue
        if rows and t.dim() == 2 and t.is_cuda and t.stride(1) == 1:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors" + (" (matrices: unit column stride)"
                                                                            if rows else ""))


def _expect(t, numel, dtype, name):
    """t is a tensor of `dtype` with exactly `numel` elements (None passes: the C side rejects a
    missing required pointer)."""
    import torch
    if t is None:
        return
    dt = {"f32": torch.float32, "i32": torch.int32, "u8": torch.uint8}[dtype]
    if t.dtype != dt:
        raise ValueError(f"{name} must be {dt}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


_KIND = {"conv": CONV, "relu": RELU, "pool": MAXPOOL, "fc": FC, "softmax_ce": SOFTMAX_CE}


def to_layers(layers):
    """Convert ("conv", out, c, pad) / ("relu",) / ("pool", p) / ("fc", out) / ("softmax_ce",) tuples."""
    arr = (SgdLayer * len(layers))()
    for j, L in enumerate(layers):
        k = _KIND[L[0]]
        a = arr[j]
        a.kind = k
        if k == CONV:
            a.out, a.kernel, a.pad = L[1], L[2], L[3]
        elif k == MAXPOOL:
            a.pool = L[1]
        elif k == FC:
            a.out = L[1]
    return arr


class Net:
    """A planned network (sgd_create_net)."""

    def __init__(self, nchw, layers, reduce_sum=False):
        L = lib()
        inp = SgdInput(*[int(v) for v in nchw])
        arr = to_layers(layers)
        h = C.c_void_p()
        _check(L.sgd_create_net(C.byref(inp), arr, len(layers), REDUCE_SUM if reduce_sum else REDUCE_MEAN,
                                C.byref(h)))
        self._h = h
        self.nchw = tuple(nchw)
        self.layers = list(layers)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.sgd_destroy_net(h)
            self._h = None

    def param_count(self):
        return lib().sgd_param_count(self._h)

    def param_offsets(self):
        n = lib().sgd_param_offsets(self._h, None, None, 0)
        if n < 0:
            _check(n)
        w = (C.c_int64 * n)()
        b = (C.c_int64 * n)()
        lib().sgd_param_offsets(self._h, w, b, n)
        return list(w), list(b)

    def workspace_bytes(self):
        return lib().sgd_workspace_bytes(self._h)

    def tensor_info(self, layer, which):
        off = C.c_int64()
        dims = (C.c_int64 * 4)()
        lay = C.c_int()
        _check(lib().sgd_tensor_info(self._h, layer, which, C.byref(off), dims, C.byref(lay)))
        return off.value, tuple(dims), lay.value

    def workspace(self, device="cuda"):
        import torch
        return torch.empty(self.workspace_bytes(), dtype=torch.uint8, device=device)

    def view(self, ws, layer, which):
        """A torch view of a workspace tensor (float32, or uint8 for T_ARGMAX)."""
        import torch
        off, dims, lay = self.tensor_info(layer, which)
        if lay == LAYOUT_ROWS:
            shape = (dims[0], dims[2])   # rows x row stride; logical columns are dims[1]
        else:
            shape = dims
        n = 1
        for d in shape:
            n *= d
        if which == T_ARGMAX:
            return ws[off:off + n].view(shape)
        return ws[off:off + 4 * n].view(torch.float32).view(shape)

    def set_implicit_conv(self, enable):
        """Implicit-GEMM convolutions where the shapes allow (default on); re-plans the workspace."""
        _check(lib().sgd_set_implicit_conv(self._h, 1 if enable else 0))

    def _check_step(self, W, X, y, loss, ws, state=None, grad=None, need_state=False):
        n = self.param_count()
        N = self.nchw[0]
        nx = 1
        for d in self.nchw:
            nx *= int(d)
        _expect(W, n, "f32", "W")
        _expect(X, nx, "f32", "X")
        _expect(y, N, "i32", "y")
        _expect(loss, None, "f32", "loss")
        if loss is not None and loss.numel() < 1:
            raise ValueError("loss must hold at least one float")
        _expect(ws, None, "u8", "ws")
        _expect(state, n, "f32", "state")
        _expect(grad, n, "f32", "grad")
        if need_state and state is None:
            raise ValueError("this rule needs a state tensor")

    def set_debug(self, enable):
        """Validate the labels on the host before every step (sgd_set_debug)."""
        _check(lib().sgd_set_debug(self._h, 1 if enable else 0))

    def set_overlap(self, enable):
        """Run the dedw products on a second stream, overlapping the next layer: True, False, or None for the
        library's default (on when the weight-gradient products total at least 2^30 flops per step)."""
        _check(lib().sgd_set_overlap(self._h, -1 if enable is None else 1 if enable else 0))

    @property
    def overlap(self):
        """The overlap setting in effect (the default resolved)."""
        v = C.c_int()
        _check(lib().sgd_get_overlap(self._h, C.byref(v)))
        return bool(v.value)

    def profile(self, enable):
        """Start (clearing old records) or stop per-launch kernel timing."""
        _check(lib().sgd_profile(self._h, 1 if enable else 0))

    def profile_read(self):
        """[(kernel, layer, phase, ms, flops, bytes, (m, n, k, product))] for every recorded launch.

        The last field is (0, 0, 0, -1) for launches outside a matrix product."""
        n = lib().sgd_profile_read(self._h, None, 0)
        if n < 0:
            _check(n)
        arr = (SgdKernelTime * max(n, 1))()
        m = lib().sgd_profile_read(self._h, arr, n)
        if m < 0:
            _check(m)
        return [(r.kernel.decode(), r.layer, r.phase, r.ms, r.flops, r.bytes, (r.m, r.n, r.k, r.product)) for r in arr[:n]]

    def compute_gradient(self, W, X, y, grad, loss, ws, stream=None):
        _require_cuda(W, X, y, grad, loss, ws)
        self._check_step(W, X, y, loss, ws, grad=grad)
        _check(lib().sgd_compute_gradient(self._h, _ptr(W), _ptr(X), _ptr(y), _ptr(grad), _ptr(loss), _ptr(ws),
                                          ws.numel() * ws.element_size(), _stream(stream)))


    def compute_gradient_into(self, W, X, y, gb, loss, ws, stream=None):
        """Gradient stored into an empty GradBuf, or added into a non-empty one."""
        _require_cuda(W, X, y, gb.data, loss, ws)
        self._check_step(W, X, y, loss, ws, grad=gb.data)
        _check(lib().sgd_compute_gradient_into(self._h, _ptr(W), _ptr(X), _ptr(y), C.byref(gb._c), _ptr(loss),
                                               _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


    def compute_gradient_into_scaled(self, W, X, y, gb, scale, loss, ws, stream=None):
        """As compute_gradient_into with every gradient value multiplied by `scale` first."""
        _require_cuda(W, X, y, gb.data, loss, ws)
        self._check_step(W, X, y, loss, ws, grad=gb.data)
        _check(lib().sgd_compute_gradient_into_scaled(self._h, _ptr(W), _ptr(X), _ptr(y), C.byref(gb._c),
                                                      C.c_float(scale), _ptr(loss), _ptr(ws),
                                                      ws.numel() * ws.element_size(), _stream(stream)))

    def train_step(self, W, X, y, state, rule, loss, ws, stream=None):
        """Gradient + update in one pass: W (and state) updated in place."""
        _require_cuda(W, X, y, state, loss, ws)
        self._check_step(W, X, y, loss, ws, state=state, need_state=rule.rule != PLAIN)
        _check(lib().sgd_train_step(self._h, _ptr(W), _ptr(X), _ptr(y), _ptr(state), C.byref(rule), _ptr(loss),
                                    _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


    def train_step_noalloc(self, W, X, y, state, rule, loss, stream=None):
        """train_step with the library's static scratch as the workspace (sgd_train_step_noalloc)."""
        _require_cuda(W, X, y, state, loss)
        self._check_step(W, X, y, loss, None, state=state, need_state=rule.rule != PLAIN)
        _check(lib().sgd_train_step_noalloc(self._h, _ptr(W), _ptr(X), _ptr(y), _ptr(state), C.byref(rule),
                                            _ptr(loss), _stream(stream)))


class StepGraph:
    """sgd_train_step recorded as a HIP graph (sgd_train_step_graph); launch() replays one step.
    Holds references to the net and the buffers the graph is bound to."""

    def __init__(self, net, W, X, y, state, rule, loss, ws):
        _require_cuda(W, X, y, state, loss, ws)
        net._check_step(W, X, y, loss, ws, state=state, need_state=rule.rule != PLAIN)
        self._keep = (net, W, X, y, state, loss, ws)
        self._rule = rule
        h = C.c_void_p()
        _check(lib().sgd_train_step_graph(net._h, _ptr(W), _ptr(X), _ptr(y), _ptr(state), C.byref(rule), _ptr(loss),
                                          _ptr(ws), ws.numel() * ws.element_size(), C.byref(h)))
        self._h = h

    def launch(self, stream=None):
        _check(lib().sgd_step_graph_launch(self._h, _stream(stream)))

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.sgd_step_graph_destroy(h)
            self._h = None


class GradBuf:
    """A device gradient buffer with the host-side empty flag."""

    def __init__(self, n, device="cuda", data=None):
        import torch
        self.data = data if data is not None else torch.empty(n, dtype=torch.float32, device=device)
        self._c = SgdGradBuf(self.data.data_ptr(), n, 1)

    @property
    def empty(self):
        return bool(self._c.empty)

    @empty.setter
    def empty(self, v):
        self._c.empty = 1 if v else 0


def _gemm_args(A, B, C_, a_t, b_t):
    m, n = C_.shape
    k = A.shape[0] if a_t else A.shape[1]
    if (A.shape[1] if a_t else A.shape[0]) != m or (B.shape[1] if b_t else B.shape[0]) != n or \
            (B.shape[0] if b_t else B.shape[1]) != k:
        raise ValueError(f"gemm: op(A) {tuple(A.shape)} (a_t={a_t}), op(B) {tuple(B.shape)} (b_t={b_t}) "
                         f"and C {tuple(C_.shape)} do not form a product")
    return SgdGemmArgs(m, n, k, int(a_t), int(b_t), A.data_ptr(), A.stride(0), B.data_ptr(), B.stride(0),
                       C_.data_ptr(), C_.stride(0))


PLAN_FIELDS = ("bm", "bn", "grid", "dp", "sk_iters", "rg", "cg", "edge_last", "tiles_m", "tiles_n", "ipt", "cus")


def gemm_plan(m, n, k, a_t=False, b_t=False):
    """The tile kernels' schedule for an m x n x k product (host only; see sgd_gemm_plan), as a dict."""
    out = (C.c_int64 * len(PLAN_FIELDS))()
    _check(lib().sgd_gemm_plan(int(m), int(n), int(k), int(a_t), int(b_t), out, len(PLAN_FIELDS)))
    return dict(zip(PLAN_FIELDS, (int(v) for v in out)))


def gemm_workspace_bytes(m, n, k, a_t=False, b_t=False):
    """Scratch bytes sgd_gemm needs for an m x n x k product."""
    g = SgdGemmArgs(m, n, k, int(a_t), int(b_t), None, k if not a_t else m, None, k if not b_t else n, None, n)
    return lib().sgd_gemm_workspace_bytes(C.byref(g))


def gemm(A, B, C_, a_t=False, b_t=False, ws=None, stream=None):
    """C = op(A) op(B) on the GPU: A is [m][k] (a_t: [k][m]); B is [n][k] (b_t: [k][n])."""
    _require_cuda(A, B, C_, rows=True)
    _require_cuda(ws)
    for t, name in ((A, "A"), (B, "B"), (C_, "C")):
        _expect(t, None, "f32", name)
    g = _gemm_args(A, B, C_, a_t, b_t)
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib().sgd_gemm(C.byref(g), _ptr(ws), nbytes, _stream(stream)))


def _check_gradbuf(gb):
    _expect(gb.data, None, "f32", "GradBuf data")
    if gb.data.numel() < gb._c.n:
        raise ValueError(f"GradBuf data holds {gb.data.numel()} floats, the buffer says {gb._c.n}")


def accumulate_grad(gb, grad, stream=None):
    _require_cuda(gb.data, grad)
    _check_gradbuf(gb)
    _expect(grad, gb._c.n, "f32", "grad")
    _check(lib().sgd_accumulate_grad(C.byref(gb._c), _ptr(grad), _stream(stream)))


def accumulate_grads(gb, grads, stream=None):
    _require_cuda(gb.data, *grads)
    _check_gradbuf(gb)
    for j, g in enumerate(grads):
        _expect(g, gb._c.n, "f32", f"grads[{j}]")
    arr = (C.c_void_p * len(grads))(*[g.data_ptr() for g in grads])
    _check(lib().sgd_accumulate_grads(C.byref(gb._c), arr, len(grads), _stream(stream)))


_RULES = {"plain": PLAIN, "momentum": MOMENTUM, "adagrad": ADAGRAD, "nesterov": NESTEROV}


def Rule(rule, eta, mu=0.0, eps=0.0, decay=0.0):
    return SgdRule(_RULES[rule] if isinstance(rule, str) else rule, eta, mu, eps, decay)


def apply_update(W, gb, state, rule, stream=None):
    _require_cuda(W, gb.data, state)
    _check_gradbuf(gb)
    _expect(W, gb._c.n, "f32", "W")
    _expect(state, gb._c.n, "f32", "state")
    _check(lib().sgd_apply_update(_ptr(W), C.byref(gb._c), _ptr(state), C.byref(rule), _stream(stream)))


def apply_fused(W, state, grads, rule, stream=None):
    _require_cuda(W, state, *grads)
    _expect(W, None, "f32", "W")
    _expect(state, W.numel(), "f32", "state")
    for j, g in enumerate(grads):
        _expect(g, W.numel(), "f32", f"grads[{j}]")
    arr = (C.c_void_p * len(grads))(*[g.data_ptr() for g in grads])
    _check(lib().sgd_apply_fused(_ptr(W), _ptr(state), arr, len(grads), W.numel(), C.byref(rule), _stream(stream)))


def SprintConfig(workers, iters, n_fetch=1, n_push=1, min_bufs=1, sync=False):
    """SPRINT worker/updater settings (see sgd_sprint_run): min_bufs=1, sync=False is the
    asynchronous SPRINT updater; min_bufs=workers, sync=True is bulk-synchronous SGD."""
    return SgdSprintConfig(workers, iters, n_fetch, n_push, min_bufs, 1 if sync else 0)


def sprint_workspace_bytes(net, cfg):
    return lib().sgd_sprint_workspace_bytes(net._h, C.byref(cfg))


def sprint_run(net, cfg, W, state, rule, X, y, n_batches, ws, stream=None):
    """SPRINT's workers and updater on this GPU (sgd_sprint_run).  X, y hold n_batches sub-batches of
    the net's batch.  Returns (stats dict, log) with one log entry per worker step:
    (worker, iter, push, batch, version, update)."""
    _require_cuda(W, state, X, y, ws)
    n = net.param_count()
    per = 1
    for d in net.nchw:
        per *= int(d)
    _expect(W, n, "f32", "W")
    _expect(state, n, "f32", "state")
    _expect(X, None, "f32", "X")
    _expect(y, None, "i32", "y")
    _expect(ws, None, "u8", "ws")
    if n_batches >= 1 and (X.numel() < per * int(n_batches) or y.numel() < net.nchw[0] * int(n_batches)):
        raise ValueError(f"X and y must hold {n_batches} sub-batches of {net.nchw[0]}")
    steps = cfg.workers * cfg.iters
    log = (SgdSprintContrib * max(steps, 1))()
    st = SgdSprintStats()
    nbytes = ws.numel() * ws.element_size()
    _check(lib().sgd_sprint_run(net._h, C.byref(cfg), _ptr(W), _ptr(state), C.byref(rule), _ptr(X), _ptr(y),
                                int(n_batches), _ptr(ws), nbytes, _stream(stream), C.byref(st), log, steps))
    stats = {name: getattr(st, name) for name, _ in SgdSprintStats._fields_}
    return stats, [(c.worker, c.iter, c.push, c.batch, c.version, c.update) for c in log[:steps]]


def stream_ref(outs, ins, groups=1, stream=None):
    """Reference streaming pass (sgd_stream_ref): every output = left-fold sum of the inputs."""
    _require_cuda(*outs, *ins)
    n = ins[0].numel()
    for t in list(outs) + list(ins):
        _expect(t, n, "f32", "stream tensor")
    o = (C.c_void_p * max(1, len(outs)))(*[t.data_ptr() for t in outs])
    i = (C.c_void_p * len(ins))(*[t.data_ptr() for t in ins])
    _check(lib().sgd_stream_ref(o, len(outs), i, len(ins), n, groups, _stream(stream)))
