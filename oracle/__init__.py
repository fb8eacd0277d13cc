"""Python driver for the CPU oracle (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It loads liboracle_f32.so / liboracle_f64.so (built from
oracle.c by oracle/build.py) and chains the layer functions in the order the
backpropagation algorithm fixes ("Pipelined training with stale weights of
deep CNNs", section 2: a forward pass from the first layer to the last, the
error at the output, then a backward pass from the last layer to the first
that produces each layer's weight gradient and the error of the layer below).

Shapes follow the SPRINT report (IPSJ SIG Technical Report Vol.2016-HPC-155
No.8), section 3.2 eq. (2), generalised to zero padding P (H + 2P - c + 1) and
pooling by p; the parameter count is that section's eq. (3).  The parameter
vector is flat: for each weighted layer in network order, the weight
(conv [co][ci][ky][kx], fc [out][in]) followed by the bias.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBS = {}


def lib(dtype=np.float32):
    key = np.dtype(dtype).name
    if key not in _LIBS:
        name = {"float32": "liboracle_f32.so", "float64": "liboracle_f64.so"}[key]
        path = os.path.join(_HERE, name)
        if not os.path.exists(path):
            raise RuntimeError(f"oracle library {path} is not built; run oracle/build.py")
        L = C.CDLL(path)
        P = C.c_void_p
        i, i64, d = C.c_int, C.c_int64, C.c_double
        rt = C.c_float if key == "float32" else C.c_double
        sig = {
            "or_conv_fwd": (None, [i, i, i, i, i, i, i, P, P, P, P]),
            "or_conv_bwd": (None, [i, i, i, i, i, i, i, P, P, P, P, P, P]),
            "or_conv_fwd_point": (d, [i, i, i, i, i, i, i, P, P, P, i, i, i, i]),
            "or_conv_dw_point": (d, [i, i, i, i, i, i, i, P, P, i, i, i, i]),
            "or_conv_db_point": (d, [i, i, i, i, P, i]),
            "or_conv_dx_point": (d, [i, i, i, i, i, i, i, P, P, i, i, i, i]),
            "or_relu_fwd": (None, [i64, P, P]),
            "or_relu_bwd": (None, [i64, P, P, P]),
            "or_maxpool_fwd": (None, [i, i, i, i, i, P, P, P]),
            "or_maxpool_bwd": (None, [i, i, i, i, i, P, P, P]),
            "or_fc_fwd": (None, [i, i, i, P, P, P, P]),
            "or_fc_bwd": (None, [i, i, i, P, P, P, P, P, P]),
            "or_softmax_ce": (d, [i, i, P, P, i, P]),
            "or_accumulate": (None, [P, P, P, i64]),
            "or_apply_plain": (None, [P, P, i64, rt, rt]),
            "or_apply_momentum": (None, [P, P, P, i64, rt, rt, rt]),
            "or_apply_nesterov": (None, [P, P, P, i64, rt, rt, rt]),
            "or_apply_adagrad": (None, [P, P, P, i64, rt, rt, rt]),
        }
        for fn, (res, args) in sig.items():
            f = getattr(L, fn)
            f.restype = res
            f.argtypes = args
        _LIBS[key] = L
    return _LIBS[key]


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ----------------------------------------------------------------------------
# Layer functions (thin marshalling around oracle.c; see its comments for the
# definitions and citations).  All activations are NCHW.
# ----------------------------------------------------------------------------

def conv_fwd(x, w, b, pad, dtype=np.float32):
    x, w, b = _c(x, dtype), _c(w, dtype), _c(b, dtype)
    N, Ci, H, W = x.shape
    Co, _, c, _ = w.shape
    y = np.empty((N, Co, H + 2 * pad - c + 1, W + 2 * pad - c + 1), dtype)
    lib(dtype).or_conv_fwd(N, Ci, H, W, Co, c, pad, _p(x), _p(w), _p(b), _p(y))
    return y


def conv_bwd(x, w, dy, pad, need_dx=True, dtype=np.float32):
    x, w, dy = _c(x, dtype), _c(w, dtype), _c(dy, dtype)
    N, Ci, H, W = x.shape
    Co, _, c, _ = w.shape
    dw = np.empty_like(w)
    db = np.empty(Co, dtype)
    dx = np.empty_like(x) if need_dx else None
    lib(dtype).or_conv_bwd(N, Ci, H, W, Co, c, pad, _p(x), _p(w), _p(dy), _p(dw), _p(db), _p(dx))
    return dw, db, dx


def relu_fwd(y, dtype=np.float32):
    y = _c(y, dtype)
    a = np.empty_like(y)
    lib(dtype).or_relu_fwd(y.size, _p(y), _p(a))
    return a


def relu_bwd(a, da, dtype=np.float32):
    a, da = _c(a, dtype), _c(da, dtype)
    dy = np.empty_like(a)
    lib(dtype).or_relu_bwd(a.size, _p(a), _p(da), _p(dy))
    return dy


def maxpool_fwd(x, p, dtype=np.float32):
    x = _c(x, dtype)
    N, Cc, H, W = x.shape
    y = np.empty((N, Cc, H // p, W // p), dtype)
    am = np.empty(y.shape, np.int32)
    lib(dtype).or_maxpool_fwd(N, Cc, H, W, p, _p(x), _p(y), _p(am))
    return y, am


def maxpool_bwd(dy, argmax, in_shape, p, dtype=np.float32):
    dy, am = _c(dy, dtype), _c(argmax, np.int32)
    N, Cc, H, W = in_shape
    dx = np.empty(in_shape, dtype)
    lib(dtype).or_maxpool_bwd(N, Cc, H, W, p, _p(dy), _p(am), _p(dx))
    return dx


def fc_fwd(a, w, b, dtype=np.float32):
    a, w, b = _c(a, dtype), _c(w, dtype), _c(b, dtype)
    N, In = a.shape
    Out = w.shape[0]
    z = np.empty((N, Out), dtype)
    lib(dtype).or_fc_fwd(N, In, Out, _p(a), _p(w), _p(b), _p(z))
    return z


def fc_bwd(a, w, dz, need_da=True, dtype=np.float32):
    a, w, dz = _c(a, dtype), _c(w, dtype), _c(dz, dtype)
    N, In = a.shape
    Out = w.shape[0]
    dw = np.empty_like(w)
    db = np.empty(Out, dtype)
    da = np.empty_like(a) if need_da else None
    lib(dtype).or_fc_bwd(N, In, Out, _p(a), _p(w), _p(dz), _p(dw), _p(db), _p(da))
    return dw, db, da


def softmax_ce(z, y, reduce_sum=False, dtype=np.float32):
    z, y = _c(z, dtype), _c(y, np.int32)
    N, Cc = z.shape
    if y.min(initial=0) < 0 or y.max(initial=0) >= Cc:
        raise ValueError("label out of range")
    dz = np.empty_like(z)
    loss = lib(dtype).or_softmax_ce(N, Cc, _p(z), _p(y), int(reduce_sum), _p(dz))
    return loss, dz


# Single-output spot checks (the same sums, one output at a time).

def conv_fwd_point(x, w, b, pad, n, co, oy, ox):
    N, Ci, H, W = x.shape
    Co, _, c, _ = w.shape
    return lib(np.float32).or_conv_fwd_point(N, Ci, H, W, Co, c, pad, _p(x), _p(w), _p(b), n, co, oy, ox)


def conv_dw_point(x, dy, c, pad, co, ci, ky, kx):
    N, Ci, H, W = x.shape
    Co = dy.shape[1]
    return lib(np.float32).or_conv_dw_point(N, Ci, H, W, Co, c, pad, _p(x), _p(dy), co, ci, ky, kx)


def conv_db_point(dy, co):
    N, Co, Ho, Wo = dy.shape
    return lib(np.float32).or_conv_db_point(N, Co, Ho, Wo, _p(dy), co)


def conv_dx_point(w, dy, in_hw, pad, n, ci, iy, ix):
    N, Co = dy.shape[:2]
    _, Ci, c, _ = w.shape
    H, W = in_hw
    return lib(np.float32).or_conv_dx_point(N, Ci, H, W, Co, c, pad, _p(w), _p(dy), n, ci, iy, ix)


# ----------------------------------------------------------------------------
# Update rules and GradBuf accumulation.
# ----------------------------------------------------------------------------

class GradBuf:
    """A gradient buffer with the empty state of SPRINT's Algorithms 1 and 2."""

    def __init__(self, n, dtype=np.float32):
        self.data = np.zeros(n, dtype)
        self.empty = True

    def accumulate(self, g):
        g = _c(g, self.data.dtype)
        e = C.c_int(1 if self.empty else 0)
        lib(self.data.dtype).or_accumulate(_p(self.data), C.byref(e), _p(g), g.size)
        self.empty = bool(e.value)


def apply_plain(W, g, eta, decay=0.0):
    lib(W.dtype).or_apply_plain(_p(W), _p(g), W.size, eta, decay)


def apply_momentum(W, V, g, mu, eta, decay=0.0):
    lib(W.dtype).or_apply_momentum(_p(W), _p(V), _p(g), W.size, mu, eta, decay)


def apply_nesterov(W, V, g, mu, eta, decay=0.0):
    lib(W.dtype).or_apply_nesterov(_p(W), _p(V), _p(g), W.size, mu, eta, decay)


def apply_adagrad(W, A, g, eta, eps, decay=0.0):
    lib(W.dtype).or_apply_adagrad(_p(W), _p(A), _p(g), W.size, eta, eps, decay)


def apply_rule(rule, W, state, g, eta, mu=0.0, eps=0.0, decay=0.0):
    """Apply one update in place; g None means an empty GradBuf (zero gradient)."""
    if rule == "plain":
        apply_plain(W, g, eta, decay)
    elif rule == "momentum":
        apply_momentum(W, state, g, mu, eta, decay)
    elif rule == "nesterov":
        apply_nesterov(W, state, g, mu, eta, decay)
    elif rule == "adagrad":
        apply_adagrad(W, state, g, eta, eps, decay)
    else:
        raise ValueError(rule)


# ----------------------------------------------------------------------------
# Whole network.
# ----------------------------------------------------------------------------

class OracleNet:
    """A CNN/MLP described by a layer list, run layer by layer on the CPU.

    layers: ("conv", out, c, pad) | ("relu",) | ("pool", p) | ("fc", out) |
    ("softmax_ce",), applied in order to images of shape chw.
    """

    def __init__(self, chw, layers, reduce_sum=False, dtype=np.float32):
        self.chw = tuple(chw)
        self.layers = list(layers)
        self.reduce_sum = reduce_sum
        self.dtype = np.dtype(dtype)
        self.params = {}   # layer index -> (w_off, w_shape, b_off, b_len)
        c, h, w = self.chw
        flat = None
        off = 0
        for i, L in enumerate(self.layers):
            k = L[0]
            if k == "conv":
                co, cc, pad = L[1], L[2], L[3]
                if flat is not None:
                    raise ValueError("conv after fc")
                shape = (co, c, cc, cc)
                nw = co * c * cc * cc
                self.params[i] = (off, shape, off + nw, co)
                off += nw + co
                c, h, w = co, h + 2 * pad - cc + 1, w + 2 * pad - cc + 1
            elif k == "pool":
                if h % L[1] or w % L[1]:
                    raise ValueError("pool does not divide the feature map")
                h, w = h // L[1], w // L[1]
            elif k == "fc":
                fan_in = c * h * w if flat is None else flat
                shape = (L[1], fan_in)
                self.params[i] = (off, shape, off + L[1] * fan_in, L[1])
                off += L[1] * fan_in + L[1]
                flat = L[1]
            elif k in ("relu", "softmax_ce"):
                pass
            else:
                raise ValueError(k)
        self.n_params = off
        self.classes = flat

    def param_count(self):
        return self.n_params

    def weight(self, W, i):
        wo, shape, bo, nb = self.params[i]
        return W[wo:wo + int(np.prod(shape))].reshape(shape), W[bo:bo + nb]

    def gradient(self, W, X, y, keep=False):
        """Loss and flat gradient for one sub-batch (and, with keep, every intermediate)."""
        dt = self.dtype
        W = _c(W, dt)
        a = _c(X, dt)
        acts = [a]          # acts[j] = input of layer j
        pools = {}
        loss = None
        dz = None
        for i, L in enumerate(self.layers):
            k = L[0]
            if k == "conv":
                w, b = self.weight(W, i)
                a = conv_fwd(a, w, b, L[3], dt)
            elif k == "relu":
                a = relu_fwd(a, dt)
            elif k == "pool":
                a, am = maxpool_fwd(a, L[1], dt)
                pools[i] = am
            elif k == "fc":
                w, b = self.weight(W, i)
                a = fc_fwd(a.reshape(a.shape[0], -1), w, b, dt)
            elif k == "softmax_ce":
                loss, dz = softmax_ce(a, y, self.reduce_sum, dt)
            acts.append(a)
        grad = np.zeros(self.n_params, dt)
        douts = {}
        d = dz
        first_weighted = min(self.params)
        for i in range(len(self.layers) - 2, -1, -1):
            L = self.layers[i]
            k = L[0]
            x_in = acts[i]
            douts[i] = d
            if k == "fc":
                w, _ = self.weight(W, i)
                wo, shape, bo, nb = self.params[i]
                dw, db, da = fc_bwd(x_in.reshape(x_in.shape[0], -1), w, d, need_da=i > first_weighted,
                                    dtype=dt)
                grad[wo:wo + dw.size] = dw.ravel()
                grad[bo:bo + nb] = db
                d = None if da is None else da.reshape(x_in.shape)
            elif k == "conv":
                w, _ = self.weight(W, i)
                wo, shape, bo, nb = self.params[i]
                dw, db, dx = conv_bwd(x_in, w, d.reshape(acts[i + 1].shape), L[3],
                                      need_dx=i > first_weighted, dtype=dt)
                grad[wo:wo + dw.size] = dw.ravel()
                grad[bo:bo + nb] = db
                d = dx
            elif k == "relu":
                d = relu_bwd(acts[i + 1], d.reshape(acts[i + 1].shape), dt)
            elif k == "pool":
                d = maxpool_bwd(d.reshape(acts[i + 1].shape), pools[i], x_in.shape, L[1], dt)
            if d is None:
                break
        if keep:
            return loss, grad, dict(acts=acts, douts=douts, pools=pools)
        return loss, grad

    def loss(self, W, X, y):
        """Forward pass only (used by the finite-difference checks)."""
        dt = self.dtype
        W = _c(W, dt)
        a = _c(X, dt)
        for i, L in enumerate(self.layers):
            k = L[0]
            if k == "conv":
                w, b = self.weight(W, i)
                a = conv_fwd(a, w, b, L[3], dt)
            elif k == "relu":
                a = relu_fwd(a, dt)
            elif k == "pool":
                a, _ = maxpool_fwd(a, L[1], dt)
            elif k == "fc":
                w, b = self.weight(W, i)
                a = fc_fwd(a.reshape(a.shape[0], -1), w, b, dt)
            elif k == "softmax_ce":
                return softmax_ce(a, y, self.reduce_sum, dt)[0]
        raise ValueError("network has no softmax_ce layer")


# ----------------------------------------------------------------------------
# SPRINT's workers and updater, replayed from a recorded schedule.
# ----------------------------------------------------------------------------

def sprint_replay(net, W0, state0, rule, batches, log, eta, mu=0.0, eps=0.0, decay=0.0):
    """The weights SPRINT reaches on one node for a given schedule (SPRINT report section 3.4,
    Algorithms 1 and 2).

    log holds one (worker, iter, push, batch, version, update) per worker step: the step's
    gradient is taken at the weights after `version` updates, on batches[batch] = (X, y)
    (Algorithm 1's gradient).  A worker's steps with the same push index are summed in iter
    order (the first stored, the rest added) and that sum goes into its GradBuf: copied when
    the buffer is empty, else added (Algorithm 1's push).  Update u takes the buffers holding
    the steps with update == u, in worker order, folds them the same way into one sum, and
    applies the rule to the weights (Algorithm 2 with one node).  A buffer taken by update u
    holds exactly the pushes of its steps, in push order.

    Returns (W, state, versions): the final weights and rule state, and W after each update
    (versions[0] is W0)."""
    n = net.param_count()
    dt = net.dtype
    W = np.array(W0, dtype=dt, copy=True)
    st = None if state0 is None else np.array(state0, dtype=dt, copy=True)
    versions = [W.copy()]
    if not log:
        return W, st, versions
    if any(e[5] < 0 for e in log):
        raise ValueError("a step was never applied")
    if any(e[4] > e[5] for e in log):
        raise ValueError("a step used weights newer than the update that applied it")
    for u in range(max(e[5] for e in log) + 1):
        steps = [e for e in log if e[5] == u]
        send = GradBuf(n, dt)                                 # SendBuf
        for t in sorted({e[0] for e in steps}):
            buf = GradBuf(n, dt)                              # GradBuf_t as update u takes it
            mine = [e for e in steps if e[0] == t]
            for p in sorted({e[2] for e in mine}):
                push = GradBuf(n, dt)                         # Grad summed over one push interval
                for e in sorted((e for e in mine if e[2] == p), key=lambda e: e[1]):
                    X, y = batches[e[3]]
                    push.accumulate(net.gradient(versions[e[4]], X, y)[1])
                buf.accumulate(push.data)
            send.accumulate(buf.data)
        apply_rule(rule, W, st, send.data if not send.empty else None, eta, mu, eps, decay)
        versions.append(W.copy())
    return W, st, versions
