"""The SPRINT report's model of the gradient step's time, refitted to this library's kernels.

The SPRINT report (IPSJ SIG Technical Report, section 3.3) writes the time of
ComputeGradient as a sum over layers of CUDA-kernel times and SGEMM times
(eq. 4).  It models im2col as linear in the size of the column matrix it
writes (eq. 5) and every SGEMM as a polynomial in its m, n, k with eight
coefficients (eq. 6), fitted to products timed on a grid of powers of two and
checked on shapes between the grid points (section 4.1, Figs. 5 and 6).

This module does the same for this library:

* ``gemm_grid`` times ``sgd_gemm`` launches on the device (host work only:
  buffers, events, a call per shape);
* ``fit_eq6`` and ``fit_linear`` fit eq. 6 and the linear CUDA-kernel models
  of eq. 5 / Fig. 5 by least squares on relative error;
* ``products_of`` and ``predict_step`` evaluate eq. 4 for a step recorded
  with ``Net.profile``, whose records carry each product's shape.

The page fits one model for one library routine.  Here the library picks
between two kernel families by operand alignment, which m, n, k alone do not
show: the direct-load kernels (rows of whole 16-byte groups) and the staged
kernels (any layout).  Each family and form gets its own eight coefficients,
the staged family fitted on the same grid moved by 2 in the dimension whose
alignment the direct loads need (``staged_shape``).

The forms are named as the kernels are, with BLAS's letters for C = op(A)
op(B) where op(A) is m x k and op(B) is k x n: 'n' for an operand stored in
that shape, 't' for one stored transposed.  The forward and fc products are
"nt" (B = W stored [n][k]), dedw with dedb as its extra ones column is "tn",
and dedx is "nn".
"""

import numpy as np

EQ6_TERMS = ("mnk", "mn", "mk", "nk", "m", "n", "k", "1")
FORMS = {"nt": (False, False), "tn": (True, True), "nn": (False, True), "tt": (True, False)}
# the gathered (implicit im2col) kernels compute the same algebra as these forms
_CONV_FORMS = {"fwd": "nt", "dw": "tn", "dx": "nn"}


def eq6_features(m, n, k):
    """Rows [mnk, mn, mk, nk, m, n, k, 1] of eq. 6 for arrays of m, n, k."""
    m, n, k = (np.asarray(v, dtype=np.float64) for v in (m, n, k))
    return np.stack([m * n * k, m * n, m * k, n * k, m, n, k, np.ones_like(m)], axis=-1)


def _rel_lstsq(X, t):
    """Least squares of X a = t on relative error (each row divided by t), with
    the columns scaled to unit size first so the solve is well conditioned."""
    X = np.asarray(X, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    if X.shape[0] < X.shape[1] or np.any(t <= 0):
        raise ValueError("need at least as many positive samples as coefficients")
    Xr = X / t[:, None]
    scale = np.abs(Xr).max(axis=0)
    scale[scale == 0] = 1.0
    a, *_ = np.linalg.lstsq(Xr / scale, np.ones_like(t), rcond=None)
    return a / scale


def fit_eq6(m, n, k, t):
    """The eight coefficients (alpha_mnk .. alpha_k, beta) of eq. 6 for times t."""
    return _rel_lstsq(eq6_features(m, n, k), t)


def eq6(alpha, m, n, k):
    return eq6_features(m, n, k) @ np.asarray(alpha, dtype=np.float64)


def fit_linear(x, t):
    """(alpha, beta) of t = alpha * x + beta (eq. 5's form), on relative error.
    With a single distinct x there is nothing to fit a slope to: (0, mean t)."""
    x = np.asarray(x, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    if len(np.unique(x)) < 2:
        return 0.0, float(np.mean(t))
    a, b = _rel_lstsq(np.stack([x, np.ones_like(x)], axis=-1), t)
    return float(a), float(b)


def grid_points(lo=3, hi=22, max_mnk_log2=38, max_pair_log2=29):
    """(m, n, k) = (2^x, 2^y, 2^z) with lo <= x, y, z <= hi.  Products beyond
    2^max_mnk_log2 multiply-adds or with an operand beyond 2^max_pair_log2
    elements are left out: none of the networks here comes near them."""
    pts = []
    for x in range(lo, hi + 1):
        for y in range(lo, hi + 1):
            for z in range(lo, hi + 1):
                if x + y + z <= max_mnk_log2 and max(x + y, x + z, y + z) <= max_pair_log2:
                    pts.append((1 << x, 1 << y, 1 << z))
    return pts


def offgrid_points(count, seed, lo=3, hi=22, max_mnk_log2=38, max_pair_log2=29, shift=0.25):
    """A seeded sample of grid points moved to 2^(x + shift) in every
    dimension, rounded to integers: shapes the fit has not seen, most of them
    not multiples of 4."""
    base = grid_points(lo, hi - 1, max_mnk_log2 - 1, max_pair_log2 - 1)
    rng = np.random.default_rng(seed)
    pick = rng.choice(len(base), size=min(count, len(base)), replace=False)
    out = []
    for i in sorted(pick):
        m, n, k = base[i]
        out.append(tuple(int(round(v * 2.0 ** shift)) for v in (m, n, k)))
    return out


def staged_shape(form, m, n, k):
    """A grid shape moved so the form's direct-load precondition fails: k by 2
    where A is stored [m][k] (nt, nn), else m by 2 (A stored [k][m])."""
    return (m, n, k + 2) if form in ("nt", "nn") else (m + 2, n, k)


def family_for(form, m, n, k):
    """The kernel family the library picks for a product whose operands sit
    at 16-byte aligned addresses with row strides a multiple of 4 floats: the
    direct loads need each operand's contiguous dimension (k for A [m][k] and
    B [n][k], m for A [k][m], n for B [k][n]) to be a multiple of 4."""
    a_t, b_t = FORMS[form]
    ok = (m % 4 == 0 if a_t else k % 4 == 0) and (n % 4 == 0 if b_t else k % 4 == 0)
    return "dma" if ok else "staged"


def family_of_kernel(name):
    """"staged" for the staged kernels, "dma" for the direct-load ones (the
    gathered convolution kernels share their main loop, and the streaming
    weight-gradient kernel of short reductions is what the library picks for
    the same aligned operands, as are the skinny kernels of a logits layer's
    products)."""
    return "staged" if name.startswith("gemm_staged_") else "dma"


def form_of_kernel(name):
    """The product form of a GEMM kernel name, e.g. gemm_dma_128x128_tn -> "tn"."""
    if name.startswith("gemm_conv_"):
        return _CONV_FORMS[name.split("_")[2]]
    if name.startswith("gemm_dw_short_"):
        return "tn"
    if name.startswith(("gemm_skinny_", "gemm_smallk_")):
        return name.rsplit("_", 1)[-1]
    suffix = name.rsplit("_", 1)[-1]
    if name.startswith(("gemm_dma_", "gemm_staged_")) and suffix in FORMS:
        return suffix
    return None


def products_of(records):
    """Split profile records into matrix products and other kernels.

    Returns (products, others): products is a list of dicts {form, family,
    m, n, k, ms, kernels} with ms summed over every launch of the product
    (main kernel, stream-K fixup, split-K reduce); others is a list of
    (kernel, bytes, ms)."""
    prods = {}
    others = []
    for (name, _layer, _phase, ms, _flops, nbytes, shape) in records:
        m, n, k, pid = shape
        if pid < 0:
            others.append((name, nbytes, ms))
            continue
        p = prods.setdefault(pid, {"form": None, "family": None, "m": m, "n": n, "k": k, "ms": 0.0,
                                   "kernels": []})
        p["ms"] += ms
        p["kernels"].append(name)
        if p["form"] is None:
            p["form"] = form_of_kernel(name)
            p["family"] = family_of_kernel(name)
    return [prods[i] for i in sorted(prods)], others


def fit_kernel_models(records):
    """Per CUDA kernel (everything outside the products), (alpha, beta) of
    time = alpha * algorithmic bytes + beta, the linear form eq. 5 gives
    im2col and Fig. 5 applies to each CUDA kernel."""
    _, others = products_of(records)
    by = {}
    for name, nbytes, ms in others:
        by.setdefault(name, ([], []))
        by[name][0].append(nbytes)
        by[name][1].append(ms)
    return {name: fit_linear(x, t) for name, (x, t) in by.items()}


def predict_step(records, alphas, kernel_models):
    """Eq. 4 for one recorded step: the sum over its products of eq. 6 with the
    coefficients of the product's kernel family and form (alphas[family][form]),
    plus the sum over its other kernels of their linear models.  Returns a
    dict with the predicted and measured sums (ms) split into the SGEMM and
    CUDA parts, and the per-product rows (family, form, m, n, k, pred, meas)."""
    prods, others = products_of(records)
    rows = []
    sg_pred = sg_meas = 0.0
    for p in prods:
        a = alphas.get(p["family"], {}).get(p["form"])
        if a is None:
            raise KeyError(f"no eq. 6 fit for {p['family']} form {p['form']!r} ({p['kernels'][0]})")
        pred = float(eq6(a, p["m"], p["n"], p["k"]))
        rows.append((p["family"], p["form"], p["m"], p["n"], p["k"], pred, p["ms"]))
        sg_pred += pred
        sg_meas += p["ms"]
    cu_pred = cu_meas = 0.0
    missing = set()
    for name, nbytes, ms in others:
        if name not in kernel_models:
            missing.add(name)
            continue
        a, b = kernel_models[name]
        cu_pred += a * nbytes + b
        cu_meas += ms
    if missing:
        raise KeyError(f"no CUDA-kernel model for {sorted(missing)}")
    return {"sgemm_pred": sg_pred, "sgemm_meas": sg_meas, "cuda_pred": cu_pred, "cuda_meas": cu_meas,
            "pred": sg_pred + cu_pred, "meas": sg_meas + cu_meas, "products": rows}


def gemm_grid(shapes, reps=5, device="cuda", progress=None):
    """Median time (ms) of one sgd_gemm launch for every form and (m, n, k) of
    shapes = {form: [(m, n, k), ...]}.

    Operands are stored as the networks store theirs: row strides rounded up
    to a multiple of 4 floats.  Every launch is bracketed by its own events,
    as the step profiler brackets its kernels, behind a device sleep that
    lets the host queue the launches ahead of the GPU, so host call overhead
    is not timed.  Returns {form: np.array of [m, n, k, ms] rows}."""
    import torch

    from . import gemm, gemm_workspace_bytes

    def r4(v):
        return (v + 3) // 4 * 4

    dev = torch.device(device)
    big = max(max(r4(m) * r4(k), r4(k) * r4(n), m * r4(n)) for pts in shapes.values() for (m, n, k) in pts)
    bufs = [torch.rand(big, device=dev) for _ in range(2)]
    out = torch.empty(big, device=dev)
    wsz = max(gemm_workspace_bytes(m, n, k, *FORMS[f]) for f, pts in shapes.items() for (m, n, k) in pts)
    ws = torch.empty(max(wsz, 256) // 4 + 64, device=dev)
    stream = torch.cuda.current_stream()
    events = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]

    def mat(buf, rows, cols):
        return buf[: rows * r4(cols)].view(rows, r4(cols))[:, :cols]

    res = {}
    for fi, (f, pts) in enumerate(shapes.items()):
        a_t, b_t = FORMS[f]
        rows = []
        for i, (m, n, k) in enumerate(pts):
            A = mat(bufs[0], k, m) if a_t else mat(bufs[0], m, k)
            B = mat(bufs[1], k, n) if b_t else mat(bufs[1], n, k)
            Cm = mat(out, m, n)
            gemm(A, B, Cm, a_t, b_t, ws, stream)  # warm-up (and first-touch of the shape)
            # queue-ahead: a sleep of 100k clocks (40 us at 2.4 GHz) per launch to queue
            torch.cuda._sleep(100_000 * reps)
            for r in range(reps):
                events[r].record(stream)
                gemm(A, B, Cm, a_t, b_t, ws, stream)
            events[reps].record(stream)
            events[reps].synchronize()
            t = sorted(events[r].elapsed_time(events[r + 1]) for r in range(reps))
            rows.append((m, n, k, t[reps // 2]))
            if progress and (i + 1) % 1000 == 0:
                progress(f"form {f} ({fi + 1}/{len(shapes)}): {i + 1}/{len(pts)} shapes")
        res[f] = np.array(rows, dtype=np.float64)
    return res


def rel_errors(pred, meas):
    pred = np.asarray(pred, dtype=np.float64)
    meas = np.asarray(meas, dtype=np.float64)
    return (pred - meas) / meas


def summarize_errors(err):
    a = np.abs(np.asarray(err))
    return {"median": float(np.median(a)), "p90": float(np.percentile(a, 90)), "max": float(a.max()),
            "n": int(a.size)}
