#!/usr/bin/env python3
"""Benchmark one data-parallel worker's full SGD step on one MI355X.

A step is the gradient (forward, softmax-CE, backward through every layer)
and the update rule applied to the weights (sgd_train_step: each layer's
update is applied in the epilogue of its dedw product, bitwise equal to
gradient-into-GradBuf + apply_update), through the C ABI on one stream, with
inputs already resident in HBM.  The unfused pair is timed too, for
reference.  The default
workload is the 5000-unit MLP (fc 3072-5000x5-10, ReLU, softmax-CE, batch 512,
momentum SGD mu = 0.9, eta = 0.01), synthetic inputs from the seeded
generators, He-normal weights.

Printed: one JSON line with images/s (value), the roofline of the dominant
kernel (HIP-event durations of every launch inside the timed region,
algorithmic flops per launch), per-kernel totals, the parameter-server Adagrad
apply in GB/s, and the CPU oracle timed on a bounded sample of the same
workload on this host's cores.

    python bench.py [--steps 50] [--warmup 5] [--workload mlp5000] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3   # MI355X dense fp32 matrix (MFMA) peak
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
METRIC = "images/sec per fwd+bwd+update SGD step (fp32); GEMM MFMA util %, update GB/s"


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE/WRITE_SIZE counter runs, or None
    when there is no record for it or the kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = b"".join(open(os.path.join(ROOT, "sgd_cnns_amd", "csrc", f), "rb").read() for f in ("gemm.hip", "update.hip"))
    if rec.get("workload") != workload or rec.get("source_sha256(gemm.hip+update.hip)") != hashlib.sha256(src).hexdigest():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k["traffic_bytes"]


def describe(wl):
    arch = {"mlp5000": "fc 3072-5000x5-10, ReLU, softmax-CE",
            "lenet5": "LeNet-5 (conv5x5 6, pool, conv5x5 16, pool, fc 400-120-84-10)",
            "vgg_cifar": "VGG-style 13 conv3x3 + 5 pool + fc 512-512-10 at 3x32x32",
            "vgg16": "VGG-16 (13 conv3x3 + 5 pool + fc 25088-4096-4096-1000) at 3x224x224"}[wl.name]
    rule = {"plain": f"plain SGD eta={wl.eta}", "momentum": f"momentum SGD mu={wl.mu} eta={wl.eta}",
            "adagrad": f"Adagrad eta={wl.eta}"}[wl.rule]
    return f"{wl.name}: {arch}, batch {wl.batch}, {rule}"


def gpu_step_bench(wl, steps, warmup, use_graph=True):
    import numpy as np
    import torch

    import sgd_cnns_amd as S
    import workloads

    dev = torch.device("cuda")
    X, y, W = workloads.make_inputs(wl)
    net = S.Net((wl.batch,) + tuple(wl.chw), wl.layers)
    n = net.param_count()
    Wd = torch.from_numpy(W).to(dev)
    Xd = torch.from_numpy(X).to(dev)
    yd = torch.from_numpy(y).to(dev)
    grad = torch.empty(n, device=dev)
    loss = torch.empty(1, device=dev)
    ws = net.workspace(dev)
    gb = S.GradBuf(n, device=dev)
    state = None
    if wl.rule == "momentum":
        state = torch.zeros(n, device=dev)
    elif wl.rule == "adagrad":
        state = torch.full((n,), 0.1, device=dev)
    rule = S.Rule(wl.rule, wl.eta, wl.mu, wl.eps)
    stream = torch.cuda.current_stream()

    def step(record=False):
        # one sub-batch per update: gradient and rule fused (sgd_train_step)
        net.train_step(Wd, Xd, yd, state, rule, loss, ws, stream)

    warm_losses = []
    for _ in range(warmup):
        step()
        warm_losses.append(float(loss.item()))
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    # the timed region, twice: the steps launched one call at a time, then (unless disabled) the step
    # recorded once as a HIP graph (sgd_train_step_graph) and replayed, one launch per step.  Both are
    # whole steps with no per-launch events; value takes the faster.  The graph removes the host
    # launch gaps (small networks) but its replay may not overlap the dedw stream with the main one.
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    eager_ms = t0.elapsed_time(t1)
    graph_ms = None
    graph = None
    if use_graph:
        graph = S.StepGraph(net, Wd, Xd, yd, state, rule, loss, ws)
        graph.launch(stream)
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        t0.record(stream)
        for _ in range(steps):
            graph.launch(stream)
        t1.record(stream)
        torch.cuda.synchronize()
        graph_ms = t0.elapsed_time(t1)
        if graph_ms < eager_ms:
            wall = time.perf_counter() - g0
    total_ms = eager_ms if graph_ms is None else min(eager_ms, graph_ms)
    loss_v = float(loss.item())
    # the same number of steps again with an event pair around every launch (sgd_profile): the
    # per-kernel durations of the roofline and the kernel table.  The events add a few
    # microseconds per launch, so this pass is not the one the throughput is taken from.
    net.profile(True)
    t0.record(stream)
    for _ in range(steps):
        step(record=True)
    t1.record(stream)
    torch.cuda.synchronize()
    net.profile(False)
    prof_ms = t0.elapsed_time(t1)
    recs = net.profile_read()
    if warm_losses:
        print(f"[bench] warmup losses {['%.4g' % v for v in warm_losses]}, last timed step {loss_v:.4g}",
              file=sys.stderr, flush=True)

    # per-kernel totals over the timed region
    kern = kernel_totals(recs)
    # the same step with the dedw products on the caller's stream (no
    # overlap): each kernel then has the GPU to itself, so its event time is
    # its own duration
    reps = max(3, min(steps, 10))
    net.set_overlap(False)
    step()
    torch.cuda.synchronize()
    i0, i1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    net.profile(True)
    i0.record(stream)
    for _ in range(reps):
        step()
    i1.record(stream)
    torch.cuda.synchronize()
    net.profile(False)
    net.set_overlap(True)
    kern_iso = kernel_totals(net.profile_read())
    iso_ms = i0.elapsed_time(i1) / reps
    # the unfused pair for reference: gradient into the GradBuf, then the
    # standalone apply kernel (its bandwidth is the update kernel's figure)
    u0, u1, u2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    upd_ms = 0.0
    # one untimed pair first: the timed step never launches the standalone
    # update kernels, so their first launch (code-object load) is kept out
    net.compute_gradient_into(Wd, Xd, yd, gb, loss, ws, stream)
    S.apply_update(Wd, gb, state, rule, stream)
    torch.cuda.synchronize()
    u0.record(stream)
    for _ in range(reps):
        net.compute_gradient_into(Wd, Xd, yd, gb, loss, ws, stream)
        u1.record(stream)
        S.apply_update(Wd, gb, state, rule, stream)
        u2.record(stream)
        torch.cuda.synchronize()
        upd_ms += u1.elapsed_time(u2)
    unfused_ms = u0.elapsed_time(u2) / reps
    upd_b = {"plain": 12.0, "momentum": 20.0, "adagrad": 20.0}[wl.rule] * n
    return dict(total_ms=total_ms, prof_ms=prof_ms, eager_ms=eager_ms, graph_ms=graph_ms,
                graph=graph_ms is not None and graph_ms < eager_ms, wall_s=wall,
                kern=kern, loss=loss_v, n_params=n,
                loss_first=warm_losses[0] if warm_losses else None,
                update={"kernel": f"apply_{wl.rule}", "avg_us": 1e3 * upd_ms / reps,
                        "GB/s": upd_b / (upd_ms / reps / 1e3) / 1e9},
                unfused_ms=unfused_ms, kern_iso=kern_iso, iso_ms=iso_ms, iso_reps=reps)


def kernel_totals(recs):
    # per kernel name: launches, event ms, algorithmic flops and bytes, and the roofline time
    # sum over launches of max(flops / fp32 MFMA peak, bytes / HBM peak), with how many launches
    # the flop term bounds
    kern = {}
    for (name, layer, phase, ms, flops, nbytes, _shape) in recs:
        k = kern.setdefault(name, {"launches": 0, "ms": 0.0, "flops": 0.0, "bytes": 0.0, "bound_ms": 0.0,
                                   "flop_bound": 0})
        k["launches"] += 1
        k["ms"] += ms
        k["flops"] += flops
        k["bytes"] += nbytes
        t_f = flops / (PEAK_FP32_TFLOPS * 1e9)
        t_b = nbytes / (PEAK_HBM_GBS * 1e6)
        k["bound_ms"] += max(t_f, t_b)
        k["flop_bound"] += t_f >= t_b and flops > 0
    return kern


def kernel_table(kern, total_ms):
    rows = []
    for name, v in sorted(kern.items(), key=lambda kv: -kv[1]["ms"]):
        e = {"kernel": name, "launches": v["launches"], "avg_us": 1e3 * v["ms"] / v["launches"],
             "share_of_step": v["ms"] / total_ms}
        if v["flops"] and name.startswith("gemm_"):
            e["TFLOP/s"] = v["flops"] / (v["ms"] / 1e3) / 1e12
            e["frac_fp32_peak"] = e["TFLOP/s"] / PEAK_FP32_TFLOPS
            # against each launch's attainable time min(peak, AI * 8 TB/s), AI from its algorithmic
            # operand bytes (A, B and C once)
            e["frac_attainable"] = v["bound_ms"] / v["ms"] if v["ms"] > 0 else None
            e["attainable_bound"] = ("mfma" if v["flop_bound"] == v["launches"] else
                                     "hbm" if v["flop_bound"] == 0 else "mixed")
        if v["bytes"]:
            e["GB/s"] = v["bytes"] / (v["ms"] / 1e3) / 1e9
            e["frac_hbm_peak"] = e["GB/s"] / PEAK_HBM_GBS
        rows.append(e)
    return rows


def variant_apply_bench(n, reps=20):
    """Standalone update kernels for the rule variants (weight decay, Nesterov) on n parameters."""
    import torch

    import sgd_cnns_amd as S

    dev = torch.device("cuda")
    W = torch.randn(n, device=dev)
    V = torch.zeros(n, device=dev)
    G = torch.randn(n, device=dev) * 1e-3
    stream = torch.cuda.current_stream()
    out = {}
    for name, rule, nbytes in (("apply_nesterov_decay", S.Rule("nesterov", 0.01, 0.9, 0.0, 5e-4), 20.0),
                               ("apply_plain_decay", S.Rule("plain", 0.01, 0.0, 0.0, 5e-4), 12.0)):
        st = V if name.startswith("apply_nesterov") else None
        S.apply_fused(W, st, [G], rule, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            S.apply_fused(W, st, [G], rule, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"params": n, "bytes_per_param": nbytes, "avg_us": 1e3 * ms,
                     "GB/s": nbytes * n / ms / 1e6, "frac_hbm_peak": nbytes * n / ms / 1e6 / PEAK_HBM_GBS}
    return out


def ps_apply_bench(steps=100, pool=16):
    """Parameter-server apply: 138,357,544 params, K = 8 buffers left-folded + Adagrad, fresh buffers per step."""
    import torch

    import sgd_cnns_amd as S
    import workloads

    ps = workloads.PS_APPLY
    n, k = ps["n"], ps["k"]
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(ps["seed"])
    W = torch.randn(n, device=dev, generator=g)
    A = torch.full((n,), ps["acc0"], device=dev)
    bufs = [torch.randn(n, device=dev, generator=g) * ps["grad_std"] for _ in range(pool)]
    rule = S.Rule("adagrad", ps["eta"], 0.0, ps["eps"])
    stream = torch.cuda.current_stream()
    evs = []
    for s in range(steps + 2):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        S.apply_fused(W, A, [bufs[(k * s + i) % pool] for i in range(k)], rule, stream)
        e1.record(stream)
        if s >= 2:
            evs.append((e0, e1))
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
    nbytes = (k + 4) * 4.0 * n
    del bufs
    return {"workload": f"{n} params, K={k} gradient buffers (fresh each step, pool {pool}) left-folded + Adagrad",
            "kernel": "apply_fused_adagrad", "ms_per_step": ms, "bytes_per_step": nbytes,
            "GB/s": nbytes / ms / 1e6, "frac_of_hbm_peak": nbytes / ms / 1e6 / PEAK_HBM_GBS, "steps": steps}


def cpu_baseline(wl, sample):
    """The CPU oracle on a bounded sample: gradient of `sample` images + a full accumulate + apply."""
    import numpy as np

    import oracle as O
    import workloads

    X, y, W = workloads.make_inputs(wl)
    net = O.OracleNet(wl.chw, wl.layers)
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    _, g = net.gradient(W, X[:sample], y[:sample])
    t_grad = time.perf_counter() - t0
    gb = O.GradBuf(W.size)
    state = np.zeros_like(W) if wl.rule != "adagrad" else np.full_like(W, 0.1)
    t0 = time.perf_counter()
    gb.accumulate(g)
    O.apply_rule(wl.rule, W, state, gb.data, wl.eta, wl.mu, wl.eps)
    t_upd = time.perf_counter() - t0
    t_step = t_grad * wl.batch / sample + t_upd
    return {"value": wl.batch / t_step, "unit": "images/s", "cores": cores, "kind": "oracle",
            "sample": (f"gradient of the first {sample} of {wl.batch} images ({t_grad:.1f} s) scaled per image to the "
                       f"full batch, plus one accumulate+apply over all {W.size} parameters ({t_upd:.2f} s)")}


def timing_model_report(out_path, raw_prefix=None, reps=3):
    """Refit the SPRINT report's timing model (section 3.3, eqs. 4-6) to these kernels and check its
    step predictions: eq. 6 on a power-of-two grid of sgd_gemm launches for each kernel family and
    form, validated off the grid (section 4.1, Fig. 6); the CUDA kernels' linear models (eq. 5,
    Fig. 5) from each workload's explicit-im2col gradient step at a quarter and a half of its batch;
    eq. 4 at the full batch."""
    import numpy as np
    import torch

    import sgd_cnns_amd as S
    import workloads
    from sgd_cnns_amd import timing_model as TM

    def say(msg):
        print(f"[timing-model] {msg}", file=sys.stderr, flush=True)

    t_start = time.perf_counter()
    forms = ("nt", "tn", "nn")
    grid = TM.grid_points()
    say(f"grid: {len(grid)} shapes x {len(forms)} forms x 2 kernel families")
    g = {"dma": TM.gemm_grid({f: grid for f in forms}, progress=say),
         "staged": TM.gemm_grid({f: [TM.staged_shape(f, *p) for p in grid] for f in forms}, progress=say)}
    alphas = {fam: {} for fam in g}
    fit_err = {fam: {} for fam in g}
    for fam in g:
        for f in forms:
            m, n, k, t = g[fam][f].T
            alphas[fam][f] = TM.fit_eq6(m, n, k, t)
            fit_err[fam][f] = TM.rel_errors(TM.eq6(alphas[fam][f], m, n, k), t)
    off = TM.offgrid_points(400, seed=6)
    say(f"off-grid validation: {len(off)} shapes")
    go = TM.gemm_grid({f: off for f in forms}, progress=say)
    off_err, off_err_big, off_fam = {}, {}, {}
    for f in forms:
        m, n, k, t = go[f].T
        fams = [TM.family_for(f, int(a), int(b), int(c)) for a, b, c in zip(m, n, k)]
        pred = np.array([float(TM.eq6(alphas[fam][f], a, b, c)) for fam, a, b, c in zip(fams, m, n, k)])
        e = TM.rel_errors(pred, t)
        off_err[f] = e
        off_err_big[f] = e[m * n * k >= 2.0 ** 27]
        off_fam[f] = sum(1 for x in fams if x == "dma")

    def step_records(wl, batch):
        w = wl.with_batch(batch)
        X, y, W = workloads.make_inputs(w)
        net = S.Net((batch,) + tuple(w.chw), w.layers)
        net.set_implicit_conv(False)
        net.set_overlap(False)
        dev = torch.device("cuda")
        Wd, Xd, yd = (torch.from_numpy(a).to(dev) for a in (W, X, y))
        grad = torch.empty(net.param_count(), device=dev)
        loss = torch.empty(1, device=dev)
        ws = net.workspace(dev)
        stream = torch.cuda.current_stream()
        for _ in range(2):
            net.compute_gradient(Wd, Xd, yd, grad, loss, ws, stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # as the step runs normally: launched back to back, host launch gaps included
        e0.record(stream)
        for _ in range(reps):
            net.compute_gradient(Wd, Xd, yd, grad, loss, ws, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = e0.elapsed_time(e1) / reps
        # profiled, each step queued behind a 2 ms device sleep so the GPU runs it without waiting
        # for the host: the kernels' event times are their device times, as on the grid
        steps, dev_ms = [], 0.0
        for _ in range(reps):
            net.profile(True)
            torch.cuda._sleep(5_000_000)
            e0.record(stream)
            net.compute_gradient(Wd, Xd, yd, grad, loss, ws, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            net.profile(False)
            steps.append(net.profile_read())
            dev_ms += e0.elapsed_time(e1)
        del ws
        torch.cuda.empty_cache()
        return steps, wall, dev_ms / reps

    names = ["lenet5", "mlp5000", "vgg_cifar", "vgg16"]
    fit_recs = []
    raw_steps = {}
    for name in names:
        wl = workloads.WORKLOADS[name]
        for b in (max(1, wl.batch // 4), max(1, wl.batch // 2)):
            say(f"{name} batch {b} (CUDA-kernel fit)")
            steps, _, _ = step_records(wl, b)
            raw_steps[f"{name}_{b}"] = steps
            for rec in steps:
                fit_recs.extend(rec)
    kmodels = TM.fit_kernel_models(fit_recs)
    preds = {}
    for name in names:
        wl = workloads.WORKLOADS[name]
        say(f"{name} batch {wl.batch} (eq. 4 prediction)")
        steps, wall, dev_ms = step_records(wl, wl.batch)
        raw_steps[f"{name}_{wl.batch}"] = steps
        per = [TM.predict_step(rec, alphas, kmodels) for rec in steps]
        avg = {key: float(np.mean([p[key] for p in per])) for key in
               ("sgemm_pred", "sgemm_meas", "cuda_pred", "cuda_meas", "pred", "meas")}
        avg["wall"], avg["device"] = wall, dev_ms
        avg["products"] = per[0]["products"]
        # the same products as lone sgd_gemm launches: splits eq. 4's SGEMM error into the fit's own
        # error and what the step's context adds (fused epilogues, operands not in cache).  A dedw
        # product records its ones column (dedb) in n; alone it is timed without it, so it runs on the
        # same direct-load kernels.
        alone = {}
        for (fam, f, m, n, k, _pr, _me) in avg["products"]:
            if fam == "dma" and TM.family_for(f, m, n, k) == "staged" and TM.family_for(f, m, n - 1, k) == "dma":
                n -= 1
            alone.setdefault(f, set()).add((m, n, k))
        shapes = {f: sorted(v) for f, v in alone.items()}
        t_alone = TM.gemm_grid(shapes)
        lookup = {(f, int(r[0]), int(r[1]), int(r[2])): r[3] for f in t_alone for r in t_alone[f]}
        tot = 0.0
        for (fam, f, m, n, k, _pr, _me) in avg["products"]:
            key = (f, m, n - 1, k) if (f, m, n, k) not in lookup else (f, m, n, k)
            tot += lookup[key]
        avg["sgemm_alone"] = tot
        preds[name] = avg
    if raw_prefix:
        np.savez(raw_prefix + "_grid.npz", **{f"{fam}_{f}": g[fam][f] for fam in g for f in forms},
                 **{f"off_{f}": go[f] for f in forms})
        with open(raw_prefix + "_steps.json", "w") as fh:
            json.dump(raw_steps, fh)

    L = []
    L.append("# SPRINT timing model (eqs. 4-6) refitted on MI355X")
    L.append("")
    L.append("Command (from the repository root): `python bench.py --timing-model profiles/timing_model_fit.md`")
    L.append("")
    L.append(f"Run time {time.perf_counter() - t_start:.0f} s.  Times are event-bracketed launches, fp32: the "
             "median of 5 per grid shape, queued ahead of the GPU; steps averaged over "
             f"{reps} profiled gradient steps (sgd_compute_gradient with im2col explicit, the page's method, "
             "and the dedw products on the caller's stream), each queued ahead the same way.")
    L.append("")
    L.append(f"## Eq. 6 fit: {len(grid)} shapes (m, n, k) = (2^x, 2^y, 2^z), 3 <= x, y, z <= 22, "
             "x+y+z <= 38, every operand <= 2^29 elements; least squares on relative error")
    L.append("")
    L.append("The staged family is timed on the same grid with k + 2 (nt, nn) or m + 2 (tn), which the "
             "direct-load kernels cannot take.")
    L.append("")
    L.append("| family | form | " + " | ".join(f"alpha_{t}" if t != "1" else "beta (ms)" for t in TM.EQ6_TERMS)
             + " | asymptotic TFLOP/s | on-grid median abs. rel. error | p90 |")
    L.append("|---|---|" + "---|" * (len(TM.EQ6_TERMS) + 3))
    for fam in g:
        for f in forms:
            a = alphas[fam][f]
            e = TM.summarize_errors(fit_err[fam][f])
            L.append(f"| {fam} | {f} | " + " | ".join(f"{v:.4g}" for v in a) +
                     f" | {2 / a[0] / 1e9:.1f} | {e['median']:.1%} | {e['p90']:.1%} |")
    L.append("")
    L.append("alpha_mnk is ms per multiply-add, so 2 / alpha_mnk / 1e9 is the fitted asymptotic TFLOP/s.")
    L.append("")
    L.append(f"## Off-grid check (Fig. 6's method): {len(off)} seeded grid shapes moved to 2^(x + 1/4), "
             "each predicted with the family the library picks for it")
    L.append("")
    L.append("| form | direct-load / staged | median abs. rel. error | p90 | max | mnk >= 2^27: median | p90 | n |")
    L.append("|---|---|---|---|---|---|---|---|")
    for f in forms:
        b, c = TM.summarize_errors(off_err[f]), TM.summarize_errors(off_err_big[f])
        L.append(f"| {f} | {off_fam[f]} / {len(off) - off_fam[f]} | {b['median']:.1%} | {b['p90']:.1%} | "
                 f"{b['max']:.1%} | {c['median']:.1%} | {c['p90']:.1%} | {c['n']} |")
    L.append("")
    L.append("## CUDA-kernel models: time = alpha * algorithmic bytes + beta (eq. 5's form; im2col's bytes are "
             "its column matrix plus its input)")
    L.append("")
    L.append("Fitted on the explicit-im2col gradient steps of all four workloads at a quarter and a half of "
             "their batch.")
    L.append("")
    L.append("| kernel | 1/alpha (GB/s) | beta (us) |")
    L.append("|---|---|---|")
    for kname in sorted(kmodels):
        a, b = kmodels[kname]
        L.append(f"| {kname} | {'-' if a <= 0 else f'{1e-6 / a:.0f}'} | {1e3 * b:.2f} |")
    L.append("")
    L.append("## Eq. 4: predicted vs measured gradient step at the full batch (ms per step)")
    L.append("")
    L.append("'same products alone' times each of the step's products as a lone sgd_gemm launch (plain store "
             "epilogue); 'device' is the profiled step queued ahead of the GPU, event records between kernels "
             "included; 'wall' the same step unprofiled and launched back to back as in training.")
    L.append("")
    L.append("| workload | batch | SGEMM pred | same products alone | SGEMM meas | CUDA pred | CUDA meas | eq. 4 pred "
             "| sum of kernels | error | device | error | wall | error |")
    L.append("|---|---|---|---|---|---|---|---|---|---|---|---|---|---|")
    for name in names:
        p = preds[name]
        L.append(f"| {name} | {workloads.WORKLOADS[name].batch} | {p['sgemm_pred']:.3f} | {p['sgemm_alone']:.3f} | "
                 f"{p['sgemm_meas']:.3f} | "
                 f"{p['cuda_pred']:.3f} | {p['cuda_meas']:.3f} | {p['pred']:.3f} | {p['meas']:.3f} | "
                 f"{(p['pred'] - p['meas']) / p['meas']:+.1%} | {p['device']:.3f} | "
                 f"{(p['pred'] - p['device']) / p['device']:+.1%} | {p['wall']:.3f} | "
                 f"{(p['pred'] - p['wall']) / p['wall']:+.1%} |")
    L.append("")
    L.append("## Largest products of each step: eq. 6 vs measured (ms)")
    for name in names:
        rows = sorted(preds[name]["products"], key=lambda r: -r[6])[:6]
        L.append("")
        L.append(f"{name}:")
        L.append("")
        L.append("| family | form | m | n | k | eq. 6 | measured | error |")
        L.append("|---|---|---|---|---|---|---|---|")
        for (fam, f, m, n, k, pr, me) in rows:
            L.append(f"| {fam} | {f} | {m} | {n} | {k} | {pr:.4f} | {me:.4f} | {(pr - me) / me:+.1%} |")
    text = "\n".join(L) + "\n"
    with open(out_path, "w") as fh:
        fh.write(text)
    print(text)


def sprint_report(out_path, workload="mlp5000"):
    """SPRINT's asynchronous workers and updater on one GPU (section 3.4, Algorithms 1 and 2): for
    several worker counts and sub-batch sizes, the throughput, T_GPU, T_Update, the measured average
    minibatch per update against eq. (9), and the staleness of the applied gradients."""
    import numpy as np
    import torch

    import sgd_cnns_amd as S
    import workloads

    def say(msg):
        print(f"[sprint] {msg}", file=sys.stderr, flush=True)

    base = workloads.WORKLOADS[workload]
    dev = torch.device("cuda")
    rows = []
    t_start = time.perf_counter()
    for sub in (128, 512):
        wl = base.with_batch(sub)
        n_batches = 16
        X = workloads.uniform01(wl.seed, 0, (n_batches * sub,) + tuple(wl.chw))
        y = workloads.labels(wl.seed, 1, n_batches * sub, wl.classes)
        W0 = workloads.he_normal_params(wl.seed, wl.chw, wl.layers)
        Xd, yd = torch.from_numpy(X).to(dev), torch.from_numpy(y).to(dev)
        net = S.Net((sub,) + tuple(wl.chw), wl.layers)
        rule = S.Rule(wl.rule, wl.eta, wl.mu, wl.eps)
        # the single-stream step at this sub-batch (sgd_train_step), for reference
        Wd = torch.from_numpy(W0).to(dev)
        V = torch.zeros_like(Wd)
        ws1 = net.workspace(dev)
        loss = torch.empty(1, device=dev)
        for _ in range(3):
            net.train_step(Wd, Xd[:sub], yd[:sub], V, rule, loss, ws1)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        e0.record()
        for r in range(reps):
            b = r % n_batches
            net.train_step(Wd, Xd[b * sub:(b + 1) * sub], yd[b * sub:(b + 1) * sub], V, rule, loss, ws1)
        e1.record()
        torch.cuda.synchronize()
        single_ms = e0.elapsed_time(e1) / reps
        del ws1
        for workers in (1, 2, 4, 8):
            iters = max(8, int(round(400.0 / (single_ms * workers))))
            cfg = S.SprintConfig(workers=workers, iters=iters)
            ws = torch.empty(S.sprint_workspace_bytes(net, cfg), dtype=torch.uint8, device=dev)
            Wd.copy_(torch.from_numpy(W0))
            V.zero_()
            S.sprint_run(net, S.SprintConfig(workers=workers, iters=2), Wd, V, rule, Xd, yd, n_batches, ws)  # warm-up
            Wd.copy_(torch.from_numpy(W0))
            V.zero_()
            torch.cuda.synchronize()
            st, log = S.sprint_run(net, cfg, Wd, V, rule, Xd, yd, n_batches, ws)
            torch.cuda.synchronize()
            finite = bool(torch.isfinite(Wd).all().item())
            say(f"sub-batch {sub}, {workers} workers x {iters}: {st['steps'] * sub / st['wall_ms'] * 1e3:.0f} img/s")
            rows.append(dict(sub=sub, workers=workers, iters=iters, single_ms=single_ms, finite=finite, **st))
            del ws
            torch.cuda.empty_cache()
    L = ["# SPRINT Algorithms 1 and 2 on one MI355X", "",
         f"Command (from the repository root): `python bench.py --sprint {os.path.relpath(out_path, ROOT)}`", "",
         f"Workload: {describe(base)} with the sub-batch below per worker step; 16 seeded synthetic sub-batches "
         "taken in turn by a shared counter.  Asynchronous SPRINT: every worker fetches LatestWeights at every "
         "step (n_fetch = 1) and pushes every step (n_push = 1); the updater applies whatever buffers are "
         "non-empty as soon as one is (min_bufs = 1), summing them and applying the momentum rule in one pass.  "
         f"Run time {time.perf_counter() - t_start:.0f} s.", "",
         "T_GPU is a worker's mean step (fetch, gradient, push, wait for its stream); T_Update the mean time "
         "between update completions.  Eq. (9) with one node: N_Minibatch_avg = N_GPU x N_Subbatch x "
         "T_Update / T_GPU.  Staleness: updates between the version a gradient was computed at and the update "
         "that applied it.  'single stream' is sgd_train_step at the same sub-batch, one step per update.", "",
         "| N_Subbatch | workers (N_GPU) | steps | images/s | single stream images/s | T_GPU ms | T_Update ms "
         "| updates | N_Minibatch_avg measured | eq. (9) | staleness mean | max | weights finite |",
         "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        L.append(f"| {r['sub']} | {r['workers']} | {r['steps']} | {r['steps'] * r['sub'] / r['wall_ms'] * 1e3:.0f} | "
                 f"{r['sub'] / r['single_ms'] * 1e3:.0f} | {r['t_gpu_ms']:.3f} | {r['t_update_ms']:.3f} | "
                 f"{r['updates']} | {r['n_minibatch_avg']:.1f} | {r['n_minibatch_eq9']:.1f} | "
                 f"{r['staleness_mean']:.2f} | {r['staleness_max']} | {r['finite']} |")
    text = "\n".join(L) + "\n"
    with open(out_path, "w") as fh:
        fh.write(text)
    print(text)


def main():
    import numpy as np
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mlp5000", choices=["mlp5000", "lenet5", "vgg_cifar", "vgg16"])
    ap.add_argument("--cpu-sample", type=int, default=0, help="images in the oracle sample (0 = per workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of HIP-graph replays")
    ap.add_argument("--no-ps-apply", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (a known-size kernel for counter scaling)")
    ap.add_argument("--timing-model", metavar="OUT_MD", default=None,
                    help="refit the SPRINT timing model (eqs. 4-6) and write its report instead of the step bench")
    ap.add_argument("--timing-model-raw", metavar="PREFIX", default=None,
                    help="also save the timing model's raw grid times and step records under this prefix")
    ap.add_argument("--sprint", metavar="OUT_MD", default=None,
                    help="run SPRINT's asynchronous workers and updater (Algorithms 1 and 2) and write the report")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}); the multi-GPU path is not built",
              file=sys.stderr)
        sys.exit(2)

    if args.sprint:
        sprint_report(args.sprint)
        return
    if args.timing_model:
        timing_model_report(args.timing_model, args.timing_model_raw)
        return
    import workloads
    wl = workloads.WORKLOADS[args.workload]
    if args.copy_calibration_mib:
        import torch
        n = args.copy_calibration_mib * 2 ** 20 // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty(n, device="cuda")
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(f"[bench] {describe(wl)}; warmup {args.warmup}, steps {args.steps}", file=sys.stderr, flush=True)
    r = gpu_step_bench(wl, args.steps, args.warmup, use_graph=not args.no_graph)
    ms_step = r["total_ms"] / args.steps
    value = wl.batch * args.steps / (r["total_ms"] / 1e3)
    kern = r["kern"]
    gemms = {k: v for k, v in kern.items() if k.startswith("gemm_")}
    dom = max(gemms, key=lambda k: gemms[k]["ms"])
    d = gemms[dom]
    achieved = d["flops"] / (d["ms"] / 1e3) / 1e12
    g_flops = sum(v["flops"] for v in gemms.values())
    g_ms = sum(v["ms"] for v in gemms.values())
    upd = r["update"]
    kernels = kernel_table(kern, r["prof_ms"])
    iso = r["kern_iso"].get(dom)
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "images/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded Philox inputs of the workload's shape; He-normal random-init weights)",
        "config": {"workload": describe(wl), "global_batch": wl.batch, "params": r["n_params"],
                   "update": wl.rule},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_TFLOPS,
                     "traffic": measured_traffic(dom, wl.name),
                     "launches": d["launches"], "avg_launch_us": 1e3 * d["ms"] / d["launches"],
                     "flops_per_launch": d["flops"] / d["launches"],
                     "ms_per_step_profiled": r["prof_ms"] / args.steps,
                     "note": "kernel durations from HIP events around every launch over the same number of steps, "
                             "run right after the timed region (the events cost a few microseconds per launch, so "
                             "value is timed without them).  Each layer's dedw product runs on a second stream, "
                             "overlapping the next layer's dedx product, so avg_launch_us is the launch's duration "
                             "while it shares the GPU; roofline_isolated is the same kernel with the overlap "
                             "switched off"},
        "roofline_isolated": None if iso is None else {
            "kernel": dom, "achieved": iso["flops"] / (iso["ms"] / 1e3) / 1e12, "peak": PEAK_FP32_TFLOPS,
            "unit": "TFLOP/s", "frac": iso["flops"] / (iso["ms"] / 1e3) / 1e12 / PEAK_FP32_TFLOPS,
            "launches": iso["launches"], "avg_launch_us": 1e3 * iso["ms"] / iso["launches"],
            "ms_per_step_no_overlap": r["iso_ms"]},
        "kernels_isolated": kernel_table(r["kern_iso"], r["iso_ms"] * r["iso_reps"])[:8],
        "gemm_mfma_util": {"achieved_TFLOP/s": g_flops / (g_ms / 1e3) / 1e12,
                           "frac_fp32_peak": g_flops / (g_ms / 1e3) / 1e12 / PEAK_FP32_TFLOPS,
                           "share_of_step": g_ms / r["prof_ms"]},
        "update_GB/s": {"kernel": upd["kernel"], "GB/s": upd["GB/s"], "frac_hbm_peak": upd["GB/s"] / PEAK_HBM_GBS,
                        "avg_us": upd["avg_us"],
                        "note": "standalone apply after gradient-into-GradBuf; the timed step fuses the update into "
                                "the dedw epilogues (sgd_train_step)"},
        "timed_as": "HIP graph replay of sgd_train_step (one launch per step)" if r["graph"] else
                    "sgd_train_step launched per step",
        "eager_ms_per_step": r["eager_ms"] / args.steps,
        "graph_ms_per_step": None if r["graph_ms"] is None else r["graph_ms"] / args.steps,
        "unfused_ms_per_step": r["unfused_ms"],
        "kernels": kernels,
        "loss_first_step": r["loss_first"],
        "loss_last_step": r["loss"] if np.isfinite(r["loss"]) else str(r["loss"]),
    }
    out["update_variants"] = variant_apply_bench(r["n_params"])
    if not args.no_ps_apply:
        print("[bench] parameter-server apply", file=sys.stderr, flush=True)
        out["ps_apply"] = ps_apply_bench()
    if not args.no_cpu_baseline:
        sample = args.cpu_sample or {"mlp5000": 512, "lenet5": 16, "vgg_cifar": 16, "vgg16": 1}[wl.name]
        print(f"[bench] CPU oracle baseline on {sample} images", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, sample)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
