#!/usr/bin/env python3
"""Benchmark one data-parallel worker's full SGD step on one MI355X, for the five workloads.

A step is the gradient (forward, softmax-CE, backward through every layer) and
the update rule applied to the weights (sgd_train_step: each layer's update is
applied in the epilogue of its dedw product, bitwise equal to
gradient-into-GradBuf + apply_update), through the C ABI on one stream, with
inputs resident in HBM.  Before every step -- warm-up, timed, profiled -- the
weights and optimiser state are restored from a pristine device copy (outside
the step's events), so every timed step is the same first step from the
workload's He-normal weights, and every step's loss is checked to be finite.
Each step is bracketed by its own HIP events on the caller's stream; the
figures are the mean and median of the steps' event times (images/s =
batch / mean step time, SPRINT report eq. (9) with one GPU).

Workloads (seeded synthetic inputs):
  lenet5     LeNet-5, batch 16 of 1x28x28, plain SGD eta 0.01
  mlp5000    fc 3072-5000x5-10, batch 512, momentum mu 0.9 eta 0.01 (the headline `value`)
  vgg_cifar  VGG-style 13 conv + 5 pool + fc 512-512-10 at 3x32x32, batch 128, plain SGD
  vgg16      VGG-16 at 3x224x224, batch 32, 1000 classes, plain SGD
  ps_adagrad the parameter-server apply: 138,357,544 parameters, 8 fresh seeded gradient buffers
             left-folded + Adagrad, 100 steps; beside it the unfused chain and plain streaming
             kernels with the same read and write streams (the memory-traffic ceiling)

Printed: one JSON line.  Top level: the MLP's images/s (value), the roofline
of its dominant kernel (HIP-event durations of every launch in an
event-bracketed pass over the same steps, algorithmic flops per launch), its
CPU-oracle baseline.  `configs`: one record per workload with the same
figures, the isolated (no-overlap) roofline, and eq. (4)'s prediction from the
committed timing-model fit.

    python bench.py [--steps 20] [--warmup 5] [--workload all|mlp5000|...] [--no-cpu-baseline]
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3   # MI355X dense fp32 matrix (MFMA) peak
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
METRIC = "images/sec per fwd+bwd+update SGD step (fp32); GEMM MFMA util %, update GB/s"
STEP_WORKLOADS = ["mlp5000", "lenet5", "vgg_cifar", "vgg16"]


def say(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def kernel_code_sha256(files=("gemm.hip", "update.hip")):
    """SHA-256 of the kernel sources' code: C/C++ comments, trailing blanks and empty lines removed, so an
    edit of a comment does not mark counters taken on the same code as stale."""
    import hashlib
    out = []
    for f in files:
        text = open(os.path.join(ROOT, "sgd_cnns_amd", "csrc", f), encoding="utf-8").read()
        code, i, n, quote = [], 0, len(text), None
        while i < n:
            c = text[i]
            if quote:
                code.append(c)
                if c == "\\" and i + 1 < n:
                    code.append(text[i + 1])
                    i += 2
                    continue
                if c == quote:
                    quote = None
                i += 1
            elif c in "\"'":
                quote = c
                code.append(c)
                i += 1
            elif text.startswith("//", i):
                j = text.find("\n", i)
                i = n if j < 0 else j
            elif text.startswith("/*", i):
                j = text.find("*/", i + 2)
                i = n if j < 0 else j + 2
            else:
                code.append(c)
                i += 1
        lines = [ln.rstrip() for ln in "".join(code).split("\n")]
        out.append("\n".join(ln for ln in lines if ln))
    return hashlib.sha256("\n".join(out).encode()).hexdigest()


TRAFFIC_KEY = "code_sha256(gemm.hip+update.hip, comments stripped)"


def measured_traffic(kernel, workload):
    """(HBM bytes per launch, source) of `kernel` from the committed FETCH_SIZE/WRITE_SIZE counter
    runs, or (None, reason) when there is no record for it or the kernel sources changed since the
    counters were taken (the record stores a SHA-256 of the sources)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None, "no counter record"
    rec = json.load(open(path))
    recs = rec if isinstance(rec, list) else [rec]
    digest = kernel_code_sha256()
    for r in recs:
        if r.get("workload") != workload:
            continue
        if r.get(TRAFFIC_KEY) != digest:
            return None, f"profiles/traffic.json ({workload}) predates the current kernel sources"
        k = r.get("kernels", {}).get(kernel)
        if k is None:
            return None, f"no counter record for {kernel}"
        return k["traffic_bytes"], (f"profiles/traffic.json: rocprofv3 FETCH_SIZE x {r['fetch_scale']:.3f} + "
                                    f"WRITE_SIZE x {r['write_scale']:.3f} per dispatch ({r['calibration']})")
    return None, f"no counter record for {workload}"


def describe(wl):
    arch = {"mlp5000": "fc 3072-5000x5-10, ReLU, softmax-CE",
            "lenet5": "LeNet-5 (conv5x5 6, pool, conv5x5 16, pool, fc 400-120-84-10)",
            "vgg_cifar": "VGG-style 13 conv3x3 + 5 pool + fc 512-512-10 at 3x32x32",
            "vgg16": "VGG-16 (13 conv3x3 + 5 pool + fc 25088-4096-4096-1000) at 3x224x224"}[wl.name]
    rule = {"plain": f"plain SGD eta={wl.eta}", "momentum": f"momentum SGD mu={wl.mu} eta={wl.eta}",
            "adagrad": f"Adagrad eta={wl.eta}"}[wl.rule]
    return f"{wl.name}: {arch}, batch {wl.batch}, {rule}"


def _stats(ms):
    return {"mean": statistics.fmean(ms), "median": statistics.median(ms), "min": min(ms), "max": max(ms)}


def step_bench(wl, steps, warmup, use_graph=True):
    """Time `steps` training steps of workload wl (each from the pristine weights), eagerly and as HIP
    graph replays, then the same steps with per-launch events (overlapped and isolated) and the
    unfused gradient + apply pair."""
    import numpy as np
    import torch

    import sgd_cnns_amd as S
    import workloads

    dev = torch.device("cuda")
    X, y, W = workloads.make_inputs(wl)
    net = S.Net((wl.batch,) + tuple(wl.chw), wl.layers)
    overlap = net.overlap  # the library's default for this net (dedw products on a second stream or not)
    n = net.param_count()
    W0 = torch.from_numpy(W).to(dev)
    Wd = W0.clone()
    Xd = torch.from_numpy(X).to(dev)
    yd = torch.from_numpy(y).to(dev)
    loss = torch.empty(1, device=dev)
    ws = net.workspace(dev)
    st0 = None
    if wl.rule == "momentum":
        st0 = torch.zeros(n, device=dev)
    elif wl.rule == "adagrad":
        st0 = torch.full((n,), 0.1, device=dev)
    state = None if st0 is None else st0.clone()
    rule = S.Rule(wl.rule, wl.eta, wl.mu, wl.eps)
    stream = torch.cuda.current_stream()
    hist = torch.full((5 * steps + warmup + 64,), float("nan"), device=dev)
    n_hist = [0]

    def restore():
        Wd.copy_(W0)
        if state is not None:
            state.copy_(st0)

    def keep_loss():
        i = n_hist[0]
        hist[i:i + 1].copy_(loss)
        n_hist[0] += 1

    def eager():
        net.train_step(Wd, Xd, yd, state, rule, loss, ws, stream)

    def timed(run, count):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(count)]
        first = n_hist[0]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            restore()
            e0.record(stream)
            run()
            e1.record(stream)
            keep_loss()
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) for e0, e1 in evs], hist[first:n_hist[0]].cpu().numpy()

    for _ in range(warmup):
        restore()
        eager()
        keep_loss()
    torch.cuda.synchronize()
    warm_losses = hist[:n_hist[0]].cpu().numpy()
    eager_ms, eager_loss = timed(eager, steps)
    graph_ms = graph_loss = None
    if use_graph:
        graph = S.StepGraph(net, Wd, Xd, yd, state, rule, loss, ws)
        restore()
        graph.launch(stream)
        torch.cuda.synchronize()
        graph_ms, graph_loss = timed(lambda: graph.launch(stream), steps)
        del graph
    losses = np.concatenate([warm_losses, eager_loss] + ([graph_loss] if graph_loss is not None else []))
    if not np.isfinite(losses).all():
        raise RuntimeError(f"{wl.name}: non-finite loss in a warm-up or timed step: {losses.tolist()}")
    use_g = graph_ms is not None and statistics.fmean(graph_ms) < statistics.fmean(eager_ms)
    ms = graph_ms if use_g else eager_ms

    # the same steps with an event pair around every launch (sgd_profile): the per-kernel durations of
    # the roofline and the kernel table.  The events cost a few microseconds per launch, so the
    # throughput is not taken from this pass.
    net.profile(True)
    prof_ms, _ = timed(eager, steps)
    net.profile(False)
    prof_recs = net.profile_read()
    kern = kernel_totals(prof_recs)
    # the same with the dedw products on the caller's stream (no overlap): each kernel has the GPU to
    # itself, so its event time is its own duration; eq. (4) models this serial sum
    reps = max(3, min(steps, 10))
    net.set_overlap(False)
    restore()
    eager()
    net.profile(True)
    iso_ms, _ = timed(eager, reps)
    net.profile(False)
    iso_recs = net.profile_read()
    net.set_overlap(None)
    kern_iso = kernel_totals(iso_recs)
    # the unfused pair for reference: gradient into the GradBuf, then the standalone apply kernel
    gb = S.GradBuf(n, device=dev)
    restore()
    net.compute_gradient_into(Wd, Xd, yd, gb, loss, ws, stream)
    S.apply_update(Wd, gb, state, rule, stream)
    torch.cuda.synchronize()
    unf = []
    upd = []
    for _ in range(reps):
        u0, u1, u2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        restore()
        u0.record(stream)
        net.compute_gradient_into(Wd, Xd, yd, gb, loss, ws, stream)
        u1.record(stream)
        S.apply_update(Wd, gb, state, rule, stream)
        u2.record(stream)
        keep_loss()
        torch.cuda.synchronize()
        unf.append(u0.elapsed_time(u2))
        upd.append(u1.elapsed_time(u2))
    upd_b = {"plain": 12.0, "momentum": 20.0, "adagrad": 20.0}[wl.rule] * n
    final = hist[:n_hist[0]].cpu().numpy()
    if not np.isfinite(final).all():
        raise RuntimeError(f"{wl.name}: non-finite loss in a profiled step")
    del ws, gb
    torch.cuda.empty_cache()
    return dict(ms=ms, eager_ms=eager_ms, graph_ms=graph_ms, graph=use_g, overlap=overlap, prof_ms=prof_ms, iso_ms=iso_ms,
                kern=kern, kern_iso=kern_iso, iso_recs=iso_recs, prof_recs=prof_recs, n_params=n, losses=losses,
                update={"kernel": f"apply_{wl.rule}", "avg_us": 1e3 * statistics.fmean(upd),
                        "GB/s": upd_b / (statistics.fmean(upd) / 1e3) / 1e9},
                unfused_ms=unf)


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


def is_product(name):
    return name.startswith(("gemm_dma_", "gemm_staged_", "gemm_conv_", "gemm_dw_short_", "gemm_skinny_",
                            "gemm_smallk_"))


def kernel_table(kern, total_ms, top=10):
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
    return rows[:top]


def dominant(kern):
    """The kernel with the largest total time: a matrix product if any product is within a factor
    of two of the largest kernel, else the largest kernel."""
    top = max(kern, key=lambda k: kern[k]["ms"])
    prods = {k: v for k, v in kern.items() if is_product(k)}
    if prods:
        p = max(prods, key=lambda k: prods[k]["ms"])
        if 2 * prods[p]["ms"] >= kern[top]["ms"]:
            return p
    return top


def roofline_of(kern, name, steps):
    d = kern[name]
    if is_product(name) or (d["flops"] and d["flop_bound"] == d["launches"]):
        ach = d["flops"] / (d["ms"] / 1e3) / 1e12
        out = {"bound": "mfma", "kernel": name, "achieved": ach, "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
               "frac": ach / PEAK_FP32_TFLOPS, "flops_per_launch": d["flops"] / d["launches"]}
    else:
        ach = d["bytes"] / (d["ms"] / 1e3) / 1e9
        out = {"bound": "hbm", "kernel": name, "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
               "frac": ach / PEAK_HBM_GBS, "bytes_per_launch": d["bytes"] / d["launches"]}
    out.update({"launches": d["launches"], "launches_per_step": d["launches"] / steps,
                "avg_launch_us": 1e3 * d["ms"] / d["launches"]})
    return out


def per_product(recs, steps):
    """The last recorded step's launches grouped by matrix product (main kernel + stream-K fixup +
    split-K reduce) and other kernels, in launch order: [phase, layer, kernels, m, n, k, us, TFLOP/s or
    GB/s].  The last step, because the first one after an idle GPU runs slower."""
    per = max(1, len(recs) // steps)
    out = []
    by = {}
    for (name, layer, phase, ms, flops, nbytes, shape) in recs[len(recs) - per:]:
        m, n, k, pid = shape
        if pid < 0:
            out.append([phase, layer, name, 0, 0, 0, round(1e3 * ms, 1), round(nbytes / (ms / 1e3) / 1e9, 1)])
            continue
        if pid not in by:
            by[pid] = [phase, layer, name, m, n, k, 0.0, 0.0]
            out.append(by[pid])
        e = by[pid]
        if name != e[2] and name not in e[2].split("+"):
            e[2] += "+" + name
        e[6] += 1e3 * ms
        e[7] += flops if is_product(name) else 0.0
    for e in out:
        if e[3]:
            e[7] = round(e[7] / (e[6] / 1e6) / 1e12, 1)
            e[6] = round(e[6], 1)
    return out


def load_timing_fit():
    path = os.path.join(ROOT, "profiles", "timing_model_fit.json")
    if not os.path.exists(path):
        return None
    return json.load(open(path))


def eq4_record(fit, iso_recs, reps, iso_step_ms, step_ms):
    """Eq. (4) of the SPRINT report with the committed eq. (6) / CUDA-kernel fit, for the products and
    kernels this step launches, against the measured serial (no-overlap) step and the timed step."""
    if fit is None:
        return {"pred_ms": None, "note": "no committed timing-model fit (profiles/timing_model_fit.json)"}
    from sgd_cnns_amd import timing_model as TM
    per = max(1, len(iso_recs) // reps)
    recs = iso_recs[:per]
    try:
        p = TM.predict_step(recs, fit["alphas"], {k: tuple(v) for k, v in fit["kernel_models"].items()})
    except KeyError as e:
        return {"pred_ms": None, "note": f"fit does not cover this step: {e}"}
    return {"pred_ms": p["pred"], "sgemm_pred_ms": p["sgemm_pred"], "cuda_pred_ms": p["cuda_pred"],
            "kernels_sum_ms": p["meas"], "no_overlap_step_ms": iso_step_ms, "timed_step_ms": step_ms,
            "err_vs_no_overlap": (p["pred"] - iso_step_ms) / iso_step_ms,
            "err_vs_timed_step": (p["pred"] - step_ms) / step_ms,
            "fit": "profiles/timing_model_fit.json (eq. 6 per kernel family and form, eq. 5-form CUDA kernels)"}


def cpu_baseline_step(wl, sample, min_seconds=2.0):
    """The CPU oracle on a bounded sample: the gradient of `sample` images (repeated until about
    min_seconds have passed when the sample is small) scaled per image to the full batch, plus one
    accumulate + apply over all parameters."""
    import numpy as np

    import oracle as O
    import workloads

    X, y, W = workloads.make_inputs(wl)
    net = O.OracleNet(wl.chw, wl.layers)
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    reps = 0
    t0 = time.perf_counter()
    while True:
        net.gradient(W, X[:sample], y[:sample])
        reps += 1
        if time.perf_counter() - t0 >= min_seconds or reps >= 1000:
            break
    t_grad = (time.perf_counter() - t0) / reps
    _, g = net.gradient(W, X[:sample], y[:sample])
    gb = O.GradBuf(W.size)
    state = np.zeros_like(W) if wl.rule != "adagrad" else np.full_like(W, 0.1)
    t0 = time.perf_counter()
    gb.accumulate(g)
    O.apply_rule(wl.rule, W, state, gb.data, wl.eta, wl.mu, wl.eps)
    t_upd = time.perf_counter() - t0
    t_step = t_grad * wl.batch / sample + t_upd
    return {"value": wl.batch / t_step, "unit": "images/s", "cores": cores, "cpu_model": cpu_model(),
            "kind": "oracle", "ms_per_step": 1e3 * t_step,
            "sample": (f"gradient of the first {sample} of {wl.batch} images ({1e3 * t_grad:.1f} ms, mean of {reps}) "
                       f"scaled per image to the full batch, plus one accumulate+apply over all {W.size} "
                       f"parameters ({1e3 * t_upd:.1f} ms)")}


def ps_bench(steps=100, reps=20):
    """Parameter-server apply (config 5): 138,357,544 parameters, K = 8 gradient buffers from the
    seeded pool of 16 (step s folds buffers 8s .. 8s+7 mod 16), left-folded + Adagrad in one pass,
    one event pair per step.  Beside it, in the same run: the unfused chain (copy + 7 adds into a
    GradBuf, then the standalone apply: 112 B per parameter) and plain streaming kernels with the
    apply's read and write streams (sgd_stream_ref), the memory-traffic ceiling of that mix."""
    import numpy as np
    import torch

    import sgd_cnns_amd as S
    import workloads

    ps = workloads.PS_APPLY
    n, k = ps["n"], ps["k"]
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    pool_h = workloads.ps_pool(ps, threads=min(16, len(os.sched_getaffinity(0))))
    bufs = [torch.from_numpy(g).to(dev) for g in pool_h]
    del pool_h
    W0 = torch.from_numpy(workloads.normal(ps["seed"], 2, n)).to(dev)
    say(f"ps_adagrad: pool of {len(bufs)} seeded buffers ready in {time.perf_counter() - t0:.1f} s")
    W = W0.clone()
    A = torch.full((n,), ps["acc0"], device=dev)
    rule = S.Rule("adagrad", ps["eta"], 0.0, ps["eps"])

    def events(count):
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(count)]

    def fused(s):
        S.apply_fused(W, A, [bufs[i] for i in workloads.ps_step_buffers(s, k, len(bufs))], rule, stream)

    fused(0)
    W.copy_(W0)
    A.fill_(ps["acc0"])
    torch.cuda.synchronize()
    evs = events(steps)
    for s, (e0, e1) in enumerate(evs):
        e0.record(stream)
        fused(s)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    finite = bool(torch.isfinite(W).all().item()) and bool(torch.isfinite(A).all().item())
    if not finite:
        raise RuntimeError("ps_adagrad: non-finite weights after 100 steps")
    nbytes = (k + 4) * 4.0 * n
    st = _stats(ms)
    # unfused chain: GradBuf <- g_0 (copy), += g_1 .. g_7, then the standalone Adagrad apply
    gb = S.GradBuf(n, device=dev)

    def unfused(s):
        for i in workloads.ps_step_buffers(s, k, len(bufs)):
            S.accumulate_grad(gb, bufs[i], stream)
        S.apply_update(W, gb, A, rule, stream)

    unfused(0)
    torch.cuda.synchronize()
    evs = events(reps)
    for s, (e0, e1) in enumerate(evs):
        e0.record(stream)
        unfused(s)
        e1.record(stream)
    torch.cuda.synchronize()
    ums = [a.elapsed_time(b) for a, b in evs]
    ubytes = (8.0 + 12.0 * (k - 1) + 20.0) * n
    # the plain streaming references with the same streams (on the same buffers)
    ref = {}
    for name, outs, ins, groups in (("copy_1r1w", [gb.data], [bufs[0]], 1),
                                    ("read_10r", [], bufs[:8] + [W, A], 1),
                                    ("stream_10r2w_g1", [W, A], bufs[:8] + [W, A], 1),
                                    ("stream_10r2w_g4", [W, A], bufs[:8] + [W, A], 4)):
        S.stream_ref(outs, ins, groups, stream)
        torch.cuda.synchronize()
        evs = events(reps)
        for s, (e0, e1) in enumerate(evs):
            sh = [bufs[(j + 8 * s) % len(bufs)] for j in range(len(ins) - 2)] + ins[-2:] if len(ins) == 10 else ins
            e0.record(stream)
            S.stream_ref(outs, sh, groups, stream)
            e1.record(stream)
        torch.cuda.synchronize()
        rms = statistics.fmean(a.elapsed_time(b) for a, b in evs)
        rb = 4.0 * (len(ins) + len(outs)) * n
        ref[name] = {"reads": len(ins), "writes": len(outs), "floats_per_thread": 4 * groups, "avg_us": 1e3 * rms,
                     "GB/s": rb / rms / 1e6, "frac_hbm_peak": rb / rms / 1e6 / PEAK_HBM_GBS}
    ceiling = max(ref["stream_10r2w_g1"]["GB/s"], ref["stream_10r2w_g4"]["GB/s"])
    gbs = nbytes / st["mean"] / 1e6
    traffic, source = measured_traffic("apply_kernel<2, 8>", "ps_adagrad")
    del bufs, gb
    torch.cuda.empty_cache()
    return {"workload": (f"ps_adagrad: {n} parameters, K={k} fresh seeded gradient buffers N(0, 1e-3^2) per step "
                         f"(pool {ps['pool']}), left-folded + Adagrad eta={ps['eta']} eps={ps['eps']} A0={ps['acc0']}, "
                         f"{steps} steps"),
            "metric": "update GB/s (48 B per parameter: 8 gradients + W + A read, W + A written)",
            "steps": steps, "ms_per_step": st["mean"], "median_ms_per_step": st["median"],
            "min_ms_per_step": st["min"], "max_ms_per_step": st["max"],
            "bytes_per_step": nbytes, "GB/s": gbs, "frac_of_hbm_peak": gbs / PEAK_HBM_GBS,
            "roofline": {"bound": "hbm", "kernel": "apply_kernel<2, 8> (sgd_apply_fused, Adagrad, K = 8)",
                         "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                         "bytes_per_launch": nbytes, "avg_launch_us": 1e3 * st["mean"], "traffic": traffic,
                         "traffic_source": source if traffic is not None else f"null: {source}"},
            "frac_of_stream_10r2w_ceiling": gbs / ceiling,
            "stream_ref": ref,
            "unfused": {"chain": "accumulate copy + 7 accumulate adds + apply_update (Adagrad)",
                        "bytes_per_param": ubytes / n, "ms_per_step": statistics.fmean(ums),
                        "GB/s": ubytes / statistics.fmean(ums) / 1e6,
                        "frac_hbm_peak": ubytes / statistics.fmean(ums) / 1e6 / PEAK_HBM_GBS},
            "weights_finite_after_100_steps": finite}


def cpu_baseline_ps(frac=16):
    """The oracle's 8-buffer fold + Adagrad on 1/frac of the parameters, scaled to all of them."""
    import numpy as np

    import oracle as O
    import workloads

    ps = workloads.PS_APPLY
    n, k = ps["n"], ps["k"]
    m = n // frac
    gs = [workloads.normal(ps["seed"], 100 + j, m, ps["grad_std"]) for j in range(k)]
    W = workloads.normal(ps["seed"], 2, m)
    A = np.full(m, ps["acc0"], np.float32)
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    gb = O.GradBuf(m)
    for g in gs:
        gb.accumulate(g)
    O.apply_adagrad(W, A, gb.data, ps["eta"], ps["eps"])
    t = (time.perf_counter() - t0) * n / m
    return {"value": 48.0 * n / t / 1e9, "unit": "GB/s", "ms_per_step": 1e3 * t, "cores": cores,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"one step (8-buffer fold + Adagrad) on the first {m} of {n} parameters, scaled to all"}


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
    # the fit itself, for the step benchmark's per-workload eq. (4) prediction
    import hashlib
    src = b"".join(open(os.path.join(ROOT, "sgd_cnns_amd", "csrc", f), "rb").read()
                   for f in ("gemm.hip", "layers.hip", "update.hip"))
    fit = {"command": f"python bench.py --timing-model {os.path.relpath(out_path, ROOT)}",
           "alphas": {fam: {f: [float(v) for v in alphas[fam][f]] for f in alphas[fam]} for fam in alphas},
           "eq6_terms": list(TM.EQ6_TERMS),
           "kernel_models": {k: [float(a), float(b)] for k, (a, b) in kmodels.items()},
           "source_sha256(gemm.hip+layers.hip+update.hip)": hashlib.sha256(src).hexdigest()}
    with open(os.path.splitext(out_path)[0] + ".json", "w") as fh:
        json.dump(fit, fh, indent=1)
    print(text)


def vendor_compare(out_path, reps=15):
    """Context for the rooflines: every distinct matrix product of each workload's step (its form and
    m, n, k, as the step profiler records them, with its count per step), timed as one plain sgd_gemm
    launch (the same main loop and schedule as the step's product, with a plain store in place of the
    fused epilogue and the explicit operand in place of a convolution gather) and as torch.mm, the
    vendor's fp32 GEMM (TF32 off), on the same operands.  Median of `reps` event-bracketed launches
    each; both results are compared (max |difference| / max |result|)."""
    import numpy as np
    import torch

    import sgd_cnns_amd as S
    import workloads
    from sgd_cnns_amd import timing_model as TM

    torch.backends.cuda.matmul.allow_tf32 = False
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()

    def median_us(fn):
        fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda._sleep(100_000 * reps)  # queue the launches ahead of the GPU
        for r in range(reps):
            ev[r].record(stream)
            fn()
        ev[reps].record(stream)
        ev[reps].synchronize()
        return 1e3 * sorted(ev[r].elapsed_time(ev[r + 1]) for r in range(reps))[reps // 2]

    lines = ["# Step products: sgd_gemm against the vendor fp32 GEMM (torch.mm)", "",
             "Command (repository root, one MI355X): `python bench.py --vendor-compare OUT.md`", "",
             "Every distinct product of each workload's step (form, m, n, k as the step profiler records "
             "them, with a weight gradient's n taken without the bias's implicit ones column; count = "
             "launches per step), timed as one plain sgd_gemm launch (the step product's "
             "main loop and schedule, with a plain store in place of the fused epilogue and the explicit "
             "operand in place of a convolution gather) and as torch.mm on the same operands (fp32, TF32 "
             f"off).  Median of {reps} event-bracketed launches.  `diff` = max |ours - torch| / max |torch|.", ""]
    summary = {}
    for name in STEP_WORKLOADS:
        wl = workloads.WORKLOADS[name]
        say(f"vendor compare: {name}")
        X, y, W = workloads.make_inputs(wl)
        net = S.Net((wl.batch,) + tuple(wl.chw), wl.layers)
        net.set_overlap(False)
        Wd, Xd, yd = (torch.from_numpy(a).to(dev) for a in (W, X, y))
        grad = torch.empty(net.param_count(), device=dev)
        loss = torch.empty(1, device=dev)
        ws = net.workspace(dev)
        net.compute_gradient(Wd, Xd, yd, grad, loss, ws, stream)
        net.profile(True)
        net.compute_gradient(Wd, Xd, yd, grad, loss, ws, stream)
        net.profile(False)
        torch.cuda.synchronize()
        prods, _ = TM.products_of(net.profile_read())
        del ws, grad, Wd, Xd
        count = {}
        for pr in prods:
            if pr["form"] in TM.FORMS:
                # A weight gradient's recorded n counts the bias's implicit ones column, which the
                # stored operand does not hold: both sides take the stored width.
                n = pr["n"] - 1 if pr["form"] == "tn" and pr["n"] % 4 == 1 else pr["n"]
                key = (pr["form"], pr["m"], n, pr["k"])
                count[key] = count.get(key, 0) + 1
        lines += [f"## {name}", "", "| form | m | n | k | per step | ours µs | torch.mm µs | ours / torch | ours TFLOP/s | "
                  "torch TFLOP/s | diff |", "|---|---|---|---|---|---|---|---|---|---|---|"]
        tot_o = tot_t = 0.0
        for (form, m, n, k), c in sorted(count.items(), key=lambda kv: -2.0 * kv[0][1] * kv[0][2] * kv[0][3] * kv[1]):
            a_t, b_t = TM.FORMS[form]
            A = torch.randn((k, m) if a_t else (m, k), device=dev)
            B = torch.randn((k, n) if b_t else (n, k), device=dev)
            Co = torch.empty(m, n, device=dev)
            Ct = torch.empty(m, n, device=dev)
            opA = A.t() if a_t else A
            opB = B if b_t else B.t()
            wsz = S.gemm_workspace_bytes(m, n, k, a_t, b_t)
            gws = torch.empty(max(wsz, 256) // 4 + 64, device=dev)
            t_o = median_us(lambda: S.gemm(A, B, Co, a_t, b_t, gws, stream))
            t_t = median_us(lambda: torch.mm(opA, opB, out=Ct))
            torch.cuda.synchronize()
            diff = float((Co - Ct).abs().max() / Ct.abs().max().clamp_min(1e-30))
            fl = 2.0 * m * n * k
            tot_o += c * t_o
            tot_t += c * t_t
            lines.append(f"| {form} | {m} | {n} | {k} | {c} | {t_o:.1f} | {t_t:.1f} | {t_o / t_t:.2f} | "
                         f"{fl / t_o / 1e6:.1f} | {fl / t_t / 1e6:.1f} | {diff:.1e} |")
            del A, B, Co, Ct, gws
        torch.cuda.empty_cache()
        lines += ["", f"Sum over one step's products: ours {tot_o / 1e3:.3f} ms, torch.mm {tot_t / 1e3:.3f} ms "
                  f"(ratio {tot_o / tot_t:.2f}).", ""]
        summary[name] = {"ours_ms": tot_o / 1e3, "torch_ms": tot_t / 1e3}
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({"vendor_compare": summary}))


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
            diverged = None
            if not finite:
                # where it diverged: shorter runs from the same start, doubling the steps per worker, until
                # the weights are non-finite (the schedule is asynchronous, so this brackets the update)
                last_ok = 0
                it = 1
                while it <= iters:
                    Wd.copy_(torch.from_numpy(W0))
                    V.zero_()
                    st2, _ = S.sprint_run(net, S.SprintConfig(workers=workers, iters=it), Wd, V, rule, Xd, yd,
                                          n_batches, ws)
                    torch.cuda.synchronize()
                    if not bool(torch.isfinite(Wd).all().item()):
                        diverged = (last_ok, st2["updates"], it)
                        break
                    last_ok = st2["updates"]
                    it *= 2
            rows.append(dict(sub=sub, workers=workers, iters=iters, single_ms=single_ms, finite=finite,
                             diverged=diverged, **st))
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
    div = [r for r in rows if not r["finite"]]
    if div:
        L += ["", "Rows whose weights were not finite at the end, re-run from the same weights with 1, 2, 4, ... "
                  "steps per worker until they were not finite (an asynchronous schedule, so this brackets the "
                  "update at which the run diverged; each update applies the sum of the buffers it takes, so "
                  "more workers put more summed samples into one update):", "",
              "| N_Subbatch | workers | finite after (updates) | non-finite after (updates) | steps per worker |",
              "|---|---|---|---|---|"]
        for r in div:
            d = r["diverged"]
            if d is None:
                L.append(f"| {r['sub']} | {r['workers']} | - | only in the full run | - |")
            else:
                L.append(f"| {r['sub']} | {r['workers']} | {d[0]} | {d[1]} | {d[2]} |")
    text = "\n".join(L) + "\n"
    with open(out_path, "w") as fh:
        fh.write(text)
    print(text)




# --------------------------------------------------------------- rocprofv3 summaries ----
_EM_NAMES = {"0": "generic", "1": "store", "2": "bias", "3": "mask", "4": "dw", "5": "update"}


def bench_kernel_name(instance):
    """The name the library's profiler gives a launch of this kernel instance (as printed by
    rocprofv3, demangled), or the instance itself for kernels outside the products."""
    import re
    ms = re.search(r"dw_short<(\d+), \d+, -?\d+>", instance)
    if ms:
        return f"gemm_dw_short_k{2 * int(ms.group(1))}"
    if "dw_long_kernel" in instance:
        return "gemm_staged_long_tn"
    if "skinny_nt_kernel" in instance:
        return "gemm_skinny_nt"
    if "smallk_nn_kernel" in instance:
        return "gemm_smallk_nn"
    m = re.search(r"gemm_(dma|staged)<(\d+), (\d+), (?:(\d+), )?(true|false), (true|false), (\d+)"
                  r"(?:, (true|false), (true|false))?(?:, (?:true|false))?(?:, \d+)?>", instance)
    if not m:
        return short_instance(instance).split("<")[0]
    fam, bm, bn, _bk, at, bt, em, ga, gb = m.groups()
    if ga == "true":
        return f"gemm_conv_{'fwd' if em == '2' else 'dx'}_{bm}x{bn}"
    if gb == "true":
        return f"gemm_conv_dw_{bm}x{bn}"
    form = {("false", "false"): "nt", ("true", "true"): "tn", ("false", "true"): "nn", ("true", "false"): "tt"}[(at, bt)]
    return f"gemm_{fam}_{bm}x{bn}_{form}"


def short_instance(name):
    """A demangled kernel name without its return type, namespaces and parameter list."""
    n = name.replace("(anonymous namespace)::", "")
    if n.startswith("void "):
        n = n[5:]
    n = n.split("(")[0]
    for ns in ("sgd::", "at::native::"):
        n = n.replace(ns, "")
    return n.strip()


def _csv_rows(directory, suffix):
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *{suffix} under {directory}")
    return rows


def summarize_stats(directory, out_md, title, command):
    """Markdown table of a rocprofv3 --kernel-trace --stats run (its *kernel_stats.csv)."""
    rows = _csv_rows(directory, "kernel_stats.csv")
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    L = [f"# rocprofv3 kernel statistics — {title}", "", "Command (repository root, one MI355X):", "", "```",
         command, "```", "", "Every dispatch of the run (warm-up, timed steps, graph replays, the event-bracketed "
         "and no-overlap passes, the unfused reference).  The library's own name for each instance is in "
         "parentheses.", "", "| kernel | calls | avg µs | total ms | % |", "|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"]))[:40]:
        inst = short_instance(r["Name"])
        L.append(f"| `{inst}` ({bench_kernel_name(r['Name'])}) | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                 f"{float(r['TotalDurationNs']) / 1e6:.2f} | {100 * float(r['TotalDurationNs']) / total:.1f} |")
    open(out_md, "w").write("\n".join(L) + "\n")
    print("\n".join(L))


def _counter_table(directory, counter):
    """{instance: [per-dispatch values]} of one counter, and the calibration copy's value (the largest
    copy-kernel dispatch)."""
    per = {}
    copy = 0.0
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        name = r["Kernel_Name"]
        v = float(r["Counter_Value"])
        if "copyBuffer" in name or "copy_kernel" in name:
            copy = max(copy, v)
        per.setdefault(name, []).append(v)
    return per, copy


def summarize_traffic(fetch_dir, write_dir, workload, calib_mib, out_md, out_json, command):
    """HBM bytes per dispatch from a FETCH_SIZE pass and a WRITE_SIZE pass (KiB per dispatch), each
    scaled so the calibration copy of calib_mib MiB counts its bytes once, per kernel instance; merged
    into out_json under the workload (with a hash of the kernel sources)."""
    import hashlib
    f, fcopy = _counter_table(fetch_dir, "FETCH_SIZE")
    w, wcopy = _counter_table(write_dir, "WRITE_SIZE")
    nbytes = calib_mib * 2 ** 20
    fs = nbytes / (fcopy * 1024) if fcopy else 1.0
    ws = nbytes / (wcopy * 1024) if wcopy else 1.0
    kern = {}
    for inst, vals in f.items():
        if "sgd::" not in inst:   # the library's kernels only (not the calibration copy or torch's own)
            continue
        name = bench_kernel_name(inst) if ("gemm_dma<" in inst or "gemm_staged<" in inst) else short_instance(inst)
        fb = 1024 * fs * statistics.fmean(vals)
        wb = 1024 * ws * statistics.fmean(w.get(inst, [0.0]))
        rec = {"instance": short_instance(inst), "dispatches": len(vals), "fetch_bytes": fb, "write_bytes": wb,
               "traffic_bytes": fb + wb}
        if name not in kern or kern[name]["dispatches"] < len(vals):
            kern[name] = rec
    entry = {"workload": workload, TRAFFIC_KEY: kernel_code_sha256(),
             "fetch_scale": fs, "write_scale": ws,
             "calibration": f"one {calib_mib} MiB device copy in the same runs", "command": command, "kernels": kern}
    old = json.load(open(out_json)) if os.path.exists(out_json) else []
    old = old if isinstance(old, list) else [old]
    old = [e for e in old if e.get("workload") != workload] + [entry]
    json.dump(old, open(out_json, "w"), indent=1)
    L = [f"# HBM traffic per launch — {workload} (FETCH_SIZE / WRITE_SIZE)", "",
         "Commands (repository root, one MI355X; two separate counter passes, then this summary):", "", "```",
         command, "```", "",
         f"Calibration: the same runs copy {calib_mib} MiB once; FETCH_SIZE is scaled by {fs:.3f} and WRITE_SIZE by "
         f"{ws:.3f} so that copy counts its bytes once.  FETCH_SIZE counts L2-to-fabric reads, so Infinity Cache "
         "(MALL) hits are included.  Averages over every dispatch of the instance.", "",
         "| kernel (instance) | dispatches | fetch MB/launch | write MB/launch | traffic MB/launch |",
         "|---|---|---|---|---|"]
    for name, r in sorted(kern.items(), key=lambda kv: -kv[1]["traffic_bytes"] * kv[1]["dispatches"])[:25]:
        L.append(f"| `{name}` (`{r['instance']}`) | {r['dispatches']} | {r['fetch_bytes'] / 1e6:.1f} | "
                 f"{r['write_bytes'] / 1e6:.1f} | {r['traffic_bytes'] / 1e6:.1f} |")
    open(out_md, "w").write("\n".join(L) + "\n")
    print("\n".join(L))


def summarize_mfma(directory, out_md, title, command, min_us=50.0):
    """Matrix-core busy fraction and clock per GEMM instance from GRBM_GUI_ACTIVE and
    SQ_VALU_MFMA_BUSY_CYCLES (one pass)."""
    rows = _csv_rows(directory, "counter_collection.csv")
    by = {}
    for r in rows:
        key = (r["Kernel_Name"], r.get("Dispatch_Id") or r.get("Correlation_Id"))
        d = by.setdefault(key, {"dur": (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) / 1e3})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    agg = {}
    for (name, _), d in by.items():
        if "GRBM_GUI_ACTIVE" not in d or "SQ_VALU_MFMA_BUSY_CYCLES" not in d or d["dur"] < min_us:
            continue
        a = agg.setdefault(name, {"n": 0, "dur": 0.0, "clk": 0.0, "busy": 0.0})
        a["n"] += 1
        a["dur"] += d["dur"]
        gui = d["GRBM_GUI_ACTIVE"] / 8.0          # the counter sums the 8 XCDs
        a["clk"] += gui / d["dur"]               # cycles per microsecond = MHz
        a["busy"] += d["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * 1024.0)
    L = [f"# Matrix-core busy fraction and clock — {title}", "", "Command (repository root, one MI355X):", "", "```",
         command, "```", "",
         "Per GEMM instance, averaged over its dispatches: duration from the counter run's timestamps; clock = "
         "GRBM_GUI_ACTIVE / 8 (the counter sums the 8 XCDs) over that duration; matrix cores busy = "
         "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs).  Dispatches under "
         f"{min_us:.0f} µs are left out (the timestamps do not bracket them closely).", "",
         "| kernel | dispatches | avg µs | MHz | MFMA busy % |", "|---|---|---|---|---|"]
    for name, a in sorted(agg.items(), key=lambda kv: -kv[1]["dur"]):
        if not name.startswith(("void sgd", "sgd")) and "gemm" not in name:
            continue
        L.append(f"| `{short_instance(name)}` ({bench_kernel_name(name)}) | {a['n']} | {a['dur'] / a['n']:.1f} | "
                 f"{a['clk'] / a['n']:.0f} | {100 * a['busy'] / a['n']:.1f} |")
    open(out_md, "w").write("\n".join(L) + "\n")
    print("\n".join(L))


def step_record(wl, r, steps, fit, cpu):
    """The JSON record of one step workload."""
    ms = r["ms"]
    st = _stats(ms)
    kern, kern_iso = r["kern"], r["kern_iso"]
    dom = dominant(kern)
    prof_total = sum(r["prof_ms"])
    roof = roofline_of(kern, dom, steps)
    traffic, source = measured_traffic(dom, wl.name)
    roof["traffic"] = traffic
    roof["traffic_source"] = source if traffic is not None else f"null: {source}"
    roof["ms_per_step_profiled"] = prof_total / steps
    roof["note"] = ("durations from HIP events around every launch over the same steps, right after the timed "
                    "steps (the events cost a few microseconds per launch, so value is timed without them); with "
                    "the dedw products on a second stream, a launch's duration is its time while it shares the GPU")
    iso = None
    if dom in kern_iso:
        iso = roofline_of(kern_iso, dom, len(r["iso_ms"]))
        iso["ms_per_step_no_overlap"] = statistics.fmean(r["iso_ms"])
    gflops = sum(v["flops"] for k, v in kern.items() if is_product(k)) / steps
    rec = {
        "workload": describe(wl), "name": wl.name, "batch": wl.batch, "params": r["n_params"], "update": wl.rule,
        "images_per_s": wl.batch / (st["mean"] / 1e3), "ms_per_step": st["mean"],
        "median_ms_per_step": st["median"], "min_ms_per_step": st["min"], "max_ms_per_step": st["max"],
        "steps": steps, "timed_as": "HIP graph replay of sgd_train_step" if r["graph"] else "sgd_train_step per call",
        "dedw_side_stream": r["overlap"],
        "eager_ms_per_step": statistics.fmean(r["eager_ms"]),
        "eager_median_ms_per_step": statistics.median(r["eager_ms"]),
        "graph_ms_per_step": None if r["graph_ms"] is None else statistics.fmean(r["graph_ms"]),
        "graph_median_ms_per_step": None if r["graph_ms"] is None else statistics.median(r["graph_ms"]),
        "no_overlap_ms_per_step": statistics.fmean(r["iso_ms"]),
        "unfused_ms_per_step": statistics.fmean(r["unfused_ms"]),
        "loss_first": float(r["losses"][0]), "loss_last": float(r["losses"][-1]),
        "losses_finite": True,
        "gemm_step_util": {"gemm_gflop_per_step": gflops / 1e9,
                           "TFLOP/s": gflops / (st["mean"] / 1e3) / 1e12,
                           "frac_fp32_peak": gflops / (st["mean"] / 1e3) / 1e12 / PEAK_FP32_TFLOPS,
                           "note": "sum of 2mnk over the step's products / ms_per_step"},
        "roofline": roof, "roofline_isolated": iso,
        "kernels": kernel_table(kern, prof_total), "kernels_isolated": kernel_table(kern_iso, sum(r["iso_ms"])),
        "update_GB/s": {"kernel": r["update"]["kernel"], "GB/s": r["update"]["GB/s"],
                        "frac_hbm_peak": r["update"]["GB/s"] / PEAK_HBM_GBS, "avg_us": r["update"]["avg_us"],
                        "note": "standalone apply after gradient-into-GradBuf (the unfused pair); the timed step "
                                "applies the rule in the dedw epilogues"},
        "eq4": eq4_record(fit, r["iso_recs"], len(r["iso_ms"]), statistics.fmean(r["iso_ms"]), st["mean"]),
        "products_fields": ["phase (0 fwd, 1 bwd)", "layer", "kernels", "m", "n", "k", "us",
                            "TFLOP/s (products) or GB/s (others)"],
        "products": per_product(r["prof_recs"], steps),
        "products_isolated": per_product(r["iso_recs"], len(r["iso_ms"])),
        "cpu_baseline": cpu,
    }
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all", choices=["all", "ps_adagrad"] + STEP_WORKLOADS,
                    help="one workload only (the headline fields then describe it), or all five")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only (no HIP-graph replays)")
    ap.add_argument("--no-ps-apply", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (a known-size kernel for counter scaling)")
    ap.add_argument("--timing-model", metavar="OUT_MD", default=None,
                    help="refit the SPRINT timing model (eqs. 4-6) and write its report (and a .json of the fit "
                         "beside it) instead of the step bench")
    ap.add_argument("--timing-model-raw", metavar="PREFIX", default=None,
                    help="also save the timing model's raw grid times and step records under this prefix")
    ap.add_argument("--sprint", metavar="OUT_MD", default=None,
                    help="run SPRINT's asynchronous workers and updater (Algorithms 1 and 2) and write the report")
    ap.add_argument("--summarize", nargs="+", metavar="ARG", default=None,
                    help="summarize rocprofv3 output instead of running: 'stats DIR OUT.md TITLE', "
                         "'traffic FETCH_DIR WRITE_DIR WORKLOAD CALIB_MIB OUT.md OUT.json', 'mfma DIR OUT.md TITLE' "
                         "(with --summary-command giving the command text to record)")
    ap.add_argument("--summary-command", default="", help="the command(s) that produced the summarized output")
    ap.add_argument("--vendor-compare", metavar="OUT_MD", default=None,
                    help="time every distinct product of each workload's step on sgd_gemm and on torch.mm (the "
                         "vendor fp32 GEMM) and write the comparison instead of the step bench")
    args = ap.parse_args()
    if args.summarize:
        kind, rest = args.summarize[0], args.summarize[1:]
        if kind == "stats":
            summarize_stats(rest[0], rest[1], rest[2], args.summary_command)
        elif kind == "traffic":
            summarize_traffic(rest[0], rest[1], rest[2], int(rest[3]), rest[4], rest[5], args.summary_command)
        elif kind == "mfma":
            summarize_mfma(rest[0], rest[1], rest[2], args.summary_command)
        else:
            raise SystemExit(f"unknown summary kind {kind}")
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): this build runs the step on a "
              "single MI355X; the multi-GPU exchange is a design, not code", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    if args.sprint:
        sprint_report(args.sprint)
        return
    if args.timing_model:
        timing_model_report(args.timing_model, args.timing_model_raw)
        return
    if args.vendor_compare:
        vendor_compare(args.vendor_compare)
        return
    import workloads
    if args.copy_calibration_mib:
        import torch
        n = args.copy_calibration_mib * 2 ** 20 // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty(n, device="cuda")
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    names = STEP_WORKLOADS if args.workload == "all" else [w for w in STEP_WORKLOADS if w == args.workload]
    fit = load_timing_fit()
    cpu_sample = {"mlp5000": 64, "lenet5": 16, "vgg_cifar": 8, "vgg16": 1}
    configs = []
    t_start = time.perf_counter()
    for name in names:
        wl = workloads.WORKLOADS[name]
        say(f"{describe(wl)}; warmup {args.warmup}, steps {args.steps}")
        r = step_bench(wl, args.steps, args.warmup, use_graph=not args.no_graph)
        say(f"{name}: {statistics.fmean(r['ms']):.3f} ms/step ({'graph' if r['graph'] else 'eager'}), "
            f"losses {r['losses'][0]:.4g} .. {r['losses'][-1]:.4g}")
        cpu = None
        if not args.no_cpu_baseline:
            say(f"{name}: CPU oracle baseline on {cpu_sample[name]} images")
            cpu = cpu_baseline_step(wl, cpu_sample[name])
        configs.append(step_record(wl, r, args.steps, fit, cpu))
    ps = None
    if not args.no_ps_apply and args.workload in ("all", "ps_adagrad"):
        say("ps_adagrad: parameter-server apply, 100 steps")
        ps = ps_bench()
        if not args.no_cpu_baseline:
            say("ps_adagrad: CPU oracle baseline")
            ps["cpu_baseline"] = cpu_baseline_ps()
        ps["name"] = "ps_adagrad"
        configs.append(ps)
    say(f"all workloads done in {time.perf_counter() - t_start:.0f} s")
    head = next((c for c in configs if c["name"] == "mlp5000"), configs[0])
    if head["name"] == "ps_adagrad":
        out = {"metric": METRIC, "value": head["GB/s"], "unit": "GB/s", "n_gpus": 1, "steps": head["steps"],
               "warmup": 1, "ms_per_step": head["ms_per_step"], "median_ms_per_step": head["median_ms_per_step"],
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
               "data": "synthetic (seeded Philox gradient buffers and weights)",
               "config": {"workload": head["workload"]}, "roofline": head["roofline"],
               "cpu_baseline": head.get("cpu_baseline"), "configs": configs}
        print(json.dumps(out))
        return
    out = {
        "metric": METRIC,
        "value": head["images_per_s"],
        "unit": "images/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "median_ms_per_step": head["median_ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded Philox inputs of the workload's shape; He-normal random-init weights, restored "
                "before every step)",
        "config": {"workload": head["workload"], "global_batch": head["batch"], "params": head["params"],
                   "update": head["update"]},
        "roofline": head["roofline"],
        "roofline_isolated": head["roofline_isolated"],
        "cpu_baseline": head["cpu_baseline"],
        "gemm_step_util": head["gemm_step_util"],
        "timed_as": head["timed_as"],
        "loss_first": head["loss_first"],
        "loss_last": head["loss_last"],
        "configs": configs,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
