"""Seeded synthetic workloads: layer specs and input generators.

This module holds no arithmetic of the training step.  It only describes the
five workloads (layer lists, batch shapes, update rule parameters) and draws
their random inputs from a counter-based generator (numpy's Philox4x32-10, the
generator of Salmon et al., "Parallel random numbers: as easy as 1, 2, 3",
SC 2011), keyed by (workload seed, tensor id).  The same host arrays are given
to the HIP path and to the CPU oracle.

Tensor ids: 0 = images X, 1 = labels y, 2 = flat parameter vector W,
3 = optimizer state, 100 + j = gradient buffer j (parameter-server workload).

The pages train on MNIST, CIFAR-10 and ILSVRC2012 images; none of those
datasets is used.  Inputs here only share their shapes and simple value
distributions (uniform [0,1) pixels for the MNIST/CIFAR-like inputs, N(0,1)
for the normalised ones, labels uniform over the classes).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# A layer is a tuple: ("conv", out_channels, kernel, pad) | ("relu",) |
# ("pool", p) | ("fc", out) | ("softmax_ce",).


def _vgg_convs(widths, pool_after):
    layers = []
    for i, w in enumerate(widths):
        layers += [("conv", w, 3, 1), ("relu",)]
        if i in pool_after:
            layers.append(("pool", 2))
    return layers


LENET5 = [
    ("conv", 6, 5, 2), ("relu",), ("pool", 2),
    ("conv", 16, 5, 0), ("relu",), ("pool", 2),
    ("fc", 120), ("relu",), ("fc", 84), ("relu",), ("fc", 10), ("softmax_ce",),
]

MLP5000 = ([("fc", 5000), ("relu",)] * 5) + [("fc", 10), ("softmax_ce",)]

VGG_CIFAR = _vgg_convs([64, 64, 128, 128, 256, 256, 256, 512, 512, 512, 512, 512, 512],
                       {1, 3, 6, 9, 12}) + [("fc", 512), ("relu",), ("fc", 10), ("softmax_ce",)]

VGG16 = _vgg_convs([64, 64, 128, 128, 256, 256, 256, 512, 512, 512, 512, 512, 512],
                   {1, 3, 6, 9, 12}) + [("fc", 4096), ("relu",), ("fc", 4096), ("relu",),
                                        ("fc", 1000), ("softmax_ce",)]


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    chw: tuple            # (C, H, W) of one input image
    layers: list = field(default_factory=list)
    classes: int = 10
    x_dist: str = "uniform"   # "uniform" -> U[0,1), "normal" -> N(0,1)
    rule: str = "plain"       # plain | momentum | adagrad
    eta: float = 0.01
    mu: float = 0.0
    eps: float = 0.0

    def with_batch(self, batch: int) -> "Workload":
        d = dict(self.__dict__)
        d["batch"] = batch
        return Workload(**d)


WORKLOADS = {
    "lenet5": Workload("lenet5", 1, 16, (1, 28, 28), LENET5, 10, "uniform", "plain", 0.01),
    "mlp5000": Workload("mlp5000", 2, 512, (3072, 1, 1), MLP5000, 10, "uniform", "momentum",
                        0.01, 0.9),
    "vgg_cifar": Workload("vgg_cifar", 3, 128, (3, 32, 32), VGG_CIFAR, 10, "normal", "plain", 0.01),
    "vgg16": Workload("vgg16", 4, 32, (3, 224, 224), VGG16, 1000, "normal", "plain", 0.01),
}

# The parameter-server apply: a flat W of VGG-16's size, K gradient buffers
# summed in a fixed order, then per-parameter Adagrad.
PS_APPLY = dict(name="ps_adagrad", seed=5, n=138_357_544, k=8, grad_std=1e-3,
                eta=0.01, eps=1e-8, acc0=0.1, steps=100, pool=16)


def rng(seed: int, tensor_id: int) -> np.random.Generator:
    """Philox4x32-10 stream keyed by (seed, tensor id); platform independent."""
    key = (np.uint64(seed) << np.uint64(32)) | np.uint64(tensor_id)
    return np.random.Generator(np.random.Philox(key=int(key)))


def uniform01(seed, tensor_id, shape):
    """U[0,1) float32 with 24 random mantissa bits."""
    return rng(seed, tensor_id).random(size=shape, dtype=np.float32)


def normal(seed, tensor_id, shape, std=1.0):
    """N(0, std^2), drawn in float64 and rounded once to float32."""
    g = rng(seed, tensor_id).standard_normal(size=shape, dtype=np.float64)
    if std != 1.0:
        g *= std
    return g.astype(np.float32)


def labels(seed, tensor_id, n, classes):
    return rng(seed, tensor_id).integers(0, classes, size=n, dtype=np.int32)


def weighted_layers(chw, layers):
    """Walk a layer list; yield (index, kind, fan_in, n_weight, n_bias) per weighted layer.

    Shapes follow the valid-convolution recurrence generalised to zero
    padding P: H_out = H + 2P - c + 1, pooling divides by p, fc flattens.
    """
    c, h, w = chw
    flat = None
    out = []
    for i, L in enumerate(layers):
        if L[0] == "conv":
            co, k, p = L[1], L[2], L[3]
            fan_in = c * k * k
            out.append((i, "conv", fan_in, co * fan_in, co))
            c, h, w = co, h + 2 * p - k + 1, w + 2 * p - k + 1
        elif L[0] == "pool":
            h, w = h // L[1], w // L[1]
        elif L[0] == "fc":
            fan_in = c * h * w if flat is None else flat
            out.append((i, "fc", fan_in, L[1] * fan_in, L[1]))
            flat = L[1]
    return out


def he_normal_params(seed, chw, layers):
    """Flat parameter vector: per weighted layer, weight (std sqrt(2/fan_in)) then zero bias."""
    parts = []
    g = rng(seed, 2)
    for (_, _, fan_in, nw, nb) in weighted_layers(chw, layers):
        wv = g.standard_normal(size=nw, dtype=np.float64)
        wv *= math.sqrt(2.0 / fan_in)
        parts.append(wv.astype(np.float32))
        parts.append(np.zeros(nb, dtype=np.float32))
    return np.concatenate(parts)


def make_inputs(wl: Workload):
    """(X float32 NCHW, y int32, W float32 flat) for a workload."""
    shape = (wl.batch,) + tuple(wl.chw)
    if wl.x_dist == "uniform":
        X = uniform01(wl.seed, 0, shape)
    else:
        X = normal(wl.seed, 0, shape)
    y = labels(wl.seed, 1, wl.batch, wl.classes)
    W = he_normal_params(wl.seed, wl.chw, wl.layers)
    return X, y, W


def ps_gradient(seed, j, n, std):
    """Gradient buffer j of the parameter-server workload: N(0, std^2)."""
    return normal(seed, 100 + j, n, std)


def ps_pool(ps=None, count=None, threads=8):
    """The pool of `count` (default ps["pool"]) gradient buffers of the parameter-server workload,
    drawn in parallel host threads (each buffer is its own Philox stream, so the bits do not
    depend on the thread count)."""
    from concurrent.futures import ThreadPoolExecutor
    ps = PS_APPLY if ps is None else ps
    count = ps["pool"] if count is None else count
    with ThreadPoolExecutor(max(1, min(threads, count))) as ex:
        return list(ex.map(lambda j: ps_gradient(ps["seed"], j, ps["n"], ps["grad_std"]), range(count)))


def ps_step_buffers(step, k, pool):
    """Pool indices of the k fresh gradient buffers of step `step` (0-based), in fold order."""
    return [(k * step + i) % pool for i in range(k)]
