"""Seeded synthetic inputs for the MLP training step.

This module only draws random numbers; it holds none of the step's arithmetic
(no matmul, activation, loss or update), so the float64 oracle and the HIP
path can both consume its output without sharing any of the method's code.

Shapes and distributions follow the two-layer MNIST-style MLP of the
Meganeura README ("Example" section: x [32,784], one-hot labels [32,10],
w1 [784,128], w2 [128,10], no bias) and the wider/skinnier workloads built on
the same graph.  MNIST itself is not available, so x is drawn uniform in
[0,1) (the pixel range) or standard normal, and class ids are uniform.

Draw order (fixed, so that any consumer reproduces the same values):
  * weights: ``default_rng([seed, 0])``; layer by layer, ``uniform(-a, a,
    (d_in, d_out))`` in float64, then rounded to float32;
  * batch s: ``default_rng([seed, 1, s])``; x first, then the class ids
    ``integers(0, C, B)``; labels are the float32 one-hot rows of the ids.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Sequence, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    """One named MLP workload: layer widths, batch, data recipe, step count."""

    name: str
    dims: Tuple[int, ...]          # d0 -> d1 -> ... -> dL
    batch: int
    x_dist: str                    # "uniform01" | "normal"
    init: str                      # "glorot" | "kaiming"
    lr: float
    steps: int                     # steps the workload is defined over
    fresh_batch: bool              # new seeded batch every step?
    precision: str = "f32"         # "f32" | "bf16"
    seed: int = 0

    @property
    def n_layers(self) -> int:
        return len(self.dims) - 1

    @property
    def classes(self) -> int:
        return self.dims[-1]

    def forward_flops(self) -> int:
        """2*M*N*K summed over the forward products of one pass."""
        B, d, L = self.batch, self.dims, self.n_layers
        return sum(2 * B * d[l] * d[l + 1] for l in range(L))

    def gemm_flops(self) -> int:
        """2*M*N*K summed over the forward, dX and dW products of one step."""
        B, d, L = self.batch, self.dims, self.n_layers
        fwd = sum(2 * B * d[l] * d[l + 1] for l in range(L))
        dw = fwd
        dx = sum(2 * B * d[l] * d[l + 1] for l in range(1, L))
        return fwd + dw + dx


# The five workloads: the README's MLP at its own batch and at batch 1024,
# a wide 3-layer MLP (f32 and bf16 operands) and a skinny batch-8 MLP whose
# step is dominated by streaming the weights.
WORKLOADS = {
    "mnist_b32": Workload("mnist_b32", (784, 128, 10), 32, "uniform01",
                          "glorot", 0.1, 10, False),
    "mnist_b1024": Workload("mnist_b1024", (784, 128, 10), 1024, "uniform01",
                            "glorot", 0.05, 100, True),
    "wide_f32": Workload("wide_f32", (1024, 4096, 4096, 1000), 4096, "normal",
                         "kaiming", 0.01, 1, False),
    "wide_bf16": Workload("wide_bf16", (1024, 4096, 4096, 1000), 4096,
                          "normal", "kaiming", 0.01, 1, False,
                          precision="bf16"),
    "skinny_b8": Workload("skinny_b8", (4096, 11008, 4096), 8, "normal",
                          "glorot", 1e-3, 1, False),
    # One GPU's share of skinny_b8 under 8-way tensor parallelism: W1 split by
    # columns and W2 by rows (11008 / 8 = 1376 hidden units per GPU).  Run on
    # one GPU it measures the per-GPU kernels at their real shapes; the
    # exchange of partial logits between GPUs is not part of it.
    "skinny_b8_tp8_shard": Workload("skinny_b8_tp8_shard", (4096, 1376, 4096), 8, "normal",
                                    "glorot", 1e-3, 1, False),
}


def init_bound(init: str, fan_in: int, fan_out: int) -> float:
    """Half-width of the uniform initialiser for a [fan_in, fan_out] weight.

    Glorot-uniform: sqrt(6/(fan_in+fan_out)); Kaiming-uniform (ReLU gain
    sqrt 2): sqrt(6/fan_in)."""
    if init == "glorot":
        return math.sqrt(6.0 / (fan_in + fan_out))
    if init == "kaiming":
        return math.sqrt(6.0 / fan_in)
    if init == "zeros":
        return 0.0
    raise ValueError(f"unknown initialiser {init!r}")


def make_weights(dims: Sequence[int], init: str, seed: int = 0) -> List[np.ndarray]:
    """Float32 weights W_l of shape [d_{l-1}, d_l], drawn in layer order."""
    rng = np.random.default_rng([seed, 0])
    out = []
    for l in range(len(dims) - 1):
        a = init_bound(init, dims[l], dims[l + 1])
        w = rng.uniform(-a, a, (dims[l], dims[l + 1])) if a > 0 else \
            np.zeros((dims[l], dims[l + 1]))
        out.append(np.ascontiguousarray(w, dtype=np.float32))
    return out


def make_batch(batch: int, d_in: int, classes: int, x_dist: str,
               seed: int = 0, step: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(x [B,d_in] f32, labels [B,C] f32 one-hot, class ids [B] int64)."""
    rng = np.random.default_rng([seed, 1, step])
    if x_dist == "uniform01":
        x = rng.random((batch, d_in))
    elif x_dist == "normal":
        x = rng.standard_normal((batch, d_in))
    else:
        raise ValueError(f"unknown x distribution {x_dist!r}")
    ids = rng.integers(0, classes, batch)
    t = np.zeros((batch, classes), dtype=np.float32)
    t[np.arange(batch), ids] = 1.0
    return np.ascontiguousarray(x, dtype=np.float32), t, ids


def workload_weights(w: Workload) -> List[np.ndarray]:
    return make_weights(w.dims, w.init, w.seed)


def workload_batch(w: Workload, step: int = 0):
    s = step if w.fresh_batch else 0
    return make_batch(w.batch, w.dims[0], w.classes, w.x_dist, w.seed, s)


def integer_operands(shape: Tuple[int, ...], lo: int, hi: int, seed: int) -> np.ndarray:
    """Float32 array of integers drawn uniformly from [lo, hi] (inclusive)."""
    rng = np.random.default_rng([seed, 7])
    return rng.integers(lo, hi + 1, shape).astype(np.float32)
