"""Seeded synthetic LiSA workloads (shapes and value distributions only).

This module draws inputs; it holds none of the LiSA arithmetic.  Both the
GPU path's tests/benchmark and the CPU oracle consume what it returns.

The shapes stand in for the token grids of the reading note "LiSA:面向长程视觉
建模的线性随机注意力" (§3 experiments, §4.5 efficiency): DeiT-T at 224^2 and
384^2 input (14x14 and 24x24 patch grids), PVT-T stage 1 (56x56), a stride-4
map of a 1280x800 COCO image (200x320), and square grids up to the 2048^2 /
128^2-grid efficiency point.  No dataset or trained weight is used: the
projections of a trained network are replaced by

  Q, K = ReLU(N(0, 1)),  V ~ N(0, 1)       (drawn in fp32, then rounded to
                                            bf16 round-to-nearest-even unless
                                            the workload is fp32)
  adaptive weights = softmax over T of N(0, 1) logits   (fp32)
  alpha ~ U(0, 1) per head                              (fp32)

drawn with numpy.random.default_rng(seed) in the order Q, K, V, logits, alpha.
"""

from dataclasses import dataclass, replace

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "get", "make_inputs", "small"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    heads: int
    H: int
    W: int
    T: int
    dtype: str = "bf16"  # "bf16" or "fp32"
    mode: str = "adaptive"  # "adaptive" or "geometric"
    beta: float = 0.5  # geometric mode only
    alpha: float = None  # fixed alpha for every head, else U(0, 1) per head
    eps: float = 1e-6
    d_h: int = 64
    d_v: int = 64
    seed: int = 1000

    @property
    def n(self):
        return self.H * self.W

    @property
    def token_heads(self):
        return self.B * self.heads * self.n

    def describe(self):
        return (
            f"{self.name}: [B={self.B}, heads={self.heads}, {self.H}x{self.W}, "
            f"d={self.d_h}] {self.dtype} T={self.T} {self.mode}"
        )


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_oracle_14x14", 1, 1, 14, 14, 3, dtype="fp32", mode="geometric",
                 beta=0.5, alpha=0.5, seed=1000),
        Workload("deit_t_224", 64, 3, 14, 14, 3, seed=1001),
        Workload("deit_t_384", 64, 3, 24, 24, 3, seed=1002),
        Workload("deit_t_384_t5", 64, 3, 24, 24, 5, seed=1002),
        Workload("pvt_t_stage1", 32, 1, 56, 56, 3, seed=1003),
        Workload("long_range_200x320", 1, 1, 200, 320, 5, seed=1004),
        Workload("square_64x64", 1, 1, 64, 64, 5, seed=1005),
        Workload("square_128x128", 1, 1, 128, 128, 5, seed=1006),
        Workload("square_256x256", 1, 1, 256, 256, 5, seed=1007),
    ]
}


def get(name):
    return WORKLOADS[name]


def small(name, B, heads, H, W, T, **kw):
    """An ad-hoc workload for tests (ragged grids, edge cases)."""
    return Workload(name, B, heads, H, W, T, **kw)


def _to_dtype(x32, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)  # round-to-nearest-even
    if dtype == "fp32":
        return t
    raise ValueError(dtype)


def make_inputs(w, seed=None):
    """Draw one input set for workload ``w`` on the host.

    Returns a dict of CPU torch tensors: q, k [B, heads, n, d_h] and v
    [B, heads, n, d_v] in the workload dtype, weights [B, heads, n, T] fp32
    (None in geometric mode), alpha [heads] fp32; plus the scalars T, H, W,
    beta, eps.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shp = (w.B, w.heads, w.n)
    q = np.maximum(rng.standard_normal(shp + (w.d_h,), dtype=np.float32), 0)
    k = np.maximum(rng.standard_normal(shp + (w.d_h,), dtype=np.float32), 0)
    v = rng.standard_normal(shp + (w.d_v,), dtype=np.float32)
    weights = None
    if w.mode == "adaptive":
        logits = rng.standard_normal(shp + (w.T,)).astype(np.float64)
        e = np.exp(logits - logits.max(axis=-1, keepdims=True))
        weights = torch.from_numpy((e / e.sum(axis=-1, keepdims=True)).astype(np.float32))
    elif w.mode != "geometric":
        raise ValueError(w.mode)
    if w.alpha is None:
        alpha = rng.uniform(0.0, 1.0, size=w.heads).astype(np.float32)
    else:
        alpha = np.full(w.heads, w.alpha, dtype=np.float32)
    return {
        "q": _to_dtype(q, w.dtype),
        "k": _to_dtype(k, w.dtype),
        "v": _to_dtype(v, w.dtype),
        "weights": weights,
        "alpha": torch.from_numpy(alpha),
        "T": w.T,
        "H": w.H,
        "W": w.W,
        "beta": w.beta if w.mode == "geometric" else None,
        "eps": w.eps,
    }


def mlp_params(heads, hidden, T, d_h=64, seed=0):
    """Random parameters of the walk-weight predictor, as CPU fp32 tensors:
    w1 [heads, hidden, 2 d_h], b1 [heads, hidden], w2 [heads, T, hidden],
    b2 [heads, T].  Scales keep the hidden pre-activations and the logits of
    order one for ReLU(N(0, 1)) queries and keys."""
    rng = np.random.default_rng(seed)
    f = lambda *shape, scale: torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32))  # noqa: E731
    return {
        "w1": f(heads, hidden, 2 * d_h, scale=1.0 / np.sqrt(d_h)),
        "b1": f(heads, hidden, scale=0.1),
        "w2": f(heads, T, hidden, scale=2.0 / np.sqrt(hidden)),
        "b2": f(heads, T, scale=0.1),
    }


def layer_params(w, seed=None):
    """Input and parameters of a LiSA attention layer for workload ``w``
    (C = 64 heads channels), as CPU tensors: x [B, n, C] and w_qkv [3C, C],
    w_o [C, C] in the workload dtype, b_qkv [3C] and b_o [C] fp32.  The
    projections keep Q, K, V of unit scale."""
    rng = np.random.default_rng((w.seed if seed is None else seed) + 7)
    C = 64 * w.heads
    x = rng.standard_normal((w.B, w.n, C), dtype=np.float32)
    wqkv = (rng.standard_normal((3 * C, C)) / np.sqrt(C)).astype(np.float32)
    wo = (rng.standard_normal((C, C)) / np.sqrt(C)).astype(np.float32)
    return {
        "x": _to_dtype(x, w.dtype),
        "w_qkv": _to_dtype(wqkv, w.dtype),
        "b_qkv": torch.from_numpy((rng.standard_normal(3 * C) * 0.1).astype(np.float32)),
        "w_o": _to_dtype(wo, w.dtype),
        "b_o": torch.from_numpy((rng.standard_normal(C) * 0.1).astype(np.float32)),
    }


def with_changes(w, **kw):
    return replace(w, **kw)
