"""Seeded synthetic inputs for the fast-weight scan (shared by tests and bench).

This module holds no arithmetic of the method: it only draws random tensors
with the shapes and value distributions of the five workloads and rounds them
to the io dtype.  Both the HIP path and the CPU oracle are fed from it: the HIP
path gets the rounded tensors, the oracle gets their exact fp64 upcast.

Distribution notation: N(mu, v) takes v as the VARIANCE, so N(0, 1/d) has
standard deviation 1/sqrt(d).  sigmoid(z) = 1 / (1 + exp(-z)).

Workloads (the model shapes echo the 340M / 1.3B scales named in the ParaTTT
summary, ai4snews.wisdomeyes.cn, section "Perspective"):
  c1  B=1 H=1  T=256   d=32   fp64
  c2  B=4 H=8  T=1024  d=64   fp32 (chunk 64)
  c3  B=8 H=16 T=4096  d=64   bf16 io, fp32 gates  (340M-shape layer)
  c4  B=4 H=16 T=4096  d=128  bf16 io, alpha = sigmoid(N(5, 0.5))  (1.3B shape)
  c5  B=1 H=16 T=32768 d=128  bf16 io, alpha mixture, unit-norm x  (long context)
Common: x, g, W0 ~ N(0, 1/d); eta = 0.1 * sigmoid(N(-1, 1));
alpha = sigmoid(N(3, 1)); dy ~ N(0, 1).  Seeds: numpy PCG64(1000 + k) for ck,
drawn in the fixed order W0, x, g, eta, [coin], alpha, dy.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

DTYPES = ("f64", "f32", "bf16")


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    d_in: int
    d_out: int
    dtype: str          # io dtype: "f64" | "f32" | "bf16"
    alpha_kind: str     # "base" | "near1" | "mix"
    x_kind: str         # "gauss" | "unit"
    seed: int
    chunk: int = 0      # 0 = library default

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def token_heads(self) -> int:
        return self.B * self.H * self.T


CONFIGS = {
    "c1": Workload("c1", 1, 1, 256, 32, 32, "f64", "base", "gauss", 1001),
    "c2": Workload("c2", 4, 8, 1024, 64, 64, "f32", "base", "gauss", 1002, 64),
    "c3": Workload("c3", 8, 16, 4096, 64, 64, "bf16", "base", "gauss", 1003),
    "c4": Workload("c4", 4, 16, 4096, 128, 128, "bf16", "near1", "gauss", 1004),
    "c5": Workload("c5", 1, 16, 32768, 128, 128, "bf16", "mix", "unit", 1005),
}


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def round_to(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to the io dtype and return their exact fp64 upcast."""
    if dtype == "f64":
        return np.ascontiguousarray(a, np.float64)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(a, np.float64))
        return t.to(torch.bfloat16).to(torch.float64).numpy()
    raise ValueError(dtype)


def gate_dtype(io_dtype: str) -> str:
    return "f64" if io_dtype == "f64" else "f32"


def make_inputs(w: Workload) -> dict:
    """Draw one batch.  Returns fp64 numpy arrays holding values exactly
    representable in the io dtype (x, g, W0, dy) or gate dtype (eta, alpha)."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    B, H, T, di, do = w.B, w.H, w.T, w.d_in, w.d_out
    W0 = rng.standard_normal((H, do, di)) / np.sqrt(di)
    if w.x_kind == "unit":
        z = rng.standard_normal((B, H, T, di))
        x = z / np.linalg.norm(z, axis=-1, keepdims=True)
    else:
        x = rng.standard_normal((B, H, T, di)) / np.sqrt(di)
    g = rng.standard_normal((B, H, T, do)) / np.sqrt(do)
    eta = 0.1 * _sigmoid(rng.normal(-1.0, 1.0, (B, H, T)))
    if w.alpha_kind == "near1":
        alpha = _sigmoid(rng.normal(5.0, np.sqrt(0.5), (B, H, T)))
    elif w.alpha_kind == "mix":
        coin = rng.random((B, H, T)) < 0.5
        slow = _sigmoid(rng.normal(6.0, np.sqrt(0.5), (B, H, T)))
        fast = _sigmoid(rng.normal(0.0, 1.0, (B, H, T)))
        alpha = np.where(coin, slow, fast)
    else:
        alpha = _sigmoid(rng.normal(3.0, 1.0, (B, H, T)))
    dy = rng.standard_normal((B, H, T, do))
    gd = gate_dtype(w.dtype)
    return {
        "x": round_to(x, w.dtype),
        "g": round_to(g, w.dtype),
        "eta": round_to(eta, gd),
        "alpha": round_to(alpha, gd),
        "W0": round_to(W0, w.dtype),
        "dy": round_to(dy, w.dtype),
    }
