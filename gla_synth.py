"""Seeded synthetic inputs for the key-only GLA token mixer.

This module only draws random numbers. It holds none of the mixer's arithmetic,
and both sides of every parity check (the HIP path and the fp64 oracle) take
their inputs from here.

The workloads stand in for GTR's activations. The pages measure the operator in
isolation at 256, 1.6K and 16.4K tokens (GTR summary page, section 实验结果 and
its table of results; the 0539edu.com page, section 3.3), and real activations
would need trained weights and images, so every input here is synthetic.
Tokens are the positions of the stride-16 patch grid, so L = grid_h * grid_w.

Recipe (numpy PCG64, ``default_rng(seed)``). q, k, v and g are drawn in that
order, each standard normal float32 in layout [B, L, H, d].
  * fp16 workloads: q, k, v are scaled by ``qkv_std`` (1/8 = 1/sqrt(64));
    log_gamma = logsigmoid(g + gate_mu) / 16, evaluated in float32.
    The 1/16 is the gate temperature tau = 16 of the low-rank gate
    gamma = sigmoid(.)^(1/tau) (summary page, section 核心方法).
    Everything is then rounded to fp16 (round-to-nearest-even).
  * fp32 workload ("tiny"): the same, without the 1/8 and without rounding.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    grid_h: int
    grid_w: int
    d_k: int
    d_v: int
    dtype: str          # "fp16" or "fp32"
    seed: int
    qkv_std: float = 0.125
    gate_mu: float = 0.0
    chunk: int = 64
    note: str = ""

    @property
    def L(self) -> int:
        return self.grid_h * self.grid_w

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny", 1, 1, 16, 16, 32, 32, "fp32", 0, qkv_std=1.0,
                 note="256-token oracle check, fp32"),
        Workload("img640", 1, 6, 40, 40, 64, 64, "fp16", 1,
                 note="640x640 image, 1600 tokens, 6 heads"),
        Workload("img1024", 1, 12, 64, 64, 64, 64, "fp16", 2,
                 note="1024x1024 image, 4096 tokens, 12 heads"),
        Workload("batched640", 8, 6, 40, 40, 64, 64, "fp16", 3,
                 note="batch 8 of 640x640 images"),
        Workload("long2048", 1, 12, 128, 128, 64, 64, "fp16", 4,
                 note="2048x2048 image, 16384 tokens, 12 heads"),
        Workload("long2048_near1", 1, 12, 128, 128, 64, 64, "fp16", 5, gate_mu=3.0,
                 note="16384 tokens with gates near 1 (long memory)"),
        Workload("img640_dk32", 1, 6, 40, 40, 32, 64, "fp16", 6,
                 note="640x640 image with the pages' operator head shape, d_k = 32, d_v = 64"),
    ]
}


def _logsigmoid_f32(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float32)
    return (np.minimum(x, np.float32(0)) - np.log1p(np.exp(-np.abs(x)))).astype(np.float32)


def generate(w: Workload) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Return (q, k, v, log_gamma) as numpy arrays in [B, L, H, d] layout and w.dtype."""
    rng = np.random.default_rng(w.seed)
    shp_k = (w.B, w.L, w.H, w.d_k)
    shp_v = (w.B, w.L, w.H, w.d_v)
    q = rng.standard_normal(shp_k, dtype=np.float32)
    k = rng.standard_normal(shp_k, dtype=np.float32)
    v = rng.standard_normal(shp_v, dtype=np.float32)
    g = rng.standard_normal(shp_k, dtype=np.float32)
    lg = _logsigmoid_f32(g + np.float32(w.gate_mu)) / np.float32(16.0)
    if w.dtype == "fp16":
        s = np.float32(w.qkv_std)
        return ((q * s).astype(np.float16), (k * s).astype(np.float16),
                (v * s).astype(np.float16), lg.astype(np.float16))
    if w.dtype == "fp32":
        s = np.float32(w.qkv_std)
        return (q * s), (k * s), (v * s), lg
    raise ValueError(f"unknown dtype {w.dtype}")


def generate_lowrank(w: Workload, C: int, seed: int, bias_std: float = 0.5
                     ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Inputs of the data-dependent low-rank gate (rank 16): (x, W1, W2, bias).

    x [B, L, C] standard normal (rounded to fp16 for fp16 workloads, as a
    layer-normed feature map); W1 [C, 16] normal with std 1/sqrt(C) and W2
    [16, H d_k] normal with std 1/4, so that x W1 W2 is about unit normal;
    bias [H d_k] = gate_mu + bias_std * normal. W1, W2 and bias are float32.
    """
    rng = np.random.default_rng(seed)
    K = w.H * w.d_k
    x = rng.standard_normal((w.B, w.L, C), dtype=np.float32)
    w1 = rng.standard_normal((C, 16), dtype=np.float32) * np.float32(1.0 / np.sqrt(C))
    w2 = rng.standard_normal((16, K), dtype=np.float32) * np.float32(0.25)
    bias = (np.float32(w.gate_mu) + np.float32(bias_std) *
            rng.standard_normal(K, dtype=np.float32)).astype(np.float32)
    if w.dtype == "fp16":
        x = x.astype(np.float16)
    return x, w1, w2, bias


def generate_sswiglu(B: int, grid_h: int, grid_w: int, C: int, Hd: int, seed: int,
                     bias: bool = True):
    """Inputs of the Spatial SwiGLU mixer: (x, W_g, W_v, conv_w, conv_b, W_o).

    x [B, L, C] standard normal (a layer-normed feature map); W_g, W_v [Hd, C]
    normal with std 1/sqrt(C) and W_o [C, Hd] with std 1/sqrt(Hd) (unit-scale
    activations at every stage), all rounded to fp16; conv_w [Hd, 3, 3] normal
    with std 1/3 and conv_b [Hd] normal with std 0.1 (or None), float32.
    """
    rng = np.random.default_rng(seed)
    L = grid_h * grid_w
    x = rng.standard_normal((B, L, C), dtype=np.float32).astype(np.float16)
    wg = (rng.standard_normal((Hd, C), dtype=np.float32) / np.float32(np.sqrt(C))).astype(np.float16)
    wv = (rng.standard_normal((Hd, C), dtype=np.float32) / np.float32(np.sqrt(C))).astype(np.float16)
    cw = (rng.standard_normal((Hd, 3, 3), dtype=np.float32) / np.float32(3.0)).astype(np.float32)
    cb = (np.float32(0.1) * rng.standard_normal(Hd, dtype=np.float32)) if bias else None
    wo = (rng.standard_normal((C, Hd), dtype=np.float32) / np.float32(np.sqrt(Hd))).astype(np.float16)
    return x, wg, wv, cw, cb, wo


def np_dtype(w: Workload):
    return np.float16 if w.dtype == "fp16" else np.float32
