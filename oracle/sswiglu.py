"""fp64 CPU oracle of GTR's Spatial SwiGLU channel mixer.

TEST INFRASTRUCTURE ONLY (as the rest of this package): the tests, the smoke
check and the benchmark's CPU-baseline leg use it; the product path never
imports it, and it imports nothing from there.

Definition followed (GTR summary page "GTR:门控Token循环实现高效稠密预测",
section 前置知识 › SwiGLU前馈块 and section 核心方法): the SwiGLU channel
mixer Y = SiLU(X W_g) ⊙ (X W_v) W_o with a 3x3 depthwise convolution inserted
in the value branch,

    Y = (SiLU(X W_g) ⊙ DWConv3x3(X W_v)) W_o,    SiLU(z) = z sigma(z),

over the tokens of the stride-16 patch grid. Readings where the pages are
silent: the weights are given as linear-layer weights [out, in] (so X W_g is
x @ w_g.T); the depthwise convolution is a per-channel cross-correlation
(out[i, j] = sum_{a, c} K[a, c] u[i + a - 1, j + c - 1]) over the grid with
zero padding and the same output size, plus an optional per-channel bias.

Every step is one line of numpy in fp64 in the pages' order; the convolution
is the nine taps written out. Pins: ``tests/test_oracle_sswiglu.py``.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + e^{-z}) in fp64 (e^{-z} overflowing to inf gives -0)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def dwconv3x3(u: np.ndarray, grid_h: int, grid_w: int, weight: np.ndarray,
              bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Depthwise 3x3 cross-correlation with zero padding over the patch grid.

    u [B, L, Hd] with L = grid_h * grid_w (row-major tokens); weight [Hd, 3, 3];
    bias [Hd] or None. Returns [B, L, Hd] in fp64.
    """
    u = np.asarray(u, dtype=np.float64)
    B, L, Hd = u.shape
    if L != grid_h * grid_w:
        raise ValueError("L must equal grid_h * grid_w")
    w = np.asarray(weight, dtype=np.float64)
    if w.shape != (Hd, 3, 3):
        raise ValueError("weight must be [Hd, 3, 3]")
    img = u.reshape(B, grid_h, grid_w, Hd)
    pad = np.zeros((B, grid_h + 2, grid_w + 2, Hd), dtype=np.float64)
    pad[:, 1:-1, 1:-1, :] = img
    out = np.zeros_like(img)
    for a in range(3):          # row offset a - 1
        for c in range(3):      # column offset c - 1
            out += w[:, a, c] * pad[:, a:a + grid_h, c:c + grid_w, :]
    if bias is not None:
        out += np.asarray(bias, dtype=np.float64)
    return out.reshape(B, L, Hd)


def sswiglu(x, w_g, w_v, conv_w, conv_b, w_o, grid_h: int, grid_w: int) -> np.ndarray:
    """Y = (SiLU(x W_g) ⊙ DWConv3x3(x W_v)) W_o for x [B, L, C].

    w_g, w_v [Hd, C]; conv_w [Hd, 3, 3]; conv_b [Hd] or None; w_o [C_out, Hd].
    Returns Y [B, L, C_out] in fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    wg = np.asarray(w_g, dtype=np.float64)
    wv = np.asarray(w_v, dtype=np.float64)
    wo = np.asarray(w_o, dtype=np.float64)
    if wg.shape != wv.shape or wg.shape[1] != x.shape[-1] or wo.shape[1] != wg.shape[0]:
        raise ValueError("w_g, w_v must be [Hd, C] and w_o [C_out, Hd]")
    g = x @ wg.T
    u = x @ wv.T
    a = silu(g) * dwconv3x3(u, grid_h, grid_w, conv_w, conv_b)
    return a @ wo.T
