"""fp64 CPU oracle for key-only gated linear attention (GTR's token mixer).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark use this package to check and time the HIP path. The product
path (``chunkwise_gated_recurrence_amd``) never imports it, and this package
imports nothing from there.

The arithmetic lives in ``gla_oracle.c`` (plain C, fp64, threads only across the
independent (batch, head) sequences). This module builds it with gcc, loads it
with ctypes and converts arrays. Every input is upcast to float64 exactly
(fp16 and fp32 values are representable in fp64), so the oracle sees the very
values the GPU receives.

Definitions followed (GTR summary page "GTR:门控Token循环实现高效稠密预测",
section 前置知识 › 门控线性注意力(GLA) and section 核心方法):

    S_t = Diag(gamma_t) S_{t-1} + k_t^T v_t,   o_t = d_k^{-1/2} q_t S_t,   S_0 = 0

(``recurrent_init``: the same from a given S_0), the data-dependent gate
gamma_t = sigma(x_t W1 W2 + b)^{1/tau} of section 核心方法 (rank 16, tau = 16;
``lowrank_gate`` gives log_gamma), and the output epilogue that the end-to-end
operator fuses (0539edu.com page, appendix E.3.1; ``rmsnorm_gate``)

with gamma_t = exp(log_gamma_t) per key dimension, walked along one of four
scan orders over the patch grid (same sections; see ``scan_order``).

``sswiglu`` (module ``oracle.sswiglu``, numpy fp64) is the block's other
token-grid operator, the Spatial SwiGLU channel mixer (same page, section
前置知识 › SwiGLU前馈块), pinned in ``tests/test_oracle_sswiglu.py``.

Pins: every function here is pinned by tests in ``tests/test_oracle.py`` against
closed forms (causal linear attention, retention with a constant gate, the
gamma -> 0 limit), hand-computed examples in ``tests/golden/``, the brute-force
double sum, and the direction/linearity invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libglaoracle.so")
_lib = None

DIRS = {"l2r": 0, "r2l": 1, "t2b": 2, "b2t": 3}


def build(force: bool = False) -> str:
    """Compile gla_oracle.c into libglaoracle.so next to it (gcc, -O2)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        for name in ("gla_oracle_recurrent", "gla_oracle_bruteforce"):
            fn = getattr(lib, name)
            fn.restype = i
            fn.argtypes = [dp, dp, dp, dp, i, i, i, i, i, i, i, dp, dp, i]
        lib.gla_oracle_chunked.restype = i
        lib.gla_oracle_chunked.argtypes = [dp, dp, dp, dp, i, i, i, i, i, i, i, i, dp, dp, i]
        lib.gla_oracle_recurrent_init.restype = i
        lib.gla_oracle_recurrent_init.argtypes = [dp, dp, dp, dp, dp, i, i, i, i, i, i, i, dp, dp,
                                                  i]
        lib.gla_oracle_lowrank_gate.restype = i
        lib.gla_oracle_lowrank_gate.argtypes = [dp, dp, dp, dp, ctypes.c_double, ctypes.c_long, i,
                                                i, i, dp]
        lib.gla_oracle_rmsnorm_gate.restype = i
        lib.gla_oracle_rmsnorm_gate.argtypes = [dp, dp, dp, ctypes.c_double, ctypes.c_long, i, dp]
        lib.gla_oracle_scan_position.restype = ctypes.c_long
        lib.gla_oracle_scan_position.argtypes = [ctypes.c_long, i, i, i]
        _lib = lib
    return _lib


def _dir(d) -> int:
    if isinstance(d, str):
        return DIRS[d]
    return int(d)


def _f64(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x), dtype=np.float64)


def _ptr(x: np.ndarray):
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def scan_order(grid_h: int, grid_w: int, direction) -> np.ndarray:
    """Spatial token visited at each scan step, as an int64 array of length L."""
    lib = _load()
    L = grid_h * grid_w
    d = _dir(direction)
    return np.array([lib.gla_oracle_scan_position(t, grid_h, grid_w, d) for t in range(L)],
                    dtype=np.int64)


def _shapes(q, k, v, lg, grid_h, grid_w):
    q = np.asarray(q)
    v = np.asarray(v)
    if q.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, log_gamma must be [B, L, H, d_k] and v [B, L, H, d_v]")
    B, L, H, dk = q.shape
    dv = v.shape[3]
    if L != grid_h * grid_w:
        raise ValueError(f"L={L} does not match grid {grid_h}x{grid_w}")
    if np.asarray(k).shape != q.shape or np.asarray(lg).shape != q.shape:
        raise ValueError("k and log_gamma must have q's shape")
    if v.shape[:3] != (B, L, H):
        raise ValueError("v must be [B, L, H, d_v]")
    return B, L, H, dk, dv


def _call(name, q, k, v, lg, grid_h, grid_w, direction, threads, chunk=None):
    lib = _load()
    B, L, H, dk, dv = _shapes(q, k, v, lg, grid_h, grid_w)
    q64, k64, v64, g64 = _f64(q), _f64(k), _f64(v), _f64(lg)
    out = np.zeros((B, L, H, dv), dtype=np.float64)
    fs = np.zeros((B, H, dk, dv), dtype=np.float64)
    nt = default_threads() if threads is None else int(threads)
    args = [_ptr(q64), _ptr(k64), _ptr(v64), _ptr(g64), B, H, grid_h, grid_w, dk, dv,
            _dir(direction)]
    if chunk is not None:
        args.append(int(chunk))
    args += [_ptr(out), _ptr(fs), nt]
    r = getattr(lib, name)(*args)
    if r != 0:
        raise RuntimeError(f"{name} failed with status {r}")
    return out, fs


def recurrent(q, k, v, log_gamma, grid_h: int, grid_w: int, direction,
              threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Token-by-token fp64 recurrence. Returns (o [B,L,H,d_v], final_state [B,H,d_k,d_v])."""
    return _call("gla_oracle_recurrent", q, k, v, log_gamma, grid_h, grid_w, direction, threads)


def recurrent_init(q, k, v, log_gamma, initial_state, grid_h: int, grid_w: int, direction,
                   threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """The recurrence from S_0 = initial_state [B,H,d_k,d_v] instead of zero."""
    lib = _load()
    B, L, H, dk, dv = _shapes(q, k, v, log_gamma, grid_h, grid_w)
    s0 = _f64(initial_state)
    if s0.shape != (B, H, dk, dv):
        raise ValueError("initial_state must be [B, H, d_k, d_v]")
    q64, k64, v64, g64 = _f64(q), _f64(k), _f64(v), _f64(log_gamma)
    out = np.zeros((B, L, H, dv), dtype=np.float64)
    fs = np.zeros((B, H, dk, dv), dtype=np.float64)
    nt = default_threads() if threads is None else int(threads)
    r = lib.gla_oracle_recurrent_init(_ptr(q64), _ptr(k64), _ptr(v64), _ptr(g64), _ptr(s0), B, H,
                                      grid_h, grid_w, dk, dv, _dir(direction), _ptr(out), _ptr(fs),
                                      nt)
    if r != 0:
        raise RuntimeError(f"gla_oracle_recurrent_init failed with status {r}")
    return out, fs


def lowrank_gate(x, w1, w2, bias, inv_tau: float = 1.0 / 16) -> np.ndarray:
    """log_gamma = inv_tau * logsigmoid(x W1 W2 + bias) over the last axis of x
    ([..., C] -> [..., K]); W1 [C, R], W2 [R, K], bias [K]."""
    lib = _load()
    x64, a64, b64, c64 = _f64(x), _f64(w1), _f64(w2), _f64(bias)
    C = x64.shape[-1]
    R = a64.shape[1]
    K = b64.shape[1]
    if a64.shape != (C, R) or b64.shape != (R, K) or c64.shape != (K,):
        raise ValueError("W1 must be [C, R], W2 [R, K] and bias [K]")
    rows = x64.size // C
    lg = np.zeros(x64.shape[:-1] + (K,), dtype=np.float64)
    r = lib.gla_oracle_lowrank_gate(_ptr(x64), _ptr(a64), _ptr(b64), _ptr(c64), float(inv_tau),
                                    rows, C, R, K, _ptr(lg))
    if r != 0:
        raise RuntimeError(f"gla_oracle_lowrank_gate failed with status {r}")
    return lg


def rmsnorm_gate(o, gate, weight, eps: float) -> np.ndarray:
    """Output epilogue over the last axis: o / sqrt(mean(o^2) + eps) * weight * SiLU(gate)."""
    lib = _load()
    o64, z64, w64 = _f64(o), _f64(gate), _f64(weight)
    if z64.shape != o64.shape or w64.shape != (o64.shape[-1],):
        raise ValueError("gate must have o's shape and weight o's last dimension")
    d = o64.shape[-1]
    rows = o64.size // d
    y = np.zeros_like(o64)
    r = lib.gla_oracle_rmsnorm_gate(_ptr(o64), _ptr(z64), _ptr(w64), float(eps), rows, d, _ptr(y))
    if r != 0:
        raise RuntimeError(f"gla_oracle_rmsnorm_gate failed with status {r}")
    return y


def bruteforce(q, k, v, log_gamma, grid_h: int, grid_w: int, direction,
               threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Explicit O(L^2) double sum of the same outputs (small inputs only)."""
    return _call("gla_oracle_bruteforce", q, k, v, log_gamma, grid_h, grid_w, direction, threads)


def chunked(q, k, v, log_gamma, grid_h: int, grid_w: int, direction, chunk: int,
            threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Three-phase chunkwise evaluation in fp64 (chunk summaries, boundary scan, outputs)."""
    return _call("gla_oracle_chunked", q, k, v, log_gamma, grid_h, grid_w, direction, threads,
                 chunk=chunk)


def rel_err(x, ref) -> float:
    """max|x - ref| / max|ref| over the whole tensor (absolute max-abs if ref is all zero)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    return num / den if den > 0 else num
