"""Python binding of libgtrgla: key-only gated linear attention forward on MI355X.

Thin ctypes marshalling over the C ABI in ``include/gtr_gla.h``. The functions
have the C names and argument order. They take torch tensors that live on the
GPU, check dtype, device, contiguity and element count against the sizes
passed, and pass raw pointers plus the current HIP stream. Every step of the
computation runs in the HIP kernels of ``libgtrgla.so``. If the library is not
built, importing works but every call raises.

Operation (GTR summary page "GTR:门控Token循环实现高效稠密预测", section
前置知识 › 门控线性注意力(GLA)): S_t = Diag(gamma_t) S_{t-1} + k_t^T v_t,
o_t = d_k^{-1/2} q_t S_t, S_0 = 0, along one of four scan orders over the
patch grid, evaluated chunkwise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgtrgla.so")

# status codes (gtr_gla_status)
OK, ERR_NULL, ERR_SHAPE, ERR_DIR, ERR_CHUNK, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, \
    ERR_ALIAS, ERR_POLICY, ERR_VALUE, ERR_EXCHANGE, ERR_WS_STATE, ERR_SCRATCH = range(14)
NOALLOC_SCRATCH_BYTES = 32 << 20   # GTR_GLA_NOALLOC_SCRATCH_BYTES
# scan orders (gtr_gla_dir)
L2R, R2L, T2B, B2T = 0, 1, 2, 3
DIRS = {"l2r": L2R, "r2l": R2L, "t2b": T2B, "b2t": B2T}
# policies (gtr_gla_policy)
POLICY_AUTO, POLICY_GENERIC, POLICY_FUSED, POLICY_FUSED_ONE = 0, 1, 2, 3

EXPORTED = (
    "gtr_gla_fwd", "gtr_gla_fwd_f32", "gtr_gla_workspace_bytes", "gtr_gla_workspace_init",
    "gtr_gla_fwd_ws", "gtr_gla_fwd_f32_ws", "gtr_gla_fwd_ex", "gtr_gla_fwd_lowrank",
    "gtr_gla_lowrank_workspace_bytes", "gtr_gla_set_policy", "gtr_gla_get_policy",
    "gtr_gla_plan", "gtr_gla_plan_lowrank", "gtr_gla_status_str", "gtr_sswiglu_fwd",
    "gtr_sswiglu_workspace_bytes", "gtr_gla_workspace_status", "gtr_gla_set_exchange_wait",
    "gtr_gla_fwd_noalloc",
)


class GtrGlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {gtr_gla_status_str(status)} (status {status})")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgtrgla.so (raises if it has not been built).

    PyTorch-ROCm ships its own HIP and HSA runtimes (same sonames as ROCm's). The
    library links libamdhip64.so.7 by soname: loaded after torch it binds to the
    runtime torch already holds. Loaded first, it would pull in the system's copy
    and the process would hold two HIP runtimes competing for the GPU (one of
    them then sees no device). So torch's runtime is loaded first here."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m chunkwise_gated_recurrence_amd.build`")
    try:
        import torch  # noqa: F401  (loads torch's HIP runtime before the library binds one)
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    fwd = [P, P, P, P, I, I, I, I, I, I, I, I, P, P]
    lib.gtr_gla_fwd.argtypes = fwd + [P]
    lib.gtr_gla_fwd_f32.argtypes = fwd + [P]
    lib.gtr_gla_fwd_ws.argtypes = fwd + [P, Z, P]
    lib.gtr_gla_fwd_noalloc.argtypes = fwd + [P]
    lib.gtr_gla_fwd_noalloc.restype = I
    lib.gtr_gla_fwd_f32_ws.argtypes = fwd + [P, Z, P]
    for f in (lib.gtr_gla_fwd, lib.gtr_gla_fwd_f32, lib.gtr_gla_fwd_ws, lib.gtr_gla_fwd_f32_ws):
        f.restype = I
    lib.gtr_gla_fwd_ex.argtypes = [P, P, P, P, P, P, P, ctypes.c_float, I, I, I, I, I, I, I, I, I,
                                   P, P, P, Z, P]
    lib.gtr_gla_fwd_ex.restype = I
    lib.gtr_gla_fwd_lowrank.argtypes = [P, P, P, P, P, P, P, ctypes.c_float, I, P, P, P,
                                        ctypes.c_float, I, I, I, I, I, I, I, I, I, P, P, P, Z, P]
    lib.gtr_gla_fwd_lowrank.restype = I
    lib.gtr_gla_lowrank_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
    lib.gtr_gla_lowrank_workspace_bytes.restype = Z
    lib.gtr_gla_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
    lib.gtr_gla_workspace_bytes.restype = Z
    lib.gtr_gla_workspace_init.argtypes = [P, Z, P]
    lib.gtr_gla_workspace_init.restype = I
    lib.gtr_gla_set_policy.argtypes = [I]
    lib.gtr_gla_set_policy.restype = I
    lib.gtr_gla_get_policy.argtypes = []
    lib.gtr_gla_get_policy.restype = I
    IP = ctypes.POINTER(ctypes.c_int)
    lib.gtr_gla_plan.argtypes = [I, I, I, I, I, I, I, I, IP, IP, IP]
    lib.gtr_gla_plan.restype = I
    lib.gtr_gla_plan_lowrank.argtypes = [I, I, I, I, I, I, I, I, IP, IP, IP]
    lib.gtr_gla_plan_lowrank.restype = I
    lib.gtr_sswiglu_fwd.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P, P, Z, P]
    lib.gtr_sswiglu_fwd.restype = I
    lib.gtr_sswiglu_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.gtr_sswiglu_workspace_bytes.restype = Z
    lib.gtr_gla_status_str.argtypes = [I]
    lib.gtr_gla_status_str.restype = ctypes.c_char_p
    lib.gtr_gla_workspace_status.argtypes = [P, Z, P]
    lib.gtr_gla_workspace_status.restype = I
    lib.gtr_gla_set_exchange_wait.argtypes = [ctypes.c_uint, I]
    lib.gtr_gla_set_exchange_wait.restype = I
    _lib = lib
    return lib


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def _check(t, name: str, dtype, numel: int):
    if t is None:
        return
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def _check_all(q, k, v, lg, B, H, gh, gw, dk, dv, out, fs, dtype):
    import torch
    if min(B, H, gh, gw, dk, dv) < 1:
        return  # let the library report the invalid size
    rows = B * gh * gw * H
    for t, n in ((q, "q"), (k, "k"), (lg, "log_gamma")):
        _check(t, n, dtype, rows * dk)
    _check(v, "v", dtype, rows * dv)
    _check(out, "out", dtype, rows * dv)
    _check(fs, "final_state", torch.float32, B * H * dk * dv)


def _raise(status: int, where: str):
    if status != OK:
        raise GtrGlaError(status, where)


def gtr_gla_fwd(q, k, v, log_gamma, B: int, H: int, grid_h: int, grid_w: int, d_k: int, d_v: int,
                dir: int, chunk: int, out, final_state=None, stream=None) -> None:
    """fp16 forward; writes `out` [B,L,H,d_v] fp16 and `final_state` [B,H,d_k,d_v] fp32."""
    import torch
    _check_all(q, k, v, log_gamma, B, H, grid_h, grid_w, d_k, d_v, out, final_state, torch.float16)
    r = load_library().gtr_gla_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_gamma), B, H, grid_h,
                                   grid_w, d_k, d_v, dir, chunk, _ptr(out), _ptr(final_state),
                                   _stream(stream))
    _raise(r, "gtr_gla_fwd")


def gtr_gla_fwd_noalloc(q, k, v, log_gamma, B: int, H: int, grid_h: int, grid_w: int, d_k: int,
                        d_v: int, dir: int, chunk: int, out, final_state=None,
                        stream=None) -> None:
    """gtr_gla_fwd with the library's static per-GPU scratch (allocates nothing)."""
    import torch
    _check_all(q, k, v, log_gamma, B, H, grid_h, grid_w, d_k, d_v, out, final_state, torch.float16)
    r = load_library().gtr_gla_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_gamma), B, H,
                                           grid_h, grid_w, d_k, d_v, dir, chunk, _ptr(out),
                                           _ptr(final_state), _stream(stream))
    _raise(r, "gtr_gla_fwd_noalloc")


def gtr_gla_fwd_f32(q, k, v, log_gamma, B: int, H: int, grid_h: int, grid_w: int, d_k: int,
                    d_v: int, dir: int, chunk: int, out, final_state=None, stream=None) -> None:
    """fp32 forward (generic kernels)."""
    import torch
    _check_all(q, k, v, log_gamma, B, H, grid_h, grid_w, d_k, d_v, out, final_state, torch.float32)
    r = load_library().gtr_gla_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(log_gamma), B, H, grid_h,
                                       grid_w, d_k, d_v, dir, chunk, _ptr(out), _ptr(final_state),
                                       _stream(stream))
    _raise(r, "gtr_gla_fwd_f32")


def gtr_gla_workspace_bytes(B: int, H: int, grid_h: int, grid_w: int, d_k: int, d_v: int,
                            chunk: int, is_fp32: int) -> int:
    return int(load_library().gtr_gla_workspace_bytes(B, H, grid_h, grid_w, d_k, d_v, chunk,
                                                      int(is_fp32)))


def gtr_gla_workspace_init(workspace, workspace_bytes: int, stream=None) -> None:
    r = load_library().gtr_gla_workspace_init(_ptr(workspace), workspace_bytes, _stream(stream))
    _raise(r, "gtr_gla_workspace_init")


def gtr_gla_fwd_ws(q, k, v, log_gamma, B, H, grid_h, grid_w, d_k, d_v, dir, chunk, out,
                   final_state, workspace, workspace_bytes: int, stream=None) -> None:
    import torch
    _check_all(q, k, v, log_gamma, B, H, grid_h, grid_w, d_k, d_v, out, final_state, torch.float16)
    r = load_library().gtr_gla_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(log_gamma), B, H, grid_h,
                                      grid_w, d_k, d_v, dir, chunk, _ptr(out), _ptr(final_state),
                                      _ptr(workspace), workspace_bytes, _stream(stream))
    _raise(r, "gtr_gla_fwd_ws")


def gtr_gla_fwd_f32_ws(q, k, v, log_gamma, B, H, grid_h, grid_w, d_k, d_v, dir, chunk, out,
                       final_state, workspace, workspace_bytes: int, stream=None) -> None:
    import torch
    _check_all(q, k, v, log_gamma, B, H, grid_h, grid_w, d_k, d_v, out, final_state, torch.float32)
    r = load_library().gtr_gla_fwd_f32_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(log_gamma), B, H,
                                          grid_h, grid_w, d_k, d_v, dir, chunk, _ptr(out),
                                          _ptr(final_state), _ptr(workspace), workspace_bytes,
                                          _stream(stream))
    _raise(r, "gtr_gla_fwd_f32_ws")


def gtr_gla_fwd_ex(q, k, v, log_gamma, initial_state, gate, norm_weight, norm_eps: float, B: int,
                   H: int, grid_h: int, grid_w: int, d_k: int, d_v: int, dir: int, chunk: int,
                   is_fp32: int, out, final_state=None, workspace=None, workspace_bytes: int = 0,
                   stream=None) -> None:
    """Forward from an initial state and/or with the RMSNorm + SiLU output gate."""
    import torch
    dtype = torch.float32 if is_fp32 else torch.float16
    _check_all(q, k, v, log_gamma, B, H, grid_h, grid_w, d_k, d_v, out, final_state, dtype)
    if min(B, H, grid_h, grid_w, d_k, d_v) >= 1:
        _check(initial_state, "initial_state", torch.float32, B * H * d_k * d_v)
        _check(gate, "gate", dtype, B * grid_h * grid_w * H * d_v)
        _check(norm_weight, "norm_weight", torch.float32, d_v)
    r = load_library().gtr_gla_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(log_gamma),
                                      _ptr(initial_state), _ptr(gate), _ptr(norm_weight),
                                      float(norm_eps), B, H, grid_h, grid_w, d_k, d_v, dir, chunk,
                                      int(is_fp32), _ptr(out), _ptr(final_state), _ptr(workspace),
                                      workspace_bytes, _stream(stream))
    _raise(r, "gtr_gla_fwd_ex")


def gtr_gla_fwd_lowrank(q, k, v, x, w1, w2, gate_bias, inv_tau: float, C: int, initial_state,
                        gate, norm_weight, norm_eps: float, B: int, H: int, grid_h: int,
                        grid_w: int, d_k: int, d_v: int, dir: int, chunk: int, is_fp32: int, out,
                        final_state=None, workspace=None, workspace_bytes: int = 0,
                        stream=None) -> None:
    """Forward with the gate computed from x by the rank-16 projection:
    log_gamma = inv_tau * log sigmoid(x w1 w2 + gate_bias)."""
    import torch
    dtype = torch.float32 if is_fp32 else torch.float16
    _check_all(q, k, v, None, B, H, grid_h, grid_w, d_k, d_v, out, final_state, dtype)
    if min(B, H, grid_h, grid_w, d_k, d_v, C) >= 1:
        _check(x, "x", dtype, B * grid_h * grid_w * C)
        _check(w1, "w1", torch.float32, C * 16)
        _check(w2, "w2", torch.float32, 16 * H * d_k)
        _check(gate_bias, "gate_bias", torch.float32, H * d_k)
        _check(initial_state, "initial_state", torch.float32, B * H * d_k * d_v)
        _check(gate, "gate", dtype, B * grid_h * grid_w * H * d_v)
        _check(norm_weight, "norm_weight", torch.float32, d_v)
    r = load_library().gtr_gla_fwd_lowrank(
        _ptr(q), _ptr(k), _ptr(v), _ptr(x), _ptr(w1), _ptr(w2), _ptr(gate_bias), float(inv_tau),
        C, _ptr(initial_state), _ptr(gate), _ptr(norm_weight), float(norm_eps), B, H, grid_h,
        grid_w, d_k, d_v, dir, chunk, int(is_fp32), _ptr(out), _ptr(final_state),
        _ptr(workspace), workspace_bytes, _stream(stream))
    _raise(r, "gtr_gla_fwd_lowrank")


def gtr_gla_lowrank_workspace_bytes(B: int, H: int, grid_h: int, grid_w: int, d_k: int,
                                    d_v: int, chunk: int, is_fp32: int) -> int:
    return int(load_library().gtr_gla_lowrank_workspace_bytes(B, H, grid_h, grid_w, d_k, d_v,
                                                              chunk, int(is_fp32)))


def gtr_gla_set_policy(policy: int) -> None:
    _raise(load_library().gtr_gla_set_policy(int(policy)), "gtr_gla_set_policy")


def gtr_gla_get_policy() -> int:
    return int(load_library().gtr_gla_get_policy())


def gtr_gla_plan(B, H, grid_h, grid_w, d_k, d_v, chunk, is_fp32,
                 lowrank: bool = False) -> Tuple[int, int, int]:
    """(kernel, span, grid) of the launch a call would make: kernel 1 generic, 2 fused,
    3 fused with the outputs kept in registers (long sequences), 4 the span
    kernels. lowrank: of a gtr_gla_fwd_lowrank call (gtr_gla_plan_lowrank)."""
    kern, span, grid = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    lib = load_library()
    fn = lib.gtr_gla_plan_lowrank if lowrank else lib.gtr_gla_plan
    r = fn(B, H, grid_h, grid_w, d_k, d_v, chunk, int(is_fp32), ctypes.byref(kern),
           ctypes.byref(span), ctypes.byref(grid))
    _raise(r, "gtr_gla_plan_lowrank" if lowrank else "gtr_gla_plan")
    return kern.value, span.value, grid.value


def gtr_gla_workspace_status(workspace=None, workspace_bytes: int = 0, stream=None) -> int:
    """Wait for the stream, read and clear a workspace's error word (None: the library's
    own workspaces for this stream), re-initialising a flagged workspace. Returns the
    status (OK, ERR_EXCHANGE or ERR_WS_STATE) rather than raising on those two."""
    r = load_library().gtr_gla_workspace_status(_ptr(workspace), workspace_bytes,
                                                _stream(stream))
    if r not in (OK, ERR_EXCHANGE, ERR_WS_STATE):
        _raise(r, "gtr_gla_workspace_status")
    return r


def gtr_gla_set_exchange_wait(wait_us: int, fault: int = 0) -> None:
    _raise(load_library().gtr_gla_set_exchange_wait(int(wait_us), int(fault)),
           "gtr_gla_set_exchange_wait")


def gtr_gla_status_str(status: int) -> str:
    try:
        return load_library().gtr_gla_status_str(int(status)).decode()
    except RuntimeError:
        return f"status {status}"


def forward(q, k, v, log_gamma, grid_h: int, grid_w: int, dir, chunk: int = 64,
            out=None, final_state=None, stream=None, initial_state=None, gate=None,
            norm_weight=None, norm_eps: float = 1e-5):
    """Allocate outputs (if not given) and run the forward for [B, L, H, d] tensors.

    Returns (out, final_state). fp16 inputs take gtr_gla_fwd, fp32 gtr_gla_fwd_f32;
    with an initial state or an output gate, gtr_gla_fwd_ex.
    """
    import torch
    if isinstance(dir, str):
        dir = DIRS[dir]
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, L, H, dv), dtype=q.dtype, device=q.device)
    if final_state is None:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    if initial_state is not None or gate is not None:
        gtr_gla_fwd_ex(q, k, v, log_gamma, initial_state, gate, norm_weight, norm_eps, B, H,
                       grid_h, grid_w, dk, dv, int(dir), chunk, int(q.dtype == torch.float32), out,
                       final_state, stream=stream)
        return out, final_state
    fn = gtr_gla_fwd_f32 if q.dtype == torch.float32 else gtr_gla_fwd
    fn(q, k, v, log_gamma, B, H, grid_h, grid_w, dk, dv, int(dir), chunk, out, final_state, stream)
    return out, final_state


def forward_lowrank(q, k, v, x, w1, w2, gate_bias, grid_h: int, grid_w: int, dir,
                    chunk: int = 64, inv_tau: float = 1.0 / 16, out=None, final_state=None,
                    stream=None, initial_state=None, gate=None, norm_weight=None,
                    norm_eps: float = 1e-5):
    """forward() with the gate projected from x [B, L, C] (gtr_gla_fwd_lowrank).

    w1 [C, 16], w2 [16, H d_k] and gate_bias [H d_k] are fp32. Returns (out, final_state).
    """
    import torch
    if isinstance(dir, str):
        dir = DIRS[dir]
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    C = x.shape[-1]
    if out is None:
        out = torch.empty((B, L, H, dv), dtype=q.dtype, device=q.device)
    if final_state is None:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    gtr_gla_fwd_lowrank(q, k, v, x, w1, w2, gate_bias, inv_tau, C, initial_state, gate,
                        norm_weight, norm_eps, B, H, grid_h, grid_w, dk, dv, int(dir), chunk,
                        int(q.dtype == torch.float32), out, final_state, stream=stream)
    return out, final_state


def gtr_sswiglu_fwd(x, w_g, w_v, conv_w, conv_b, w_o, B: int, grid_h: int, grid_w: int, C: int,
                    Hd: int, y, workspace=None, workspace_bytes: int = 0, stream=None) -> None:
    """Spatial SwiGLU: y = (SiLU(x w_g^T) * DWConv3x3(x w_v^T)) w_o^T (fp16 tensors,
    fp32 convolution weights [Hd, 3, 3] and bias [Hd] or None)."""
    import torch
    if min(B, grid_h, grid_w, C, Hd) >= 1:
        L = grid_h * grid_w
        _check(x, "x", torch.float16, B * L * C)
        _check(w_g, "w_g", torch.float16, Hd * C)
        _check(w_v, "w_v", torch.float16, Hd * C)
        _check(conv_w, "conv_w", torch.float32, Hd * 9)
        _check(conv_b, "conv_b", torch.float32, Hd)
        _check(w_o, "w_o", torch.float16, C * Hd)
        _check(y, "y", torch.float16, B * L * C)
    r = load_library().gtr_sswiglu_fwd(_ptr(x), _ptr(w_g), _ptr(w_v), _ptr(conv_w), _ptr(conv_b),
                                       _ptr(w_o), B, grid_h, grid_w, C, Hd, _ptr(y),
                                       _ptr(workspace), workspace_bytes, _stream(stream))
    _raise(r, "gtr_sswiglu_fwd")


def gtr_sswiglu_workspace_bytes(B: int, grid_h: int, grid_w: int, C: int, Hd: int) -> int:
    return int(load_library().gtr_sswiglu_workspace_bytes(B, grid_h, grid_w, C, Hd))


def sswiglu(x, w_g, w_v, conv_w, conv_b, w_o, grid_h: int, grid_w: int, y=None, stream=None):
    """Allocate y (if not given) and run the Spatial SwiGLU mixer for x [B, L, C]."""
    import torch
    B, L, C = x.shape
    Hd = w_g.shape[0]
    if y is None:
        y = torch.empty((B, L, w_o.shape[0]), dtype=x.dtype, device=x.device)
    gtr_sswiglu_fwd(x, w_g, w_v, conv_w, conv_b, w_o, B, grid_h, grid_w, C, Hd, y,
                    stream=stream)
    return y
