"""The C ABI on the host: the library loads, exports every declared symbol, and
rejects invalid arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

import chunkwise_gated_recurrence_amd as gla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("gtr_gla.h", "gtr_sswiglu.h")]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gla.LIB_PATH):
        from chunkwise_gated_recurrence_amd import build
        build.build()
    return gla.load_library()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(gtr_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_header_declares_the_api():
    names = declared_functions()
    assert "gtr_gla_fwd" in names and "gtr_gla_fwd_ws" in names and "gtr_sswiglu_fwd" in names
    assert set(names) == set(gla.EXPORTED)


def test_one_hip_runtime_per_process(lib):
    """Loaded before anything else touches torch, the binding still leaves one HIP
    runtime and one HSA runtime in the process (torch's): two would compete for
    the GPU and one of them would report no device."""
    import subprocess
    import sys
    code = ("import chunkwise_gated_recurrence_amd as g; g.load_library(); import torch; "
            "print(open('/proc/self/maps').read())")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                         check=True).stdout
    hip = {l.split()[-1] for l in out.splitlines() if "libamdhip64" in l}
    hsa = {l.split()[-1] for l in out.splitlines() if "libhsa-runtime64" in l}
    assert len(hip) == 1 and len(hsa) == 1, (hip, hsa)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def _fwd(lib, ptrs, B=1, H=2, gh=4, gw=4, dk=64, dv=64, d=0, C=64, f32=False, ws=None, nws=0):
    q, k, v, g, o, fs = ptrs
    if ws is None and nws == 0:
        fn = lib.gtr_gla_fwd_f32 if f32 else lib.gtr_gla_fwd
        return fn(q, k, v, g, B, H, gh, gw, dk, dv, d, C, o, fs, None)
    fn = lib.gtr_gla_fwd_f32_ws if f32 else lib.gtr_gla_fwd_ws
    return fn(q, k, v, g, B, H, gh, gw, dk, dv, d, C, o, fs, ws, nws, None)


# Fake, well separated, never dereferenced device addresses: every call below
# fails validation before any HIP call.
BASE = 1 << 40
SEP = 1 << 32
PTRS = [BASE + i * SEP for i in range(6)]


@pytest.mark.parametrize("f32", [False, True])
def test_null_pointers(lib, f32):
    for i in range(5):
        ptrs = list(PTRS)
        ptrs[i] = None
        assert _fwd(lib, ptrs, f32=f32) == gla.ERR_NULL


@pytest.mark.parametrize("f32", [False, True])
def test_bad_sizes(lib, f32):
    for kw in (dict(B=0), dict(H=-1), dict(gh=0), dict(gw=0), dict(dk=0), dict(dv=0)):
        assert _fwd(lib, PTRS, f32=f32, **kw) == gla.ERR_SHAPE, kw
    assert _fwd(lib, PTRS, f32=f32, gh=1 << 16, gw=1 << 16) == gla.ERR_SHAPE
    assert _fwd(lib, PTRS, f32=f32, d=4) == gla.ERR_DIR
    assert _fwd(lib, PTRS, f32=f32, d=-1) == gla.ERR_DIR
    for C in (0, 1, 48, 256):
        assert _fwd(lib, PTRS, f32=f32, C=C) == gla.ERR_CHUNK
    assert _fwd(lib, PTRS, f32=f32, dk=129) == gla.ERR_UNSUPPORTED
    assert _fwd(lib, PTRS, f32=f32, dv=513) == gla.ERR_UNSUPPORTED


def test_aliasing_outputs(lib):
    p = list(PTRS)
    p[4] = p[2] + 64          # out inside v
    assert _fwd(lib, p) == gla.ERR_ALIAS
    p = list(PTRS)
    p[5] = p[0]               # final_state on q
    assert _fwd(lib, p) == gla.ERR_ALIAS
    p = list(PTRS)
    p[5] = p[4]               # final_state on out
    assert _fwd(lib, p) == gla.ERR_ALIAS


def test_workspace_checks(lib):
    # fp32 always takes the generic kernels: the 256-byte header, then U/S (d_k*d_v)
    # and d (d_k) per chunk
    n = lib.gtr_gla_workspace_bytes(2, 3, 10, 13, 32, 16, 64, 1)
    chunks = 2 * 3 * ((10 * 13 + 63) // 64)
    assert n == 256 + chunks * (32 * 16 + 32) * 4
    assert lib.gtr_gla_workspace_bytes(0, 3, 10, 13, 32, 16, 64, 1) == 0
    assert lib.gtr_gla_workspace_bytes(2, 3, 10, 13, 32, 16, 48, 1) == 0
    assert _fwd(lib, PTRS, B=2, H=3, gh=10, gw=13, dk=32, dv=16, f32=True, ws=None, nws=1) == \
        gla.ERR_WORKSPACE
    assert _fwd(lib, PTRS, B=2, H=3, gh=10, gw=13, dk=32, dv=16, f32=True,
                ws=BASE + 7 * SEP, nws=n - 1) == gla.ERR_WORKSPACE
    assert lib.gtr_gla_workspace_init(None, 16, None) == gla.ERR_NULL
    assert lib.gtr_gla_workspace_init(BASE, 0, None) == gla.ERR_WORKSPACE


def test_policy_and_plan(lib):
    assert lib.gtr_gla_set_policy(7) == gla.ERR_POLICY
    assert lib.gtr_gla_set_policy(-1) == gla.ERR_POLICY
    old = lib.gtr_gla_get_policy()
    assert lib.gtr_gla_set_policy(gla.POLICY_GENERIC) == gla.OK
    assert lib.gtr_gla_get_policy() == gla.POLICY_GENERIC
    k, s, g = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    assert lib.gtr_gla_plan(1, 6, 40, 40, 64, 64, 64, 0, ctypes.byref(k), ctypes.byref(s),
                            ctypes.byref(g)) == gla.OK
    assert (k.value, s.value, g.value) == (1, 1, 6 * 25)
    # fp32 never takes the fused kernel
    assert lib.gtr_gla_set_policy(gla.POLICY_FUSED) == gla.OK
    assert lib.gtr_gla_plan(1, 6, 40, 40, 64, 64, 64, 1, ctypes.byref(k), None, None) == gla.OK
    assert k.value == 1
    assert lib.gtr_gla_plan(1, 6, 40, 40, 64, 64, 48, 1, None, None, None) == gla.ERR_CHUNK
    assert lib.gtr_gla_set_policy(old) == gla.OK


def test_status_strings(lib):
    seen = set()
    for s in range(10):
        txt = lib.gtr_gla_status_str(s).decode()
        assert txt and txt != "unknown status"
        seen.add(txt)
    assert len(seen) == 10
    assert lib.gtr_gla_status_str(99).decode() == "unknown status"


def _fwd_ex(lib, ptrs, init=None, gate=None, nw=None, eps=1e-5, B=1, H=2, gh=4, gw=4, dk=64,
            dv=64, f32=0, fs="auto"):
    q, k, v, g, o, f = ptrs
    if fs != "auto":
        f = fs
    return lib.gtr_gla_fwd_ex(q, k, v, g, init, gate, nw, eps, B, H, gh, gw, dk, dv, 0, 64, f32,
                              o, f, None, 0, None)


def test_fwd_ex_checks_its_additions(lib):
    """gtr_gla_fwd_ex: a gate needs a weight and a finite eps >= 0; an addition may not
    overlap an output, except an initial state that is the final state itself."""
    far = BASE + 10 * SEP
    # a gate without a weight
    assert _fwd_ex(lib, PTRS, gate=far) == gla.ERR_NULL
    # eps must be finite and >= 0
    for eps in (-1e-3, float("nan"), float("inf")):
        assert _fwd_ex(lib, PTRS, gate=far, nw=far + SEP, eps=eps) == gla.ERR_VALUE
    # the additions must not overlap the outputs
    out, fs = PTRS[4], PTRS[5]
    assert _fwd_ex(lib, PTRS, gate=out + 64, nw=far) == gla.ERR_ALIAS
    assert _fwd_ex(lib, PTRS, gate=far, nw=out) == gla.ERR_ALIAS
    assert _fwd_ex(lib, PTRS, gate=far, nw=fs + 8) == gla.ERR_ALIAS
    assert _fwd_ex(lib, PTRS, init=out + 16) == gla.ERR_ALIAS
    assert _fwd_ex(lib, PTRS, init=fs + 16) == gla.ERR_ALIAS
    # the base checks still apply first
    assert _fwd_ex(lib, PTRS, gate=far, nw=far + SEP, B=0) == gla.ERR_SHAPE
    ptrs = list(PTRS)
    ptrs[0] = None
    assert _fwd_ex(lib, ptrs, init=far) == gla.ERR_NULL
    assert "norm_eps" in gla.gtr_gla_status_str(gla.ERR_VALUE)


def _fwd_lr(lib, ptrs, x="far", w1="far", w2="far", bias="far", inv_tau=1.0 / 16, C=96, B=1,
            H=2, gh=4, gw=4, dk=64, dv=64, f32=0, init=None):
    q, k, v, _, o, f = ptrs
    far = BASE + 10 * SEP
    x = far if x == "far" else x
    w1 = far + SEP if w1 == "far" else w1
    w2 = far + 2 * SEP if w2 == "far" else w2
    bias = far + 3 * SEP if bias == "far" else bias
    return lib.gtr_gla_fwd_lowrank(q, k, v, x, w1, w2, bias, inv_tau, C, init, None, None, 1e-5,
                                   B, H, gh, gw, dk, dv, 0, 64, f32, o, f, None, 0, None)


def test_fwd_lowrank_checks_its_inputs(lib):
    """gtr_gla_fwd_lowrank: x, W1, W2 and the bias are required, C >= 1, inv_tau finite and
    > 0, and none of them may overlap an output; log_gamma is not an input."""
    for name in ("x", "w1", "w2", "bias"):
        assert _fwd_lr(lib, PTRS, **{name: None}) == gla.ERR_NULL, name
    assert _fwd_lr(lib, PTRS, C=0) == gla.ERR_SHAPE
    for t in (0.0, -1.0, float("nan"), float("inf")):
        assert _fwd_lr(lib, PTRS, inv_tau=t) == gla.ERR_VALUE, t
    out, fs = PTRS[4], PTRS[5]
    assert _fwd_lr(lib, PTRS, x=out + 64) == gla.ERR_ALIAS
    assert _fwd_lr(lib, PTRS, w2=fs + 4) == gla.ERR_ALIAS
    assert _fwd_lr(lib, PTRS, bias=out) == gla.ERR_ALIAS
    # the base checks still apply; no log_gamma is needed
    assert _fwd_lr(lib, PTRS, B=0) == gla.ERR_SHAPE
    ptrs = list(PTRS)
    ptrs[3] = None
    assert _fwd_lr(lib, ptrs, B=0) == gla.ERR_SHAPE
    ptrs[0] = None
    assert _fwd_lr(lib, ptrs) == gla.ERR_NULL
    assert "inv_tau" in gla.gtr_gla_status_str(gla.ERR_VALUE)


def test_lowrank_workspace_size(lib):
    """The low-rank call's workspace: the kernels' own, then x W1 in fp32 (16 per token), and
    on the generic path log_gamma too."""
    B, H, gh, gw, dk, dv = 2, 3, 10, 13, 32, 16
    base = lib.gtr_gla_workspace_bytes(B, H, gh, gw, dk, dv, 64, 1)
    up = lambda n: (n + 255) // 256 * 256
    rows = B * gh * gw
    n = lib.gtr_gla_lowrank_workspace_bytes(B, H, gh, gw, dk, dv, 64, 1)
    assert n == up(base) + up(rows * 16 * 4) + up(rows * H * dk * 4)
    assert lib.gtr_gla_lowrank_workspace_bytes(0, H, gh, gw, dk, dv, 64, 1) == 0


def _ss(lib, x=BASE, wg=BASE + SEP, wv=BASE + 2 * SEP, cw=BASE + 3 * SEP, cb=BASE + 4 * SEP,
        wo=BASE + 5 * SEP, y=BASE + 6 * SEP, B=1, gh=4, gw=5, C=64, Hd=128, ws=None, nws=0):
    return lib.gtr_sswiglu_fwd(x, wg, wv, cw, cb, wo, B, gh, gw, C, Hd, y, ws, nws, None)


def test_sswiglu_checks():
    """gtr_sswiglu_fwd: required pointers, sizes (C, Hd multiples of 64), aliasing of y
    and of a caller workspace, workspace size; nothing launches on a failed check."""
    lib = gla.load_library()
    for name in ("x", "wg", "wv", "cw", "wo", "y"):
        assert _ss(lib, **{name: None}) == gla.ERR_NULL, name
    for kw in (dict(B=0), dict(gh=0), dict(gw=-1), dict(C=0), dict(Hd=0)):
        assert _ss(lib, **kw) == gla.ERR_SHAPE, kw
    for kw in (dict(C=96), dict(Hd=100), dict(Hd=192), dict(C=8256), dict(gh=1 << 15, gw=1 << 15)):
        assert _ss(lib, **kw) == gla.ERR_UNSUPPORTED, kw
    assert _ss(lib, y=BASE + 64) == gla.ERR_ALIAS
    assert _ss(lib, y=BASE + 5 * SEP + 2) == gla.ERR_ALIAS
    n = lib.gtr_sswiglu_workspace_bytes(2, 4, 5, 64, 128)
    assert n == 2 * 20 * 128 * 2
    assert lib.gtr_sswiglu_workspace_bytes(2, 4, 5, 96, 128) == 0
    assert lib.gtr_sswiglu_workspace_bytes(2, 4, 5, 64, 64) == 0
    assert _ss(lib, B=2, ws=BASE + 8 * SEP, nws=n - 1) == gla.ERR_WORKSPACE
    assert _ss(lib, B=2, ws=BASE + 6 * SEP + 16, nws=n) == gla.ERR_ALIAS
    assert _ss(lib, B=2, ws=BASE + 16, nws=n) == gla.ERR_ALIAS


def test_status_and_exchange_wait_validation(lib):
    """The status query and the exchange-wait hook check their arguments before
    any HIP call; the new status codes have descriptions."""
    assert lib.gtr_gla_workspace_status(BASE, 255, None) == gla.ERR_WORKSPACE
    assert lib.gtr_gla_workspace_status(BASE, 0, None) == gla.ERR_WORKSPACE
    assert lib.gtr_gla_set_exchange_wait(0, 0) == gla.ERR_VALUE
    assert lib.gtr_gla_set_exchange_wait(10 ** 7 + 1, 0) == gla.ERR_VALUE
    assert lib.gtr_gla_set_exchange_wait(20000, 0) == gla.OK
    for st in (gla.ERR_EXCHANGE, gla.ERR_WS_STATE):
        text = gla.gtr_gla_status_str(st)
        assert text and "unknown" not in text and "NaN" in text


def test_noalloc_scratch_limit(lib):
    """gtr_gla_fwd_noalloc refuses a call whose workspace exceeds its static scratch
    (before any HIP call), and reports invalid sizes as gtr_gla_fwd does."""
    need = lib.gtr_gla_workspace_bytes(1, 16, 128, 128, 64, 32, 64, 0)
    assert need > gla.NOALLOC_SCRATCH_BYTES
    q, k, v, g, o, fs = PTRS
    assert lib.gtr_gla_fwd_noalloc(q, k, v, g, 1, 16, 128, 128, 64, 32, 0, 64, o, fs,
                                   None) == gla.ERR_SCRATCH
    assert lib.gtr_gla_fwd_noalloc(q, k, v, g, 0, 16, 128, 128, 64, 32, 0, 64, o, fs,
                                   None) == gla.ERR_SHAPE
    assert lib.gtr_gla_fwd_noalloc(q, k, v, g, 1, 2, 8, 8, 64, 64, 9, 64, o, fs,
                                   None) == gla.ERR_DIR
    assert "scratch" in gla.gtr_gla_status_str(gla.ERR_SCRATCH)
