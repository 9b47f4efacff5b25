"""GPU parity of the Spatial SwiGLU mixer (gtr_sswiglu_fwd) against the fp64
oracle (oracle/sswiglu.py; GTR summary page, section 前置知识 › SwiGLU前馈块),
on the pages' model widths (C = 192 / 384 with Hd = 4 C, and Hd = 6 C), ragged
grids whose 8x8 tiles and 64-token output tiles are partial, degenerate grids,
batches, and without the convolution bias. The down projection uses 64x64
output tiles when they number at least the CU count and 64x32 tiles below
that: batch2-640 (300 tiles of 64x64) takes the first, the other cases the
second.

Bar: max|gpu - oracle| / max|oracle| <= 5e-3 over y (fp16 operands with fp32
accumulation; the gated hidden tensor and y are each rounded to fp16 once,
about 2^-11 of their size).
"""
import sys

import numpy as np
import pytest

import gla_synth
from oracle import sswiglu as ss

torch = pytest.importorskip("torch")
import chunkwise_gated_recurrence_amd as gla  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = 5e-3

# (name, B, grid_h, grid_w, C, Hd, bias)
CASES = [
    ("img640-L", 1, 40, 40, 384, 1536, True),
    ("batch2-640", 2, 40, 40, 384, 1536, True),
    ("ragged-S", 2, 30, 34, 192, 768, True),
    ("ratio6-X", 1, 24, 20, 384, 2304, True),
    ("no-bias", 1, 17, 23, 128, 256, False),
    ("grid-1x1", 1, 1, 1, 64, 128, True),
    ("grid-1x9", 2, 1, 9, 64, 128, True),
    ("grid-9x1", 1, 9, 1, 64, 256, True),
    ("grid-3x3", 3, 3, 3, 64, 384, True),
]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def rel_err(x, ref):
    return float(np.max(np.abs(x.astype(np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-30))


@pytest.fixture(autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    gla.load_library()


@pytest.mark.parametrize("name,B,gh,gw,C,Hd,bias", CASES, ids=[c[0] for c in CASES])
def test_sswiglu_parity(name, B, gh, gw, C, Hd, bias):
    ins = gla_synth.generate_sswiglu(B, gh, gw, C, Hd, seed=70 + len(name), bias=bias)
    y = gla.sswiglu(*[dev(a) for a in ins], gh, gw)
    torch.cuda.synchronize()
    ref = ss.sswiglu(*ins, gh, gw)
    err = rel_err(y.cpu().numpy(), ref)
    say(f"[case] sswiglu/{name} B={B} grid={gh}x{gw} C={C} Hd={Hd} bias={bias} err={err:.3e} (tol {TOL:g})")
    assert np.isfinite(y.cpu().numpy().astype(np.float64)).all()
    assert err <= TOL


def test_sswiglu_caller_workspace_matches():
    """A caller workspace of gtr_sswiglu_workspace_bytes gives the library-workspace
    result bit for bit, on two calls in a row with different shapes."""
    outs = []
    for (B, gh, gw, C, Hd) in ((1, 40, 40, 384, 1536), (2, 13, 11, 192, 768)):
        ins = [dev(a) for a in gla_synth.generate_sswiglu(B, gh, gw, C, Hd, seed=90)]
        ref = gla.sswiglu(*ins, gh, gw)
        n = gla.gtr_sswiglu_workspace_bytes(B, gh, gw, C, Hd)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(ref)
        gla.gtr_sswiglu_fwd(*ins, B, gh, gw, C, Hd, y, workspace=ws, workspace_bytes=n)
        outs.append((ref, y))
    torch.cuda.synchronize()
    for ref, y in outs:
        assert torch.equal(ref, y)
