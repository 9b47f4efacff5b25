"""GPU parity of gtr_gla_fwd_lowrank against the fp64 oracle: the gate computed
from the input by the rank-16 projection, log_gamma = (1/tau) logsigmoid(x W1
W2 + b) (GTR summary page, section 核心方法), on every kernel family (fused
one-chunk spans, parked spans, register-kept spans, streamed spans, generic
fp16 and fp32), every scan order, feature widths that take the tiled and the
plain projection kernel, a gate range wide enough for the exact score path,
and together with the initial state and the output gate.

Expected values: oracle.lowrank_gate (fp64) on the same rounded x, W1, W2 and
bias, then oracle.recurrent / recurrent_init / rmsnorm_gate. Bar: max|gpu -
oracle| / max|oracle| over a tensor, 5e-3 for fp16 and 1e-5 for fp32 inputs.
"""
import os
import sys

import numpy as np
import pytest

import gla_synth
import oracle

torch = pytest.importorskip("torch")
import chunkwise_gated_recurrence_amd as gla  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = {"fp16": 5e-3, "fp32": 1e-5}
DIRS = ["l2r", "r2l", "t2b", "b2t"]
EPS = 1e-5
INV_TAU = 1.0 / 16

BASE = gla_synth.WORKLOADS["img640"]
TINY = gla_synth.WORKLOADS["tiny"]
# (name, workload, feature width C, policy, span env, register-kept env)
CASES = [
    ("fused-one", BASE.with_(H=3, seed=61), 384, gla.POLICY_AUTO, None, None),
    ("fused-parked", BASE.with_(B=2, H=2, grid_h=30, grid_w=30, seed=62), 384, gla.POLICY_FUSED,
     "4", None),
    ("fused-rk", BASE.with_(B=2, H=2, grid_h=30, grid_w=30, seed=63), 384, gla.POLICY_FUSED,
     "3", "1"),
    ("fused-streamed", BASE.with_(H=2, grid_h=40, grid_w=40, seed=64), 384, gla.POLICY_FUSED,
     "3", None),
    ("generic-fp16", BASE.with_(H=2, grid_h=24, grid_w=20, seed=65), 384, gla.POLICY_GENERIC,
     None, None),
    ("generic-fp32", TINY.with_(d_k=64, d_v=64, grid_h=20, grid_w=21, H=2, seed=66), 96,
     gla.POLICY_AUTO, None, None),
    # the pages' operator shape, d_k = 32
    ("fused-one-dk32", BASE.with_(d_k=32, H=3, seed=67), 384, gla.POLICY_AUTO, None, None),
    ("fused-rk-dk32", BASE.with_(d_k=32, B=2, H=2, grid_h=30, grid_w=30, seed=68), 768,
     gla.POLICY_FUSED, "3", "1"),
]


@pytest.fixture(autouse=True)
def clean_env():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    gla.load_library()
    yield
    gla.gtr_gla_set_policy(gla.POLICY_AUTO)
    os.environ.pop("GTR_GLA_SPAN", None)
    os.environ.pop("GTR_GLA_RK", None)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def setup(policy, span, rk):
    gla.gtr_gla_set_policy(policy)
    for key, val in (("GTR_GLA_SPAN", span), ("GTR_GLA_RK", rk)):
        if val is None:
            os.environ.pop(key, None)
        else:
            os.environ[key] = val


def reference_gate(w, x, w1, w2, bias, inv_tau=INV_TAU):
    lg = oracle.lowrank_gate(x, w1, w2, bias, inv_tau)
    return lg.reshape(w.B, w.L, w.H, w.d_k)


def check(tag, w, d, o, s, o_ref, s_ref):
    eo, es = oracle.rel_err(o, o_ref), oracle.rel_err(s, s_ref)
    tol = TOL[w.dtype]
    say(f"[case] {tag} B={w.B} H={w.H} grid={w.grid_h}x{w.grid_w} d_k={w.d_k} {w.dtype} dir={d} "
        f"plan={gla.gtr_gla_plan(w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, w.chunk, int(w.dtype == 'fp32'), lowrank=True)} "
        f"err_o={eo:.3e} err_S={es:.3e} (tol {tol:g})")
    assert np.isfinite(o.astype(np.float64)).all() and np.isfinite(s).all()
    assert eo <= tol and es <= tol


def run_case(w, C, d, seed, inv_tau=INV_TAU, bias_std=0.5, x_offset=0, **kw):
    q, k, v, _ = gla_synth.generate(w)
    x, w1, w2, bias = gla_synth.generate_lowrank(w, C, seed, bias_std=bias_std)
    if x_offset:
        # x starting x_offset elements into its allocation (not 16-byte aligned)
        buf = torch.empty(x.size + x_offset, dtype=torch.float16 if w.dtype == "fp16"
                          else torch.float32, device="cuda")
        xd = buf[x_offset:].view(x.shape)
        xd.copy_(dev(x))
    else:
        xd = dev(x)
    out, fs = gla.forward_lowrank(dev(q), dev(k), dev(v), xd, dev(w1), dev(w2), dev(bias),
                                  w.grid_h, w.grid_w, d, inv_tau=inv_tau, **kw)
    torch.cuda.synchronize()
    lg = reference_gate(w, x, w1, w2, bias, inv_tau)
    return (q, k, v, lg), out.cpu().numpy(), fs.cpu().numpy()


@pytest.mark.parametrize("d", DIRS)
@pytest.mark.parametrize("name,w,C,policy,span,rk", CASES, ids=[c[0] for c in CASES])
def test_lowrank_gate(name, w, C, policy, span, rk, d):
    setup(policy, span, rk)
    arrays, o, s = run_case(w, C, d, w.seed + 400)
    o_ref, s_ref = oracle.recurrent(*arrays, w.grid_h, w.grid_w, d)
    check(f"lowrank/{name}/C={C}", w, d, o, s, o_ref, s_ref)


# feature widths: 1 and 36 take the plain projection kernel, 96 the tiled fp32
# one, 256 (and 384, 768 above) the fp16 MFMA one; an x that starts 2 bytes
# into its allocation takes the plain kernel too
@pytest.mark.parametrize("C,x_offset", [(1, 0), (36, 0), (96, 0), (256, 0), (384, 1)])
@pytest.mark.parametrize("name,w,_c,policy,span,rk", [CASES[0], CASES[4]],
                         ids=[CASES[0][0], CASES[4][0]])
def test_lowrank_feature_widths(name, w, _c, policy, span, rk, C, x_offset):
    setup(policy, span, rk)
    arrays, o, s = run_case(w, C, "t2b", w.seed + 500 + C, x_offset=x_offset)
    o_ref, s_ref = oracle.recurrent(*arrays, w.grid_h, w.grid_w, "t2b")
    check(f"lowrank-C/{name}/C={C}/off={x_offset}", w, "t2b", o, s, o_ref, s_ref)


@pytest.mark.parametrize("name,w,C,policy,span,rk", CASES[:5], ids=[c[0] for c in CASES[:5]])
def test_lowrank_wide_gate_range(name, w, C, policy, span, rk):
    """tau = 1 and a bias near -4: about -4 of log decay per token, far past the
    range the factorised in-chunk scores cover, so the exact score path runs."""
    setup(policy, span, rk)
    ww = w.with_(gate_mu=-4.0)
    arrays, o, s = run_case(ww, C, "b2t", w.seed + 600, inv_tau=1.0, bias_std=1.0)
    assert arrays[3].min() < -4.0
    o_ref, s_ref = oracle.recurrent(*arrays, ww.grid_h, ww.grid_w, "b2t")
    check(f"lowrank-wide/{name}", ww, "b2t", o, s, o_ref, s_ref)


@pytest.mark.parametrize("name,w,C,policy,span,rk", CASES, ids=[c[0] for c in CASES])
def test_lowrank_with_initial_state_and_output_gate(name, w, C, policy, span, rk):
    setup(policy, span, rk)
    rng = np.random.default_rng(w.seed + 700)
    S0 = (0.5 * rng.standard_normal((w.B, w.H, w.d_k, w.d_v))).astype(np.float32)
    dt = np.float16 if w.dtype == "fp16" else np.float32
    gate = (2.0 * rng.standard_normal((w.B, w.L, w.H, w.d_v))).astype(dt)
    nw = rng.uniform(0.5, 1.5, w.d_v).astype(np.float32)
    arrays, y, s = run_case(w, C, "r2l", w.seed + 800, initial_state=dev(S0), gate=dev(gate),
                            norm_weight=dev(nw), norm_eps=EPS)
    o_ref, s_ref = oracle.recurrent_init(*arrays, S0, w.grid_h, w.grid_w, "r2l")
    y_ref = oracle.rmsnorm_gate(o_ref, gate, nw, EPS)
    check(f"lowrank-both/{name}", w, "r2l", y, s, y_ref, s_ref)


@pytest.mark.parametrize("name,w,C,policy,span,rk", [CASES[0], CASES[2], CASES[4]],
                         ids=[CASES[0][0], CASES[2][0], CASES[4][0]])
def test_lowrank_caller_workspace(name, w, C, policy, span, rk):
    """A caller-managed workspace of gtr_gla_lowrank_workspace_bytes, used by two
    calls in a row (a plain forward between them): the same results as the
    library's own workspace, bit for bit."""
    setup(policy, span, rk)
    q, k, v, lg0 = [dev(a) for a in gla_synth.generate(w)]
    x, w1, w2, bias = [dev(a) for a in gla_synth.generate_lowrank(w, C, w.seed + 900)]
    is32 = int(w.dtype == "fp32")
    nbytes = gla.gtr_gla_lowrank_workspace_bytes(w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v,
                                                 w.chunk, is32)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    gla.gtr_gla_workspace_init(ws, nbytes)
    ref_o, ref_s = gla.forward_lowrank(q, k, v, x, w1, w2, bias, w.grid_h, w.grid_w, "l2r")
    outs = []
    for _ in range(2):
        o = torch.empty_like(ref_o)
        s = torch.empty_like(ref_s)
        gla.gtr_gla_fwd_lowrank(q, k, v, x, w1, w2, bias, INV_TAU, C, None, None, None, EPS,
                                w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, gla.L2R, w.chunk,
                                is32, o, s, workspace=ws, workspace_bytes=nbytes)
        gla.forward(q, k, v, lg0, w.grid_h, w.grid_w, "l2r")
        outs.append((o, s))
    torch.cuda.synchronize()
    say(f"[case] lowrank-ws/{name} bytes={nbytes}")
    for o, s in outs:
        assert torch.equal(o, ref_o) and torch.equal(s, ref_s)
