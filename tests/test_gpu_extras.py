"""GPU parity of gtr_gla_fwd_ex's additions against the fp64 oracle: a nonzero
initial state, and the RMSNorm + SiLU output-gate epilogue (0539edu.com page,
appendix E.3.1), on every kernel family (fused one-chunk spans, parked spans,
register-kept spans, streamed spans, the span kernels at d_k = 64 and 32, the
gla_fused.hip kernels at d_k = 32 zero-padded to 64, generic fp16 and fp32)
and scan order.

Bar: as for the plain forward, max|gpu - oracle| / max|oracle| over a tensor,
5e-3 for fp16 and 1e-5 for fp32 inputs; the gated outputs are compared with
the oracle's epilogue applied to the oracle's (unrounded) outputs.
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

BASE = gla_synth.WORKLOADS["img640"]
TINY = gla_synth.WORKLOADS["tiny"]
# (name, workload, policy, span env, register-kept env, kernel-family env)
CASES = [
    ("fused-one", BASE.with_(H=3, seed=51), gla.POLICY_AUTO, None, None, "1"),
    ("fused-parked", BASE.with_(B=2, H=2, grid_h=30, grid_w=30, seed=52), gla.POLICY_FUSED, "4", None,
     "1"),
    ("fused-rk", BASE.with_(B=2, H=2, grid_h=30, grid_w=30, seed=53), gla.POLICY_FUSED, "3", "1", "1"),
    ("fused-streamed", BASE.with_(H=2, grid_h=40, grid_w=40, seed=54), gla.POLICY_FUSED, "3", None,
     "1"),
    ("generic-fp16", BASE.with_(H=2, grid_h=24, grid_w=20, seed=55), gla.POLICY_GENERIC, None, None,
     None),
    ("generic-fp32", TINY.with_(d_k=64, d_v=64, grid_h=20, grid_w=21, H=2, seed=56),
     gla.POLICY_AUTO, None, None, None),
    # the pages' operator shape, d_k = 32: the span kernels' 32-wide tiles (the default) ...
    ("span-one-dk32", BASE.with_(d_k=32, H=3, seed=57), gla.POLICY_AUTO, None, None, None),
    ("span-3-dk32", BASE.with_(d_k=32, B=2, H=2, grid_h=30, grid_w=30, seed=58),
     gla.POLICY_FUSED, "3", None, None),
    # ... and the gla_fused.hip kernels, zero-padded to 64
    ("fused-one-dk32", BASE.with_(d_k=32, H=3, seed=60), gla.POLICY_AUTO, None, None, "1"),
    ("fused-rk-dk32", BASE.with_(d_k=32, B=2, H=2, grid_h=30, grid_w=30, seed=61),
     gla.POLICY_FUSED, "3", "1", "1"),
    # the span kernels at d_k = 64
    ("span-one-dk64", BASE.with_(H=3, seed=62), gla.POLICY_AUTO, None, None, "2"),
    ("span-3-dk64", BASE.with_(B=2, H=2, grid_h=30, grid_w=30, seed=63), gla.POLICY_FUSED, "3", None,
     "2"),
]


@pytest.fixture(autouse=True)
def clean_env():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    gla.load_library()
    yield
    gla.gtr_gla_set_policy(gla.POLICY_AUTO)
    for key in ("GTR_GLA_SPAN", "GTR_GLA_RK", "GTR_GLA_KERNEL"):
        os.environ.pop(key, None)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def setup(policy, span, rk, kernel=None):
    gla.gtr_gla_set_policy(policy)
    for key, val in (("GTR_GLA_SPAN", span), ("GTR_GLA_RK", rk), ("GTR_GLA_KERNEL", kernel)):
        if val is None:
            os.environ.pop(key, None)
        else:
            os.environ[key] = val


def extras(w, seed):
    rng = np.random.default_rng(seed)
    S0 = (0.5 * rng.standard_normal((w.B, w.H, w.d_k, w.d_v))).astype(np.float32)
    dt = np.float16 if w.dtype == "fp16" else np.float32
    gate = (2.0 * rng.standard_normal((w.B, w.L, w.H, w.d_v))).astype(dt)
    nw = rng.uniform(0.5, 1.5, w.d_v).astype(np.float32)
    return S0, gate, nw


def errs(tag, w, d, o, s, o_ref, s_ref):
    eo, es = oracle.rel_err(o, o_ref), oracle.rel_err(s, s_ref)
    tol = TOL[w.dtype]
    say(f"[case] {tag} B={w.B} H={w.H} grid={w.grid_h}x{w.grid_w} {w.dtype} dir={d} "
        f"plan={gla.gtr_gla_plan(w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, w.chunk, int(w.dtype == 'fp32'))} "
        f"err_o={eo:.3e} err_S={es:.3e} (tol {tol:g})")
    assert np.isfinite(o.astype(np.float64)).all() and np.isfinite(s).all()
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("d", DIRS)
@pytest.mark.parametrize("name,w,policy,span,rk,kernel", CASES, ids=[c[0] for c in CASES])
def test_initial_state(name, w, policy, span, rk, kernel, d):
    arrays = gla_synth.generate(w)
    S0, _, _ = extras(w, w.seed + 100)
    setup(policy, span, rk, kernel)
    q, k, v, lg = [dev(a) for a in arrays]
    o, s = gla.forward(q, k, v, lg, w.grid_h, w.grid_w, d, initial_state=dev(S0))
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrent_init(*arrays, S0, w.grid_h, w.grid_w, d)
    errs(f"init/{name}", w, d, o.cpu().numpy(), s.cpu().numpy(), o_ref, s_ref)


@pytest.mark.parametrize("d", DIRS)
@pytest.mark.parametrize("name,w,policy,span,rk,kernel", CASES, ids=[c[0] for c in CASES])
def test_output_gate(name, w, policy, span, rk, kernel, d):
    arrays = gla_synth.generate(w)
    _, gate, nw = extras(w, w.seed + 200)
    setup(policy, span, rk, kernel)
    q, k, v, lg = [dev(a) for a in arrays]
    y, s = gla.forward(q, k, v, lg, w.grid_h, w.grid_w, d, gate=dev(gate), norm_weight=dev(nw),
                       norm_eps=EPS)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrent(*arrays, w.grid_h, w.grid_w, d)
    y_ref = oracle.rmsnorm_gate(o_ref, gate, nw, EPS)
    errs(f"gate/{name}", w, d, y.cpu().numpy(), s.cpu().numpy(), y_ref, s_ref)


@pytest.mark.parametrize("name,w,policy,span,rk,kernel", CASES[:3] + CASES[-2:],
                         ids=[c[0] for c in CASES[:3] + CASES[-2:]])
def test_both_additions_and_in_place_chaining(name, w, policy, span, rk, kernel):
    """Two calls over the top and bottom rows of an L->R scan, the second from the
    first's final state updated in place, with the output gate: the outputs and
    final state of one scan of the whole grid (oracle), and of one GPU call."""
    arrays = gla_synth.generate(w)
    _, gate, nw = extras(w, w.seed + 300)
    setup(policy, span, rk, kernel)
    gh, gw, h1 = w.grid_h, w.grid_w, w.grid_h // 3
    top = lambda x: np.ascontiguousarray(x[:, : h1 * gw])
    bot = lambda x: np.ascontiguousarray(x[:, h1 * gw:])
    fs = torch.empty((w.B, w.H, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
    y1, _ = gla.forward(*[dev(top(a)) for a in arrays], h1, gw, "l2r", final_state=fs,
                        gate=dev(top(gate)), norm_weight=dev(nw), norm_eps=EPS)
    y2, _ = gla.forward(*[dev(bot(a)) for a in arrays], gh - h1, gw, "l2r", final_state=fs,
                        initial_state=fs, gate=dev(bot(gate)), norm_weight=dev(nw), norm_eps=EPS)
    yw, sw = gla.forward(*[dev(a) for a in arrays], gh, gw, "l2r", gate=dev(gate),
                         norm_weight=dev(nw), norm_eps=EPS)
    torch.cuda.synchronize()
    y = np.concatenate([y1.cpu().numpy(), y2.cpu().numpy()], axis=1)
    o_ref, s_ref = oracle.recurrent(*arrays, gh, gw, "l2r")
    y_ref = oracle.rmsnorm_gate(o_ref, gate, nw, EPS)
    errs(f"chain/{name}", w, "l2r", y, fs.cpu().numpy(), y_ref, s_ref)
    errs(f"whole/{name}", w, "l2r", yw.cpu().numpy(), sw.cpu().numpy(), y_ref, s_ref)
