"""GPU parity: the HIP path against the fp64 oracle, element by element.

Bar (max|gpu - oracle| / max|oracle| over a whole tensor, separately for the
outputs and the final state): 5e-3 for fp16 inputs, 1e-5 for fp32 inputs.
Workloads are the seeded synthetic grids of gla_synth (full sizes), in the
launch configuration the benchmark times, plus ragged and degenerate shapes,
every scan order, every launch policy and span, and the decay extremes.
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
_oracle_cache = {}


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    gla.load_library()
    yield
    gla.gtr_gla_set_policy(gla.POLICY_AUTO)
    for key in ("GTR_GLA_SPAN", "GTR_GLA_RK", "GTR_GLA_KERNEL"):
        os.environ.pop(key, None)


@pytest.fixture
def old_family():
    """The kernels of gla_fused.hip (one-chunk, parked, streamed and register-kept
    spans), selected with GTR_GLA_KERNEL=1 for the duration of a test."""
    os.environ["GTR_GLA_KERNEL"] = "1"
    yield
    os.environ.pop("GTR_GLA_KERNEL", None)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run_gpu(w, arrays, d, chunk=None):
    q, k, v, lg = [dev(a) for a in arrays]
    out, fs = gla.forward(q, k, v, lg, w.grid_h, w.grid_w, d, chunk=chunk or w.chunk)
    torch.cuda.synchronize()
    return out.cpu().numpy(), fs.cpu().numpy()


def ref(w, arrays, d, key=None):
    if key is not None and (key, d) in _oracle_cache:
        return _oracle_cache[(key, d)]
    r = oracle.recurrent(*arrays, w.grid_h, w.grid_w, d)
    if key is not None:
        _oracle_cache[(key, d)] = r
    return r


def check(w, arrays, d, tag, key=None, chunk=None, tol=None):
    say(f"[case] {tag} {w.name} B={w.B} H={w.H} grid={w.grid_h}x{w.grid_w} dk={w.d_k} dv={w.d_v} "
        f"{w.dtype} dir={d} chunk={chunk or w.chunk} policy={gla.gtr_gla_get_policy()} "
        f"span_env={os.environ.get('GTR_GLA_SPAN')} rk_env={os.environ.get('GTR_GLA_RK')} "
        f"kernel_env={os.environ.get('GTR_GLA_KERNEL')}")
    o, s = run_gpu(w, arrays, d, chunk)
    o_ref, s_ref = ref(w, arrays, d, key)
    eo, es = oracle.rel_err(o, o_ref), oracle.rel_err(s, s_ref)
    tol = tol or TOL[w.dtype]
    say(f"       err_o={eo:.3e} err_S={es:.3e} (tol {tol:g})")
    assert np.isfinite(o.astype(np.float64)).all() and np.isfinite(s).all()
    assert eo <= tol, f"outputs: {eo}"
    assert es <= tol, f"final state: {es}"
    return o, s


# --------------------------------------------------------------------------- workloads
@pytest.mark.parametrize("d", DIRS)
@pytest.mark.parametrize("name", list(gla_synth.WORKLOADS))
def test_workload_parity(name, d):
    gla.gtr_gla_set_policy(gla.POLICY_AUTO)
    w = gla_synth.WORKLOADS[name]
    arrays = gla_synth.generate(w)
    check(w, arrays, d, "auto", key=name)


@pytest.mark.parametrize("d", DIRS)
@pytest.mark.parametrize("name", ["img640", "img1024"])
def test_generic_policy_parity(name, d):
    gla.gtr_gla_set_policy(gla.POLICY_GENERIC)
    try:
        w = gla_synth.WORKLOADS[name]
        check(w, gla_synth.generate(w), d, "generic", key=name)
    finally:
        gla.gtr_gla_set_policy(gla.POLICY_AUTO)


@pytest.mark.parametrize("name,plan", [("img640", (2, 1, 150)), ("img1024", (3, 2, 384)),
                                       ("batched640", (4, 3, 432)), ("long2048", (3, 7, 444)),
                                       ("img640_dk32", (4, 1, 150))])
def test_default_plans(name, plan):
    """The launch policy's choice for the benchmark workloads (kernel 2: one
    chunk per workgroup while the grid fits at two per CU; kernel 3: the
    shortest register-kept span whose grid is resident; kernel 4, the span
    kernels, for 32-wide keys, and for 64-wide keys when a sequence takes at
    most 16 spans: batched640's 48 sequences of 9 spans). The grids assume the
    MI355X's 256 CUs and take at most 7/8 of the resident slots."""
    w = gla_synth.WORKLOADS[name]
    assert gla.gtr_gla_plan(w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, w.chunk, 0) == plan


@pytest.mark.parametrize("span", [1, 2, 4, 8])
@pytest.mark.parametrize("name", ["img1024", "ragged30"])
def test_fused_spans(name, span, old_family):
    w = gla_synth.WORKLOADS["img1024"]
    if name == "ragged30":
        w = w.with_(name="ragged30", B=2, H=3, grid_h=30, grid_w=30, seed=17)
    arrays = gla_synth.generate(w)
    gla.gtr_gla_set_policy(gla.POLICY_FUSED)
    os.environ["GTR_GLA_SPAN"] = str(span)
    try:
        kern, sp, _ = gla.gtr_gla_plan(w.B, w.H, w.grid_h, w.grid_w, 64, 64, 64, 0)
        assert (kern, sp) == (2, span)
        for d in DIRS:
            check(w, arrays, d, f"fused-span{span}", key=w.name)
    finally:
        os.environ.pop("GTR_GLA_SPAN", None)
        gla.gtr_gla_set_policy(gla.POLICY_AUTO)


@pytest.mark.parametrize("span", [2, 3, 5, 7])
@pytest.mark.parametrize("name", ["img1024", "ragged30"])
def test_fused_register_kept(name, span, old_family):
    """Spans whose every chunk's outputs stay in registers through the exchange
    while the next chunk's g, k, v are staged in LDS (the long-sequence variant);
    ragged30's last span is shorter than the others and its last chunk partial."""
    w = gla_synth.WORKLOADS["img1024"]
    if name == "ragged30":
        w = w.with_(name="ragged30", B=2, H=3, grid_h=30, grid_w=30, seed=17)
    arrays = gla_synth.generate(w)
    gla.gtr_gla_set_policy(gla.POLICY_FUSED)
    os.environ["GTR_GLA_SPAN"] = str(span)
    os.environ["GTR_GLA_RK"] = "1"
    try:
        kern, sp, _ = gla.gtr_gla_plan(w.B, w.H, w.grid_h, w.grid_w, 64, 64, 64, 0)
        assert (kern, sp) == (3, span)
        for d in DIRS:
            check(w, arrays, d, f"fused-rk-span{span}", key=w.name)
    finally:
        os.environ.pop("GTR_GLA_SPAN", None)
        os.environ.pop("GTR_GLA_RK", None)
        gla.gtr_gla_set_policy(gla.POLICY_AUTO)


@pytest.mark.parametrize("span,rk,kernel", [(1, None, 2), (4, None, 2), (3, None, 2), (3, "1", 3)],
                         ids=["one-chunk", "parked4", "streamed3", "rk3"])
def test_fused_dk32(span, rk, kernel, old_family):
    """The pages' operator shape (d_k = 32, d_v = 64) on every fused kernel family:
    the key dim is zero-padded to 64 on load, the final state keeps its 32 rows."""
    w = gla_synth.WORKLOADS["img640_dk32"].with_(name="dk32-30x30", B=2, H=2, grid_h=30, grid_w=30,
                                                 seed=19)
    arrays = gla_synth.generate(w)
    gla.gtr_gla_set_policy(gla.POLICY_FUSED)
    os.environ["GTR_GLA_SPAN"] = str(span)
    if rk:
        os.environ["GTR_GLA_RK"] = rk
    try:
        kern, sp, _ = gla.gtr_gla_plan(w.B, w.H, w.grid_h, w.grid_w, 32, 64, 64, 0)
        assert (kern, sp) == (kernel, span)
        for d in DIRS:
            check(w, arrays, d, f"fused-dk32-span{span}", key=w.name)
    finally:
        os.environ.pop("GTR_GLA_SPAN", None)
        os.environ.pop("GTR_GLA_RK", None)
        gla.gtr_gla_set_policy(gla.POLICY_AUTO)


@pytest.mark.parametrize("span", [1, 2, 3, 4, 5, 6, 7])
@pytest.mark.parametrize("dk", [64, 32])
@pytest.mark.parametrize("name", ["img1024", "ragged30"])
def test_span_kernels(name, dk, span):
    """The span kernels (GTR_GLA_KERNEL=2) at every span length, for both key
    widths they hold natively: every chunk's outputs stay in registers through
    the exchange while the next chunk's tiles stream into LDS; ragged30's last
    span is shorter than the others and its last chunk partial."""
    w = gla_synth.WORKLOADS["img1024"].with_(d_k=dk)
    if name == "ragged30":
        w = w.with_(name="ragged30", B=2, H=3, grid_h=30, grid_w=30, seed=17)
    key = w.name if dk == 64 else f"{w.name}-dk32"   # the dk=64 cases share the oracle runs above
    arrays = gla_synth.generate(w)
    os.environ["GTR_GLA_SPAN"] = str(span)
    os.environ["GTR_GLA_KERNEL"] = "2"
    try:
        kern, sp, _ = gla.gtr_gla_plan(w.B, w.H, w.grid_h, w.grid_w, dk, 64, 64, 0)
        assert (kern, sp) == (4, span)
        for d in DIRS:
            check(w, arrays, d, f"span-kernel-span{span}", key=key)
    finally:
        os.environ.pop("GTR_GLA_SPAN", None)
        os.environ.pop("GTR_GLA_KERNEL", None)


# --------------------------------------------------------------------------- odd shapes
BASE16 = gla_synth.WORKLOADS["img640"]
BASE32 = gla_synth.WORKLOADS["tiny"]
SHAPES = [
    ("tail30x30", BASE16.with_(grid_h=30, grid_w=30, H=2, seed=21)),
    ("nonsquare24x40", BASE16.with_(grid_h=24, grid_w=40, H=3, seed=22)),
    ("batch3", BASE16.with_(B=3, H=2, grid_h=20, grid_w=17, seed=23)),
    ("row1x100", BASE16.with_(grid_h=1, grid_w=100, H=2, seed=24)),
    ("col100x1", BASE16.with_(grid_h=100, grid_w=1, H=2, seed=25)),
    ("single1x1", BASE16.with_(grid_h=1, grid_w=1, H=2, seed=26)),
    ("dk32dv64", BASE16.with_(d_k=32, d_v=64, grid_h=24, grid_w=24, seed=27)),
    ("dk32dv32", BASE16.with_(d_k=32, d_v=32, grid_h=16, grid_w=16, seed=28)),
    ("dk128dv96", BASE16.with_(d_k=128, d_v=96, grid_h=12, grid_w=20, H=2, seed=29)),
    ("fp32_d64", BASE32.with_(d_k=64, d_v=64, grid_h=30, grid_w=30, H=2, seed=30)),
    ("fp32_ragged", BASE32.with_(d_k=32, d_v=48, grid_h=13, grid_w=11, B=2, H=3, seed=31)),
]


@pytest.mark.parametrize("d", DIRS)
@pytest.mark.parametrize("name,w", SHAPES, ids=[s[0] for s in SHAPES])
def test_shapes(name, w, d):
    check(w, gla_synth.generate(w), d, name, key=name)


@pytest.mark.parametrize("chunk", [16, 32, 64, 128])
def test_chunk_sizes(chunk):
    w = BASE16.with_(name="chunks", grid_h=20, grid_w=30, H=2, seed=41)
    arrays = gla_synth.generate(w)
    for d in DIRS:
        check(w, arrays, d, f"chunk{chunk}", key="chunks", chunk=chunk)


def _with_gates(w, lg_value, seed):
    q, k, v, _ = gla_synth.generate(w.with_(seed=seed))
    lg = np.full(q.shape, lg_value, dtype=q.dtype)
    return q, k, v, lg


@pytest.mark.parametrize("policy", [gla.POLICY_AUTO, gla.POLICY_GENERIC])
@pytest.mark.parametrize("lg_value", [0.0, -1.0, -1e4])
def test_decay_extremes(lg_value, policy):
    """gamma = 1 (plain causal linear attention), strong decay, and gamma -> 0."""
    w = BASE16.with_(name=f"decay{lg_value}", grid_h=32, grid_w=40, H=2)
    arrays = _with_gates(w, lg_value, 51)
    gla.gtr_gla_set_policy(policy)
    try:
        for d in DIRS:
            check(w, arrays, d, f"lg={lg_value}", key=w.name)
    finally:
        gla.gtr_gla_set_policy(gla.POLICY_AUTO)


@pytest.mark.parametrize("kernel_env,span", [("1", None), ("2", None), ("2", 3), ("2", 7)],
                         ids=["fused-auto", "span-auto", "span3", "span7"])
def test_mixed_decay_chunks(kernel_env, span):
    """Some chunks inside the factorised-score range and some far outside it,
    on spans of one chunk and of several (where a wide chunk sits between
    ordinary ones of the same span)."""
    w = BASE16.with_(name="mixed", grid_h=32, grid_w=64, H=2)
    q, k, v, lg = gla_synth.generate(w.with_(seed=61))
    lg = lg.astype(np.float32)
    lg[:, 640:1280] = -0.6          # ~ 55 log2 units per chunk: exact-score path
    lg[:, 1500] = -30.0             # one very small gate
    arrays = (q, k, v, lg.astype(np.float16))
    for key, val in (("GTR_GLA_KERNEL", kernel_env), ("GTR_GLA_SPAN", span)):
        if val is not None:
            os.environ[key] = str(val)
    try:
        if span is not None:
            kern, sp, _ = gla.gtr_gla_plan(w.B, w.H, w.grid_h, w.grid_w, 64, 64, 64, 0)
            assert (kern, sp) == (4, span)
        for d in DIRS:
            check(w, arrays, d, "mixed", key="mixed")
    finally:
        os.environ.pop("GTR_GLA_KERNEL", None)
        os.environ.pop("GTR_GLA_SPAN", None)


@pytest.mark.parametrize("lg_value", [0.0, -1.0, -1e4])
def test_span_decay_extremes(lg_value):
    """The decay extremes on a span of four chunks of the span kernels."""
    w = BASE16.with_(name=f"decay{lg_value}", grid_h=32, grid_w=40, H=2)
    arrays = _with_gates(w, lg_value, 51)
    os.environ["GTR_GLA_SPAN"] = "4"
    os.environ["GTR_GLA_KERNEL"] = "2"
    try:
        assert gla.gtr_gla_plan(w.B, w.H, w.grid_h, w.grid_w, 64, 64, 64, 0)[:2] == (4, 4)
        for d in DIRS:
            check(w, arrays, d, f"span4 lg={lg_value}", key=w.name)
    finally:
        os.environ.pop("GTR_GLA_SPAN", None)
        os.environ.pop("GTR_GLA_KERNEL", None)
