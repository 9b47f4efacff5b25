"""HIP-graph capture of the entry points that take a caller workspace (they
allocate nothing): gtr_gla_fwd_ex with both additions, gtr_gla_fwd_lowrank and
gtr_sswiglu_fwd. Each call is first made eagerly (the reference), then captured
once and replayed several times with other eager work in between; every replay
must reproduce the eager result bit for bit (same kernels, same inputs, same
plan). A workspace of gtr_gla_workspace_bytes also serves gtr_gla_fwd_ex (the
size covers the kernel variant with the additions).
"""
import numpy as np
import pytest

import gla_synth

torch = pytest.importorskip("torch")
import chunkwise_gated_recurrence_amd as gla  # noqa: E402

pytestmark = pytest.mark.gpu

W = gla_synth.WORKLOADS["img640"].with_(H=3, grid_h=30, grid_w=34, seed=81)


@pytest.fixture(autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    gla.load_library()
    yield
    gla.gtr_gla_set_policy(gla.POLICY_AUTO)


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def replay_matches(call, outs, eager_between):
    """Capture call() into a graph (after a warm-up on the capture stream), then
    replay it four times, zeroing the outputs first and running eager work
    after each replay; every replay must equal the eager result."""
    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, ref):
            assert torch.equal(t, r), rep
        eager_between()
        torch.cuda.synchronize()


def eager_other():
    """A plain forward on other data and shape (the library's own workspace)."""
    w = gla_synth.WORKLOADS["img640"].with_(H=2, grid_h=17, grid_w=23, seed=82)
    o, s = gla.forward(*[dev(a) for a in gla_synth.generate(w)], w.grid_h, w.grid_w, "t2b")
    assert torch.isfinite(o.float()).all()


@pytest.mark.parametrize("d_k,family", [(64, None), (32, None), (64, "2")],
                         ids=["dk64-fused", "dk32-span", "dk64-span"])
def test_graph_fwd_ex_caller_workspace(d_k, family, monkeypatch):
    """On the gla_fused.hip kernels (d_k = 64 by default) and the span kernels
    (d_k = 32 by default, d_k = 64 forced)."""
    if family is not None:
        monkeypatch.setenv("GTR_GLA_KERNEL", family)
    w = W.with_(d_k=d_k)
    q, k, v, lg = [dev(a) for a in gla_synth.generate(w)]
    rng = np.random.default_rng(83)
    s0 = dev((0.5 * rng.standard_normal((w.B, w.H, w.d_k, w.d_v))).astype(np.float32))
    gate = dev(rng.standard_normal((w.B, w.L, w.H, w.d_v)).astype(np.float16))
    nw = dev(rng.uniform(0.5, 1.5, w.d_v).astype(np.float32))
    n = gla.gtr_gla_workspace_bytes(w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, w.chunk, 0)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    gla.gtr_gla_workspace_init(ws, n)
    o = torch.empty((w.B, w.L, w.H, w.d_v), dtype=torch.float16, device="cuda")
    fs = torch.empty((w.B, w.H, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
    # the library-workspace call gives the same result
    o_lib, fs_lib = gla.forward(q, k, v, lg, w.grid_h, w.grid_w, "b2t", initial_state=s0,
                                gate=gate, norm_weight=nw, norm_eps=1e-5)

    def call():
        gla.gtr_gla_fwd_ex(q, k, v, lg, s0, gate, nw, 1e-5, w.B, w.H, w.grid_h, w.grid_w,
                           w.d_k, w.d_v, gla.B2T, w.chunk, 0, o, fs, ws, n)

    call()
    torch.cuda.synchronize()
    assert torch.equal(o, o_lib) and torch.equal(fs, fs_lib)
    print(f"[case] graph fwd_ex plan={gla.gtr_gla_plan(w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, 64, 0)}",
          flush=True)
    replay_matches(call, [o, fs], eager_other)


def test_graph_fwd_lowrank():
    w = W
    q, k, v, _ = [dev(a) for a in gla_synth.generate(w)]
    C = 384
    x, w1, w2, b = [dev(a) for a in gla_synth.generate_lowrank(w, C, 84)]
    n = gla.gtr_gla_lowrank_workspace_bytes(w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, w.chunk, 0)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    gla.gtr_gla_workspace_init(ws, n)
    o = torch.empty((w.B, w.L, w.H, w.d_v), dtype=torch.float16, device="cuda")
    fs = torch.empty((w.B, w.H, w.d_k, w.d_v), dtype=torch.float32, device="cuda")

    def call():
        gla.gtr_gla_fwd_lowrank(q, k, v, x, w1, w2, b, 1.0 / 16, C, None, None, None, 1e-5,
                                w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, gla.L2R, w.chunk, 0,
                                o, fs, ws, n)

    print("[case] graph fwd_lowrank", flush=True)
    replay_matches(call, [o, fs], eager_other)


def test_graph_sswiglu():
    B, gh, gw, C, Hd = 1, 30, 34, 192, 768
    ins = [dev(a) for a in gla_synth.generate_sswiglu(B, gh, gw, C, Hd, seed=85)]
    n = gla.gtr_sswiglu_workspace_bytes(B, gh, gw, C, Hd)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    y = torch.empty((B, gh * gw, C), dtype=torch.float16, device="cuda")

    def call():
        gla.gtr_sswiglu_fwd(*ins, B, gh, gw, C, Hd, y, workspace=ws, workspace_bytes=n)

    print("[case] graph sswiglu", flush=True)
    replay_matches(call, [y], eager_other)
