"""GPU invariants of the HIP path that hold at any size.

* Direction folding changes addresses only: the output for scan order `dir`
  equals the left-to-right output on the correspondingly reversed/transposed
  inputs, bit for bit, for the generic kernels and both fused families (the
  gla_fused.hip kernels and the span kernels, each at d_k = 64 and 32) alike
  (the two calls have the same B, H and L, so the same plan, chunk contents
  and arithmetic; the exchange's fold order is fixed).
* Repeated calls agree bit for bit, and workspaces are reusable across calls
  and shapes (per-slot epochs; a layout change re-initialises the workspace).
* The caller-managed workspace entry point equals the library-managed one,
  under HIP-graph capture and replay, and on a non-default stream.
"""
import numpy as np
import pytest

import gla_synth
import oracle

torch = pytest.importorskip("torch")
import chunkwise_gated_recurrence_amd as gla  # noqa: E402

pytestmark = pytest.mark.gpu

W = gla_synth.WORKLOADS["img1024"]
RAG = W.with_(name="rag", B=2, H=3, grid_h=30, grid_w=34, seed=71)
RAG32 = RAG.with_(name="rag32", d_k=32, seed=72)
TIGHT = 1e-3
# (policy, GTR_GLA_KERNEL): generic; the fused kernels' default family for the
# key dim; the gla_fused.hip kernels; the span kernels
FAMILIES = [(gla.POLICY_GENERIC, None), (gla.POLICY_AUTO, None), (gla.POLICY_AUTO, "1"),
            (gla.POLICY_AUTO, "2")]


@pytest.fixture(autouse=True)
def reset_policy():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    gla.gtr_gla_set_policy(gla.POLICY_AUTO)
    yield
    gla.gtr_gla_set_policy(gla.POLICY_AUTO)


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def fwd(arrays, gh, gw, d):
    q, k, v, lg = [dev(a) for a in arrays]
    o, s = gla.forward(q, k, v, lg, gh, gw, d)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64), s.cpu().numpy()


def same(a, b, bitwise):
    if bitwise:
        return np.array_equal(a, b)
    return oracle.rel_err(a, b) <= TIGHT


def rev(x):
    return x[:, ::-1].copy()


def tr(x, gh, gw):
    B, L, H, d = x.shape
    return x.reshape(B, gh, gw, H, d).transpose(0, 2, 1, 3, 4).reshape(B, L, H, d).copy()


@pytest.mark.parametrize("policy,family", FAMILIES, ids=["generic", "auto", "fused", "span"])
@pytest.mark.parametrize("w", [W, RAG, RAG32], ids=["img1024", "ragged", "ragged-dk32"])
def test_direction_folding(w, policy, family, monkeypatch):
    gla.gtr_gla_set_policy(policy)
    if family is not None:
        monkeypatch.setenv("GTR_GLA_KERNEL", family)
    bitwise = True
    x = gla_synth.generate(w)
    gh, gw = w.grid_h, w.grid_w
    print(f"[case] direction folding {w.name} policy={policy} family={family}", flush=True)
    o, s = fwd(x, gh, gw, "r2l")
    o2, s2 = fwd([rev(a) for a in x], gh, gw, "l2r")
    assert same(o, rev(o2), bitwise) and same(s, s2, bitwise)
    o, s = fwd(x, gh, gw, "t2b")
    o2, s2 = fwd([tr(a, gh, gw) for a in x], gw, gh, "l2r")
    assert same(o, tr(o2, gw, gh), bitwise) and same(s, s2, bitwise)
    o, s = fwd(x, gh, gw, "b2t")
    o2, s2 = fwd([tr(a, gh, gw) for a in x], gw, gh, "r2l")
    assert same(o, tr(o2, gw, gh), bitwise) and same(s, s2, bitwise)


@pytest.mark.parametrize("policy,family", FAMILIES, ids=["generic", "auto", "fused", "span"])
def test_repeat_calls_and_shape_changes(policy, family, monkeypatch):
    """Alternating shapes (and, with the default family, key dims: d_k = 32
    takes the span kernels) on the library's workspace."""
    gla.gtr_gla_set_policy(policy)
    if family is not None:
        monkeypatch.setenv("GTR_GLA_KERNEL", family)
    bitwise = True
    big = gla_synth.generate(W)
    small = gla_synth.generate(RAG)
    small32 = gla_synth.generate(RAG32)
    print(f"[case] repeat calls policy={policy} family={family}", flush=True)
    o0, s0 = fwd(big, W.grid_h, W.grid_w, "t2b")
    r0 = fwd(small, RAG.grid_h, RAG.grid_w, "l2r")
    q0 = fwd(small32, RAG32.grid_h, RAG32.grid_w, "b2t")
    for _ in range(3):
        o, s = fwd(big, W.grid_h, W.grid_w, "t2b")
        assert same(o, o0, bitwise) and same(s, s0, bitwise)
        r = fwd(small, RAG.grid_h, RAG.grid_w, "l2r")
        assert same(r[0], r0[0], bitwise) and same(r[1], r0[1], bitwise)
        q = fwd(small32, RAG32.grid_h, RAG32.grid_w, "b2t")
        assert same(q[0], q0[0], bitwise) and same(q[1], q0[1], bitwise)


@pytest.mark.parametrize("w", [W, W.with_(name="img1024_dk32", d_k=32)], ids=["dk64", "dk32"])
def test_many_back_to_back_launches(w):
    """Launch after launch without host synchronisation: the ticket/epoch
    protocol must hand a clean workspace to every launch (d_k = 32: the span
    kernels)."""
    x = [dev(a) for a in gla_synth.generate(w)]
    B, L, H, dk = x[0].shape
    dv = x[2].shape[3]
    outs = []
    for i in range(20):
        o = torch.empty((B, L, H, dv), dtype=torch.float16, device="cuda")
        s = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
        gla.gtr_gla_fwd(*x, B, H, w.grid_h, w.grid_w, dk, dv, i % 4, 64, o, s)
        outs.append((i % 4, o, s))
    torch.cuda.synchronize()
    first = {}
    for d, o, s in outs:
        o, s = o.cpu().numpy().astype(np.float64), s.cpu().numpy()
        if d in first:
            assert same(o, first[d][0], True) and same(s, first[d][1], True)
        else:
            first[d] = (o, s)


def _ws_call(x, w, d, ws, nbytes, o, s, stream=None):
    B, L, H, dk = x[0].shape
    gla.gtr_gla_fwd_ws(*x, B, H, w.grid_h, w.grid_w, dk, x[2].shape[3], d, 64, o, s, ws, nbytes,
                       stream)


@pytest.mark.parametrize("policy", [gla.POLICY_AUTO, gla.POLICY_GENERIC])
def test_workspace_entry_point_and_graph_replay(policy):
    gla.gtr_gla_set_policy(policy)
    bitwise = True
    w = W
    x = [dev(a) for a in gla_synth.generate(w)]
    B, L, H, dk = x[0].shape
    nbytes = gla.gtr_gla_workspace_bytes(B, H, w.grid_h, w.grid_w, dk, dk, 64, 0)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    gla.gtr_gla_workspace_init(ws, nbytes)
    ref_o, ref_s = fwd([a.cpu().numpy() for a in x], w.grid_h, w.grid_w, 3)
    o = torch.empty((B, L, H, dk), dtype=torch.float16, device="cuda")
    s = torch.empty((B, H, dk, dk), dtype=torch.float32, device="cuda")
    print(f"[case] ws eager policy={policy}", flush=True)
    _ws_call(x, w, 3, ws, nbytes, o, s)
    torch.cuda.synchronize()
    assert same(o.cpu().numpy().astype(np.float64), ref_o, bitwise)
    assert same(s.cpu().numpy(), ref_s, bitwise)
    # too small a workspace is refused
    with pytest.raises(gla.GtrGlaError):
        _ws_call(x, w, 3, ws, nbytes - 1, o, s)
    # capture into a graph and replay several times, with eager work between
    print(f"[case] ws graph capture policy={policy}", flush=True)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _ws_call(x, w, 3, ws, nbytes, o, s)   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        _ws_call(x, w, 3, ws, nbytes, o, s)
    for rep in range(4):
        o.fill_(0)
        s.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert same(o.cpu().numpy().astype(np.float64), ref_o, bitwise), rep
        assert same(s.cpu().numpy(), ref_s, bitwise), rep
        eager = fwd([a.cpu().numpy() for a in x], w.grid_h, w.grid_w, 1)  # eager work between
        assert np.isfinite(eager[0]).all()


def test_non_default_stream():
    x = gla_synth.generate(RAG)
    ref_o, ref_s = fwd(x, RAG.grid_h, RAG.grid_w, "b2t")
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        q, k, v, lg = [dev(a) for a in x]
        o, s = gla.forward(q, k, v, lg, RAG.grid_h, RAG.grid_w, "b2t")
    st.synchronize()
    o, s = o.cpu().numpy().astype(np.float64), s.cpu().numpy()
    o_or, s_or = oracle.recurrent(*x, RAG.grid_h, RAG.grid_w, "b2t")
    print(f"[case] default stream err_o={oracle.rel_err(ref_o, o_or):.3e} "
          f"err_S={oracle.rel_err(ref_s, s_or):.3e}; other stream err_o={oracle.rel_err(o, o_or):.3e} "
          f"err_S={oracle.rel_err(s, s_or):.3e}", flush=True)
    assert oracle.rel_err(ref_o, o_or) <= 5e-3 and oracle.rel_err(o, o_or) <= 5e-3
    assert same(o, ref_o, True)
    assert same(s, ref_s, True)


def test_null_final_state_is_allowed():
    x = [dev(a) for a in gla_synth.generate(RAG)]
    B, L, H, dk = x[0].shape
    o = torch.empty((B, L, H, dk), dtype=torch.float16, device="cuda")
    gla.gtr_gla_fwd(*x, B, H, RAG.grid_h, RAG.grid_w, dk, dk, 2, 64, o, None)
    torch.cuda.synchronize()
    ref_o, _ = fwd([a.cpu().numpy() for a in x], RAG.grid_h, RAG.grid_w, 2)
    assert same(o.cpu().numpy().astype(np.float64), ref_o, True)


def test_validation_leaves_outputs_untouched():
    x = [dev(a) for a in gla_synth.generate(RAG)]
    B, L, H, dk = x[0].shape
    o = torch.full((B, L, H, dk), 7.0, dtype=torch.float16, device="cuda")
    with pytest.raises(gla.GtrGlaError) as e:
        gla.gtr_gla_fwd(*x, B, H, RAG.grid_h, RAG.grid_w, dk, dk, 5, 64, o, None)
    assert e.value.status == gla.ERR_DIR
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
