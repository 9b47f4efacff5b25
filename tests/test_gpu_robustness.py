"""Failure paths and launch-loop coverage of the fused kernels on the GPU.

* The in-kernel boundary exchange gives up within its deadline when a span's
  summary never arrives (forced from the host: the exchange's test hook makes
  span 0 of every sequence publish nothing). Every kernel still exits; the
  call writes NaN outputs and final state; gtr_gla_workspace_status reports
  GTR_GLA_ERR_EXCHANGE and re-initialises the workspace; the next call matches
  the oracle. Covered for one-chunk spans, register-kept spans, and a ranged
  fold (two span ranges per owner element), and for the library's own
  workspace.
* A workspace the kernel cannot trust (its bytes overwritten after use, or
  last used by a call of another layout while a captured graph still expects
  the old one) gives NaN outputs and GTR_GLA_ERR_WS_STATE instead of silently
  wrong numbers; after the status call the same call is correct again.
* The multi-launch loop (more sequences than fit on the chip at once) matches
  the oracle: a test-only cap on resident workgroups forces several launches.
"""
import os

import numpy as np
import pytest

import gla_synth
import oracle

torch = pytest.importorskip("torch")
import chunkwise_gated_recurrence_amd as gla  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = 5e-3
SMALL = gla_synth.WORKLOADS["img640"].with_(name="robust", B=1, H=2, grid_h=24, grid_w=20, seed=91)


@pytest.fixture(autouse=True)
def clean_state():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    saved = {k: os.environ.pop(k, None) for k in ("GTR_GLA_SPAN", "GTR_GLA_RK",
                                                  "GTR_GLA_MAX_RESIDENT", "GTR_GLA_KERNEL")}
    gla.gtr_gla_set_policy(gla.POLICY_AUTO)
    gla.gtr_gla_set_exchange_wait(20000, 0)
    yield
    gla.gtr_gla_set_exchange_wait(20000, 0)
    gla.gtr_gla_set_policy(gla.POLICY_AUTO)
    for k, v in saved.items():
        os.environ.pop(k, None)
        if v is not None:
            os.environ[k] = v


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def outputs(w):
    o = torch.zeros((w.B, w.L, w.H, w.d_v), dtype=torch.float16, device="cuda")
    s = torch.zeros((w.B, w.H, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
    return o, s


def ws_call(x, w, d, ws, o, s):
    gla.gtr_gla_fwd_ws(*x, w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, d, 64, o, s, ws,
                       ws.numel())


def check_oracle(arrays, w, d, o, s):
    o_ref, s_ref = oracle.recurrent(*arrays, w.grid_h, w.grid_w, d)
    eo = oracle.rel_err(o.cpu().numpy().astype(np.float64), o_ref)
    es = oracle.rel_err(s.cpu().numpy(), s_ref)
    assert eo <= TOL and es <= TOL, (eo, es)


def all_nan(t):
    return bool(torch.isnan(t.float()).all())


GIVE_UP_CASES = {
    # name: (workload, GTR_GLA_SPAN, GTR_GLA_RK, GTR_GLA_KERNEL, expected kernel of gtr_gla_plan)
    "one_chunk": (SMALL, "1", None, "1", 2),
    "register_kept": (SMALL, "2", "1", "1", 3),
    "ranged_fold": (SMALL.with_(name="ranged", grid_h=64, grid_w=32), "1", None, "1", 2),
    "span_one_chunk": (SMALL, "1", None, "2", 4),
    "span_three": (SMALL, "3", None, "2", 4),
    "span_ranged_fold": (SMALL.with_(name="ranged", grid_h=64, grid_w=32), "1", None, "2", 4),
    "span_dk32": (SMALL.with_(name="dk32", d_k=32), "2", None, "2", 4),
}


@pytest.mark.parametrize("case", sorted(GIVE_UP_CASES))
def test_exchange_gives_up_loudly_and_recovers(case):
    w, span, rk, family, kernel = GIVE_UP_CASES[case]
    os.environ["GTR_GLA_SPAN"] = span
    os.environ["GTR_GLA_KERNEL"] = family
    if rk:
        os.environ["GTR_GLA_RK"] = rk
    assert gla.gtr_gla_plan(w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, 64, 0)[0] == kernel
    arrays = gla_synth.generate(w)
    x = [dev(a) for a in arrays]
    nbytes = gla.gtr_gla_workspace_bytes(w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, 64, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    gla.gtr_gla_workspace_init(ws, nbytes)
    o, s = outputs(w)
    print(f"[case] forced give-up {case}", flush=True)
    gla.gtr_gla_set_exchange_wait(2000, 1)
    ws_call(x, w, 1, ws, o, s)
    torch.cuda.synchronize()
    assert all_nan(o) and all_nan(s)
    assert gla.gtr_gla_workspace_status(ws, nbytes) == gla.ERR_EXCHANGE
    assert gla.gtr_gla_workspace_status(ws, nbytes) == gla.OK   # cleared
    print(f"[case] recovery after give-up {case}", flush=True)
    gla.gtr_gla_set_exchange_wait(20000, 0)
    for d in (1, 2):
        ws_call(x, w, d, ws, o, s)
        torch.cuda.synchronize()
        check_oracle(arrays, w, d, o, s)
    assert gla.gtr_gla_workspace_status(ws, nbytes) == gla.OK


def test_library_workspace_give_up_is_reported():
    w = SMALL
    arrays = gla_synth.generate(w)
    x = [dev(a) for a in arrays]
    o, s = outputs(w)
    print("[case] library workspace give-up", flush=True)
    gla.gtr_gla_fwd(*x, w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, 0, 64, o, s)   # warm
    assert gla.gtr_gla_workspace_status() == gla.OK
    gla.gtr_gla_set_exchange_wait(2000, 1)
    gla.gtr_gla_fwd(*x, w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, 0, 64, o, s)
    torch.cuda.synchronize()
    assert all_nan(o) and all_nan(s)
    assert gla.gtr_gla_workspace_status() == gla.ERR_EXCHANGE
    gla.gtr_gla_set_exchange_wait(20000, 0)
    gla.gtr_gla_fwd(*x, w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, 0, 64, o, s)
    torch.cuda.synchronize()
    check_oracle(arrays, w, 0, o, s)


def test_overwritten_workspace_is_not_trusted():
    w = SMALL
    arrays = gla_synth.generate(w)
    x = [dev(a) for a in arrays]
    nbytes = gla.gtr_gla_workspace_bytes(w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, 64, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    gla.gtr_gla_workspace_init(ws, nbytes)
    o, s = outputs(w)
    ws_call(x, w, 0, ws, o, s)
    torch.cuda.synchronize()
    check_oracle(arrays, w, 0, o, s)
    # the same memory rewritten by someone else (as a caching allocator may hand it out)
    print("[case] overwritten workspace", flush=True)
    ws.copy_(torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda"))
    ws_call(x, w, 0, ws, o, s)
    torch.cuda.synchronize()
    assert all_nan(o)
    assert gla.gtr_gla_workspace_status(ws, nbytes) == gla.ERR_WS_STATE
    ws_call(x, w, 0, ws, o, s)
    torch.cuda.synchronize()
    check_oracle(arrays, w, 0, o, s)


def test_graph_after_other_layout_on_same_workspace():
    """A captured call keeps the layout it was captured with; an eager call of another
    layout on the same workspace in between makes the replay fail loudly (NaN and a
    status), not read the other layout's words; after the status call it replays right."""
    wa, wb = SMALL, SMALL.with_(name="other", H=3, grid_h=40, grid_w=40, seed=92)
    xa_np, xb_np = gla_synth.generate(wa), gla_synth.generate(wb)
    xa, xb = [dev(a) for a in xa_np], [dev(a) for a in xb_np]
    la = gla.gtr_gla_plan(wa.B, wa.H, wa.grid_h, wa.grid_w, 64, 64, 64, 0)
    lb = gla.gtr_gla_plan(wb.B, wb.H, wb.grid_h, wb.grid_w, 64, 64, 64, 0)
    assert la != lb   # two exchange layouts
    nbytes = max(gla.gtr_gla_workspace_bytes(w.B, w.H, w.grid_h, w.grid_w, 64, 64, 64, 0)
                 for w in (wa, wb))
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    gla.gtr_gla_workspace_init(ws, nbytes)
    oa, sa = outputs(wa)
    ob, sb = outputs(wb)
    ws_call(xa, wa, 2, ws, oa, sa)   # eager warm-up of the captured call
    torch.cuda.synchronize()
    ref = oa.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ws_call(xa, wa, 2, ws, oa, sa)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(oa, ref)
    print("[case] eager call of another layout, then replay", flush=True)
    ws_call(xb, wb, 0, ws, ob, sb)
    torch.cuda.synchronize()
    check_oracle(xb_np, wb, 0, ob, sb)
    g.replay()
    torch.cuda.synchronize()
    assert all_nan(oa)
    assert gla.gtr_gla_workspace_status(ws, nbytes) == gla.ERR_WS_STATE
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(oa, ref)


MULTI = gla_synth.WORKLOADS["img640"].with_(name="multi", B=2, H=4, grid_h=16, grid_w=17, seed=93)


@pytest.mark.parametrize("span,rk,cap,family", [("1", None, "6", "1"), ("2", "1", "6", "1"),
                                                ("2", None, "6", "1"), (None, None, "4", "1"),
                                                ("1", None, "6", "2"), ("3", None, "6", "2")],
                         ids=["one_chunk", "register_kept", "parked", "auto_streamed", "span1",
                              "span3"])
def test_multi_launch_loop_parity(span, rk, cap, family):
    w = MULTI
    if span:
        os.environ["GTR_GLA_SPAN"] = span
    if rk:
        os.environ["GTR_GLA_RK"] = rk
    os.environ["GTR_GLA_MAX_RESIDENT"] = cap
    os.environ["GTR_GLA_KERNEL"] = family
    kern, sp, grid = gla.gtr_gla_plan(w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, 64, 0)
    n_spans = -(-(-(-w.L // 64)) // sp)
    assert kern in ((2, 3) if family == "1" else (4,)) and grid < w.B * w.H * n_spans, (kern, sp, grid)
    arrays = gla_synth.generate(w)
    x = [dev(a) for a in arrays]
    for d in range(4):
        print(f"[case] multi-launch span={span} rk={rk} cap={cap} dir={d}", flush=True)
        o, s = gla.forward(*x, w.grid_h, w.grid_w, d)
        torch.cuda.synchronize()
        check_oracle(arrays, w, d, o, s)


def test_library_workspace_alternates_kernel_families():
    """The library's own workspace, reused by calls of the two fused kernel
    families whose plans agree on spans per sequence and sequences per launch
    (a forced cap of six resident workgroups): the exchange layouts still differ,
    so each call re-initialises the workspace instead of tripping the other
    family's header (which would give NaN); every call matches the oracle."""
    w = MULTI
    arrays = gla_synth.generate(w)
    x = [dev(a) for a in arrays]
    os.environ["GTR_GLA_SPAN"] = "1"
    os.environ["GTR_GLA_MAX_RESIDENT"] = "6"
    plans = {}
    for family in ("1", "2", "1", "2"):
        os.environ["GTR_GLA_KERNEL"] = family
        plans[family] = gla.gtr_gla_plan(w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, 64, 0)
        print(f"[case] family {family} plan {plans[family]}", flush=True)
        o, s = gla.forward(*x, w.grid_h, w.grid_w, 1)
        torch.cuda.synchronize()
        check_oracle(arrays, w, 1, o, s)
        assert gla.gtr_gla_workspace_status() == gla.OK
    assert plans["1"][1:] == plans["2"][1:] and plans["1"][0] != plans["2"][0]


ALT64 = gla_synth.WORKLOADS["img1024"].with_(name="alt64", B=2, H=3, grid_h=30, grid_w=34, seed=95)
ALT32 = ALT64.with_(name="alt32", d_k=32, seed=96)


@pytest.mark.parametrize("own_ws", [False, True], ids=["library-ws", "caller-ws"])
def test_span_key_widths_alternate_on_one_workspace(own_ws):
    """Span-kernel calls at d_k = 64 and 32 with the same spans per sequence and
    sequences per launch (16 and 6 here) hold differently sized exchange slots,
    so their exchange layouts must differ: a call after one of the other key
    width then starts from a re-initialised workspace instead of reading the
    incoming-state words that a call two launches back left, whose tag parity
    matches (a regression: the span plans once carried the default key width in
    their layout word). The scan order changes from call to call, so that
    stale states would give wrong outputs."""
    os.environ["GTR_GLA_KERNEL"] = "2"
    p64 = gla.gtr_gla_plan(ALT64.B, ALT64.H, ALT64.grid_h, ALT64.grid_w, 64, 64, 64, 0)
    p32 = gla.gtr_gla_plan(ALT32.B, ALT32.H, ALT32.grid_h, ALT32.grid_w, 32, 64, 64, 0)
    assert p64 == p32 and p64[0] == 4, (p64, p32)   # same kernel family, span and grid
    ws = None
    if own_ws:
        nbytes = max(gla.gtr_gla_workspace_bytes(w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, 64, 0)
                     for w in (ALT64, ALT32))
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        gla.gtr_gla_workspace_init(ws, nbytes)
    data = {w.name: (gla_synth.generate(w), w) for w in (ALT64, ALT32)}
    for i, (name, d) in enumerate([("alt64", 0), ("alt32", 3), ("alt64", 3), ("alt32", 2),
                                   ("alt64", 1), ("alt64", 2), ("alt32", 0), ("alt64", 0)]):
        arrays, w = data[name]
        x = [dev(a) for a in arrays]
        o, s = outputs(w)
        print(f"[case] alternate key widths {'caller' if own_ws else 'library'} ws call {i}: "
              f"{name} dir={d}", flush=True)
        if own_ws:
            ws_call(x, w, d, ws, o, s)
        else:
            o, s = gla.forward(*x, w.grid_h, w.grid_w, d)
        torch.cuda.synchronize()
        check_oracle(arrays, w, d, o, s)


def test_mixed_call_history_matches_the_oracle():
    """A call history that mixes kernel families, key widths, shapes of equal
    and unequal exchange layouts, scan orders and the two streams' library
    workspaces, each call checked against the oracle (a repeat of the same call
    cannot show stale exchange words: they would hold the same values)."""
    shapes = {
        "a64": ALT64, "a32": ALT32,
        "b64": ALT64.with_(name="b64", grid_h=34, grid_w=30, seed=97),      # the same layout as a64
        "c64": ALT64.with_(name="c64", B=1, H=4, grid_h=20, grid_w=40, seed=98),
    }
    data = {k: gla_synth.generate(w) for k, w in shapes.items()}
    side = torch.cuda.Stream()
    history = [("a64", 0, None, None), ("b64", 3, None, None), ("a32", 1, None, None),
               ("a64", 2, "2", None), ("c64", 3, None, None), ("a64", 1, "1", None),
               ("b64", 0, None, side), ("a32", 3, "2", side), ("a64", 3, None, side),
               ("a64", 2, None, None), ("c64", 0, "2", None), ("a32", 2, None, None),
               ("b64", 1, None, None), ("a64", 0, "2", None)]
    for i, (name, d, family, stream) in enumerate(history):
        w, arrays = shapes[name], data[name]
        if family is None:
            os.environ.pop("GTR_GLA_KERNEL", None)
        else:
            os.environ["GTR_GLA_KERNEL"] = family
        plan = gla.gtr_gla_plan(w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, 64, 0)
        print(f"[case] history call {i}: {name} dir={d} family={family} "
              f"stream={'side' if stream is not None else 'default'} plan={plan}", flush=True)
        x = [dev(a) for a in arrays]
        if stream is None:
            o, s = gla.forward(*x, w.grid_h, w.grid_w, d)
            torch.cuda.synchronize()
        else:
            stream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(stream):
                o, s = gla.forward(*x, w.grid_h, w.grid_w, d)
            stream.synchronize()
        check_oracle(arrays, w, d, o, s)


@pytest.mark.parametrize("span,rk,family", [("1", None, "1"), ("2", "1", "1"), ("1", None, "2"),
                                            ("3", None, "2")],
                         ids=["one_chunk", "register_kept", "span1", "span3"])
def test_multi_launch_with_initial_state_and_gate(span, rk, family):
    """The multi-launch loop with the optional inputs that are indexed per
    sequence (initial states, final states) or per token (the output gate): the
    later launches must take their sequences' rows, not the first launch's."""
    w = MULTI
    os.environ["GTR_GLA_SPAN"] = span
    if rk:
        os.environ["GTR_GLA_RK"] = rk
    os.environ["GTR_GLA_MAX_RESIDENT"] = "6"
    os.environ["GTR_GLA_KERNEL"] = family
    kern, sp, grid = gla.gtr_gla_plan(w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, 64, 0)
    n_spans = -(-(-(-w.L // 64)) // sp)
    assert grid < w.B * w.H * n_spans, (kern, sp, grid)
    arrays = gla_synth.generate(w)
    rng = np.random.default_rng(94)
    S0 = (0.5 * rng.standard_normal((w.B, w.H, w.d_k, w.d_v))).astype(np.float32)
    gate = (2.0 * rng.standard_normal((w.B, w.L, w.H, w.d_v))).astype(np.float16)
    nw = rng.uniform(0.5, 1.5, w.d_v).astype(np.float32)
    x = [dev(a) for a in arrays]
    for d in range(4):
        print(f"[case] multi-launch with additions span={span} family={family} dir={d}", flush=True)
        y, s = gla.forward(*x, w.grid_h, w.grid_w, d, initial_state=dev(S0), gate=dev(gate),
                           norm_weight=dev(nw), norm_eps=1e-5)
        torch.cuda.synchronize()
        o_ref, s_ref = oracle.recurrent_init(*arrays, S0, w.grid_h, w.grid_w, d)
        y_ref = oracle.rmsnorm_gate(o_ref, gate, nw, 1e-5)
        ey = oracle.rel_err(y.cpu().numpy().astype(np.float64), y_ref)
        es = oracle.rel_err(s.cpu().numpy(), s_ref)
        assert ey <= TOL and es <= TOL, (ey, es)


def test_multi_launch_lowrank():
    """The low-rank gate (projection per token, gate per head) across several
    launches of the fused kernels."""
    w = MULTI
    C = 96
    os.environ["GTR_GLA_MAX_RESIDENT"] = "6"
    os.environ["GTR_GLA_SPAN"] = "1"
    kern, sp, grid = gla.gtr_gla_plan(w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, 64, 0,
                                      lowrank=True)
    n_spans = -(-(-(-w.L // 64)) // sp)
    assert grid < w.B * w.H * n_spans, (kern, sp, grid)
    q, k, v, _ = gla_synth.generate(w)
    xin, w1, w2, bias = gla_synth.generate_lowrank(w, C, 95)
    lg = oracle.lowrank_gate(xin, w1, w2, bias, 1.0 / 16).reshape(w.B, w.L, w.H, w.d_k)
    for d in range(4):
        print(f"[case] multi-launch lowrank dir={d}", flush=True)
        out, fs = gla.forward_lowrank(dev(q), dev(k), dev(v), dev(xin), dev(w1), dev(w2), dev(bias),
                                      w.grid_h, w.grid_w, d, inv_tau=1.0 / 16)
        torch.cuda.synchronize()
        check_oracle((q, k, v, lg), w, d, out, fs)
