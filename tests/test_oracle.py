"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: closed forms
from the mathematics, values worked by hand in tests/golden/, the brute-force
double sum, or invariants that the definition fixes. Together they are chosen
so that a plausible slip in the oracle (a dropped term, a gate applied on the
value side or one step late, a wrong scale, a transposed grid walk, a wrong
index) fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")
DIRS = ["l2r", "r2l", "t2b", "b2t"]


def np_order(gh, gw, d):
    """Scan order written with numpy reshapes (independent of the oracle's index math)."""
    grid = np.arange(gh * gw).reshape(gh, gw)
    return {"l2r": grid.ravel(), "r2l": grid.ravel()[::-1],
            "t2b": grid.T.ravel(), "b2t": grid.T.ravel()[::-1]}[d]


def rand_inputs(seed, B, gh, gw, H, dk, dv, lg_lo=-0.6, lg_hi=0.0):
    rng = np.random.default_rng(seed)
    L = gh * gw
    q = rng.standard_normal((B, L, H, dk))
    k = rng.standard_normal((B, L, H, dk))
    v = rng.standard_normal((B, L, H, dv))
    lg = rng.uniform(lg_lo, lg_hi, (B, L, H, dk))
    return q, k, v, lg


# --------------------------------------------------------------------------- golden
def test_scan_orders_match_hand_lists():
    g = json.load(open(GOLDEN))
    for grid in g["scan_orders"]["grids"]:
        for d in DIRS:
            got = oracle.scan_order(grid["grid_h"], grid["grid_w"], d)
            assert got.tolist() == grid[d], (grid, d)
            assert np_order(grid["grid_h"], grid["grid_w"], d).tolist() == grid[d]


@pytest.mark.parametrize("fn", [oracle.recurrent, oracle.bruteforce])
def test_hand_examples(fn):
    g = json.load(open(GOLDEN))
    for ex in g["examples"]:
        q = np.array(ex["q"])[None, :, None, :]
        k = np.array(ex["k"])[None, :, None, :]
        v = np.array(ex["v"])[None, :, None, :]
        lg = np.log(np.array(ex["gamma"]))[None, :, None, :]
        for d, e in ex["expect"].items():
            o, S = fn(q, k, v, lg, ex["grid_h"], ex["grid_w"], d)
            np.testing.assert_allclose(o[0, :, 0, :], np.array(e["o"]), rtol=1e-14, atol=1e-14)
            np.testing.assert_allclose(S[0, 0], np.array(e["final_state"]), rtol=1e-14, atol=1e-14)


def test_hand_examples_chunked():
    g = json.load(open(GOLDEN))
    for ex in g["examples"]:
        q = np.array(ex["q"])[None, :, None, :]
        k = np.array(ex["k"])[None, :, None, :]
        v = np.array(ex["v"])[None, :, None, :]
        lg = np.log(np.array(ex["gamma"]))[None, :, None, :]
        for d, e in ex["expect"].items():
            for C in (1, 2, 3):
                o, S = oracle.chunked(q, k, v, lg, ex["grid_h"], ex["grid_w"], d, C)
                np.testing.assert_allclose(o[0, :, 0, :], np.array(e["o"]), rtol=1e-14, atol=1e-14)
                np.testing.assert_allclose(S[0, 0], np.array(e["final_state"]), rtol=1e-14,
                                           atol=1e-14)


# --------------------------------------------------------------------------- brute force
@pytest.mark.parametrize("shape", [(1, 4, 4, 1, 8, 8), (2, 5, 7, 2, 6, 3), (1, 16, 16, 1, 32, 32),
                                   (1, 3, 11, 3, 4, 9)])
@pytest.mark.parametrize("d", DIRS)
def test_recurrent_matches_bruteforce(shape, d):
    B, gh, gw, H, dk, dv = shape
    q, k, v, lg = rand_inputs(7, B, gh, gw, H, dk, dv)
    o1, S1 = oracle.recurrent(q, k, v, lg, gh, gw, d)
    o2, S2 = oracle.bruteforce(q, k, v, lg, gh, gw, d)
    assert oracle.rel_err(o1, o2) < 1e-12
    assert oracle.rel_err(S1, S2) < 1e-12


# --------------------------------------------------------------------------- closed forms
def _per_seq(fn, q, k, v, order):
    B, L, H, dk = q.shape
    dv = v.shape[3]
    o = np.zeros((B, L, H, dv))
    S = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            Q, K, V = q[b, order, h], k[b, order, h], v[b, order, h]
            O, Sf = fn(Q, K, V)
            o[b, order, h] = O
            S[b, h] = Sf
    return o, S


@pytest.mark.parametrize("d", DIRS)
def test_gate_one_is_causal_linear_attention(d):
    """gamma == 1: o_t = d_k^{-1/2} sum_{s<=t} (q_t . k_s) v_s and S_L = K^T V."""
    B, gh, gw, H, dk, dv = 2, 6, 9, 2, 8, 5
    q, k, v, _ = rand_inputs(11, B, gh, gw, H, dk, dv)
    lg = np.zeros_like(q)

    def cla(Q, K, V):
        return np.tril(Q @ K.T) @ V / np.sqrt(dk), K.T @ V

    o_ref, S_ref = _per_seq(cla, q, k, v, np_order(gh, gw, d))
    o, S = oracle.recurrent(q, k, v, lg, gh, gw, d)
    assert oracle.rel_err(o, o_ref) < 1e-12
    assert oracle.rel_err(S, S_ref) < 1e-12
    # the final state K^T V does not depend on the direction
    S0 = oracle.recurrent(q, k, v, lg, gh, gw, "l2r")[1]
    assert oracle.rel_err(S, S0) < 1e-12


@pytest.mark.parametrize("c", [0.5, 0.9, 0.999])
def test_constant_gate_is_retention(c):
    """gamma == c on every key dim: o_t = d_k^{-1/2} sum_{s<=t} c^{t-s} (q_t . k_s) v_s."""
    B, gh, gw, H, dk, dv = 1, 5, 8, 2, 6, 7
    q, k, v, _ = rand_inputs(12, B, gh, gw, H, dk, dv)
    lg = np.full_like(q, np.log(c))
    L = gh * gw
    t = np.arange(L)
    Dm = np.tril(c ** (t[:, None] - t[None, :]).astype(np.float64))

    def ret(Q, K, V):
        return ((Q @ K.T) * Dm) @ V / np.sqrt(dk), (K * (c ** (L - 1 - t))[:, None]).T @ V

    for d in DIRS:
        o_ref, S_ref = _per_seq(ret, q, k, v, np_order(gh, gw, d))
        o, S = oracle.recurrent(q, k, v, lg, gh, gw, d)
        assert oracle.rel_err(o, o_ref) < 1e-12
        assert oracle.rel_err(S, S_ref) < 1e-12


@pytest.mark.parametrize("fn", [oracle.recurrent, oracle.bruteforce])
def test_gate_zero_keeps_only_the_diagonal(fn):
    """gamma -> 0: o_t = d_k^{-1/2} (q_t . k_t) v_t and S_L = k_last^T v_last."""
    B, gh, gw, H, dk, dv = 1, 4, 6, 3, 5, 4
    q, k, v, _ = rand_inputs(13, B, gh, gw, H, dk, dv)
    lg = np.full_like(q, -1e4)
    o_ref = np.einsum("blhi,blhi->blh", q, k)[..., None] * v / np.sqrt(dk)
    for d in DIRS:
        o, S = fn(q, k, v, lg, gh, gw, d)
        np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-13)
        last = np_order(gh, gw, d)[-1]
        S_ref = np.einsum("bhi,bhj->bhij", k[:, last], v[:, last])
        np.testing.assert_allclose(S, S_ref, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------- chunked form
@pytest.mark.parametrize("C", [1, 2, 3, 16, 63, 64, 100, 10**6])
def test_chunked_equals_recurrent(C):
    B, gh, gw, H, dk, dv = 2, 9, 14, 2, 8, 6     # L = 126: ragged for most C
    q, k, v, lg = rand_inputs(21, B, gh, gw, H, dk, dv, lg_lo=-1.0)
    for d in DIRS:
        o1, S1 = oracle.recurrent(q, k, v, lg, gh, gw, d)
        o2, S2 = oracle.chunked(q, k, v, lg, gh, gw, d, min(C, gh * gw))
        assert oracle.rel_err(o2, o1) < 1e-12, (C, d)
        assert oracle.rel_err(S2, S1) < 1e-12, (C, d)


# --------------------------------------------------------------------------- directions
def _spatial_reverse(x):
    return x[:, ::-1].copy()


def _grid_transpose(x, gh, gw):
    B, L, H, d = x.shape
    return x.reshape(B, gh, gw, H, d).transpose(0, 2, 1, 3, 4).reshape(B, L, H, d).copy()


def test_direction_invariants():
    B, gh, gw, H, dk, dv = 2, 5, 7, 2, 6, 4
    q, k, v, lg = rand_inputs(31, B, gh, gw, H, dk, dv)
    rec = oracle.recurrent
    # right->left(x) == reverse(left->right(reverse(x)))
    o, S = rec(q, k, v, lg, gh, gw, "r2l")
    o2, S2 = rec(*[_spatial_reverse(x) for x in (q, k, v, lg)], gh, gw, "l2r")
    assert oracle.rel_err(o, _spatial_reverse(o2)) < 1e-13 and oracle.rel_err(S, S2) < 1e-13
    # top->bottom(x) on (gh, gw) == transpose(left->right(transpose(x))) on (gw, gh)
    o, S = rec(q, k, v, lg, gh, gw, "t2b")
    o2, S2 = rec(*[_grid_transpose(x, gh, gw) for x in (q, k, v, lg)], gw, gh, "l2r")
    assert oracle.rel_err(o, _grid_transpose(o2, gw, gh)) < 1e-13
    assert oracle.rel_err(S, S2) < 1e-13
    # bottom->top(x) == transpose(right->left(transpose(x)))
    o, S = rec(q, k, v, lg, gh, gw, "b2t")
    o2, S2 = rec(*[_grid_transpose(x, gh, gw) for x in (q, k, v, lg)], gw, gh, "r2l")
    assert oracle.rel_err(o, _grid_transpose(o2, gw, gh)) < 1e-13
    assert oracle.rel_err(S, S2) < 1e-13


def test_degenerate_grids():
    q, k, v, lg = rand_inputs(41, 1, 1, 12, 2, 4, 3)
    rec = oracle.recurrent
    # one row: top->bottom is left->right, bottom->top is right->left
    for a, b in (("t2b", "l2r"), ("b2t", "r2l")):
        x, y = rec(q, k, v, lg, 1, 12, a), rec(q, k, v, lg, 1, 12, b)
        assert np.array_equal(x[0], y[0]) and np.array_equal(x[1], y[1])
    # one column: left->right is top->bottom, right->left is bottom->top
    for a, b in (("l2r", "t2b"), ("r2l", "b2t")):
        x, y = rec(q, k, v, lg, 12, 1, a), rec(q, k, v, lg, 12, 1, b)
        assert np.array_equal(x[0], y[0]) and np.array_equal(x[1], y[1])
    # single token: o = d_k^{-1/2} (q . k) v whatever the gate
    q1, k1, v1, lg1 = rand_inputs(42, 1, 1, 1, 1, 5, 3)
    for d in DIRS:
        o, S = rec(q1, k1, v1, lg1, 1, 1, d)
        np.testing.assert_allclose(o[0, 0, 0], (q1[0, 0, 0] @ k1[0, 0, 0]) * v1[0, 0, 0] / np.sqrt(5),
                                   rtol=1e-14)
        np.testing.assert_allclose(S[0, 0], np.outer(k1[0, 0, 0], v1[0, 0, 0]), rtol=1e-14)


def test_first_gate_has_no_effect():
    """Zero initial state: the gate at the first scan step multiplies S_0 = 0."""
    B, gh, gw, H, dk, dv = 1, 6, 5, 2, 4, 4
    q, k, v, lg = rand_inputs(51, B, gh, gw, H, dk, dv)
    for d in DIRS:
        first = np_order(gh, gw, d)[0]
        lg2 = lg.copy()
        lg2[:, first] = -3.7
        a, b = oracle.recurrent(q, k, v, lg, gh, gw, d), oracle.recurrent(q, k, v, lg2, gh, gw, d)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        # ...while the gate at the second step does matter
        lg3 = lg.copy()
        lg3[:, np_order(gh, gw, d)[1]] -= 0.5
        c = oracle.recurrent(q, k, v, lg3, gh, gw, d)
        assert not np.allclose(a[1], c[1])


def test_linearity_and_equivariance():
    B, gh, gw, H, dk, dv = 2, 4, 5, 3, 6, 5
    q, k, v, lg = rand_inputs(61, B, gh, gw, H, dk, dv)
    _, _, v2, _ = rand_inputs(62, B, gh, gw, H, dk, dv)
    rec = oracle.recurrent
    for d in DIRS:
        o1, S1 = rec(q, k, v, lg, gh, gw, d)
        o2, S2 = rec(q, k, v2, lg, gh, gw, d)
        o3, S3 = rec(q, k, v - 2.5 * v2, lg, gh, gw, d)
        assert oracle.rel_err(o3, o1 - 2.5 * o2) < 1e-12
        assert oracle.rel_err(S3, S1 - 2.5 * S2) < 1e-12
        o4, S4 = rec(3.0 * q, k, v, lg, gh, gw, d)            # o linear in q, S independent
        assert oracle.rel_err(o4, 3.0 * o1) < 1e-13 and np.array_equal(S4, S1)
        o5, S5 = rec(q, -0.5 * k, v, lg, gh, gw, d)           # k scales o and S
        assert oracle.rel_err(o5, -0.5 * o1) < 1e-13 and oracle.rel_err(S5, -0.5 * S1) < 1e-13
    # permuting heads / batch entries permutes the outputs
    hp, bp = np.array([2, 0, 1]), np.array([1, 0])
    o, S = rec(q, k, v, lg, gh, gw, "t2b")
    oh, Sh = rec(q[:, :, hp], k[:, :, hp], v[:, :, hp], lg[:, :, hp], gh, gw, "t2b")
    assert np.array_equal(oh, o[:, :, hp]) and np.array_equal(Sh, S[:, hp])
    ob, Sb = rec(q[bp], k[bp], v[bp], lg[bp], gh, gw, "t2b")
    assert np.array_equal(ob, o[bp]) and np.array_equal(Sb, S[bp])


def test_scale_is_inverse_sqrt_dk():
    """Doubling d_k with zero padding keeps S but divides o by sqrt(2)."""
    B, gh, gw, H, dk, dv = 1, 3, 4, 1, 4, 3
    q, k, v, lg = rand_inputs(71, B, gh, gw, H, dk, dv)
    pad = lambda x: np.concatenate([x, np.zeros_like(x)], axis=3)
    o1, S1 = oracle.recurrent(q, k, v, lg, gh, gw, "l2r")
    o2, S2 = oracle.recurrent(pad(q), pad(k), v, pad(lg), gh, gw, "l2r")
    assert oracle.rel_err(o2 * np.sqrt(2.0), o1) < 1e-14
    assert oracle.rel_err(S2[:, :, :dk], S1) < 1e-14 and not S2[:, :, dk:].any()


def test_threads_do_not_change_results():
    q, k, v, lg = rand_inputs(81, 3, 6, 6, 4, 8, 8)
    a = oracle.recurrent(q, k, v, lg, 6, 6, "b2t", threads=1)
    b = oracle.recurrent(q, k, v, lg, 6, 6, "b2t", threads=5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rejects_bad_shapes():
    q, k, v, lg = rand_inputs(91, 1, 3, 3, 1, 4, 4)
    with pytest.raises(ValueError):
        oracle.recurrent(q, k, v, lg, 3, 4, "l2r")
    with pytest.raises(KeyError):
        oracle.recurrent(q, k, v, lg, 3, 3, "diag")


# --------------------------------------------------------------------------- initial state
@pytest.mark.parametrize("d", ["l2r", "r2l"])
def test_initial_state_chains_spans(d):
    """Running the first rows of the scan, then the rest from the state they leave,
    gives the outputs and final state of one run over the whole grid."""
    gh, gw, h1 = 7, 5, 3
    q, k, v, lg = rand_inputs(41, 2, gh, gw, 3, 4, 3)
    o, S = oracle.recurrent(q, k, v, lg, gh, gw, d)
    # raster rows [0, h1) are scanned first by l2r; rows [gh - h1, gh) first by r2l
    first = slice(0, h1 * gw) if d == "l2r" else slice((gh - h1) * gw, gh * gw)
    rest = slice(h1 * gw, gh * gw) if d == "l2r" else slice(0, (gh - h1) * gw)
    part = lambda x, sl: x[:, sl]
    o1, S1 = oracle.recurrent(*(part(x, first) for x in (q, k, v, lg)), h1, gw, d)
    o2, S2 = oracle.recurrent_init(*(part(x, rest) for x in (q, k, v, lg)), S1, gh - h1, gw, d)
    np.testing.assert_allclose(o1, o[:, first], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o2, o[:, rest], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-12)


def test_initial_state_alone_decays_by_the_gate_products():
    """With k = 0 nothing is added: S_t = Diag(prod_{r<=t} gamma_r) S_0, so
    o_t = d_k^{-1/2} sum_i q_t[i] prod_{r<=t} gamma_r[i] S_0[i, :]."""
    gh, gw, dk, dv = 3, 4, 5, 2
    q, k, v, lg = rand_inputs(42, 1, gh, gw, 2, dk, dv)
    S0 = np.random.default_rng(43).standard_normal((1, 2, dk, dv))
    o, S = oracle.recurrent_init(q, 0 * k, v, lg, S0, gh, gw, "t2b")
    order = np_order(gh, gw, "t2b")
    P = np.exp(np.cumsum(lg[:, order], axis=1))             # [B, L, H, dk] in scan order
    expect = np.einsum("blhi,blhi,bhij->blhj", q[:, order], P, S0) / np.sqrt(dk)
    np.testing.assert_allclose(o[:, order], expect, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, P[:, -1][..., None] * S0, rtol=1e-12, atol=1e-12)


def test_initial_state_is_additive():
    """o and S are linear in (v, S_0) jointly: the run from S_0 is the zero-state run
    plus the run of S_0 alone (v = 0)."""
    q, k, v, lg = rand_inputs(44, 2, 4, 4, 2, 3, 5)
    S0 = np.random.default_rng(45).standard_normal((2, 2, 3, 5))
    o, S = oracle.recurrent_init(q, k, v, lg, S0, 4, 4, "b2t")
    oa, Sa = oracle.recurrent(q, k, v, lg, 4, 4, "b2t")
    ob, Sb = oracle.recurrent_init(q, k, 0 * v, lg, S0, 4, 4, "b2t")
    np.testing.assert_allclose(o, oa + ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, Sa + Sb, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- output epilogue
def test_rmsnorm_gate_pins():
    rng = np.random.default_rng(46)
    o = rng.standard_normal((5, 7, 16))
    w = rng.uniform(0.5, 2.0, 16)
    ones = np.ones(16)
    big = np.full(o.shape, 40.0)     # SiLU(40) = 40 (1 - 4e-18): the gate passes the value
    # a zero gate closes the output
    assert np.all(oracle.rmsnorm_gate(o, np.zeros(o.shape), w, 1e-5) == 0)
    # wide-open gate, unit weight, eps = 0: each row is o scaled to unit mean square
    n = oracle.rmsnorm_gate(o, big, ones, 0.0) / 40.0
    np.testing.assert_allclose(np.mean(n ** 2, axis=-1), 1.0, rtol=1e-12)
    ratio = n / o
    assert np.all(ratio > 0)
    np.testing.assert_allclose(ratio, ratio[..., :1] * np.ones_like(ratio), rtol=1e-12)
    # eps equal to the row's mean square halves it
    ms = np.mean(o ** 2, axis=-1)
    half = np.stack([oracle.rmsnorm_gate(o[i, j:j + 1], big[i, j:j + 1], ones, ms[i, j])
                     for i in range(5) for j in range(7)]) / 40.0
    np.testing.assert_allclose(np.mean(half ** 2, axis=-1), 0.5, rtol=1e-12)
    # the weight multiplies per channel
    np.testing.assert_allclose(oracle.rmsnorm_gate(o, big, w, 0.0), w * n * 40.0, rtol=1e-12)
    # scale invariance without eps
    np.testing.assert_allclose(oracle.rmsnorm_gate(3.5 * o, big, w, 0.0),
                               oracle.rmsnorm_gate(o, big, w, 0.0), rtol=1e-12)
    # SiLU(z) - SiLU(-z) = z, because sigma(z) + sigma(-z) = 1
    z = rng.uniform(-6, 6, o.shape)
    diff = oracle.rmsnorm_gate(o, z, w, 1e-3) - oracle.rmsnorm_gate(o, -z, w, 1e-3)
    np.testing.assert_allclose(diff, z * oracle.rmsnorm_gate(o, big, w, 1e-3) / 40.0,
                               rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------- low-rank gate
def _lowrank_inputs(seed, rows=37, C=24, R=16, K=12):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((rows, C)), rng.standard_normal((C, R)) / np.sqrt(C),
            rng.standard_normal((R, K)) / 4.0, rng.standard_normal(K))


def test_lowrank_gate_pins():
    x, w1, w2, b = _lowrank_inputs(61)
    lg = oracle.lowrank_gate(x, w1, w2, b)
    assert lg.shape == (37, 12) and np.all(lg <= 0)
    # no projection: a constant gate; logsigmoid(0) = -ln 2, logsigmoid(ln 3) = ln(3/4)
    const = oracle.lowrank_gate(x, w1, 0 * w2, np.array([0.0, np.log(3.0)] * 6), inv_tau=1.0)
    np.testing.assert_allclose(const[:, 0], -np.log(2.0), rtol=1e-15)
    np.testing.assert_allclose(const[:, 1], np.log(0.75), rtol=1e-15)
    # sigma(y) / sigma(-y) = e^y: flipping the sign of the projection and the bias
    # moves log_gamma by exactly inv_tau * (x W1 W2 + b), a plain matrix product
    flip = oracle.lowrank_gate(x, w1, -w2, -b)
    np.testing.assert_allclose(lg - flip, (x @ w1 @ w2 + b) / 16.0, rtol=1e-12, atol=1e-14)
    # sigma(y) + sigma(-y) = 1: the two gates raised to tau add up to one
    np.testing.assert_allclose(np.exp(16 * lg) + np.exp(16 * flip), 1.0, rtol=1e-13)
    # tau divides the log
    np.testing.assert_allclose(oracle.lowrank_gate(x, w1, w2, b, inv_tau=1.0), 16 * lg, rtol=1e-14)
    # x enters only through x W1: a component outside W1's column space changes nothing
    q_, _ = np.linalg.qr(w1)
    perp = np.random.default_rng(62).standard_normal(x.shape)
    perp -= perp @ q_ @ q_.T
    np.testing.assert_allclose(oracle.lowrank_gate(x + perp, w1, w2, b), lg, rtol=1e-11, atol=1e-13)
    # no overflow for large pre-activations
    big = oracle.lowrank_gate(x, w1, 1e4 * w2, b)
    assert np.isfinite(big).all() and np.all(big <= 0)
