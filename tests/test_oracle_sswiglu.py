"""Pins of the Spatial SwiGLU oracle (oracle/sswiglu.py) against what the pages
and the mathematics fix: hand-worked examples (tests/golden/sswiglu_hand.json),
the convolution against scipy's 2-D cross-correlation per channel, the SiLU
identity SiLU(z) - SiLU(-z) = z (from sigma(z) + sigma(-z) = 1) checked with
plain matrix products, the bias-only and zero-gate cases, and translation
equivariance away from the border."""
import json
import math
import os

import numpy as np
import pytest
from scipy.signal import correlate2d

from oracle import sswiglu as ss

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sswiglu_hand.json")


def _random(seed, B=2, gh=5, gw=7, C=6, Hd=10, Co=4):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, gh * gw, C))
    wg = rng.standard_normal((Hd, C)) / math.sqrt(C)
    wv = rng.standard_normal((Hd, C)) / math.sqrt(C)
    cw = rng.standard_normal((Hd, 3, 3)) / 3.0
    cb = rng.standard_normal(Hd)
    wo = rng.standard_normal((Co, Hd)) / math.sqrt(Hd)
    return x, wg, wv, cw, cb, wo, gh, gw


def _scipy_conv(u, gh, gw, cw, cb):
    """Per-channel 2-D cross-correlation, zero fill, same size, plus bias."""
    B, L, Hd = u.shape
    img = u.reshape(B, gh, gw, Hd)
    out = np.empty_like(img)
    for b in range(B):
        for ch in range(Hd):
            out[b, :, :, ch] = correlate2d(img[b, :, :, ch], cw[ch], mode="same",
                                           boundary="fill", fillvalue=0.0) + cb[ch]
    return out.reshape(B, L, Hd)


@pytest.mark.parametrize("ex", json.load(open(GOLDEN))["examples"], ids=lambda e: e["name"])
def test_hand_examples(ex):
    ln3 = math.log(3.0)
    y = ss.sswiglu(np.array(ex["x"])[None], np.array(ex["w_g_over_ln3"]) * ln3,
                   np.array(ex["w_v"]), np.array(ex["conv_w"]), np.array(ex["conv_b"]),
                   np.array(ex["w_o"]), ex["grid_h"], ex["grid_w"])[0]
    expect = np.array([[n / d * ln3] for n, d in ex["y_over_ln3"]])
    np.testing.assert_allclose(y, expect, rtol=1e-14)


def test_conv_matches_scipy_correlate2d():
    """With W_v = I, W_o = I and a gate of exactly SiLU(40) = 40 (fp64 sigma(40)
    rounds to 1), Y / 40 is the depthwise convolution of x itself."""
    rng = np.random.default_rng(3)
    B, gh, gw, n = 2, 6, 9, 5
    x = rng.standard_normal((B, gh * gw, n))
    x[..., 0] = 1.0                      # a constant channel drives the gate
    wg = np.zeros((n, n))
    wg[:, 0] = 40.0
    cw = rng.standard_normal((n, 3, 3))
    cb = rng.standard_normal(n)
    y = ss.sswiglu(x, wg, np.eye(n), cw, cb, np.eye(n), gh, gw)
    np.testing.assert_allclose(y / 40.0, _scipy_conv(x, gh, gw, cw, cb), rtol=1e-13, atol=1e-13)


def test_silu_sign_identity():
    """SiLU(z) - SiLU(-z) = z, so Y(W_g) - Y(-W_g) = ((x W_g^T) ⊙ conv(x W_v^T)) W_o^T,
    the convolution taken from scipy (non-square weights catch a transposed operand)."""
    x, wg, wv, cw, cb, wo, gh, gw = _random(5)
    d = ss.sswiglu(x, wg, wv, cw, cb, wo, gh, gw) - ss.sswiglu(x, -wg, wv, cw, cb, wo, gh, gw)
    ref = ((x @ wg.T) * _scipy_conv(x @ wv.T, gh, gw, cw, cb)) @ wo.T
    np.testing.assert_allclose(d, ref, rtol=1e-12, atol=1e-13)


def test_bias_only_and_zero_gate():
    x, wg, wv, cw, cb, wo, gh, gw = _random(7)
    # a zero kernel leaves the bias: Y = (SiLU(x W_g^T) * b) W_o^T, SiLU by its definition
    g = x @ wg.T
    y = ss.sswiglu(x, wg, wv, 0 * cw, cb, wo, gh, gw)
    np.testing.assert_allclose(y, (g / (1 + np.exp(-g)) * cb) @ wo.T, rtol=1e-12, atol=1e-14)
    # a zero gate projection gives SiLU(0) = 0 everywhere
    assert np.all(ss.sswiglu(x, 0 * wg, wv, cw, cb, wo, gh, gw) == 0.0)
    # without a bias the convolution of a zero value branch is zero
    assert np.all(ss.sswiglu(x, wg, 0 * wv, cw, None, wo, gh, gw) == 0.0)


def test_translation_equivariance():
    """An input pattern moved by (1, 2) inside the grid (zeros around it) moves the
    output by the same amount wherever the 3x3 window stays inside the grid."""
    rng = np.random.default_rng(11)
    B, gh, gw, C, Hd = 1, 9, 10, 3, 4
    x = np.zeros((B, gh, gw, C))
    x[:, 2:5, 2:6, :] = rng.standard_normal((B, 3, 4, C))
    xs = np.roll(x, (1, 2), axis=(1, 2))
    _, wg, wv, cw, _, wo, _, _ = _random(12, C=C, Hd=Hd, Co=2)
    y = ss.sswiglu(x.reshape(B, -1, C), wg, wv, cw, None, wo, gh, gw).reshape(B, gh, gw, 2)
    ys = ss.sswiglu(xs.reshape(B, -1, C), wg, wv, cw, None, wo, gh, gw).reshape(B, gh, gw, 2)
    np.testing.assert_allclose(ys[:, 2:8, 3:9], y[:, 1:7, 1:7], rtol=1e-13, atol=1e-15)


def test_silu_extremes_and_shape_errors():
    assert ss.silu(np.array(-1000.0)) == 0.0 and ss.silu(np.array(1000.0)) == 1000.0
    x, wg, wv, cw, cb, wo, gh, gw = _random(13)
    with pytest.raises(ValueError):
        ss.sswiglu(x, wg.T, wv, cw, cb, wo, gh, gw)
    with pytest.raises(ValueError):
        ss.dwconv3x3(x @ wv.T, gh + 1, gw, cw)
    with pytest.raises(ValueError):
        ss.dwconv3x3(x @ wv.T, gh, gw, cw[:, :2])
