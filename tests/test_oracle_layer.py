"""Pins of the encoder-layer oracle (oracle/layer.py) against values fixed by
the mathematics: GELU at points where Phi is tabulated and its limits,
LayerNorm's normalised moments and its constant-row case, and the whole layer
in cases that reduce to closed forms (zero projections, zero FFN)."""
import math

import numpy as np

import oracle


def test_gelu_at_known_points():
    # Phi(0) = 1/2, Phi(1) = 0.8413447460685429, Phi(-1) = 1 - Phi(1), Phi(2) = 0.9772498680518208
    g = oracle.gelu([0.0, 1.0, -1.0, 2.0, -30.0, 30.0])
    np.testing.assert_allclose(g[:4], [0.0, 0.8413447460685429, -0.15865525393145707, 1.9544997361036416],
                               rtol=1e-15, atol=1e-16)
    assert abs(g[4]) < 1e-100 and g[5] == 30.0


def test_layernorm_moments_and_constant_rows():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64)) * 3 + 7
    y = oracle.layernorm(x, np.ones(64), np.zeros(64), 1e-12)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose((y ** 2).mean(axis=1), 1.0, rtol=1e-9)
    beta = rng.standard_normal(64)
    yc = oracle.layernorm(np.full((2, 64), 4.0), rng.standard_normal(64), beta, 1e-5)
    np.testing.assert_allclose(yc, np.broadcast_to(beta, (2, 64)), atol=1e-12)


def _weights(rng, hid, inter, zero=()):
    shapes = {"w_qkv": (hid, 3 * hid), "b_qkv": (3 * hid,), "w_g": (hid, 3 * hid), "b_g": (3 * hid,),
              "w_o": (hid, hid), "b_o": (hid,), "ln1_g": (hid,), "ln1_b": (hid,),
              "w_1": (hid, inter), "b_1": (inter,), "w_2": (inter, hid), "b_2": (hid,),
              "ln2_g": (hid,), "ln2_b": (hid,)}
    w = {k: rng.standard_normal(s) * (1 / math.sqrt(s[0]) if len(s) == 2 else 0.1) for k, s in shapes.items()}
    for k in zero:
        w[k] = np.zeros(shapes[k])
    return w


def test_layer_reduces_to_layernorms_when_projections_and_ffn_vanish():
    """w_o = 0 and w_2 = 0: H1 = LN(X + b_o), Y = LN(b_2 + H1) (GELU's input no longer matters)."""
    rng = np.random.default_rng(2)
    B, n, H, d, inter = 1, 40, 2, 8, 32
    hid = H * d
    w = _weights(rng, hid, inter, zero=("w_o", "w_2"))
    X = rng.standard_normal((B, n, hid))
    lm = np.ones((B, n), np.float32)
    gm = np.zeros((B, n), np.float32)
    gm[0, 0] = 1
    y = oracle.layer_forward(X, w, lm, gm, 8, [0, 1], H, 1e-5, threads=1)
    h1 = oracle.layernorm(X.reshape(-1, hid) + w["b_o"], w["ln1_g"], w["ln1_b"], 1e-5)
    want = oracle.layernorm(h1 + w["b_2"], w["ln2_g"], w["ln2_b"], 1e-5)
    np.testing.assert_allclose(y.reshape(-1, hid), want, rtol=1e-12, atol=1e-12)


def test_layer_attention_path_matches_direct_composition():
    """Zero value projections make the attention output zero (each output row
    is a convex combination of V rows), whatever the scores: then
    H1 = LN(X + b_o) and the FFN follows the plain formula."""
    rng = np.random.default_rng(3)
    B, n, H, d, inter = 2, 30, 2, 8, 16
    hid = H * d
    w = _weights(rng, hid, inter)
    w["w_qkv"][:, 2 * hid:] = 0.0
    w["b_qkv"][2 * hid:] = 0.0
    w["w_g"][:, 2 * hid:] = 0.0
    w["b_g"][2 * hid:] = 0.0
    X = rng.standard_normal((B, n, hid))
    lm = np.ones((B, n), np.float32)
    gm = np.zeros((B, n), np.float32)
    gm[:, 3] = 1
    y = oracle.layer_forward(X, w, lm, gm, 6, [0, 2], H, 1e-5, threads=1)
    h1 = oracle.layernorm(X.reshape(-1, hid) + w["b_o"], w["ln1_g"], w["ln1_b"], 1e-5)
    f = oracle.gelu(h1 @ w["w_1"] + w["b_1"])
    want = oracle.layernorm(f @ w["w_2"] + w["b_2"] + h1, w["ln2_g"], w["ln2_b"], 1e-5)
    np.testing.assert_allclose(y.reshape(-1, hid), want, rtol=1e-12, atol=1e-12)


def test_split_heads_is_the_head_major_reshape():
    p = np.arange(2 * 3 * 4 * 5).reshape(2 * 3, 4 * 5)
    s = oracle.layer.split_heads(p, 2, 3, 4, 5)
    assert s.shape == (2, 4, 3, 5)
    assert s[1, 2, 0, 3] == p[1 * 3 + 0, 2 * 5 + 3]
