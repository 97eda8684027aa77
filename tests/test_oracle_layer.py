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


# ---------------------------------------------------------------------------
# The attention wiring of the layer (FasterTransformer Longformer encoder guide,
# "Longformer Encoder compute flow": the [Q|K|V] and [Qg|Kg|Vg] projections
# split into heads, the local rows reading Q/K/V, the global rows Qg/Kg/Vg,
# the heads merged back before the output projection).
#
# Closed form.  X[b, j] is the one-hot row e_j (n <= hid), so a projection of
# row j is row j of its weight plus the bias.  The Q projection is the
# constant L on channel 0 of every head; the K projection puts 1 on channel 0
# of head h exactly for the positions in T_h (j % (h + 2) == 0); the global
# query/key projections vanish.  A local row's scores are then L * scale on
# its keys in T_h and 0 on the others: with L * scale = 50 the softmax puts
# weight 1 (to e^-50) uniformly on A_i n T_h, or uniformly on A_i when that is
# empty.  A global row's scores are all 0: uniform over the valid keys.  The
# value projections are distinct random matrices, so the attention output is
# a known mean of rows of W_v (W_vg) plus the bias, and the FFN is switched
# off (w_1 = b_1 = 0 gives GELU(0) = 0), so that
#     Y = LN(b_2 + H1),  H1 = LN(merge(A) w_o + b_o + X),
# merge(A)[b, i, h d + e] = A[b, h, i, e].  The key sets A_i come from
# oracle.allowed (pinned on its own in test_oracle.py).
# ---------------------------------------------------------------------------

_WIRE = dict(B=2, H=3, d=8, n=24, window=6, dilation=[0, 1, 2], inter=16, eps=1e-5)


def _wiring_case():
    c = _WIRE
    B, H, d, n, inter = c["B"], c["H"], c["d"], c["n"], c["inter"]
    hid = H * d
    assert n <= hid
    rng = np.random.default_rng(17)
    w = _weights(rng, hid, inter)
    L = 50.0 * math.sqrt(d)          # L * (1 / sqrt(d)) = 50
    w["w_qkv"][:, :2 * hid] = 0.0
    w["b_qkv"][:2 * hid] = 0.0
    T = [np.arange(n) % (h + 2) == 0 for h in range(H)]
    for h in range(H):
        w["b_qkv"][h * d] = L                              # Q: L on channel 0 of head h
        w["w_qkv"][np.flatnonzero(T[h]), hid + h * d] = 1.0  # K: 1 on channel 0 at T_h
    w["w_g"][:, :2 * hid] = 0.0
    w["b_g"][:2 * hid] = 0.0
    w["w_1"][:] = 0.0
    w["b_1"][:] = 0.0
    X = np.zeros((B, n, hid))
    X[:, np.arange(n), np.arange(n)] = 1.0
    lm = np.ones((B, n), np.float32)
    lm[1, 19:] = 0.0                                        # padded tail in row 1
    gm = np.zeros((B, n), np.float32)
    gm[0, [0, 9]] = 1.0
    gm[1, [4, 21]] = 1.0                                    # 21 is padded: not global
    return w, X, lm, gm, T


def _wiring_expected(w, X, lm, gm, T):
    c = _WIRE
    B, H, d, n = c["B"], c["H"], c["d"], c["n"]
    hid = H * d
    # the attention takes float32 copies of its inputs
    V = np.asarray(np.float32(w["w_qkv"][:n, 2 * hid:] + w["b_qkv"][2 * hid:]), np.float64)
    Vg = np.asarray(np.float32(w["w_g"][:n, 2 * hid:] + w["b_g"][2 * hid:]), np.float64)
    A = np.zeros((B, H, n, d))
    for b in range(B):
        for h in range(H):
            for i in range(n):
                kind, keys = oracle.allowed(lm[b], gm[b], c["window"], c["dilation"][h], i)
                if kind == oracle.PADDED:
                    continue
                src = Vg if kind == oracle.GLOBAL else V
                if kind == oracle.LOCAL:
                    hit = keys[T[h][keys]]
                    keys = hit if hit.size else keys
                A[b, h, i] = src[keys, h * d:(h + 1) * d].mean(axis=0)
    merged = np.zeros((B * n, hid))
    for h in range(H):
        merged[:, h * d:(h + 1) * d] = A[:, h].reshape(B * n, d)
    x2 = X.reshape(B * n, hid)
    h1 = oracle.layernorm(merged @ w["w_o"] + w["b_o"] + x2, w["ln1_g"], w["ln1_b"], c["eps"])
    y = oracle.layernorm(h1 + w["b_2"], w["ln2_g"], w["ln2_b"], c["eps"])
    return y.reshape(B, n, hid)


def _run_layer(fn, w, X, lm, gm):
    c = _WIRE
    return fn(X, w, lm, gm, c["window"], c["dilation"], c["H"], c["eps"], threads=1)


def test_layer_attention_wiring_closed_form():
    w, X, lm, gm, T = _wiring_case()
    want = _wiring_expected(w, X, lm, gm, T)
    got = _run_layer(oracle.layer_forward, w, X, lm, gm)
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-9)


def _miswired(variant):
    """The layer oracle with one wiring mistake planted (CPU only): the pin
    above must reject each of them."""
    L = oracle.layer

    def fwd(X, w, lmask, gmask, window, dilation, H, eps, threads=None):
        X = np.asarray(X, np.float64)
        B, n, hid = X.shape
        d = hid // H
        W = {k: np.asarray(v, np.float64) for k, v in w.items()}
        x2 = X.reshape(B * n, hid)
        p1 = x2 @ W["w_qkv"] + W["b_qkv"]
        p2 = x2 @ W["w_g"] + W["b_g"]
        blocks1 = [p1[:, i * hid:(i + 1) * hid] for i in range(3)]
        blocks2 = [p2[:, i * hid:(i + 1) * hid] for i in range(3)]
        if variant == "qk_swapped":
            blocks1 = [blocks1[1], blocks1[0], blocks1[2]]
        if variant == "qv_swapped":
            blocks1 = [blocks1[2], blocks1[1], blocks1[0]]
        q, k, v = (L.split_heads(x, B, n, H, d) for x in blocks1)
        qg, kg, vg = (L.split_heads(x, B, n, H, d) for x in blocks2)
        if variant == "global_rows_use_v":
            vg = v
        if variant == "local_rows_use_global_projections":
            q, k, v = qg, kg, vg
        a = oracle.forward(q, k, v, qg, kg, vg, lmask, gmask, window, dilation, 1.0 / np.sqrt(d),
                           threads=threads)
        if variant == "merge_without_transpose":
            am = a.reshape(B * n, hid)
        else:
            am = a.transpose(0, 2, 1, 3).reshape(B * n, hid)
        h1 = L.layernorm(am @ W["w_o"] + W["b_o"] + x2, W["ln1_g"], W["ln1_b"], eps)
        f = L.gelu(h1 @ W["w_1"] + W["b_1"])
        y = L.layernorm(f @ W["w_2"] + W["b_2"] + h1, W["ln2_g"], W["ln2_b"], eps)
        return y.reshape(B, n, hid)
    return fwd


def test_layer_wiring_pin_rejects_planted_miswirings():
    w, X, lm, gm, T = _wiring_case()
    want = _wiring_expected(w, X, lm, gm, T)
    np.testing.assert_allclose(_run_layer(_miswired("none"), w, X, lm, gm), want, rtol=1e-9, atol=1e-9)
    for variant in ("qk_swapped", "qv_swapped", "global_rows_use_v",
                    "local_rows_use_global_projections", "merge_without_transpose"):
        got = _run_layer(_miswired(variant), w, X, lm, gm)
        assert np.max(np.abs(got - want)) > 1e-3, variant
