"""Oracle of the encoder layer around the attention -- TEST INFRASTRUCTURE
ONLY (tests, smoke and the benchmark's CPU baseline).  It shares nothing with
the HIP path.

The plain definition, in float64 numpy, after the FasterTransformer Longformer
encoder guide (hnwysp.cn), compute flow: per layer, the Q, K, V projections
and the global path's Qg, Kg, Vg projections (GEMM plus bias, split into heads
[B, H, n, d]), the Longformer attention, the attention output projection,
AddBiasResidualLayerNorm, the FFN (intermediate GEMM, bias, GELU, output GEMM)
and AddBiasResidualLayerNorm again.  The attention itself is the oracle's
forward (oracle.forward), which reads float32 copies of its inputs.

Readings where the page is silent: LayerNorm normalises each row by its mean
and biased variance with eps inside the square root, then scales by gamma and
shifts by beta; GELU is x * Phi(x) with the normal CDF written through erf
(no tanh approximation); the attention scale is 1 / sqrt(d).
"""
import math

import numpy as np

from . import forward as _attention


def gelu(x):
    """x * Phi(x), Phi the standard normal CDF (erf form)."""
    x = np.asarray(x, np.float64)
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def layernorm(x, gamma, beta, eps):
    x = np.asarray(x, np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps) * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)


def split_heads(p, B, n, H, d):
    """[B*n, H*d] -> [B, H, n, d]."""
    return p.reshape(B, n, H, d).transpose(0, 2, 1, 3)


def layer_forward(X, w, lmask, gmask, window, dilation, H, eps, threads=None):
    """X [B, n, hid]; w: dict of weights (row-major [in, out]) w_qkv, b_qkv,
    w_g, b_g, w_o, b_o, ln1_g, ln1_b, w_1, b_1, w_2, b_2, ln2_g, ln2_b.
    Returns Y [B, n, hid] in float64."""
    X = np.asarray(X, np.float64)
    B, n, hid = X.shape
    d = hid // H
    W = {k: np.asarray(v, np.float64) for k, v in w.items()}
    x2 = X.reshape(B * n, hid)
    p1 = x2 @ W["w_qkv"] + W["b_qkv"]
    p2 = x2 @ W["w_g"] + W["b_g"]
    q, k, v = (split_heads(p1[:, i * hid:(i + 1) * hid], B, n, H, d) for i in range(3))
    qg, kg, vg = (split_heads(p2[:, i * hid:(i + 1) * hid], B, n, H, d) for i in range(3))
    a = _attention(q, k, v, qg, kg, vg, lmask, gmask, window, dilation, 1.0 / math.sqrt(d),
                   threads=threads)
    am = a.transpose(0, 2, 1, 3).reshape(B * n, hid)
    h1 = layernorm(am @ W["w_o"] + W["b_o"] + x2, W["ln1_g"], W["ln1_b"], eps)
    f = gelu(h1 @ W["w_1"] + W["b_1"])
    y = layernorm(f @ W["w_2"] + W["b_2"] + h1, W["ln2_g"], W["ln2_b"], eps)
    return y.reshape(B, n, hid)
