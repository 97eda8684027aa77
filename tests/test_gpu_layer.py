"""GPU parity of the encoder layer (lwattn_layer_* through the C ABI) against
the oracle's float64 layer, fed the same stored (bf16) inputs and weights.

Tolerance, from the arithmetic: the GEMMs accumulate in fp32 and every
intermediate is rounded to bf16 once (Q, K, V, Qg, Kg, Vg; the attention
output; the output projection and FFN-out results before their LayerNorms;
H1; the FFN-in result before the GELU; the GELU output) and Y itself (2^-9
relative each).  LayerNorm
outputs are O(1) (at most a few units); the roundings of H1 and Y alone give
up to 2^-9 of that, the earlier ones reach Y through the GEMMs' sums over hid
or inter terms of random sign.  With outputs of magnitude up to about 5 the
roundings of Y and H1 alone reach 2^-9 * 5 = 0.01.  The bound is |err| <= 4e-2
elementwise, with the mean error below a tenth of that (measured: at most
0.030 and 0.0024 over the cases).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import make_plan, say, to_np64
from long_document_sparse_amd import lwattn as lw
from long_document_sparse_amd import workloads

pytestmark = pytest.mark.gpu


def _weights(layer, seed, dev):
    rng = np.random.default_rng(seed)
    w = {}
    for name, shape in layer.shapes().items():
        if name.startswith("ln") and name.endswith("_g"):
            a = 1.0 + 0.1 * rng.standard_normal(shape)
        elif len(shape) == 2:
            a = rng.standard_normal(shape) / math.sqrt(shape[0])
        else:
            a = 0.1 * rng.standard_normal(shape)
        w[name] = torch.from_numpy(a.astype(np.float32)).to(dev).to(torch.bfloat16)
    return w


CASES = [
    # (B, H, n, window, dilation, n_global, pad_mode, pad_hi, inter)
    (2, 8, 300, 64, [0] * 6 + [1, 2], 3, "per_batch", 60, 1024),
    (1, 16, 512, 128, [0] * 16, 8, "none", 0, 4096),
    (1, 12, 1024, 256, [0] * 12, 40, "per_batch", 100, 3072),   # base-model heads (hid 768)
    (2, 4, 200, 32, [0, 1, 2, 3], 0, "none", 0, 512),           # no global token at all
    # padding anywhere in the row: the attention's register-staged paths,
    # reading Q, K, V, Kg, Vg in place from the projections
    (2, 8, 300, 64, [0] * 4 + [1] * 4, 5, "scatter", 60, 1024),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}n{c[2]}w{c[3]}i{c[8]}")
def test_layer_matches_oracle(case):
    B, H, n, window, dil, ng, pmode, phi, inter = case
    spec = workloads.custom(B, H, n, 64, window, "bf16", dil, seed=51, n_global=ng,
                            global_mode="random", pad_mode=pmode, pad_hi=phi)
    say(f"layer case {case}")
    x = workloads.generate(spec)
    dev = "cuda:0"
    plan = make_plan(spec, max_global=max(ng, 1))
    layer = lw.Layer(plan, inter, 1e-5)
    w = _weights(layer, 5, dev)
    rng = np.random.default_rng(6)
    X = torch.from_numpy(rng.standard_normal((B * n, H * 64)).astype(np.float32)).to(dev).to(torch.bfloat16)
    lm = torch.from_numpy(x.lmask).to(dev)
    gm = torch.from_numpy(x.gmask).to(dev)
    Y = layer.forward(X, w, lm, gm)
    torch.cuda.synchronize()
    assert plan.sync_status() == lw.OK
    got = to_np64(Y)
    want = oracle.layer_forward(to_np64(X).reshape(B, n, H * 64), {k: to_np64(t) for k, t in w.items()},
                                x.lmask, x.gmask, window, dil, H, 1e-5).reshape(B * n, H * 64)
    err = np.abs(got - want)
    bound = 4e-2
    say(f"max err {err.max():.4g} mean {err.mean():.4g} bound {bound:.4g}")
    assert np.all(np.isfinite(got))
    assert err.max() <= bound
    assert err.mean() <= bound / 10
    layer.close()


def test_layer_rejects_unsupported_heads_and_bad_arguments():
    spec = workloads.custom(1, 6, 128, 64, 32, "bf16", [0] * 6, n_global=1)
    plan = make_plan(spec, max_global=1)
    with pytest.raises(lw.LwattnError):
        lw.Layer(plan, 1024)
    spec = workloads.custom(1, 8, 128, 64, 32, "bf16", [0] * 8, n_global=1)
    plan = make_plan(spec, max_global=1)
    with pytest.raises(lw.LwattnError):
        lw.Layer(plan, 1023)
    layer = lw.Layer(plan, 1024)
    lib = lw.load_library()
    assert lib.lwattn_layer_forward(layer.handle, None, None, None, None, None, None) == lw.E_INVALID
    layer.close()
