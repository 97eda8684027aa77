"""GPU parity of the causal variant's backward (lwattn_backward_causal through
the C ABI) against the oracle's causal backward, element by element over dQ,
dK and dV.

Tolerance, derived from the arithmetic as for the window-and-global backward:
the HIP path accumulates in fp32 and the oracle in fp64; the matrix cores take
P and dS rounded to bf16 (2^-9 relative per term, of either sign) and the
gradients are stored in bf16 (2^-9).  Per tensor, relative to its largest
entry: |err| <= 2e-2 * max |g|.  Where the exact gradient vanishes (a window
of 0: P = 1, so dP_ii = D_i and dS = 0) only the fp32 cancellation of dP and D
remains, so the bound has a floor of 2^-16 scale d max|dO| max|V| max|Q, K|
(the size of the terms that cancel, times fp32 rounding over d products).
Rows and keys whose mask is 0 must be exactly zero in every gradient.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import make_plan, say, to_np64
from long_document_sparse_amd import workloads

pytestmark = pytest.mark.gpu

CASES = [
    # (B, H, n, window, dilation, pad_mode, pad_hi)
    (1, 2, 200, 64, [0, 1], "none", 0),
    (2, 3, 333, 40, [0, 2, 5], "per_batch", 80),
    (1, 2, 130, 400, [0, 0], "none", 0),          # window beyond the sequence
    (2, 2, 257, 16, [1, 4], "scatter", 40),       # scattered pads
    (1, 2, 1000, 300, [0, 1], "per_batch", 200),   # interior and edge tiles
    (1, 1, 65, 0, [0], "none", 0),                 # each row sees only itself
    (1, 1, 1, 32, [0], "none", 0),                 # n = 1
]


def _run(spec, strong, seed):
    x = workloads.generate(spec, strong=strong)
    dev = "cuda:0"
    q, k, v = (torch.from_numpy(a).to(dev).to(torch.bfloat16) for a in (x.Q, x.K, x.V))
    lm = torch.from_numpy(x.lmask).to(dev)
    g = torch.Generator().manual_seed(seed)
    do = torch.randn(q.shape, generator=g).to(dev).to(torch.bfloat16)
    plan = make_plan(spec, max_global=0)
    o = plan.forward_causal(q, k, v, lm)
    dq, dk, dv = plan.backward_causal(q, k, v, lm, o, do)
    torch.cuda.synchronize()
    return x, (q, k, v, do), (dq, dk, dv)


@pytest.mark.parametrize("strong", [False, True], ids=["scaled", "strong"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}n{c[2]}w{c[3]}{c[5]}")
def test_causal_backward_matches_oracle(case, strong):
    B, H, n, window, dil, pmode, phi = case
    spec = workloads.custom(B, H, n, 64, window, "bf16", dil, seed=41, n_global=0,
                            pad_mode=pmode, pad_hi=phi, max_global=0)
    say(f"causal backward case {case} strong={strong}")
    x, (q, k, v, do), got = _run(spec, strong, 43)
    want = oracle.backward_causal(to_np64(q), to_np64(k), to_np64(v), x.lmask, to_np64(do),
                                  window, dil, spec.scale)
    pad = x.lmask == 0
    amax = lambda t: float(t.abs().max())
    floor = 2.0 ** -16 * spec.scale * 64 * amax(do) * amax(v) * max(amax(q), amax(k))
    for name, g, w in zip(("dQ", "dK", "dV"), got, want):
        g = to_np64(g)
        assert np.all(np.isfinite(g)), name
        bound = max(2e-2 * np.abs(w).max(), floor)
        err = np.abs(g - w).max()
        assert err <= bound, (name, err, bound)
        for b in range(B):
            assert not np.any(g[b][:, pad[b]]), name


def test_causal_backward_charlm_sampled_heads():
    """The causal workload at full size: dQ, dK, dV of a few (batch, head)
    pairs against the oracle run on those heads alone (heads are independent)."""
    spec = workloads.named("charlm")
    say(f"causal backward charlm {spec.B}x{spec.H}x{spec.n} w={spec.window}")
    x, (q, k, v, do), got = _run(spec, False, 44)
    dil = list(spec.dilation)
    for b, h in ((0, 0), (spec.B - 1, spec.H - 1), (0, spec.H // 2)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        want = oracle.backward_causal(to_np64(q[sl]), to_np64(k[sl]), to_np64(v[sl]),
                                      x.lmask[b:b + 1], to_np64(do[sl]), spec.window, [dil[h]],
                                      spec.scale)
        for name, g, w in zip(("dQ", "dK", "dV"), got, want):
            g = to_np64(g[sl])
            bound = 2e-2 * max(np.abs(w).max(), 1e-30)
            err = np.abs(g - w).max()
            assert err <= bound, (name, b, h, err, bound)
