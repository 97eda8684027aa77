"""Pins of the oracle's backward (the gradient of the forward) against things
other than its own code: central differences of the forward oracle, torch's
autograd of dense softmax attention in float64 where the method reduces to it,
and identities of the softmax gradient (zero-sum key gradients, value-gradient
sums equal to output-gradient sums, exact zeros where no path exists).
"""
import numpy as np
import pytest
import torch

import oracle

EPS = 2.0 ** -10   # exact in float32 for the |x| < 8 of these inputs


def _problem(seed, B, H, n, d, window, gaps, n_glob, pad_tail, glob_pos=None):
    rng = np.random.default_rng(seed)
    X = [rng.standard_normal((B, H, n, d)).astype(np.float32) for _ in range(6)]
    lm = np.ones((B, n), np.float32)
    gm = np.zeros((B, n), np.float32)
    for b in range(B):
        if pad_tail:
            lm[b, n - pad_tail - b:] = 0.0
        pos = glob_pos if glob_pos is not None else rng.choice(n, n_glob, replace=False)
        gm[b, pos] = 1.0
    dO = rng.standard_normal((B, H, n, d)).astype(np.float32)
    return X, lm, gm, dO, window, list(gaps)


FD_CASES = [
    # seed, B, H, n, d, window, gaps, n_glob, pad_tail
    (1, 1, 2, 10, 4, 4, [0, 1], 1, 0),
    (2, 2, 2, 9, 3, 4, [0, 2], 2, 2),          # padding (a global inside the pad too)
    (3, 1, 1, 12, 3, 2, [1], 3, 1),
    (4, 1, 1, 7, 2, 20, [0], 0, 0),             # window wider than the sequence
]


@pytest.mark.parametrize("case", FD_CASES, ids=lambda c: f"seed{c[0]}")
def test_backward_matches_central_differences(case):
    seed, B, H, n, d, window, gaps, n_glob, pad = case
    X, lm, gm, dO, window, gaps = _problem(seed, B, H, n, d, window, gaps, n_glob, pad)
    R = dO.astype(np.float64)
    grads = oracle.backward(*X, lm, gm, dO, window, gaps, threads=1)

    def loss(xs):
        return float(np.sum(oracle.forward(*xs, lm, gm, window, gaps, threads=1) * R))

    for which in range(6):
        fd = np.zeros(X[which].shape)
        for idx in np.ndindex(X[which].shape):
            xs = [x.copy() for x in X]
            xs[which][idx] += np.float32(EPS)
            up = loss(xs)
            xs[which][idx] -= np.float32(2 * EPS)
            dn = loss(xs)
            fd[idx] = (up - dn) / (2 * EPS)
        err = np.abs(fd - grads[which])
        assert np.all(err <= 2e-5 + 1e-4 * np.abs(grads[which])), \
            f"input {which}: max err {err.max():.3e}"


@pytest.mark.parametrize("gap", [0, 2])
def test_wide_window_backward_is_dense_attention_backward(gap):
    """No padding, no globals, a window reaching every key of the row's residue
    class: the gradients are those of dense softmax attention within each class."""
    B, H, n, d = 2, 2, 18, 8
    X, lm, gm, dO, _, _ = _problem(5, B, H, n, d, 0, [gap] * H, 0, 0, glob_pos=[])
    window = 2 * n
    got = oracle.backward(*X, lm, gm, dO, window, [gap] * H, threads=2)
    scale = 1.0 / np.sqrt(d)
    s = gap + 1
    q, k, v = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in X[:3])
    go = torch.tensor(dO, dtype=torch.float64)
    outs = torch.zeros(B, H, n, d, dtype=torch.float64)
    for rho in range(s):
        sl = slice(rho, n, s)
        att = torch.softmax(scale * q[:, :, sl] @ k[:, :, sl].transpose(-1, -2), dim=-1)
        outs[:, :, sl] = att @ v[:, :, sl]
    (outs * go).sum().backward()
    for mine, ref in zip(got[:3], (q.grad, k.grad, v.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-10, atol=1e-12)
    for z in got[3:]:
        assert not np.any(z)


def test_backward_identities_and_zeros():
    B, H, n, d = 2, 3, 40, 5
    X, lm, gm, dO, window, gaps = _problem(7, B, H, n, d, 6, [0, 1, 3], 4, 5)
    dQ, dK, dV, dQg, dKg, dVg = oracle.backward(*X, lm, gm, dO, window, gaps, threads=2)
    valid = lm != 0
    glob = valid & (gm != 0)
    local = valid & ~glob
    go = dO.astype(np.float64)
    for b in range(B):
        for h in range(H):
            # every row's softmax gradient sums to zero over its keys
            np.testing.assert_allclose(dK[b, h].sum(0), 0.0, atol=1e-10)
            np.testing.assert_allclose(dKg[b, h].sum(0), 0.0, atol=1e-10)
            # every row's probabilities sum to one
            np.testing.assert_allclose(dV[b, h].sum(0), go[b, h][local[b]].sum(0), atol=1e-10)
            np.testing.assert_allclose(dVg[b, h].sum(0), go[b, h][glob[b]].sum(0), atol=1e-10)
            # no path: dQ at global/padded rows, dQg at non-global rows, padded keys
            assert not np.any(dQ[b, h][~local[b]])
            assert not np.any(dQg[b, h][~glob[b]])
            for t in (dK, dV, dKg, dVg):
                assert not np.any(t[b, h][~valid[b]])
