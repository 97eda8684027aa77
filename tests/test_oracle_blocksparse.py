"""Pins of the oracle's block-sparse attention (a per-head layout over 64 x 64
blocks of the score matrix, optionally intersected with a causal mask:
xFormers' attention-mask notes).  Reading: row i of head h sees key j when
layout[h][i/64][j/64] is set, j is valid and (causal) j <= i; a padded row, or
a row that sees no key, outputs zero.

Pinned against a dense masked softmax built here from the reading, torch's
scaled_dot_product_attention in float64 for full layouts (with and without
is_causal), the Q = 0 closed form, block-diagonal layouts as independent dense
attention per block, and the CSR form of layouts used by the GPU path.
"""
import numpy as np
import pytest
import torch

import oracle
from long_document_sparse_amd import workloads


def _inputs(seed, B, H, n, d, pad=0):
    rng = np.random.default_rng(seed)
    Q, K, V = (rng.standard_normal((B, H, n, d)).astype(np.float32) for _ in range(3))
    lm = np.ones((B, n), np.float32)
    for b in range(B):
        if pad:
            lm[b, rng.choice(n, pad, replace=False)] = 0.0
    return Q, K, V, lm


def _dense(Q, K, V, lm, layout, causal, scale):
    B, H, n, d = Q.shape
    out = np.zeros((B, H, n, d))
    blk = np.arange(n) // 64
    for b in range(B):
        valid = lm[b] != 0
        for h in range(H):
            mask = layout[h][blk[:, None], blk[None, :]] != 0
            if causal:
                mask &= np.arange(n)[None, :] <= np.arange(n)[:, None]
            mask &= valid[None, :] & valid[:, None]
            x = scale * (Q[b, h].astype(np.float64) @ K[b, h].astype(np.float64).T)
            x = np.where(mask, x, -np.inf)
            rows = mask.any(axis=1)
            x[~rows] = 0.0
            p = np.where(mask, np.exp(x - x.max(axis=1, keepdims=True)), 0.0)
            p /= np.where(rows, p.sum(axis=1), 1.0)[:, None]
            out[b, h] = p @ V[b, h].astype(np.float64)
    return out


@pytest.mark.parametrize("n,causal,pad", [(200, False, 0), (200, True, 9), (257, True, 0), (130, False, 5)])
def test_blocksparse_matches_dense_masked_softmax(n, causal, pad):
    Q, K, V, lm = _inputs(21, 2, 3, n, 8, pad)
    lay = workloads.blocksparse_layout(3, n, seed=4, local=2, extra=1, causal=causal)
    got = oracle.forward_blocksparse(Q, K, V, lm, lay, causal, 0.3, threads=2)
    np.testing.assert_allclose(got, _dense(Q, K, V, lm, lay, causal, 0.3), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_full_layout_is_dense_sdpa(causal):
    Q, K, V, lm = _inputs(22, 1, 2, 150, 8)
    lay = np.ones((2, 3, 3), np.uint8)
    got = oracle.forward_blocksparse(Q, K, V, lm, lay, causal, 1 / np.sqrt(8), threads=2)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q).double(), torch.from_numpy(K).double(), torch.from_numpy(V).double(),
        is_causal=causal).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_zero_queries_average_the_allowed_values():
    Q, K, V, lm = _inputs(23, 1, 1, 180, 4, pad=7)
    Q[:] = 0.0
    lay = workloads.blocksparse_layout(1, 180, seed=5, local=1, extra=1)
    got = oracle.forward_blocksparse(Q, K, V, lm, lay, False, 0.5, threads=1)
    for i in range(180):
        if lm[0, i] == 0:
            assert not np.any(got[0, 0, i])
            continue
        keys = [j for j in range(180) if lay[0, i // 64, j // 64] and lm[0, j] != 0]
        np.testing.assert_allclose(got[0, 0, i], V[0, 0, keys].astype(np.float64).mean(axis=0),
                                   rtol=1e-12, atol=1e-14)


def test_block_diagonal_layout_is_dense_attention_per_block():
    Q, K, V, lm = _inputs(24, 1, 1, 192, 6)
    lay = np.eye(3, dtype=np.uint8)[None]
    got = oracle.forward_blocksparse(Q, K, V, lm, lay, False, 0.4, threads=1)
    for blk in range(3):
        sl = slice(64 * blk, 64 * blk + 64)
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q[:, :, sl]).double(), torch.from_numpy(K[:, :, sl]).double(),
            torch.from_numpy(V[:, :, sl]).double(), scale=0.4).numpy()
        np.testing.assert_allclose(got[:, :, sl], want, rtol=1e-12, atol=1e-12)


def test_empty_layout_rows_output_zero():
    Q, K, V, lm = _inputs(25, 1, 1, 128, 4)
    lay = np.zeros((1, 2, 2), np.uint8)
    lay[0, 1, 0] = 1
    got = oracle.forward_blocksparse(Q, K, V, lm, lay, False, 0.5, threads=1)
    assert not np.any(got[0, 0, :64])
    assert np.all(np.any(got[0, 0, 64:] != 0, axis=1))


def test_layout_csr_lists_every_set_block_in_order():
    lay = workloads.blocksparse_layout(3, 1000, seed=6, local=3, extra=2, causal=True)
    rowptr, cols = workloads.layout_csr(lay)
    H, nb, _ = lay.shape
    for h in range(H):
        for qb in range(nb):
            r = h * nb + qb
            assert list(cols[rowptr[r]:rowptr[r + 1]]) == list(np.flatnonzero(lay[h, qb]))
            assert all(c <= qb for c in cols[rowptr[r]:rowptr[r + 1]])   # causal layout


@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_pair_counter_matches_the_reading(causal):
    from long_document_sparse_amd import flops
    rng = np.random.default_rng(26)
    n, H = 200, 2
    lm = (rng.random((2, n)) > 0.15).astype(np.float32)
    lay = workloads.blocksparse_layout(H, n, seed=7, local=2, extra=2, causal=causal)
    total = 0
    for b in range(2):
        for h in range(H):
            for i in range(n):
                if lm[b, i] == 0:
                    continue
                total += sum(1 for j in range(n) if lay[h, i // 64, j // 64] and lm[b, j] != 0
                             and (not causal or j <= i))
    assert flops.blocksparse_pairs(lm, lay, causal) == total
