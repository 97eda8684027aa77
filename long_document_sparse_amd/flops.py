"""Algorithmic work of one forward: allowed (query, key) pairs, FLOPs and bytes.

The cost model is the O(n(w+g)) count of the Longformer pages ("LongFormer: The
Long-Document Transformer" notes, "Sliding Window" and "Global Attention"; the
bmjup.com explainer's complexity formula): every allowed pair costs one
d-long dot product for Q.K^T and one d-long axpy for P.V, i.e. 4*d FLOPs.
Masked-off, padded and tile-waste work is not counted, nor is the softmax.

Bytes count each input row the forward must read once and each output row
once: Q at local rows, Qg at global rows, K and V at valid rows, Kg and Vg at
valid rows when the batch row has any global token, O at every row, and the
two float32 masks.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np


def _flags(lmask, gmask):
    v = np.asarray(lmask) != 0
    g = v & (np.asarray(gmask) != 0)
    return v, g


def row_counts(lmask_row, gmask_row, window: int, gap: int) -> np.ndarray:
    """Allowed-key count of every query row of one (batch row, head); 0 for padding."""
    v, g = _flags(lmask_row, gmask_row)
    n = v.shape[0]
    r = window // 2
    s = gap + 1
    nglob = int(g.sum())
    nvalid = int(v.sum())
    out = np.zeros(n, np.int64)
    winkey = (v & ~g).astype(np.int64)
    for rho in range(min(s, n)):
        sub = winkey[rho::s]
        m = sub.shape[0]
        pre = np.concatenate([[0], np.cumsum(sub)])
        t = np.arange(m)
        lo = np.maximum(t - r, 0)
        hi = np.minimum(t + r, m - 1)
        out[rho::s] = pre[hi + 1] - pre[lo] + nglob
    out[g] = nvalid
    out[~v] = 0
    return out


def pairs(lmask, gmask, window: int, dilation: Sequence[int]) -> int:
    lm = np.asarray(lmask)
    gm = np.asarray(gmask)
    total = 0
    for b in range(lm.shape[0]):
        for gap in dilation:
            total += int(row_counts(lm[b], gm[b], window, int(gap)).sum())
    return total


def flops(lmask, gmask, window: int, dilation: Sequence[int], d: int) -> int:
    return 4 * d * pairs(lmask, gmask, window, dilation)


def global_pairs(lmask, gmask, H: int) -> int:
    """Pairs of the global rows alone (each global row sees every valid key)."""
    v, g = _flags(lmask, gmask)
    return int(H * (v.sum(axis=1) * g.sum(axis=1)).sum())


def hbm_bytes(lmask, gmask, H: int, d: int, elt: int) -> int:
    v, g = _flags(lmask, gmask)
    n = v.shape[1]
    total = 0
    for b in range(v.shape[0]):
        nv = int(v[b].sum())
        ng = int(g[b].sum())
        rows = (nv - ng) + ng + 2 * nv + (2 * nv if ng > 0 else 0) + n
        total += H * rows * d * elt
    total += 2 * 4 * v.size
    return total


def causal_pairs(lmask, window: int, dilation: Sequence[int]) -> int:
    """Allowed pairs of the causal variant: each valid row with its valid taps
    i - k s, 0 <= k <= window // 2."""
    lm = np.asarray(lmask) != 0
    B, n = lm.shape
    r = window // 2
    total = 0
    for b in range(B):
        for gap in dilation:
            s = int(gap) + 1
            for rho in range(min(s, n)):
                sub = lm[b, rho::s].astype(np.int64)
                pre = np.concatenate([[0], np.cumsum(sub)])
                t = np.arange(sub.shape[0])
                cnt = pre[t + 1] - pre[np.maximum(t - r, 0)]
                total += int((cnt * sub).sum())
    return total


def blocksparse_pairs(lmask, layout, causal: bool = False) -> int:
    """Allowed pairs of block-sparse attention: valid rows with the valid keys
    of their listed 64-blocks (with `causal`, keys at or before the row)."""
    lm = np.asarray(lmask) != 0
    lay = np.asarray(layout) != 0
    B, n = lm.shape
    H, nb, _ = lay.shape
    total = 0
    for b in range(B):
        v = np.zeros(nb * 64, bool)
        v[:n] = lm[b]
        vb = v.reshape(nb, 64)
        cnt = vb.sum(axis=1).astype(np.int64)           # valid keys (= valid rows) per block
        # within one block: valid rows times valid keys at or before them
        tri = (vb * np.cumsum(vb, axis=1)).sum(axis=1).astype(np.int64)
        for h in range(H):
            L = lay[h]
            if not causal:
                total += int(cnt @ L.astype(np.int64) @ cnt)
            else:
                below = np.tril(L, -1).astype(np.int64)
                total += int(cnt @ below @ cnt) + int((np.diag(L).astype(np.int64) * tri).sum())
    return total


def local_global_key_pairs(lmask, gmask, H: int) -> int:
    """Pairs of local rows with global keys (every local row sees every global key)."""
    v, g = _flags(lmask, gmask)
    return int(H * (((v & ~g).sum(axis=1)) * g.sum(axis=1)).sum())


def backward_kernel_flops(lmask, gmask, window: int, dilation: Sequence[int], d: int) -> dict:
    """Matrix FLOPs each bf16 backward kernel needs for what it writes, 2 d per
    product and pair: dq_kernel S, dP, dQ over the local rows' pairs;
    global_chunk_kernel S, dP, dQg over the global rows' pairs and S, dP, dK, dV
    over the local rows' pairs with global keys; dkv_kernel S, dP, dK, dV over
    the window pairs and S, dP, dKg, dVg over the global rows' pairs."""
    H = len(dilation)
    allp = pairs(lmask, gmask, window, dilation)
    gp = global_pairs(lmask, gmask, H)
    lg = local_global_key_pairs(lmask, gmask, H)
    win = allp - gp - lg
    return {"dq_kernel": 6 * d * (win + lg), "global_chunk_kernel": 6 * d * gp + 8 * d * lg,
            "global_merge_kernel": 0, "compact_kernel": 0, "dkv_kernel": 8 * d * (win + gp)}


def backward_flops(lmask, gmask, window: int, dilation: Sequence[int], d: int) -> int:
    """Algorithmic FLOPs of the backward: per allowed pair, the five d-long
    products of the chain rule (the score q.k, dP = dO.v, and the dq, dk, dv
    accumulations), 10*d FLOPs.  Recomputation the kernels do on top (the
    scores and dP evaluated a second time for the key gradients, the
    log-sum-exp pass) is not counted."""
    return 10 * d * pairs(lmask, gmask, window, dilation)


def backward_bytes(lmask, gmask, H: int, d: int, elt: int) -> int:
    """Each row the backward must read once (Q at local rows, Qg at global rows,
    K, V at valid rows, Kg, Vg at valid rows when there is a global token, O and
    dO at valid rows) and the six gradients written at every row, plus the
    masks."""
    v, g = _flags(lmask, gmask)
    n = v.shape[1]
    total = 0
    for b in range(v.shape[0]):
        nv = int(v[b].sum())
        ng = int(g[b].sum())
        reads = (nv - ng) + ng + 2 * nv + (2 * nv if ng > 0 else 0) + 2 * nv
        total += H * (reads + 6 * n) * d * elt
    total += 2 * 4 * v.size
    return total
