"""The Q = 0 closed form of the attention (LongFormer notes, sections "Sliding
Window", "Dilated Sliding Window", "Global Attention"; FasterTransformer
Longformer encoder guide, compute flow).

With every query zero, every allowed score is 0 and the softmax weight is
uniform over a row's key set A_i.  With one-hot values V_j = e_{(j + s) mod d}
the output row is then a per-channel count over the key set divided by its
size: O_i[c] = #{j in A_i : (j + s) mod d = c} / |A_i|.  Local rows count
under the local shift, global rows under the global one (they read Vg), padded
rows are zero.  The key sets are oracle.allowed's, which test_oracle.py pins
against hand-derived sets and a dense brute force.
"""
import numpy as np

import oracle

SHIFT_LOCAL = 0
SHIFT_GLOBAL = 17


def one_hot_rows(n, d, shift):
    """[n, d] float64: row j is e_{(j + shift) mod d}."""
    e = np.zeros((n, d))
    e[np.arange(n), (np.arange(n) + shift) % d] = 1.0
    return e


def expected_rows(lmask_row, gmask_row, window, gap, d=64, rows=None):
    """[len(rows), d] float64 expected outputs of one (batch row, dilation gap)."""
    n = int(np.shape(lmask_row)[0])
    rows = np.arange(n) if rows is None else np.asarray(rows)
    out = np.zeros((rows.size, d))
    for r, i in enumerate(rows):
        kind, keys = oracle.allowed(lmask_row, gmask_row, window, gap, int(i))
        if kind == oracle.PADDED:
            continue
        sh = SHIFT_GLOBAL if kind == oracle.GLOBAL else SHIFT_LOCAL
        out[r] = np.bincount((keys + sh) % d, minlength=d) / keys.size
    return out
