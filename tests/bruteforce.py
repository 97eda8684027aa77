"""Dense brute force of the window + global attention forward, for tiny n.

A second, independent construction of the same definition as the oracle: it
builds the explicit n x n boolean attention mask of every (batch row, head) and
runs an ordinary masked softmax over whole score rows in float64.  Where the
oracle walks window taps i + k*s, this uses the distance test |i-j| <= r*s with
(i-j) divisible by s; where the oracle appends the global list, this ORs a
global-column mask, so a global key inside the window is a single mask entry.
"""
import numpy as np


def mask_for(lmask_row, gmask_row, window, gap):
    """(local_mask [n,n], global_mask [n,n], valid [n], glob [n])."""
    valid = np.asarray(lmask_row) != 0
    glob = valid & (np.asarray(gmask_row) != 0)
    n = valid.shape[0]
    idx = np.arange(n)
    dist = idx[:, None] - idx[None, :]
    s = gap + 1
    r = window // 2
    inwin = (np.abs(dist) <= r * s) & (dist % s == 0)
    local_mask = (inwin | glob[None, :]) & valid[None, :]
    global_mask = np.broadcast_to(valid[None, :], (n, n))
    return local_mask, global_mask, valid, glob


def _masked_softmax_av(q, k, v, mask, scale):
    s = scale * (q @ k.T)
    s = np.where(mask, s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    mx = np.where(np.isfinite(mx), mx, 0.0)
    e = np.where(mask, np.exp(s - mx), 0.0)
    tot = e.sum(axis=1, keepdims=True)
    p = e / np.where(tot > 0, tot, 1.0)
    return p @ v


def dense_forward(Q, K, V, Qg, Kg, Vg, lmask, gmask, window, dilation, scale):
    Q, K, V, Qg, Kg, Vg = (np.asarray(a, np.float64) for a in (Q, K, V, Qg, Kg, Vg))
    B, H, n, d = Q.shape
    out = np.zeros((B, H, n, d))
    for b in range(B):
        for h in range(H):
            lm, gm, valid, glob = mask_for(lmask[b], gmask[b], window, dilation[h])
            o_loc = _masked_softmax_av(Q[b, h], K[b, h], V[b, h], lm, scale)
            o_glb = _masked_softmax_av(Qg[b, h], Kg[b, h], Vg[b, h], gm, scale)
            o = np.where(glob[:, None], o_glb, o_loc)
            o[~valid] = 0.0
            out[b, h] = o
    return out
