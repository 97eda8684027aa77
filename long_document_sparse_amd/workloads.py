"""Seeded synthetic inputs for the window + global attention forward.

This module only draws numbers: it holds none of the attention arithmetic, and
both the HIP path (tests, bench, smoke) and the CPU oracle consume what it
produces.  Every array is float32; for bf16 workloads the values are rounded to
the nearest bf16 (ties to even) here, so that both sides see identical inputs.

The five named workloads stand in for the pages' use cases (no dataset is used):
  tiny      fp32  B=1  H=2  n=512   w=128  one global at 0
  base      bf16  B=1  H=12 n=4096  w=512  [CLS]-style global at 0 (classification)
  qa        bf16  B=4  H=16 n=4096  w=512  64 question tokens global at the start,
                                           padded tail U{0..1024} per sequence
  dilated   fp32  B=2  H=12 n=8192  w=256  per-head dilation 0/1/2, 8 random globals
  long      bf16  B=8  H=16 n=16384 w=1024 128 scattered globals, one sequence with a
                                           padded tail U{1..4096}, 1% of K rows x8
Draw order (numpy PCG64 seeded per workload): pad lengths, padded-sequence choice,
global positions, Q, K, V, Qg, Kg, Vg (standard normal / sqrt(d), or unscaled in
the "strong" variant), the x8 K rows, then the bf16 rounding.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np


def round_to_f16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest IEEE half (ties to even), kept as float32."""
    return np.asarray(a, dtype=np.float32).astype(np.float16).astype(np.float32)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


@dataclasses.dataclass
class Spec:
    name: str
    B: int
    H: int
    n: int
    d: int
    window: int
    dtype: str                      # "f32", "bf16" or "f16"
    dilation: List[int]             # gap per head
    seed: int
    max_global: int
    # structure recipe
    global_mode: str = "first"      # "first": positions [0, g); "random": uniform in valid prefix
    n_global: int = 1
    pad_mode: str = "none"          # "none" | "per_batch" (tail U{lo..hi} each) | "one_seq" (one b,
                                    # tail U{lo..hi}) | "scatter" (U{lo..hi} padded positions anywhere)
    pad_lo: int = 0
    pad_hi: int = 0
    k_boost_frac: float = 0.0       # fraction of K rows per (b,h) multiplied by k_boost
    k_boost: float = 8.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def tokens(self) -> int:
        return self.B * self.n


def named(name: str) -> Spec:
    if name == "tiny":
        return Spec("tiny", 1, 2, 512, 64, 128, "f32", [0, 0], seed=1, max_global=64)
    if name == "base":
        return Spec("base", 1, 12, 4096, 64, 512, "bf16", [0] * 12, seed=2, max_global=64)
    if name == "qa":
        return Spec("qa", 4, 16, 4096, 64, 512, "bf16", [0] * 16, seed=3, max_global=64,
                    global_mode="first", n_global=64, pad_mode="per_batch", pad_lo=0, pad_hi=1024)
    if name == "dilated":
        return Spec("dilated", 2, 12, 8192, 64, 256, "f32", [0] * 6 + [1] * 3 + [2] * 3, seed=4,
                    max_global=64, global_mode="random", n_global=8)
    if name == "long":
        return Spec("long", 8, 16, 16384, 64, 1024, "bf16", [0] * 16, seed=5, max_global=128,
                    global_mode="random", n_global=128, pad_mode="one_seq", pad_lo=1, pad_hi=4096,
                    k_boost_frac=0.01)
    if name == "bsparse":
        # block-sparse layout over 64-blocks (8 heads, n = 16384): each query
        # block sees its own and 3 previous key blocks and 4 drawn ones
        return Spec("bsparse", 1, 8, 16384, 64, 0, "bf16", [0] * 8, seed=7, max_global=0,
                    global_mode="first", n_global=0)
    if name == "ftlayer":
        # one encoder layer of the QA model the FasterTransformer guide measures:
        # 16 heads of 64, intermediate 4096, window 512; the question's 64
        # tokens global at the start
        return Spec("ftlayer", 1, 16, 4096, 64, 512, "bf16", [0] * 16, seed=8, max_global=64,
                    global_mode="first", n_global=64)
    if name == "charlm":
        # causal variant (an autoregressive character model's attention): no
        # global tokens, no padding, two dilated heads
        return Spec("charlm", 2, 12, 8192, 64, 512, "bf16", [0] * 10 + [1] * 2, seed=6, max_global=0,
                    global_mode="first", n_global=0)
    raise KeyError(name)


NAMES = ("tiny", "base", "qa", "dilated", "long")
CAUSAL_NAMES = ("charlm",)
# layout of the "bsparse" workload (blocksparse_layout arguments)
BSPARSE_LAYOUT = dict(local=4, extra=4, causal=False)
# intermediate size of the "ftlayer" workload's FFN
FTLAYER_INTER = 4096


@dataclasses.dataclass
class Inputs:
    spec: Spec
    Q: np.ndarray
    K: np.ndarray
    V: np.ndarray
    Qg: np.ndarray
    Kg: np.ndarray
    Vg: np.ndarray
    lmask: np.ndarray               # float32 [B,n], 1.0 real token / 0.0 padding
    gmask: np.ndarray               # float32 [B,n], 1.0 global / 0.0 not
    pad_len: np.ndarray             # int [B]
    global_pos: List[np.ndarray]

    def tensors(self):
        return (self.Q, self.K, self.V, self.Qg, self.Kg, self.Vg)


def _structure(spec: Spec, rng) -> tuple:
    """Draws 1-3 of the recipe: (lmask, gmask, pad_len, global_pos)."""
    B, n = spec.B, spec.n

    # 1. pad lengths (and 2. which sequence is padded)
    pad_len = np.zeros(B, np.int64)
    lmask = np.ones((B, n), np.float32)
    if spec.pad_mode == "per_batch":
        pad_len = rng.integers(spec.pad_lo, spec.pad_hi, size=B, endpoint=True)
    elif spec.pad_mode == "one_seq":
        length = int(rng.integers(spec.pad_lo, spec.pad_hi, endpoint=True))
        which = int(rng.integers(0, B))
        pad_len[which] = length
    pad_len = np.minimum(pad_len, n)
    if spec.pad_mode == "scatter":
        for b in range(B):
            cnt = min(int(rng.integers(spec.pad_lo, spec.pad_hi, endpoint=True)), n)
            lmask[b, rng.choice(n, size=cnt, replace=False)] = 0.0
            pad_len[b] = cnt
    else:
        for b in range(B):
            if pad_len[b]:
                lmask[b, n - pad_len[b]:] = 0.0

    # 3. global positions, among the real tokens
    gmask = np.zeros((B, n), np.float32)
    global_pos = []
    for b in range(B):
        valid = np.flatnonzero(lmask[b] != 0)
        g = min(spec.n_global, valid.size)
        if spec.global_mode == "first":
            pos = valid[:g]
        else:
            pos = np.sort(valid[rng.choice(valid.size, size=g, replace=False)])
        gmask[b, pos] = 1.0
        global_pos.append(pos.astype(np.int64))
    return lmask, gmask, pad_len, global_pos


def structure(spec: Spec, seed: Optional[int] = None) -> tuple:
    """The masks of a workload alone, (lmask, gmask, pad_len, global_pos): the
    same draws as generate() makes before the tensors."""
    return _structure(spec, np.random.default_rng(spec.seed if seed is None else seed))


def generate(spec: Spec, strong: bool = False, seed: Optional[int] = None) -> Inputs:
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    B, H, n, d = spec.B, spec.H, spec.n, spec.d
    lmask, gmask, pad_len, global_pos = _structure(spec, rng)

    # 4. the six projected tensors
    div = np.float32(1.0) if strong else np.float32(math.sqrt(d))
    arrs = []
    for _ in range(6):
        a = rng.standard_normal((B, H, n, d), dtype=np.float32)
        a /= div
        arrs.append(a)
    Q, K, V, Qg, Kg, Vg = arrs

    # 5. a fraction of the K rows scaled up, to stress the softmax range
    if spec.k_boost_frac > 0:
        cnt = int(math.ceil(spec.k_boost_frac * n))
        for b in range(B):
            for h in range(H):
                rows = rng.choice(n, size=cnt, replace=False)
                K[b, h, rows, :] *= np.float32(spec.k_boost)

    # 6. storage rounding
    if spec.dtype == "bf16":
        Q, K, V, Qg, Kg, Vg = (round_to_bf16(a) for a in (Q, K, V, Qg, Kg, Vg))
    elif spec.dtype == "f16":
        Q, K, V, Qg, Kg, Vg = (round_to_f16(a) for a in (Q, K, V, Qg, Kg, Vg))
    return Inputs(spec, Q, K, V, Qg, Kg, Vg, lmask, gmask, pad_len, global_pos)


def custom(B: int, H: int, n: int, d: int = 64, window: int = 128, dtype: str = "f32",
           dilation: Optional[Sequence[int]] = None, seed: int = 0, n_global: int = 1,
           global_mode: str = "random", pad_mode: str = "none", pad_lo: int = 0, pad_hi: int = 0,
           max_global: Optional[int] = None, k_boost_frac: float = 0.0) -> Spec:
    """A parity-test shape with the same recipe as the named workloads."""
    return Spec("custom", B, H, n, d, window, dtype,
                list(dilation) if dilation is not None else [0] * H, seed=seed,
                max_global=max_global if max_global is not None else max(n_global, 1),
                global_mode=global_mode, n_global=n_global, pad_mode=pad_mode,
                pad_lo=pad_lo, pad_hi=pad_hi, k_boost_frac=k_boost_frac)


# ---------------------------------------------------------------------------
# Block-sparse layouts over 64 x 64 blocks of the score matrix (xFormers'
# attention-mask notes build such layouts per head with block_size 64).  A
# synthetic stand-in for a "fixed" layout: every query block sees its own
# block and the `local` - 1 blocks before it, plus `extra` other key blocks
# drawn per head and query block (at or before it when causal).

BS_BLOCK = 64


def blocksparse_layout(H: int, n: int, seed: int, local: int = 4, extra: int = 4,
                       causal: bool = False) -> np.ndarray:
    """uint8 [H, nb, nb] layout, nb = ceil(n / 64)."""
    rng = np.random.default_rng(seed)
    nb = (n + BS_BLOCK - 1) // BS_BLOCK
    lay = np.zeros((H, nb, nb), np.uint8)
    for h in range(H):
        for qb in range(nb):
            lay[h, qb, max(0, qb - local + 1):qb + 1] = 1
            hi = qb + 1 if causal else nb
            if extra > 0 and hi > 0:
                lay[h, qb, rng.choice(hi, min(extra, hi), replace=False)] = 1
    return lay


def layout_csr(layout) -> tuple:
    """(rowptr int32 [H*nb + 1], cols int32 [nnz]) of a [H, nb, nb] layout:
    the key blocks of query block qb of head h are cols[rowptr[h*nb + qb] ..
    rowptr[h*nb + qb + 1]), ascending."""
    lay = np.asarray(layout) != 0
    H, nb, _ = lay.shape
    flat = lay.reshape(H * nb, nb)
    counts = flat.sum(axis=1)
    rowptr = np.zeros(H * nb + 1, np.int32)
    np.cumsum(counts, out=rowptr[1:])
    cols = np.nonzero(flat)[1].astype(np.int32)
    return rowptr, cols
