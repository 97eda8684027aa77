"""CPU oracle for the Longformer window + global attention forward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product path never does.  The
arithmetic lives in ``lwattn_oracle.c`` (plain C, double precision, one query
row at a time over an explicit allowed-key list); this module builds it with
gcc and marshals numpy arrays through ctypes.  It shares nothing with the HIP
path.

Definition followed (see the C file's header for the full list of readings):
"LongFormer: The Long-Document Transformer" notes, sections "Sliding Window",
"Dilated Sliding Window" and "Global Attention"; the FasterTransformer
Longformer encoder guide, "compute flow" (masked softmax, padded rows zeroed,
global-index partition).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lwattn_oracle.c")
_LIB = os.path.join(_HERE, "liblwattn_oracle.so")

PADDED, GLOBAL, LOCAL = 0, 1, 2


def build() -> str:
    """Compile the oracle with gcc (always rebuilds). Returns the .so path."""
    tmp = _LIB + ".tmp"
    # x86-64-v3 (AVX2, FMA): the library built here also runs on the GPU machine's
    # host, whose CPU model may differ from this one, so no -march=native
    cmd = ["gcc", "-O3", "-march=x86-64-v3", "-std=c11", "-fopenmp", "-shared", "-fPIC",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32),
        ("n", ctypes.c_int32), ("d", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("gap", ctypes.POINTER(ctypes.c_int32)),
        ("scale", ctypes.c_double),
        ("Q", ctypes.c_void_p), ("K", ctypes.c_void_p), ("V", ctypes.c_void_p),
        ("Qg", ctypes.c_void_p), ("Kg", ctypes.c_void_p), ("Vg", ctypes.c_void_p),
        ("lmask", ctypes.c_void_p), ("gmask", ctypes.c_void_p),
        ("causal", ctypes.c_int32),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.lwo_compact.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        lib.lwo_compact.restype = ctypes.c_int
        lib.lwo_allowed.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)]
        lib.lwo_allowed.restype = ctypes.c_int64
        lib.lwo_rows.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p, ctypes.c_int64,
                                 ctypes.c_void_p, ctypes.c_int32]
        lib.lwo_rows.restype = ctypes.c_int
        lib.lwo_forward.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p, ctypes.c_int32]
        lib.lwo_allowed_causal.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_void_p]
        lib.lwo_allowed_causal.restype = ctypes.c_int64
        lib.lwo_forward.restype = ctypes.c_int
        lib.lwo_rows_blocksparse.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_double] + \
            [ctypes.c_void_p] * 5 + [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_void_p, ctypes.c_int32]
        lib.lwo_rows_blocksparse.restype = ctypes.c_int
        lib.lwo_backward.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p] + \
            [ctypes.c_void_p] * 6 + [ctypes.c_int32]
        lib.lwo_backward.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def compact(lmask, gmask):
    """Global-index compaction: (gidx int32 [B,n], gcnt int32 [B])."""
    lm, gm = _f32(lmask), _f32(gmask)
    B, n = lm.shape
    gidx = np.empty((B, n), np.int32)
    gcnt = np.empty((B,), np.int32)
    _load().lwo_compact(lm.ctypes.data, gm.ctypes.data, B, n, gidx.ctypes.data, gcnt.ctypes.data)
    return gidx, gcnt


def allowed(lmask_row, gmask_row, window, gap, i):
    """(kind, keys) of query row i of one batch row."""
    lm, gm = _f32(lmask_row), _f32(gmask_row)
    n = lm.shape[0]
    keys = np.empty((max(n, 1),), np.int32)
    kind = ctypes.c_int32(-1)
    cnt = _load().lwo_allowed(lm.ctypes.data, gm.ctypes.data, n, int(window), int(gap), int(i),
                              keys.ctypes.data, ctypes.byref(kind))
    return kind.value, keys[:cnt].copy()


class _Bound:
    """Keeps the float32 copies alive while the C call runs."""

    def __init__(self, Q, K, V, Qg, Kg, Vg, lmask, gmask, window, dilation, scale, causal=False):
        self.arrs = [_f32(x) for x in (Q, K, V, Qg, Kg, Vg, lmask, gmask)]
        B, H, n, d = self.arrs[0].shape
        for a in self.arrs[1:6]:
            if a.shape != (B, H, n, d):
                raise ValueError("Q, K, V, Qg, Kg, Vg must share the shape [B,H,n,d]")
        for a in self.arrs[6:]:
            if a.shape != (B, n):
                raise ValueError("masks must be [B,n]")
        if dilation is None:
            dilation = [0] * H
        self.gap = np.ascontiguousarray(dilation, dtype=np.int32)
        if self.gap.shape != (H,):
            raise ValueError("dilation must have H entries")
        self.shape = (B, H, n, d)
        self.p = _Problem(B, H, n, d, int(window),
                          self.gap.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                          float(scale), *[a.ctypes.data for a in self.arrs], int(bool(causal)))


def forward(Q, K, V, Qg, Kg, Vg, lmask, gmask, window, dilation=None, scale=None,
            threads=None):
    """Every output row, float64 [B,H,n,d].  Inputs are upcast exactly to double."""
    d = np.shape(Q)[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    bound = _Bound(Q, K, V, Qg, Kg, Vg, lmask, gmask, window, dilation, scale)
    out = np.empty(bound.shape, np.float64)
    rc = _load().lwo_forward(ctypes.byref(bound.p), out.ctypes.data,
                             threads or default_threads())
    if rc:
        raise RuntimeError(f"oracle forward failed ({rc})")
    return out


def rows(Q, K, V, Qg, Kg, Vg, lmask, gmask, window, row_index, dilation=None, scale=None,
         threads=None):
    """Selected rows: row_index holds flat (b*H + h)*n + i; returns float64 [len, d]."""
    d = np.shape(Q)[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    bound = _Bound(Q, K, V, Qg, Kg, Vg, lmask, gmask, window, dilation, scale)
    idx = np.ascontiguousarray(row_index, dtype=np.int64)
    out = np.empty((idx.shape[0], d), np.float64)
    rc = _load().lwo_rows(ctypes.byref(bound.p), idx.ctypes.data, idx.shape[0],
                          out.ctypes.data, threads or default_threads())
    if rc:
        raise RuntimeError(f"oracle rows failed ({rc})")
    return out


def backward(Q, K, V, Qg, Kg, Vg, lmask, gmask, dO, window, dilation=None, scale=None,
             threads=None):
    """Gradients (dQ, dK, dV, dQg, dKg, dVg), float64 [B,H,n,d] each, of a loss whose
    gradient with respect to the forward's output is dO (inputs upcast exactly to
    double; the chain rule through the definition, see the C file)."""
    d = np.shape(Q)[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    bound = _Bound(Q, K, V, Qg, Kg, Vg, lmask, gmask, window, dilation, scale)
    go = _f32(dO)
    if go.shape != bound.shape:
        raise ValueError("dO must have the shape of the output [B,H,n,d]")
    outs = [np.empty(bound.shape, np.float64) for _ in range(6)]
    rc = _load().lwo_backward(ctypes.byref(bound.p), go.ctypes.data,
                              *[o.ctypes.data for o in outs], threads or default_threads())
    if rc:
        raise RuntimeError(f"oracle backward failed ({rc})")
    return tuple(outs)


def allowed_causal(lmask_row, window, gap, i):
    """(kind, keys) of query row i of one batch row in the causal variant."""
    lm = _f32(lmask_row)
    n = lm.shape[0]
    keys = np.empty((max(n, 1),), np.int32)
    kind = ctypes.c_int32(-1)
    cnt = _load().lwo_allowed_causal(lm.ctypes.data, n, int(window), int(gap), int(i),
                                     keys.ctypes.data, ctypes.byref(kind))
    return kind.value, keys[:cnt].copy()


def forward_causal(Q, K, V, lmask, window, dilation=None, scale=None, threads=None):
    """Causal variant (the window's taps at or before each row, no global
    attention): every output row, float64 [B,H,n,d]."""
    d = np.shape(Q)[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    gm = np.zeros_like(_f32(lmask))
    bound = _Bound(Q, K, V, Q, K, V, lmask, gm, window, dilation, scale, causal=True)
    out = np.empty(bound.shape, np.float64)
    rc = _load().lwo_forward(ctypes.byref(bound.p), out.ctypes.data, threads or default_threads())
    if rc:
        raise RuntimeError(f"oracle causal forward failed ({rc})")
    return out


def backward_causal(Q, K, V, lmask, dO, window, dilation=None, scale=None, threads=None):
    """Gradients (dQ, dK, dV), float64 [B,H,n,d] each, of the causal variant
    (the same chain rule over the causal key sets; every row is local)."""
    d = np.shape(Q)[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    gm = np.zeros_like(_f32(lmask))
    bound = _Bound(Q, K, V, Q, K, V, lmask, gm, window, dilation, scale, causal=True)
    go = _f32(dO)
    if go.shape != bound.shape:
        raise ValueError("dO must have the shape of the output [B,H,n,d]")
    outs = [np.empty(bound.shape, np.float64) for _ in range(6)]
    rc = _load().lwo_backward(ctypes.byref(bound.p), go.ctypes.data,
                              *[o.ctypes.data for o in outs], threads or default_threads())
    if rc:
        raise RuntimeError(f"oracle causal backward failed ({rc})")
    return outs[0], outs[1], outs[2]


def rows_causal(Q, K, V, lmask, window, row_index, dilation=None, scale=None, threads=None):
    """Selected rows of the causal variant: row_index holds flat (b*H + h)*n + i."""
    d = np.shape(Q)[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    gm = np.zeros_like(_f32(lmask))
    bound = _Bound(Q, K, V, Q, K, V, lmask, gm, window, dilation, scale, causal=True)
    idx = np.ascontiguousarray(row_index, dtype=np.int64)
    out = np.empty((idx.shape[0], d), np.float64)
    rc = _load().lwo_rows(ctypes.byref(bound.p), idx.ctypes.data, idx.shape[0],
                          out.ctypes.data, threads or default_threads())
    if rc:
        raise RuntimeError(f"oracle causal rows failed ({rc})")
    return out


def rows_blocksparse(Q, K, V, lmask, layout, row_index, causal=False, scale=None, threads=None):
    """Selected rows of block-sparse attention (layout: uint8/bool [H, nb, nb]
    over 64-blocks, nb = ceil(n/64); row_index holds flat (b*H + h)*n + i),
    float64 [len, d]."""
    Qf, Kf, Vf = (_f32(x) for x in (Q, K, V))
    B, H, n, d = Qf.shape
    if Kf.shape != Qf.shape or Vf.shape != Qf.shape:
        raise ValueError("Q, K, V must share the shape [B,H,n,d]")
    lm = _f32(lmask)
    nb = (n + 63) // 64
    lay = np.ascontiguousarray(np.asarray(layout) != 0, dtype=np.uint8)
    if lay.shape != (H, nb, nb):
        raise ValueError(f"layout must be [H, {nb}, {nb}]")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    idx = np.ascontiguousarray(row_index, dtype=np.int64)
    out = np.empty((idx.shape[0], d), np.float64)
    rc = _load().lwo_rows_blocksparse(B, H, n, d, float(scale), Qf.ctypes.data, Kf.ctypes.data,
                                      Vf.ctypes.data, lm.ctypes.data, lay.ctypes.data, int(bool(causal)),
                                      idx.ctypes.data, idx.shape[0], out.ctypes.data,
                                      threads or default_threads())
    if rc:
        raise RuntimeError(f"oracle block-sparse rows failed ({rc})")
    return out


def forward_blocksparse(Q, K, V, lmask, layout, causal=False, scale=None, threads=None):
    """Every output row of block-sparse attention, float64 [B,H,n,d]."""
    B, H, n, d = np.shape(Q)
    out = rows_blocksparse(Q, K, V, lmask, layout, np.arange(B * H * n), causal, scale, threads)
    return out.reshape(B, H, n, d)


from .layer import layer_forward, gelu, layernorm  # noqa: E402  (encoder layer oracle)
