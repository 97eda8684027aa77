"""Thin ctypes binding of the C ABI in include/lwattn.h.

Argument marshalling only: every step of the forward runs in the HIP kernels of
liblwattn.so.  Torch provides device memory and the current stream.  If the
library is missing, every entry point raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblwattn.so")

LWATTN_F32, LWATTN_BF16, LWATTN_F16 = 0, 1, 2
DTYPE_CODES = {"f32": LWATTN_F32, "bf16": LWATTN_BF16, "f16": LWATTN_F16}


def torch_dtype(dtype: str):
    """The torch dtype of a storage type name ("f32", "bf16", "f16")."""
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
OK, E_INVALID, E_UNSUPPORTED, E_NOMEM, E_DEVICE, E_TOO_MANY_GLOBALS, E_SCRATCH = range(7)
KERNELS = ("attention",)
# kernel slots of lwattn_timing_read_backward
BW_KERNELS = ("compact_kernel", "dq_kernel", "global_chunk_kernel", "global_merge_kernel", "dkv_kernel")

# (name, restype, argtypes) of every exported function, in header order
_c_p = ctypes.c_void_p
_i32 = ctypes.c_int32


class Config(ctypes.Structure):
    _fields_ = [
        ("B", _i32), ("H", _i32), ("n", _i32), ("d", _i32),
        ("window", _i32),
        ("dilation", ctypes.POINTER(_i32)),
        ("max_global", _i32),
        ("scale", ctypes.c_float),
        ("dtype", _i32),
    ]


SIGNATURES = [
    ("lwattn_check_config", ctypes.c_int, [ctypes.POINTER(Config)]),
    ("lwattn_plan", ctypes.c_int, [ctypes.POINTER(Config), ctypes.c_int, ctypes.POINTER(_c_p)]),
    ("lwattn_forward", ctypes.c_int, [_c_p] * 9 + [_c_p, _c_p]),
    ("lwattn_backward", ctypes.c_int, [_c_p] * 17 + [_c_p]),
    ("lwattn_forward_causal", ctypes.c_int, [_c_p] * 6 + [_c_p]),
    ("lwattn_backward_causal", ctypes.c_int, [_c_p] * 10 + [_c_p]),
    ("lwattn_forward_blocksparse", ctypes.c_int, [_c_p] * 7 + [_i32, _i32, _c_p, _c_p]),
    ("lwattn_layer_create", ctypes.c_int, [_c_p, _i32, ctypes.c_float, ctypes.POINTER(_c_p)]),
    ("lwattn_layer_forward", ctypes.c_int, [_c_p] * 7),
    ("lwattn_layer_destroy", ctypes.c_int, [_c_p]),
    ("lwattn_destroy", ctypes.c_int, [_c_p]),
    ("lwattn_global_index", ctypes.c_int, [_c_p, _c_p, _c_p, _c_p]),
    ("lwattn_sync_status", ctypes.c_int, [_c_p, _c_p]),
    ("lwattn_timing_enable", ctypes.c_int, [_c_p, _i32]),
    ("lwattn_timing_every", ctypes.c_int, [_c_p, _i32]),
    ("lwattn_timing_read", ctypes.c_int, [_c_p, ctypes.POINTER(ctypes.c_float), _i32,
                                          ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    ("lwattn_timing_read_backward", ctypes.c_int, [_c_p, ctypes.POINTER(ctypes.c_float), _i32,
                                                   ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    ("lwattn_timing_disable", ctypes.c_int, [_c_p]),
    ("lwattn_test_inject_wait_timeout", ctypes.c_int, [_c_p]),
    ("lwattn_forward_noalloc", ctypes.c_int, [ctypes.POINTER(Config), ctypes.c_int] + [_c_p] * 11),
    ("lwattn_probe_mfma", ctypes.c_int, [_i32, _c_p, _c_p]),
    ("lwattn_probe_read", ctypes.c_int, [_c_p, ctypes.c_int64, _c_p, _c_p]),
    ("lwattn_strerror", ctypes.c_char_p, [ctypes.c_int]),
]

_lib = None


class LwattnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {strerror(status)} (status {status})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is None:
        # Bind to the HIP runtime torch already carries: both export the SONAME
        # libamdhip64.so.7, so loading torch first makes the dynamic linker reuse
        # its copy instead of mapping a second runtime into the process.
        import torch  # noqa: F401
        if not os.path.exists(path):
            raise RuntimeError(
                f"HIP library {path} is not built; run `python -m long_document_sparse_amd.build` "
                "(hipcc --offload-arch=gfx950) first")
        lib = ctypes.CDLL(path)
        for name, res, args in SIGNATURES:
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def strerror(status: int) -> str:
    return load_library().lwattn_strerror(int(status)).decode()


def make_config(B: int, H: int, n: int, d: int = 64, window: int = 512,
                dilation: Optional[Sequence[int]] = None, max_global: int = 64,
                scale: Optional[float] = None, dtype: str = "bf16"):
    """Returns (Config, keepalive) -- the dilation array must outlive the call."""
    dil = None
    ptr = None
    if dilation is not None:
        dil = (_i32 * len(dilation))(*[int(x) for x in dilation])
        ptr = ctypes.cast(dil, ctypes.POINTER(_i32))
    if scale is None:
        scale = 1.0 / math.sqrt(d) if d > 0 else 1.0
    code = DTYPE_CODES.get(dtype, 99) if isinstance(dtype, str) else int(dtype)
    return Config(B, H, n, d, window, ptr, max_global, scale, code), dil


def check_config(**kw) -> int:
    cfg, keep = make_config(**kw)
    return load_library().lwattn_check_config(ctypes.byref(cfg))


def _stream_handle(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


class Plan:
    """One configuration: lwattn_plan on construction, lwattn_destroy on close()."""

    def __init__(self, B: int, H: int, n: int, d: int = 64, window: int = 512,
                 dilation: Optional[Sequence[int]] = None, max_global: int = 64,
                 scale: Optional[float] = None, dtype: str = "bf16", device: int = 0):
        self.lib = load_library()
        self.shape = (B, H, n, d)
        self.dtype = dtype
        self.device = device
        cfg, keep = make_config(B, H, n, d, window, dilation, max_global, scale, dtype)
        self.cfg = cfg
        handle = ctypes.c_void_p()
        st = self.lib.lwattn_plan(ctypes.byref(cfg), device, ctypes.byref(handle))
        if st != OK:
            raise LwattnError(st, "lwattn_plan")
        self.handle = handle
        del keep

    def close(self):
        if getattr(self, "handle", None):
            self.lib.lwattn_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, t, name, dtype):
        import torch
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a device tensor")
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    def _validate(self, q, k, v, qg, kg, vg, lmask, gmask, out):
        import torch
        tdt = torch_dtype(self.dtype)
        for t, name in ((q, "q"), (k, "k"), (v, "v"), (qg, "qg"), (kg, "kg"), (vg, "vg")):
            self._check(t, name, tdt)
            if tuple(t.shape) != self.shape:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, plan expects {self.shape}")
        B, H, n, d = self.shape
        for t, name in ((lmask, "local_attn_mask"), (gmask, "global_attn_mask")):
            self._check(t, name, torch.float32)
            if tuple(t.shape) != (B, n):
                raise ValueError(f"{name} must be [B,n]")
        if out is None:
            out = torch.empty(self.shape, dtype=tdt, device=q.device)
        else:
            self._check(out, "out", tdt)
            if tuple(out.shape) != self.shape:
                raise ValueError("out has the wrong shape")
        return out

    def forward(self, q, k, v, qg, kg, vg, lmask, gmask, out=None, stream=None):
        """Enqueue one forward; returns O (allocated if `out` is None)."""
        out = self._validate(q, k, v, qg, kg, vg, lmask, gmask, out)
        st = self.lib.lwattn_forward(self.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                     qg.data_ptr(), kg.data_ptr(), vg.data_ptr(),
                                     lmask.data_ptr(), gmask.data_ptr(), out.data_ptr(),
                                     _stream_handle(stream))
        if st != OK:
            raise LwattnError(st, "lwattn_forward")
        return out

    def forward_causal(self, q, k, v, lmask, out=None, stream=None):
        """Enqueue the causal variant (window taps at or before each row, no
        global attention; bf16 or fp16 plans); returns O (allocated if `out` is None)."""
        import torch
        tdt = torch_dtype(self.dtype)
        for t, name in ((q, "q"), (k, "k"), (v, "v")):
            self._check(t, name, tdt)
            if tuple(t.shape) != self.shape:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, plan expects {self.shape}")
        B, H, n, d = self.shape
        self._check(lmask, "local_attn_mask", torch.float32)
        if tuple(lmask.shape) != (B, n):
            raise ValueError("local_attn_mask must be [B,n]")
        if out is None:
            out = torch.empty(self.shape, dtype=tdt, device=q.device)
        else:
            self._check(out, "out", tdt)
            if tuple(out.shape) != self.shape:
                raise ValueError("out has the wrong shape")
        st = self.lib.lwattn_forward_causal(self.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                            lmask.data_ptr(), out.data_ptr(), _stream_handle(stream))
        if st != OK:
            raise LwattnError(st, "lwattn_forward_causal")
        return out

    def backward_causal(self, q, k, v, lmask, o, do, stream=None):
        """Enqueue the backward of the causal variant (bf16 plans); `o` is
        forward_causal's output on the same inputs.  Returns (dQ, dK, dV)."""
        import torch
        tdt = torch_dtype(self.dtype)
        for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
            self._check(t, name, tdt)
            if tuple(t.shape) != self.shape:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, plan expects {self.shape}")
        B, H, n, d = self.shape
        self._check(lmask, "local_attn_mask", torch.float32)
        if tuple(lmask.shape) != (B, n):
            raise ValueError("local_attn_mask must be [B,n]")
        dq, dk, dv = (torch.empty(self.shape, dtype=tdt, device=q.device) for _ in range(3))
        st = self.lib.lwattn_backward_causal(self.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                             lmask.data_ptr(), o.data_ptr(), do.data_ptr(),
                                             dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                             _stream_handle(stream))
        if st != OK:
            raise LwattnError(st, "lwattn_backward_causal")
        return dq, dk, dv

    def forward_blocksparse(self, q, k, v, lmask, rowptr, cols, causal=False, out=None, stream=None):
        """Enqueue block-sparse attention over 64-blocks (bf16 or fp16 plans): the
        layout as CSR over (head, query block), int32 device tensors rowptr
        [H*nb + 1] and cols [nnz]; returns O (allocated if `out` is None)."""
        import torch
        tdt = torch_dtype(self.dtype)
        for t, name in ((q, "q"), (k, "k"), (v, "v")):
            self._check(t, name, tdt)
            if tuple(t.shape) != self.shape:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, plan expects {self.shape}")
        B, H, n, d = self.shape
        nb = (n + 63) // 64
        self._check(lmask, "local_attn_mask", torch.float32)
        if tuple(lmask.shape) != (B, n):
            raise ValueError("local_attn_mask must be [B,n]")
        self._check(rowptr, "rowptr", torch.int32)
        self._check(cols, "cols", torch.int32)
        if tuple(rowptr.shape) != (H * nb + 1,):
            raise ValueError(f"rowptr must have H*nb + 1 = {H * nb + 1} entries")
        if out is None:
            out = torch.empty(self.shape, dtype=tdt, device=q.device)
        else:
            self._check(out, "out", tdt)
            if tuple(out.shape) != self.shape:
                raise ValueError("out has the wrong shape")
        # an empty column list still needs a valid pointer
        cptr = cols.data_ptr() if cols.numel() > 0 else rowptr.data_ptr()
        st = self.lib.lwattn_forward_blocksparse(self.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                 lmask.data_ptr(), rowptr.data_ptr(), cptr, int(cols.numel()),
                                                 int(bool(causal)), out.data_ptr(), _stream_handle(stream))
        if st != OK:
            raise LwattnError(st, "lwattn_forward_blocksparse")
        return out

    def backward(self, q, k, v, qg, kg, vg, lmask, gmask, o, do, grads=None, stream=None):
        """Enqueue the backward of the forward that produced `o`; returns
        (dQ, dK, dV, dQg, dKg, dVg), allocated if `grads` is None."""
        import torch
        self._validate(q, k, v, qg, kg, vg, lmask, gmask, o)
        tdt = torch_dtype(self.dtype)
        self._check(do, "do", tdt)
        if tuple(do.shape) != self.shape:
            raise ValueError("do has the wrong shape")
        if grads is None:
            grads = tuple(torch.empty(self.shape, dtype=tdt, device=q.device) for _ in range(6))
        for t, name in zip(grads, ("dq", "dk", "dv", "dqg", "dkg", "dvg")):
            self._check(t, name, tdt)
            if tuple(t.shape) != self.shape:
                raise ValueError(f"{name} has the wrong shape")
        st = self.lib.lwattn_backward(self.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                      qg.data_ptr(), kg.data_ptr(), vg.data_ptr(),
                                      lmask.data_ptr(), gmask.data_ptr(), o.data_ptr(),
                                      do.data_ptr(), *[t.data_ptr() for t in grads],
                                      _stream_handle(stream))
        if st != OK:
            raise LwattnError(st, "lwattn_backward")
        return grads

    def bind_backward(self, q, k, v, qg, kg, vg, lmask, gmask, o, do, grads, stream=None):
        """Like bind, for the backward: validates once, returns a no-argument
        callable that enqueues lwattn_backward into `grads` again."""
        self.backward(q, k, v, qg, kg, vg, lmask, gmask, o, do, grads=grads, stream=stream)
        fn = self.lib.lwattn_backward
        args = (self.handle,) + tuple(ctypes.c_void_p(t.data_ptr()) for t in
                                      (q, k, v, qg, kg, vg, lmask, gmask, o, do, *grads)) + \
            (_stream_handle(stream),)
        keep = (q, k, v, qg, kg, vg, lmask, gmask, o, do, grads)

        def run():
            st = fn(*args)
            if st != OK:
                raise LwattnError(st, "lwattn_backward")
            return keep[-1]
        return run

    def bind(self, q, k, v, qg, kg, vg, lmask, gmask, out=None, stream=None):
        """Validate the buffers once and return a no-argument callable that
        enqueues the same forward again (same buffers, same stream), with the
        arguments marshalled up front: the per-call host cost is one C call.
        The callable keeps the tensors alive and returns O."""
        out = self._validate(q, k, v, qg, kg, vg, lmask, gmask, out)
        fn = self.lib.lwattn_forward
        args = (self.handle,) + tuple(ctypes.c_void_p(t.data_ptr()) for t in
                                      (q, k, v, qg, kg, vg, lmask, gmask, out)) + (_stream_handle(stream),)
        keep = (q, k, v, qg, kg, vg, lmask, gmask, out)

        def run():
            st = fn(*args)
            if st != OK:
                raise LwattnError(st, "lwattn_forward")
            return keep[-1]
        return run

    __call__ = forward

    def global_index(self, stream=None):
        """(gidx [B,n] int32, gcnt [B] int32) of the last forward, as device tensors."""
        import torch
        B, H, n, d = self.shape
        dev = torch.device("cuda", self.device)
        gidx = torch.empty((B, n), dtype=torch.int32, device=dev)
        gcnt = torch.empty((B,), dtype=torch.int32, device=dev)
        st = self.lib.lwattn_global_index(self.handle, gidx.data_ptr(), gcnt.data_ptr(),
                                          _stream_handle(stream))
        if st != OK:
            raise LwattnError(st, "lwattn_global_index")
        return gidx, gcnt

    def sync_status(self, stream=None) -> int:
        return int(self.lib.lwattn_sync_status(self.handle, _stream_handle(stream)))

    def timing_enable(self, max_calls: int, every: int = 1):
        """Record per-kernel events for up to max_calls forwards, on every
        `every`-th forward."""
        st = self.lib.lwattn_timing_enable(self.handle, int(max_calls))
        if st != OK:
            raise LwattnError(st, "lwattn_timing_enable")
        st = self.lib.lwattn_timing_every(self.handle, int(every))
        if st != OK:
            raise LwattnError(st, "lwattn_timing_every")

    def timing_read(self):
        """({kernel: total ms}, calls) over the forwards recorded since timing_enable."""
        ms = (ctypes.c_float * 8)()
        nk, nc = _i32(), _i32()
        st = self.lib.lwattn_timing_read(self.handle, ms, 8, ctypes.byref(nk), ctypes.byref(nc))
        if st != OK:
            raise LwattnError(st, "lwattn_timing_read")
        return {KERNELS[i]: float(ms[i]) for i in range(nk.value)}, int(nc.value)

    def timing_read_backward(self):
        """({kernel: total ms}, calls) over the backwards recorded since timing_enable
        (kernels a call did not launch count zero)."""
        ms = (ctypes.c_float * 8)()
        nk, nc = _i32(), _i32()
        st = self.lib.lwattn_timing_read_backward(self.handle, ms, 8, ctypes.byref(nk), ctypes.byref(nc))
        if st != OK:
            raise LwattnError(st, "lwattn_timing_read_backward")
        return {BW_KERNELS[i]: float(ms[i]) for i in range(nk.value)}, int(nc.value)

    def timing_disable(self):
        self.lib.lwattn_timing_disable(self.handle)


def forward_noalloc(q, k, v, qg, kg, vg, lmask, gmask, out, window: int,
                    dilation: Optional[Sequence[int]] = None, max_global: int = 64,
                    scale: Optional[float] = None, status=None, stream=None, device: Optional[int] = None):
    """lwattn_forward_noalloc: the forward without a plan or any allocation
    (the library's static per-GPU workspace).  All tensors are caller-owned
    device tensors of the plan-based forward's shapes; `status`, if given, is a
    device int32 tensor [B + 1] (fault word, then the per-row too-many-globals
    flags).  Returns `out`."""
    import torch
    B, H, n, d = tuple(q.shape)
    tdt = q.dtype
    dtype = {torch.bfloat16: "bf16", torch.float32: "f32", torch.float16: "f16"}.get(tdt)
    if dtype is None:
        raise TypeError(f"unsupported dtype {tdt}")
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (qg, "qg"), (kg, "kg"), (vg, "vg"), (out, "out")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != tdt or not t.is_contiguous() \
                or tuple(t.shape) != (B, H, n, d):
            raise ValueError(f"{name} must be a contiguous device tensor [B,H,n,d] of {tdt}")
    for t, name in ((lmask, "local_attn_mask"), (gmask, "global_attn_mask")):
        if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (B, n):
            raise ValueError(f"{name} must be a contiguous float32 device tensor [B,n]")
    if status is not None and (status.dtype != torch.int32 or not status.is_cuda or status.numel() < B + 1):
        raise ValueError("status must be an int32 device tensor of B + 1 entries")
    cfg, keep = make_config(B, H, n, d, window, dilation, max_global, scale, dtype)
    dev = q.device.index if device is None else device
    st = load_library().lwattn_forward_noalloc(
        ctypes.byref(cfg), int(dev if dev is not None else 0), q.data_ptr(), k.data_ptr(), v.data_ptr(),
        qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), lmask.data_ptr(), gmask.data_ptr(), out.data_ptr(),
        status.data_ptr() if status is not None else None, _stream_handle(stream))
    del keep
    if st != OK:
        raise LwattnError(st, "lwattn_forward_noalloc")
    return out


LAYER_WEIGHTS = ("w_qkv", "b_qkv", "w_g", "b_g", "w_o", "b_o", "ln1_g", "ln1_b",
                 "w_1", "b_1", "w_2", "b_2", "ln2_g", "ln2_b")


class _LayerWeights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in LAYER_WEIGHTS]


class Layer:
    """Encoder layer around the attention of `plan` (lwattn_layer_*): bf16
    weights as a dict of device tensors (row-major [in, out]), X and Y [B*n, hid]."""

    def __init__(self, plan: "Plan", inter: int, eps: float = 1e-5):
        self.plan = plan
        self.lib = plan.lib
        self.inter = int(inter)
        h = ctypes.c_void_p()
        st = self.lib.lwattn_layer_create(plan.handle, self.inter, float(eps), ctypes.byref(h))
        if st != OK:
            raise LwattnError(st, "lwattn_layer_create")
        self.handle = h

    def shapes(self):
        B, H, n, d = self.plan.shape
        hid, inter = H * d, self.inter
        return {"w_qkv": (hid, 3 * hid), "b_qkv": (3 * hid,), "w_g": (hid, 3 * hid), "b_g": (3 * hid,),
                "w_o": (hid, hid), "b_o": (hid,), "ln1_g": (hid,), "ln1_b": (hid,),
                "w_1": (hid, inter), "b_1": (inter,), "w_2": (inter, hid), "b_2": (hid,),
                "ln2_g": (hid,), "ln2_b": (hid,)}

    def forward(self, x, weights, lmask, gmask, out=None, stream=None):
        import torch
        B, H, n, d = self.plan.shape
        hid = H * d
        tdt = torch_dtype(self.plan.dtype)
        self.plan._check(x, "x", tdt)
        if tuple(x.shape) != (B * n, hid):
            raise ValueError(f"x must be [{B * n}, {hid}]")
        for name, shape in self.shapes().items():
            t = weights[name]
            self.plan._check(t, name, tdt)
            if tuple(t.shape) != shape:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
        for t, name in ((lmask, "local_attn_mask"), (gmask, "global_attn_mask")):
            self.plan._check(t, name, torch.float32)
            if tuple(t.shape) != (B, n):
                raise ValueError(f"{name} must be [B,n]")
        if out is None:
            out = torch.empty_like(x)
        else:
            self.plan._check(out, "out", tdt)
            if tuple(out.shape) != tuple(x.shape):
                raise ValueError("out has the wrong shape")
        self._w = _LayerWeights(*[weights[name].data_ptr() for name in LAYER_WEIGHTS])
        st = self.lib.lwattn_layer_forward(self.handle, x.data_ptr(), ctypes.byref(self._w),
                                           lmask.data_ptr(), gmask.data_ptr(), out.data_ptr(),
                                           _stream_handle(stream))
        if st != OK:
            raise LwattnError(st, "lwattn_layer_forward")
        return out

    def close(self):
        if self.handle:
            self.lib.lwattn_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
