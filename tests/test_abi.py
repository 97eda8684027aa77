"""Host-only checks of the C ABI: the library loads, exports every function the
header declares, and validates configurations without touching a device."""
import ctypes
import os
import re

import pytest

from long_document_sparse_amd import lwattn as lw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "lwattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lwattn_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = lw.load_library()
    names = _declared()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(n for n, _, _ in lw.SIGNATURES) == names


def test_strerror_covers_every_status():
    for st in range(6):
        msg = lw.strerror(st)
        assert msg and msg != "unknown status"
    assert lw.strerror(42) == "unknown status"


BASE = dict(B=2, H=4, n=1000, d=64, window=128, dilation=[0, 1, 2, 3], max_global=8,
            scale=0.125, dtype="bf16")


@pytest.mark.parametrize("change,want", [
    ({}, lw.OK),
    ({"dtype": "f32"}, lw.OK),
    ({"dtype": "f16"}, lw.OK),
    ({"dtype": 2}, lw.OK),             # LWATTN_F16
    ({"dtype": 3}, lw.E_INVALID),
    ({"window": 0}, lw.OK),
    ({"n": 0}, lw.OK),
    ({"B": 0}, lw.OK),
    ({"max_global": 0}, lw.OK),
    ({"dilation": None}, lw.OK),
    ({"window": 7}, lw.E_INVALID),
    ({"window": -2}, lw.E_INVALID),
    ({"B": -1}, lw.E_INVALID),
    ({"n": -5}, lw.E_INVALID),
    ({"d": 0}, lw.E_INVALID),
    ({"d": 128}, lw.E_UNSUPPORTED),
    ({"d": 32}, lw.E_UNSUPPORTED),
    ({"max_global": -1}, lw.E_INVALID),
    ({"scale": 0.0}, lw.E_INVALID),
    ({"scale": -1.0}, lw.E_INVALID),
    ({"scale": float("inf")}, lw.E_INVALID),
    ({"scale": float("nan")}, lw.E_INVALID),
    ({"dtype": 7}, lw.E_INVALID),
    ({"dilation": [0, -1, 0, 0]}, lw.E_INVALID),
    ({"B": 1 << 20, "H": 1 << 10, "n": 1 << 16}, lw.E_INVALID),
    ({"B": 1, "H": 1, "n": (1 << 23) + 2}, lw.E_INVALID),
    ({"B": 4, "H": 1, "n": 1 << 23}, lw.OK),
])
def test_check_config(change, want):
    kw = dict(BASE)
    kw.update(change)
    assert lw.check_config(**kw) == want


def test_null_config_and_plan_arguments_are_rejected():
    lib = lw.load_library()
    assert lib.lwattn_check_config(None) == lw.E_INVALID
    assert lib.lwattn_destroy(None) == lw.OK
    assert lib.lwattn_forward(*([None] * 11)) == lw.E_INVALID
    assert lib.lwattn_backward(*([None] * 18)) == lw.E_INVALID
    assert lib.lwattn_forward_causal(*([None] * 7)) == lw.E_INVALID
    assert lib.lwattn_backward_causal(*([None] * 11)) == lw.E_INVALID
    assert lib.lwattn_forward_blocksparse(None, None, None, None, None, None, None, 0, 0, None, None) == lw.E_INVALID
    assert lib.lwattn_layer_create(None, 4096, 1e-5, None) == lw.E_INVALID
    assert lib.lwattn_layer_forward(*([None] * 7)) == lw.E_INVALID
    assert lib.lwattn_layer_destroy(None) == lw.OK
    assert lib.lwattn_global_index(None, None, None, None) == lw.E_INVALID
    assert lib.lwattn_sync_status(None, None) == lw.E_INVALID
    assert lib.lwattn_timing_enable(None, 4) == lw.E_INVALID
    assert lib.lwattn_timing_every(None, 2) == lw.E_INVALID
    assert lib.lwattn_test_inject_wait_timeout(None) == lw.E_INVALID
    assert lib.lwattn_timing_disable(None) == lw.E_INVALID
    nk, nc = ctypes.c_int32(), ctypes.c_int32()
    assert lib.lwattn_timing_read(None, None, 0, ctypes.byref(nk), ctypes.byref(nc)) == lw.E_INVALID
    assert lib.lwattn_timing_read_backward(None, None, 0, ctypes.byref(nk), ctypes.byref(nc)) == lw.E_INVALID
    cfg, keep = lw.make_config(**BASE)
    assert lib.lwattn_plan(ctypes.byref(cfg), 0, None) == lw.E_INVALID


def test_plan_rejects_invalid_config_before_any_device_call():
    lib = lw.load_library()
    kw = dict(BASE, window=3)
    cfg, keep = lw.make_config(**kw)
    h = ctypes.c_void_p(1234)
    assert lib.lwattn_plan(ctypes.byref(cfg), 0, ctypes.byref(h)) == lw.E_INVALID
    assert h.value is None
