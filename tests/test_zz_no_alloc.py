"""lwattn_forward_noalloc (the allocation-free forward over the library's
static per-GPU workspace) through the C ABI, against the plan-based
lwattn_forward on the same inputs: the same kernel and launch geometry, so the
outputs must agree bit for bit.  Two calls in a row, the second on a smaller
problem (the static buffer keeps the first call's contents), then the status
words, and the rejection of a problem that needs more than the buffer."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import make_plan, say, to_dev
from long_document_sparse_amd import lwattn as lw
from long_document_sparse_amd import workloads

pytestmark = pytest.mark.gpu


def _both(spec, strong=False):
    x = workloads.generate(spec, strong=strong)
    ts, lm, gm = to_dev(x)
    plan = make_plan(spec)
    want = plan(*ts, lm, gm)
    assert plan.sync_status() == lw.OK
    plan.close()
    out = torch.full_like(ts[0], float("nan"))
    status = torch.full((spec.B + 1,), -7, dtype=torch.int32, device=ts[0].device)
    lw.forward_noalloc(*ts, lm, gm, out, spec.window, spec.dilation, spec.max_global, spec.scale,
                       status=status)
    torch.cuda.synchronize()
    return want, out, status


def test_noalloc_matches_the_plan_forward_twice_second_smaller():
    big = workloads.custom(2, 3, 1500, 64, 256, "bf16", [0, 1, 2], seed=31, n_global=40,
                           global_mode="random", pad_mode="per_batch", pad_hi=300, max_global=64)
    small = workloads.custom(1, 2, 300, 64, 64, "bf16", [0, 0], seed=32, n_global=3,
                             global_mode="random", pad_mode="none", max_global=8)
    for spec in (big, small):
        say(f"noalloc vs plan: B={spec.B} H={spec.H} n={spec.n} w={spec.window}")
        want, got, status = _both(spec)
        assert torch.equal(want, got)
        assert torch.count_nonzero(status).item() == 0


def test_noalloc_fp32_and_status_of_too_many_globals():
    spec = workloads.custom(2, 2, 700, 64, 128, "f32", [0, 1], seed=33, n_global=12,
                            global_mode="random", pad_mode="per_batch", pad_hi=100, max_global=16)
    say("noalloc vs plan: fp32")
    want, got, status = _both(spec, strong=True)
    assert torch.equal(want, got)
    assert torch.count_nonzero(status).item() == 0
    # more global tokens in a row than max_global: the row's status word
    tight = workloads.custom(2, 1, 256, 64, 32, "bf16", [0], seed=34, n_global=10,
                             global_mode="random", max_global=4)
    x = workloads.generate(tight)
    ts, lm, gm = to_dev(x)
    gm[1].zero_()                      # batch row 1 keeps no global token
    out = torch.empty_like(ts[0])
    status = torch.full((3,), -7, dtype=torch.int32, device=ts[0].device)
    say("noalloc: too many globals")
    lw.forward_noalloc(*ts, lm, gm, out, tight.window, tight.dilation, 4, tight.scale, status=status)
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0, 1, 0]


def test_noalloc_rejects_problems_beyond_the_static_buffer():
    lib = lw.load_library()
    # B n flags and indices alone exceed 32 MiB; rejected before any launch
    cfg, keep = lw.make_config(8, 1, 1 << 20, 64, 64, None, 1, None, "bf16")
    p = ctypes.c_void_p(256)
    st = lib.lwattn_forward_noalloc(ctypes.byref(cfg), 0, p, p, p, p, p, p, p, p, p, None, None)
    assert st == lw.E_SCRATCH
    cfg, keep = lw.make_config(1, 33, 64, 64, 8, None, 1, None, "bf16")
    st = lib.lwattn_forward_noalloc(ctypes.byref(cfg), 0, p, p, p, p, p, p, p, p, p, None, None)
    assert st == lw.E_UNSUPPORTED
    assert lib.lwattn_forward_noalloc(None, 0, *([None] * 11)) == lw.E_INVALID
