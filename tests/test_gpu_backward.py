"""GPU parity of the backward (lwattn_backward through the C ABI) against the
oracle's backward, element by element over all six gradients.

Tolerance, derived from the arithmetic: both sides see the same stored inputs;
the HIP path accumulates in fp32 (scores, exp, every sum over up to n rows or
keys) and rounds the gradients to the storage type, the oracle works in fp64.
With bf16 storage the matrix cores also take P and dS rounded to bf16 (2^-9
relative per term, of either sign, so a sum of k terms drifts by about
2^-9 sqrt(k) of its scale) and the gradients are rounded to bf16 (2^-9).  Per
tensor, relative to its largest entry: fp32 storage |err| <= 1e-4 * max |g|;
bf16 storage |err| <= 2e-2 * max |g|.  A tensor that no path reaches must be
exactly zero.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import make_plan, say, to_dev, to_np64
from long_document_sparse_amd import lwattn as lw
from long_document_sparse_amd import workloads

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ("dQ", "dK", "dV", "dQg", "dKg", "dVg")

CASES = [
    # (B, H, n, window, dtype, dilation, n_global, global_mode, pad_mode, pad_hi)
    (1, 2, 200, 64, "f32", [0, 1], 1, "first", "none", 0),
    (2, 2, 333, 40, "bf16", [0, 2], 5, "random", "per_batch", 80),
    (1, 3, 300, 128, "f32", [0, 1, 3], 70, "random", "per_batch", 60),   # two global tiles
    (2, 2, 130, 400, "bf16", [0, 0], 3, "first", "none", 0),             # window > n
    (1, 2, 257, 16, "f32", [1, 4], 0, "first", "scatter", 40),           # no globals, scattered pads
    (1, 1, 65, 8, "bf16", [0], 65, "first", "none", 0),                  # every token global
    (1, 3, 300, 128, "bf16", [0, 1, 3], 70, "random", "per_batch", 60),  # matrix cores: two global tiles
    (1, 2, 257, 16, "bf16", [1, 4], 0, "first", "scatter", 40),          # no globals, scattered pads
    (2, 2, 1000, 256, "bf16", [0, 1], 3, "random", "per_batch", 200),    # interior and edge tiles, pads
]


def _grad_out(x, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(x.tensors()[0].shape).astype(np.float32)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}n{c[2]}w{c[3]}{c[4]}g{c[6]}{c[8]}")
def test_backward_matches_oracle(case):
    B, H, n, window, dtype, dil, ng, gmode, pmode, phi = case
    spec = workloads.custom(B, H, n, 64, window, dtype, dil, seed=21, n_global=ng,
                            global_mode=gmode, pad_mode=pmode, pad_hi=phi)
    x = workloads.generate(spec)
    ts, lm, gm = to_dev(x)
    plan = make_plan(spec, max_global=max(ng, 1))
    o = torch.empty_like(ts[0])
    plan(*ts, lm, gm, out=o)
    go_np = _grad_out(x, 3)
    tdt = ts[0].dtype
    go = torch.from_numpy(go_np).to(ts[0].device).to(tdt)
    grads = tuple(torch.full_like(ts[0], float("nan")) for _ in range(6))
    plan.backward(*ts, lm, gm, o, go, grads=grads)
    assert plan.sync_status() == lw.OK
    # the oracle sees exactly the stored values (bf16 inputs widened)
    ins = [to_np64(t) for t in ts]
    go_seen = to_np64(go)
    want = oracle.backward(*ins, x.lmask, x.gmask, go_seen, spec.window, spec.dilation, spec.scale)
    for name, g, w in zip(NAMES, grads, want):
        got = to_np64(g)
        assert np.all(np.isfinite(got)), f"{name}: non-finite values"
        err = float(np.max(np.abs(got - w)))
        ref = float(np.max(np.abs(w)))
        say(f"{name}: max abs err {err:.3e}, max |g| {ref:.3e}")
        if ref == 0.0:
            assert err == 0.0, name
        else:
            assert err <= TOL[dtype] * ref, name


def test_backward_base_size_bf16():
    """The benchmark's configuration (B=1, H=12, n=4096, w=512, one global token
    at the start, bf16), every element of every gradient."""
    spec = workloads.named("base")
    x = workloads.generate(spec)
    ts, lm, gm = to_dev(x)
    plan = make_plan(spec)
    o = torch.empty_like(ts[0])
    plan(*ts, lm, gm, out=o)
    go = torch.from_numpy(_grad_out(x, 4)).to(ts[0].device).to(ts[0].dtype)
    grads = plan.backward(*ts, lm, gm, o, go)
    assert plan.sync_status() == lw.OK
    want = oracle.backward(*[to_np64(t) for t in ts], x.lmask, x.gmask, to_np64(go),
                           spec.window, spec.dilation, spec.scale)
    for name, g, w in zip(NAMES, grads, want):
        got = to_np64(g)
        err = float(np.max(np.abs(got - w)))
        ref = float(np.max(np.abs(w)))
        say(f"base {name}: max abs err {err:.3e}, max |g| {ref:.3e}")
        assert np.all(np.isfinite(got))
        assert err <= TOL["bf16"] * ref, name


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_kernel_timing(dtype):
    """lwattn_timing_read_backward: every launched kernel slot has time, the
    slots a storage type does not launch have none."""
    spec = workloads.custom(1, 2, 512, 64, 128, dtype, [0, 1], seed=5, n_global=3)
    x = workloads.generate(spec)
    ts, lm, gm = to_dev(x)
    plan = make_plan(spec, max_global=4)
    o = torch.empty_like(ts[0])
    plan(*ts, lm, gm, out=o)
    go = torch.from_numpy(_grad_out(x, 4)).to(ts[0].device).to(ts[0].dtype)
    grads = tuple(torch.empty_like(ts[0]) for _ in range(6))
    plan.timing_enable(4)
    for _ in range(3):
        plan.backward(*ts, lm, gm, o, go, grads=grads)
    tot, calls = plan.timing_read_backward()
    plan.timing_disable()
    assert calls == 3
    launched = (("dq_kernel", "global_chunk_kernel", "dkv_kernel") if dtype == "bf16"
                else ("compact_kernel", "dq_kernel", "dkv_kernel"))
    for k in lw.BW_KERNELS:
        if k in launched:
            assert tot[k] > 0.0, (k, tot)
        else:
            assert tot[k] == 0.0, (k, tot)


# Grids that take each mix of the backward's two folds on a 256-CU MI355X
# (the compaction inside the dQ launch when its grid of 64-row blocks fits
# three per compute unit; the merge of the chunk sums inside the dK/dV launch
# when that grid's last round, two per compute unit, has room for it):
# 13 x 64 = 832 blocks: compaction launched, merge folded (192 spare slots,
# 65 merge workgroups); 8 x 64 = 512 blocks: compaction folded, merge
# launched (no spare slot).  The kernel slots that recorded time say which.
FOLD_CASES = [
    # (B, H, n, window, n_global, compaction launched, merge launched)
    (13, 1, 4096, 32, 20, True, False),
    (8, 1, 4096, 32, 10, False, True),
]


@pytest.mark.parametrize("case", FOLD_CASES, ids=lambda c: f"B{c[0]}g{c[4]}")
def test_backward_fold_modes(case):
    B, H, n, window, ng, comp_launched, merge_launched = case
    spec = workloads.custom(B, H, n, 64, window, "bf16", [0] * H, seed=33, n_global=ng,
                            global_mode="random", pad_mode="per_batch", pad_hi=300)
    x = workloads.generate(spec)
    ts, lm, gm = to_dev(x)
    plan = make_plan(spec, max_global=ng)
    o = torch.empty_like(ts[0])
    plan(*ts, lm, gm, out=o)
    go = torch.from_numpy(_grad_out(x, 7)).to(ts[0].device).to(ts[0].dtype)
    grads = tuple(torch.full_like(ts[0], float("nan")) for _ in range(6))
    plan.timing_enable(2)
    plan.backward(*ts, lm, gm, o, go, grads=grads)
    tot, calls = plan.timing_read_backward()
    plan.timing_disable()
    assert plan.sync_status() == lw.OK
    assert calls == 1
    assert (tot["compact_kernel"] > 0.0) == comp_launched, tot
    assert (tot["global_merge_kernel"] > 0.0) == merge_launched, tot
    ins = [to_np64(t) for t in ts]
    want = oracle.backward(*ins, x.lmask, x.gmask, to_np64(go), spec.window, spec.dilation, spec.scale)
    for name, g, w in zip(NAMES, grads, want):
        got = to_np64(g)
        assert np.all(np.isfinite(got)), f"{name}: non-finite values"
        err = float(np.max(np.abs(got - w)))
        ref = float(np.max(np.abs(w)))
        say(f"fold modes {case}: {name}: max abs err {err:.3e}, max |g| {ref:.3e}")
        assert err <= TOL["bf16"] * ref, name


def test_backward_folded_wait_timeout_is_reported_not_hung():
    """The dQ launch's wait for the compaction inside it is bounded: under the
    library's fault-test hook (rows published under a number nobody waits for,
    a poll limit of 64) every workgroup still exits and the fault is reported,
    stickily; the same inputs on a fresh plan give the oracle's gradients."""
    spec = workloads.custom(2, 2, 333, 64, 40, "bf16", [0, 2], seed=21, n_global=5,
                            global_mode="random", pad_mode="per_batch", pad_hi=80)
    x = workloads.generate(spec)
    ts, lm, gm = to_dev(x)
    go = torch.from_numpy(_grad_out(x, 3)).to(ts[0].device).to(ts[0].dtype)
    plan = make_plan(spec, max_global=5)
    o = torch.empty_like(ts[0])
    plan(*ts, lm, gm, out=o)
    assert plan.sync_status() == lw.OK
    grads = tuple(torch.empty_like(ts[0]) for _ in range(6))
    lib = lw.load_library()
    assert lib.lwattn_test_inject_wait_timeout(plan.handle) == lw.OK
    plan.backward(*ts, lm, gm, o, go, grads=grads)
    assert plan.sync_status() == lw.E_DEVICE
    plan.close()
    fresh = make_plan(spec, max_global=5)
    o2 = torch.empty_like(ts[0])
    fresh(*ts, lm, gm, out=o2)
    grads = tuple(torch.full_like(ts[0], float("nan")) for _ in range(6))
    fresh.backward(*ts, lm, gm, o2, go, grads=grads)
    assert fresh.sync_status() == lw.OK
    ins = [to_np64(t) for t in ts]
    want = oracle.backward(*ins, x.lmask, x.gmask, to_np64(go), spec.window, spec.dilation, spec.scale)
    for name, g, w in zip(NAMES, grads, want):
        got = to_np64(g)
        assert np.all(np.isfinite(got)), name
        ref = float(np.max(np.abs(w)))
        assert float(np.max(np.abs(got - w))) <= TOL["bf16"] * max(ref, 1e-30), name
    fresh.close()
