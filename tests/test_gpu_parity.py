"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Small shapes are compared element by element over every row; they span several
tiles and a ragged tail.  The five named workloads are compared at full size on
sampled rows (random rows plus every boundary kind), in the same launch
configuration the benchmark times, together with properties that hold at any
size (exact zeros on padded rows, every row written, no NaN).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (TOL_REL, check_rows, make_plan, oracle_rows, rel_err, run, sample_rows,
                      say, to_dev, to_np64)
from long_document_sparse_amd import lwattn as lw
from long_document_sparse_amd import workloads

pytestmark = pytest.mark.gpu


def _padded_rows_zero(out_np, x):
    for b in range(x.spec.B):
        pad = x.lmask[b] == 0
        if pad.any():
            assert np.all(out_np[b][:, pad] == 0.0)


SMALL = [
    # (B, H, n, window, dtype, dilation, n_global, global_mode, pad_mode, pad_hi)
    (1, 2, 300, 64, "f32", [0, 0], 1, "first", "none", 0),
    (2, 3, 517, 128, "bf16", [0, 1, 2], 5, "random", "per_batch", 100),
    (2, 4, 1000, 200, "f32", [0, 1, 2, 3], 40, "random", "per_batch", 300),
    (1, 2, 777, 96, "bf16", [0, 4], 33, "random", "none", 0),
    (3, 2, 260, 512, "bf16", [0, 1], 3, "first", "per_batch", 200),     # window > n
    (1, 2, 129, 0, "f32", [0, 2], 2, "random", "none", 0),             # window 0
    (2, 2, 64, 6, "bf16", [0, 0], 0, "first", "per_batch", 10),        # no globals
    (1, 1, 1, 2, "f32", [0], 1, "first", "none", 0),                   # n = 1
    (1, 1, 31, 10, "bf16", [3], 31, "first", "none", 0),               # every token global
    (2, 2, 700, 60, "bf16", [0, 1], 70, "random", "per_batch", 650),   # > 2 global tiles, long pads
    (2, 3, 600, 64, "bf16", [0, 1, 3], 6, "random", "scatter", 150),   # padding anywhere
    (2, 2, 333, 40, "f32", [0, 2], 5, "random", "scatter", 80),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"B{c[0]}H{c[1]}n{c[2]}w{c[3]}{c[4]}")
@pytest.mark.parametrize("strong", [False, True])
def test_small_full_parity(case, strong):
    B, H, n, w, dt, dil, ng, gmode, pmode, phi = case
    spec = workloads.custom(B, H, n, 64, w, dt, dil, seed=n + w, n_global=ng, global_mode=gmode,
                            pad_mode=pmode, pad_lo=0, pad_hi=phi, max_global=max(ng, 1))
    x = workloads.generate(spec, strong=strong)
    say(f"small case {case} strong={strong}")
    ts, lm, gm = to_dev(x)
    plan = make_plan(spec)
    out, st = run(plan, ts, lm, gm)
    assert st == lw.OK
    got = to_np64(out)
    assert not np.isnan(got).any(), "a row was not written"
    want = oracle.forward(*x.tensors(), x.lmask, x.gmask, w, dil, spec.scale)
    _padded_rows_zero(got, x)
    rel = rel_err(got, want)
    say(f"small case: rel err {rel:.3e} (bound {TOL_REL[dt]:.0e})")
    assert rel <= TOL_REL[dt], rel
    # compaction bit-exact
    gidx, gcnt = plan.global_index()
    og, oc = oracle.compact(x.lmask, x.gmask)
    assert np.array_equal(gidx.cpu().numpy(), og)
    assert np.array_equal(gcnt.cpu().numpy(), oc)


@pytest.mark.parametrize("name", workloads.NAMES)
def test_named_workload_parity(name):
    spec = workloads.named(name)
    say(f"named workload {name}: generating")
    x = workloads.generate(spec)
    ts, lm, gm = to_dev(x)
    plan = make_plan(spec)
    say(f"named workload {name}: forward")
    out, st = run(plan, ts, lm, gm)
    assert st == lw.OK
    assert not torch.isnan(out).any().item(), "a row was not written"
    # compaction, bit-exact over all B*n entries and the counts
    gidx, gcnt = plan.global_index()
    og, oc = oracle.compact(x.lmask, x.gmask)
    assert np.array_equal(gidx.cpu().numpy(), og)
    assert np.array_equal(gcnt.cpu().numpy(), oc)
    # padded rows exactly zero
    for b in range(spec.B):
        if x.pad_len[b]:
            tail = out[b, :, spec.n - int(x.pad_len[b]):]
            assert torch.count_nonzero(tail.float()).item() == 0
    if name == "tiny":
        want = oracle.forward(*x.tensors(), x.lmask, x.gmask, spec.window, spec.dilation, spec.scale)
        err = rel_err(to_np64(out), want)
    else:
        rows = sample_rows(x, 1500, seed=1)
        say(f"named workload {name}: oracle on {rows.size} rows")
        want = oracle_rows(x, rows)
        got = to_np64(out.reshape(-1, spec.d)[torch.from_numpy(rows).to(out.device)])
        err, _ = check_rows(x, got, want)
    say(f"named workload {name}: rel err {err:.3e}")
    assert err <= TOL_REL[spec.dtype], err


@pytest.mark.parametrize("name", workloads.NAMES)
def test_named_workload_strong_parity(name):
    """Same structure with unscaled N(0,1) inputs: O(1) outputs, relative bound."""
    spec = workloads.named(name)
    x = workloads.generate(spec, strong=True)
    ts, lm, gm = to_dev(x)
    plan = make_plan(spec)
    out, st = run(plan, ts, lm, gm)
    assert st == lw.OK
    rows = sample_rows(x, 1000, seed=2)
    want = oracle_rows(x, rows)
    got = to_np64(out.reshape(-1, spec.d)[torch.from_numpy(rows).to(out.device)])
    rel, tol = check_rows(x, got, want)
    say(f"strong {name}: rel err {rel:.3e}")
    assert rel <= tol, rel


def test_deterministic_and_poison_invariant():
    spec = workloads.custom(2, 4, 900, 64, 128, "bf16", [0, 1, 2, 0], seed=5, n_global=9,
                            pad_mode="per_batch", pad_hi=200)
    x = workloads.generate(spec)
    ts, lm, gm = to_dev(x)
    plan = make_plan(spec)
    a, _ = run(plan, ts, lm, gm)
    b, _ = run(plan, ts, lm, gm)
    assert torch.equal(a, b)
    # poison every row the method never reads (padded keys, Qg at non-globals,
    # Q at globals and padding) with NaN: the output must not change
    q, k, v, qg, kg, vg = (t.clone() for t in ts)
    for bb in range(spec.B):
        valid = torch.from_numpy(x.lmask[bb] != 0).to(q.device)
        glob = valid & torch.from_numpy(x.gmask[bb] != 0).to(q.device)
        for t in (k, v, kg, vg):
            t[bb][:, ~valid] = float("nan")
        qg[bb][:, ~glob] = float("nan")
        q[bb][:, glob | ~valid] = float("nan")
    c, _ = run(plan, [q, k, v, qg, kg, vg], lm, gm)
    assert torch.equal(a, c)


def test_bound_call_repeats_the_forward():
    """Plan.bind marshals the call once; every call of it must give exactly what
    Plan.forward gives on the same buffers."""
    spec = workloads.custom(1, 3, 700, 64, 96, "bf16", [0, 1, 0], seed=8, n_global=4,
                            pad_mode="per_batch", pad_hi=90)
    x = workloads.generate(spec)
    ts, lm, gm = to_dev(x)
    plan = make_plan(spec)
    ref, st = run(plan, ts, lm, gm)
    assert st == lw.OK
    out = torch.full_like(ref, float("nan"))
    step = plan.bind(*ts, lm, gm, out=out)
    for _ in range(3):
        out.fill_(float("nan"))
        got = step()
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got, ref)
    assert plan.sync_status() == lw.OK


def test_too_many_globals_is_reported():
    spec = workloads.custom(2, 2, 300, 64, 32, "f32", [0, 1], seed=6, n_global=20)
    x = workloads.generate(spec)
    ts, lm, gm = to_dev(x)
    plan = make_plan(spec, max_global=8)
    out, st = run(plan, ts, lm, gm)
    assert st == lw.E_TOO_MANY_GLOBALS
    plan_ok = make_plan(spec, max_global=20)
    out, st = run(plan_ok, ts, lm, gm)
    assert st == lw.OK


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_wait_timeout_is_reported_not_hung(dtype):
    """The in-kernel wait for a row's compaction is bounded: when the rows are
    published under a number nobody waits for and the poll limit is tiny (the
    library's fault-test hook), every workgroup still exits and the fault is
    reported, stickily; the same inputs on a fresh plan are correct."""
    spec = workloads.custom(2, 3, 700, 64, 128, dtype, [0, 1, 0], seed=9, n_global=5,
                            pad_mode="per_batch", pad_lo=0, pad_hi=100)
    x = workloads.generate(spec)
    ts, lm, gm = to_dev(x)
    plan = make_plan(spec)
    lib = lw.load_library()
    assert lib.lwattn_test_inject_wait_timeout(plan.handle) == lw.OK
    out, st = run(plan, ts, lm, gm)
    assert st == lw.E_DEVICE
    out, st = run(plan, ts, lm, gm)          # the fault word is sticky
    assert st == lw.E_DEVICE
    plan.close()
    fresh = make_plan(spec)
    out, st = run(fresh, ts, lm, gm)
    assert st == lw.OK
    want = oracle.forward(*x.tensors(), x.lmask, x.gmask, spec.window, spec.dilation, spec.scale)
    got = out.float().cpu().numpy().astype(np.float64)
    tol = 2e-2 if dtype == "bf16" else 1e-4
    assert float(np.max(np.abs(got - want))) <= tol


def test_one_round_band_grid_with_compaction_in_band_workgroups():
    """B=1, H=16, n=4096, window 512 (the FasterTransformer QA encoder's
    attention, 64 global tokens at the start): 512 band workgroups, one round
    of slots on a 256-CU device, so the first band workgroup also computes the
    row's compaction (no compaction workgroup ahead of the band ones).  The
    compaction is checked bit-exact, sampled rows against the oracle (strong
    inputs), and the bounded wait under the fault-test hook."""
    spec = workloads.custom(1, 16, 4096, 64, 512, "bf16", [0] * 16, seed=41, n_global=64,
                            global_mode="first", max_global=64)
    x = workloads.generate(spec, strong=True)
    ts, lm, gm = to_dev(x)
    plan = make_plan(spec)
    out, st = run(plan, ts, lm, gm)
    assert st == lw.OK
    assert not torch.isnan(out).any().item(), "a row was not written"
    gidx, gcnt = plan.global_index()
    og, oc = oracle.compact(x.lmask, x.gmask)
    assert np.array_equal(gidx.cpu().numpy(), og)
    assert np.array_equal(gcnt.cpu().numpy(), oc)
    rows = sample_rows(x, 1000, seed=4)
    want = oracle_rows(x, rows)
    got = to_np64(out.reshape(-1, spec.d)[torch.from_numpy(rows).to(out.device)])
    rel, tol = check_rows(x, got, want)
    say(f"one-round band grid: rel err {rel:.3e}")
    assert rel <= tol, rel
    lib = lw.load_library()
    assert lib.lwattn_test_inject_wait_timeout(plan.handle) == lw.OK
    _, st = run(plan, ts, lm, gm)
    assert st == lw.E_DEVICE
    plan.close()


def test_empty_problem_and_bad_pointers():
    plan = lw.Plan(0, 2, 128, 64, 16, [0, 0], 4, 0.125, "bf16")
    e = torch.empty((0, 2, 128, 64), dtype=torch.bfloat16, device="cuda:0")
    m = torch.empty((0, 128), dtype=torch.float32, device="cuda:0")
    plan(e, e, e, e, e, e, m, m, out=e)
    assert plan.sync_status() == lw.OK
    plan2 = lw.Plan(1, 1, 64, 64, 16, None, 4, 0.125, "f32")
    t = torch.zeros((1, 1, 64, 64), device="cuda:0")
    mk = torch.ones((1, 64), device="cuda:0")
    lib = lw.load_library()
    s = torch.cuda.current_stream().cuda_stream
    ptrs = [t.data_ptr()] * 6
    assert lib.lwattn_forward(plan2.handle, *ptrs, mk.data_ptr(), mk.data_ptr(), None, s) == lw.E_INVALID
    assert lib.lwattn_forward(plan2.handle, t.data_ptr() + 4, *ptrs[1:], mk.data_ptr(), mk.data_ptr(),
                              t.data_ptr(), s) == lw.E_INVALID


def test_mixed_prefix_and_scattered_padding_in_one_call():
    """Rows whose real tokens are a prefix and rows padded anywhere, in one launch."""
    spec = workloads.custom(4, 2, 500, 64, 96, "bf16", [0, 2], seed=8, n_global=7,
                            pad_mode="per_batch", pad_hi=120)
    x = workloads.generate(spec)
    rng = np.random.default_rng(3)
    x.lmask[1, rng.choice(500, size=60, replace=False)] = 0.0      # scattered in row 1
    x.lmask[3, :40] = 0.0                                          # padded head in row 3
    x.gmask[1] = 0.0
    x.gmask[1, np.flatnonzero(x.lmask[1])[[0, 5, 77]]] = 1.0
    ts, lm, gm = to_dev(x)
    plan = make_plan(spec)
    out, st = run(plan, ts, lm, gm)
    assert st == lw.OK
    got = to_np64(out)
    want = oracle.forward(*x.tensors(), x.lmask, x.gmask, spec.window, spec.dilation, spec.scale)
    _padded_rows_zero(got, x)
    assert rel_err(got, want) <= TOL_REL["bf16"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_more_global_columns_than_the_lds_list(dtype):
    """600 global tokens in a row that also has local rows: local rows take the
    first 512 global columns from the LDS list and the rest 32 at a time; 19
    global query tiles need several global-row workgroups per slice."""
    spec = workloads.custom(1, 2, 2048, 64, 128, dtype, [0, 1], seed=12, n_global=600,
                            global_mode="random", pad_mode="per_batch", pad_lo=0, pad_hi=200,
                            max_global=600)
    x = workloads.generate(spec)
    ts, lm, gm = to_dev(x)
    plan = make_plan(spec)
    out, st = run(plan, ts, lm, gm)
    assert st == lw.OK
    gidx, gcnt = plan.global_index()
    og, oc = oracle.compact(x.lmask, x.gmask)
    assert np.array_equal(gcnt.cpu().numpy(), oc) and int(oc[0]) > 512
    assert np.array_equal(gidx.cpu().numpy(), og)
    want = oracle.forward(*x.tensors(), x.lmask, x.gmask, spec.window, spec.dilation, spec.scale)
    got = to_np64(out)
    err = rel_err(got, want)
    say(f"600 globals {dtype}: rel err {err:.3e}")
    assert err <= TOL_REL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_more_heads_than_the_kernel_argument_tables(dtype):
    """40 heads with mixed dilation: band workgroups find their head through the
    device-side per-head tables instead of the kernel-argument copy."""
    H = 40
    spec = workloads.custom(1, H, 256, 64, 32, dtype, [h % 3 for h in range(H)], seed=13,
                            n_global=3, pad_mode="per_batch", pad_lo=0, pad_hi=40)
    x = workloads.generate(spec)
    ts, lm, gm = to_dev(x)
    plan = make_plan(spec)
    out, st = run(plan, ts, lm, gm)
    assert st == lw.OK
    want = oracle.forward(*x.tensors(), x.lmask, x.gmask, spec.window, spec.dilation, spec.scale)
    got = to_np64(out)
    err = rel_err(got, want)
    say(f"40 heads {dtype}: rel err {err:.3e}")
    assert err <= TOL_REL[dtype]


def test_all_padded_and_all_global_rows():
    B, H, n = 2, 2, 200
    spec = workloads.custom(B, H, n, 64, 16, "bf16", [0, 1], seed=7, n_global=0)
    x = workloads.generate(spec)
    x.lmask[0, :] = 0.0          # a fully padded sequence
    x.gmask[1, :] = 1.0          # every token global
    ts, lm, gm = to_dev(x)
    plan = make_plan(spec, max_global=n)
    out, st = run(plan, ts, lm, gm)
    assert st == lw.OK
    got = to_np64(out)
    want = oracle.forward(*x.tensors(), x.lmask, x.gmask, spec.window, spec.dilation, spec.scale)
    assert np.all(got[0] == 0.0)
    assert rel_err(got, want) <= TOL_REL["bf16"]
