"""IEEE half (fp16) storage through the C ABI: the forward against the oracle,
the allocation-free forward against the plan's, the causal and block-sparse
forwards against the oracle's, and the encoder layer against the oracle's
layer.

Tolerance, from the arithmetic (as for bf16, with fp16's unit roundoff 2^-11
in place of bf16's 2^-8): the oracle sees exactly the stored fp16 values; the
HIP path takes Q and K as stored into the matrix cores (fp32 accumulation, the
factor scale log2 e applied in fp32), rounds each probability to fp16 for the
matrix cores (2^-11 relative, the row sum taken over the same rounded values)
and the output once (2^-11).  Per compared tensor, relative to its largest
entry: |err| <= 3e-3 * max |O| (about 6 units of 2^-11, for the few
roundings that reach each output).
The closed form (Q = 0, one-hot V) has exact fp32 quotients rounded once:
|err| <= 2^-10 * expected there, and channels without keys exactly zero.
"""
import dataclasses

import numpy as np
import pytest
import torch

import closed_form as cf
import oracle
from gpu_util import make_plan, oracle_rows, run, sample_rows, say, to_dev, to_np64
from long_document_sparse_amd import lwattn as lw
from long_document_sparse_amd import workloads

pytestmark = pytest.mark.gpu

REL = 3e-3

SMALL = [
    # (B, H, n, window, dilation, n_global, global_mode, pad_mode, pad_hi)
    (2, 3, 517, 128, [0, 1, 2], 5, "random", "per_batch", 100),
    (3, 2, 260, 512, [0, 1], 3, "first", "per_batch", 200),       # window > n
    (2, 2, 700, 60, [0, 1], 70, "random", "per_batch", 650),      # > 2 global tiles, long pads
    (2, 3, 600, 64, [0, 1, 3], 6, "random", "scatter", 150),      # padding anywhere
    (1, 1, 31, 10, [3], 31, "first", "none", 0),                  # every token global
    (2, 2, 64, 6, [0, 0], 0, "first", "per_batch", 10),           # no globals
    (1, 1, 1, 2, [0], 1, "first", "none", 0),                     # n = 1
]


def _rel_err(got, want):
    return float(np.max(np.abs(got - want))) / max(float(np.max(np.abs(want))), 1e-30)


@pytest.mark.parametrize("strong", [False, True], ids=["scaled", "strong"])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"B{c[0]}H{c[1]}n{c[2]}w{c[3]}g{c[5]}{c[7]}")
def test_f16_small_full_parity(case, strong):
    B, H, n, w, dil, ng, gmode, pmode, phi = case
    spec = workloads.custom(B, H, n, 64, w, "f16", dil, seed=n + w + 1, n_global=ng, global_mode=gmode,
                            pad_mode=pmode, pad_hi=phi, max_global=max(ng, 1))
    x = workloads.generate(spec, strong=strong)
    say(f"f16 small case {case} strong={strong}")
    ts, lm, gm = to_dev(x)
    assert ts[0].dtype == torch.float16
    plan = make_plan(spec)
    out, st = run(plan, ts, lm, gm)
    assert st == lw.OK
    got = to_np64(out)
    assert not np.isnan(got).any(), "a row was not written"
    want = oracle.forward(*x.tensors(), x.lmask, x.gmask, w, dil, spec.scale)
    for b in range(B):
        pad = x.lmask[b] == 0
        assert np.all(got[b][:, pad] == 0.0)
    rel = _rel_err(got, want)
    say(f"f16 small: rel err {rel:.3e}")
    assert rel <= REL, rel


@pytest.mark.parametrize("name", ["base", "qa", "long"])
def test_f16_named_workload_sampled_rows(name):
    """The named workload's structure and sizes in fp16, sampled rows plus every
    boundary kind, strong inputs (O(1) outputs)."""
    spec = dataclasses.replace(workloads.named(name), dtype="f16")
    x = workloads.generate(spec, strong=True)
    ts, lm, gm = to_dev(x)
    plan = make_plan(spec)
    say(f"f16 {name}: forward")
    out, st = run(plan, ts, lm, gm)
    assert st == lw.OK
    assert not torch.isnan(out).any().item(), "a row was not written"
    rows = sample_rows(x, 800, seed=3)
    want = oracle_rows(x, rows)
    got = to_np64(out.reshape(-1, spec.d)[torch.from_numpy(rows).to(out.device)])
    rel = _rel_err(got, want)
    say(f"f16 {name}: rel err {rel:.3e} over {rows.size} rows")
    assert rel <= REL, rel


@pytest.mark.parametrize("name", ["base", "long"])
def test_f16_closed_form_every_row(name):
    """Q = 0, one-hot V (tests/closed_form.py) in fp16 at full size: every row."""
    spec = dataclasses.replace(workloads.named(name), dtype="f16")
    B, H, n, d = spec.B, spec.H, spec.n, spec.d
    lmask, gmask, _, _ = workloads.structure(spec)
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(spec.seed)
    Z = torch.zeros((B, H, n, d), dtype=torch.float16, device=dev)
    K = torch.randn((B, H, n, d), generator=gen, device=dev).half()
    V = torch.from_numpy(cf.one_hot_rows(n, d, cf.SHIFT_LOCAL)).to(dev).half().expand(B, H, n, d).contiguous()
    Vg = torch.from_numpy(cf.one_hot_rows(n, d, cf.SHIFT_GLOBAL)).to(dev).half().expand(B, H, n, d).contiguous()
    lm = torch.from_numpy(lmask).to(dev)
    gm = torch.from_numpy(gmask).to(dev)
    plan = make_plan(spec)
    out = torch.full((B, H, n, d), float("nan"), dtype=torch.float16, device=dev)
    plan(Z, K, V, Z, K, Vg, lm, gm, out=out)
    assert plan.sync_status() == lw.OK
    worst = 0.0
    for b in range(B):
        for gap in sorted(set(spec.dilation)):
            heads = [h for h in range(H) if spec.dilation[h] == gap]
            want = torch.from_numpy(cf.expected_rows(lmask[b], gmask[b], spec.window, gap, d)).to(dev)
            got = out[b, heads].double()
            assert not torch.isnan(got).any().item()
            zero = want == 0.0
            assert torch.all(got[:, zero] == 0.0).item()
            rel = ((got - want).abs() / torch.where(zero, torch.ones_like(want), want)).max().item()
            worst = max(worst, rel)
            assert rel <= 2.0 ** -10, (b, gap, rel)
    say(f"f16 closed form {name}: max rel err {worst:.3e}")


def test_f16_noalloc_matches_plan():
    spec = workloads.custom(2, 3, 1500, 64, 256, "f16", [0, 1, 2], seed=35, n_global=40,
                            global_mode="random", pad_mode="per_batch", pad_hi=300, max_global=64)
    x = workloads.generate(spec)
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
    assert torch.equal(want, out)
    assert torch.count_nonzero(status).item() == 0


# The backward in fp16 (the matrix-core kernels of bf16, with fp16 operands):
# the bound of the bf16 backward (2e-2 of each tensor's largest entry, from
# 2^-9 roundings of P, dS and the gradients) scaled to fp16's roundoff, 8
# times smaller: 3e-3.  The last two grids take each mix of the launch folds
# on a 256-CU device (compaction launched and merge folded; compaction folded
# and merge launched), the first ones both folds.
BWD = [
    # (B, H, n, window, dilation, n_global, global_mode, pad_mode, pad_hi)
    (2, 2, 333, 40, [0, 2], 5, "random", "per_batch", 80),
    (1, 3, 300, 128, [0, 1, 3], 70, "random", "per_batch", 60),   # two global tiles
    (1, 2, 257, 16, [1, 4], 0, "first", "scatter", 40),           # no globals
    (13, 1, 4096, 32, [0], 20, "random", "per_batch", 300),
    (8, 1, 4096, 32, [0], 10, "random", "per_batch", 300),
]
BWD_REL = 3e-3


@pytest.mark.parametrize("case", BWD, ids=lambda c: f"B{c[0]}H{c[1]}n{c[2]}w{c[3]}g{c[5]}{c[7]}")
def test_f16_backward_matches_oracle(case):
    B, H, n, window, dil, ng, gmode, pmode, phi = case
    spec = workloads.custom(B, H, n, 64, window, "f16", dil, seed=23, n_global=ng, global_mode=gmode,
                            pad_mode=pmode, pad_hi=phi)
    say(f"f16 backward case {case}")
    x = workloads.generate(spec)
    ts, lm, gm = to_dev(x)
    plan = make_plan(spec, max_global=max(ng, 1))
    o = torch.empty_like(ts[0])
    plan(*ts, lm, gm, out=o)
    go = torch.from_numpy(np.random.default_rng(3).standard_normal(x.tensors()[0].shape)).to(
        ts[0].device).to(ts[0].dtype)
    grads = tuple(torch.full_like(ts[0], float("nan")) for _ in range(6))
    plan.backward(*ts, lm, gm, o, go, grads=grads)
    assert plan.sync_status() == lw.OK
    ins = [to_np64(t) for t in ts]
    want = oracle.backward(*ins, x.lmask, x.gmask, to_np64(go), spec.window, spec.dilation, spec.scale)
    for name, g, w in zip(("dQ", "dK", "dV", "dQg", "dKg", "dVg"), grads, want):
        got = to_np64(g)
        assert np.all(np.isfinite(got)), name
        ref = float(np.max(np.abs(w)))
        err = float(np.max(np.abs(got - w)))
        say(f"f16 backward {name}: max abs err {err:.3e}, max |g| {ref:.3e}")
        if ref == 0.0:
            assert err == 0.0, name
        else:
            assert err <= BWD_REL * ref, name
    plan.close()


def test_f16_layer_matches_oracle():
    """The encoder layer in fp16 at the base model's heads (H=12): bound as for
    the bf16 layer with fp16's roundoff (8 times smaller): |err| <= 5e-3."""
    import math
    B, H, n, window, ng, inter = 1, 12, 1024, 256, 24, 3072
    dil = [0] * H
    spec = workloads.custom(B, H, n, 64, window, "f16", dil, seed=52, n_global=ng,
                            global_mode="random", pad_mode="per_batch", pad_hi=100)
    x = workloads.generate(spec)
    dev = "cuda:0"
    plan = make_plan(spec, max_global=ng)
    layer = lw.Layer(plan, inter, 1e-5)
    rng = np.random.default_rng(7)
    w = {}
    for name, shape in layer.shapes().items():
        if name.startswith("ln") and name.endswith("_g"):
            a = 1.0 + 0.1 * rng.standard_normal(shape)
        elif len(shape) == 2:
            a = rng.standard_normal(shape) / math.sqrt(shape[0])
        else:
            a = 0.1 * rng.standard_normal(shape)
        w[name] = torch.from_numpy(a.astype(np.float32)).to(dev).half()
    X = torch.from_numpy(rng.standard_normal((B * n, H * 64)).astype(np.float32)).to(dev).half()
    lm = torch.from_numpy(x.lmask).to(dev)
    gm = torch.from_numpy(x.gmask).to(dev)
    Y = layer.forward(X, w, lm, gm)
    torch.cuda.synchronize()
    assert plan.sync_status() == lw.OK
    got = to_np64(Y)
    want = oracle.layer_forward(to_np64(X).reshape(B, n, H * 64), {k: to_np64(t) for k, t in w.items()},
                                x.lmask, x.gmask, window, dil, H, 1e-5).reshape(B * n, H * 64)
    err = np.abs(got - want)
    say(f"f16 layer: max err {err.max():.4g} mean {err.mean():.4g}")
    assert np.all(np.isfinite(got))
    assert err.max() <= 5e-3
    layer.close()


CAUSAL = [
    # (B, H, n, window, dilation, pad_mode, pad_hi)
    (2, 3, 333, 40, [0, 2, 5], "per_batch", 80),
    (1, 2, 130, 400, [0, 0], "none", 0),          # window beyond the sequence
    (2, 2, 257, 16, [1, 4], "scatter", 40),       # scattered pads
    (1, 2, 1000, 300, [0, 1], "per_batch", 200),  # interior and edge tiles
]


@pytest.mark.parametrize("strong", [False, True], ids=["scaled", "strong"])
@pytest.mark.parametrize("case", CAUSAL, ids=lambda c: f"B{c[0]}H{c[1]}n{c[2]}w{c[3]}{c[5]}")
def test_f16_causal_matches_oracle(case, strong):
    B, H, n, window, dil, pmode, phi = case
    spec = workloads.custom(B, H, n, 64, window, "f16", dil, seed=31, n_global=0,
                            pad_mode=pmode, pad_hi=phi, max_global=0)
    say(f"f16 causal case {case} strong={strong}")
    x = workloads.generate(spec, strong=strong)
    q, k, v = (torch.from_numpy(a).to("cuda:0").to(torch.float16) for a in (x.Q, x.K, x.V))
    lm = torch.from_numpy(x.lmask).to("cuda:0")
    plan = make_plan(spec, max_global=0)
    out = torch.full_like(q, float("nan"))
    plan.forward_causal(q, k, v, lm, out=out)
    torch.cuda.synchronize()
    want = oracle.forward_causal(to_np64(q), to_np64(k), to_np64(v), x.lmask, window, dil, spec.scale)
    got = to_np64(out)
    assert np.all(np.isfinite(got))
    rel = _rel_err(got, want)
    say(f"f16 causal: rel err {rel:.3e}")
    assert rel <= REL, rel
    pad = x.lmask == 0
    for b in range(B):
        assert not np.any(got[b][:, pad[b]])


BSPARSE = [
    # (B, H, n, local, extra, causal, pad_mode, pad_hi)
    (2, 3, 333, 2, 2, True, "per_batch", 80),
    (1, 2, 257, 1, 3, False, "scatter", 40),
    (2, 2, 1000, 4, 4, False, "per_batch", 200),
]


@pytest.mark.parametrize("strong", [False, True], ids=["scaled", "strong"])
@pytest.mark.parametrize("case", BSPARSE, ids=lambda c: f"B{c[0]}H{c[1]}n{c[2]}l{c[3]}e{c[4]}{'c' if c[5] else ''}")
def test_f16_blocksparse_matches_oracle(case, strong):
    B, H, n, local, extra, causal, pmode, phi = case
    spec = workloads.custom(B, H, n, 64, 0, "f16", [0] * H, seed=41, n_global=0,
                            pad_mode=pmode, pad_hi=phi, max_global=0)
    layout = workloads.blocksparse_layout(H, n, seed=9, local=local, extra=extra, causal=causal)
    say(f"f16 block-sparse case {case} strong={strong}")
    x = workloads.generate(spec, strong=strong)
    q, k, v = (torch.from_numpy(a).to("cuda:0").to(torch.float16) for a in (x.Q, x.K, x.V))
    lm = torch.from_numpy(x.lmask).to("cuda:0")
    rowptr, cols = workloads.layout_csr(layout)
    plan = make_plan(spec, max_global=0)
    out = torch.full_like(q, float("nan"))
    plan.forward_blocksparse(q, k, v, lm, torch.from_numpy(rowptr).to("cuda:0"),
                             torch.from_numpy(cols).to("cuda:0"), causal=causal, out=out)
    torch.cuda.synchronize()
    want = oracle.forward_blocksparse(to_np64(q), to_np64(k), to_np64(v), x.lmask, layout, causal, spec.scale)
    got = to_np64(out)
    assert np.all(np.isfinite(got))
    rel = _rel_err(got, want)
    say(f"f16 block-sparse: rel err {rel:.3e}")
    assert rel <= REL, rel
    pad = x.lmask == 0
    for b in range(B):
        assert not np.any(got[b][:, pad[b]])


@pytest.mark.parametrize("case", CAUSAL[:3], ids=lambda c: f"B{c[0]}H{c[1]}n{c[2]}w{c[3]}{c[5]}")
def test_f16_causal_backward_matches_oracle(case):
    """The causal backward in fp16: the bound of the fp16 backward (3e-3 of
    each tensor's largest entry)."""
    B, H, n, window, dil, pmode, phi = case
    spec = workloads.custom(B, H, n, 64, window, "f16", dil, seed=35, n_global=0,
                            pad_mode=pmode, pad_hi=phi, max_global=0)
    say(f"f16 causal backward case {case}")
    x = workloads.generate(spec)
    q, k, v = (torch.from_numpy(a).to("cuda:0").to(torch.float16) for a in (x.Q, x.K, x.V))
    lm = torch.from_numpy(x.lmask).to("cuda:0")
    plan = make_plan(spec, max_global=0)
    o = plan.forward_causal(q, k, v, lm)
    go = torch.from_numpy(np.random.default_rng(4).standard_normal(x.Q.shape)).to("cuda:0").to(torch.float16)
    grads = plan.backward_causal(q, k, v, lm, o, go)
    assert plan.sync_status() == lw.OK
    want = oracle.backward_causal(to_np64(q), to_np64(k), to_np64(v), x.lmask, to_np64(go), window, dil,
                                  spec.scale)
    for name, g, w in zip(("dQ", "dK", "dV"), grads, want):
        got = to_np64(g)
        assert np.all(np.isfinite(got)), name
        ref = float(np.max(np.abs(w)))
        err = float(np.max(np.abs(got - w)))
        say(f"f16 causal backward {name}: max abs err {err:.3e}, max |g| {ref:.3e}")
        assert err <= (BWD_REL * ref if ref > 0 else 0.0), name
    plan.close()
