"""Helpers shared by the GPU tests: upload seeded inputs, run the HIP path
through the C ABI, compare with the oracle."""
import sys

import numpy as np
import torch

import oracle
from long_document_sparse_amd import lwattn as lw
from long_document_sparse_amd import workloads

# Tolerance of the forward: max |O_gpu - O_oracle| over every compared element,
# relative to max |O_oracle| over them.  Both sides see the same stored
# inputs; scores, exponentials and every sum are fp32 on the GPU (the factor
# scale log2 e applied in fp32), so fp32 storage leaves fp32 rounding over
# sums of up to a few thousand terms: 1e-5.  16-bit storage adds the rounding
# of each probability for the matrix cores and of the output, one unit
# roundoff u each (bf16 2^-9, fp16 2^-12 relative), and the drift of the row's
# O and l sums over those rounded probabilities (terms of one sign, so at most
# u of the sum): a few u in all -- 1e-2 for bf16 (5 u), 3e-3 for fp16 (12 u).
# Measured maxima over the named workloads, plain and strong inputs: bf16
# 3.5e-3, fp16 4.8e-4, fp32 7.6e-7.
TOL_REL = {"f32": 1e-5, "bf16": 1e-2, "f16": 3e-3}


def rel_err(got, want):
    """max |got - want| / max |want| (0 when both are empty or zero)."""
    if want.size == 0:
        return 0.0
    return float(np.max(np.abs(got - want))) / max(float(np.max(np.abs(want))), 1e-30)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: workloads.Inputs, dev="cuda:0"):
    tdt = lw.torch_dtype(x.spec.dtype)
    ts = [torch.from_numpy(a).to(dev).to(tdt) for a in x.tensors()]
    lm = torch.from_numpy(x.lmask).to(dev)
    gm = torch.from_numpy(x.gmask).to(dev)
    return ts, lm, gm


def make_plan(spec: workloads.Spec, max_global=None):
    return lw.Plan(spec.B, spec.H, spec.n, spec.d, spec.window, spec.dilation,
                   spec.max_global if max_global is None else max_global,
                   spec.scale, spec.dtype)


def run(plan, ts, lm, gm, poison=True):
    out = torch.empty_like(ts[0])
    if poison:
        out.fill_(float("nan"))
    plan(*ts, lm, gm, out=out)
    st = plan.sync_status()
    return out, st


def to_np64(t):
    return t.float().cpu().numpy().astype(np.float64)


def sample_rows(x: workloads.Inputs, count: int, seed: int = 0):
    """Flat row indices: random rows plus boundary rows (ends, padding edge, globals)."""
    s = x.spec
    rng = np.random.default_rng(seed)
    B, H, n = s.B, s.H, s.n
    rows = set(rng.choice(B * H * n, size=min(count, B * H * n), replace=False).tolist())
    for b in range(B):
        nv = n - int(x.pad_len[b])
        for h in (0, H - 1):
            base = (b * H + h) * n
            for i in (0, 1, 31, 32, 127, 128, n // 2, nv - 1, nv, n - 1):
                if 0 <= i < n:
                    rows.add(base + i)
            for gpos in x.global_pos[b][:8]:
                rows.add(base + int(gpos))
                for dlt in (-1, 1, s.window // 2, -(s.window // 2)):
                    if 0 <= int(gpos) + dlt < n:
                        rows.add(base + int(gpos) + dlt)
    return np.array(sorted(rows), np.int64)


def oracle_rows(x: workloads.Inputs, rows):
    s = x.spec
    return oracle.rows(*x.tensors(), x.lmask, x.gmask, s.window, rows, s.dilation, s.scale)


def check_rows(x, got_np64_flat_rows, want):
    """(error relative to max |want|, the storage type's bound)."""
    return rel_err(got_np64_flat_rows, want), TOL_REL[x.spec.dtype]
