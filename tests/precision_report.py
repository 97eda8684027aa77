"""Achieved forward error per named workload on the GPU (plain and strong
inputs; the workload's storage type, and fp16 beside bf16), and what rounding
the scaled queries Q c back to the storage type would add (the oracle on
Q' = round(Q c) / c against the oracle on Q, on the CPU).  One JSON line per
case, and the list in gpurun_out/precision.json.  Run from the repository
root on a GPU: python3 tests/precision_report.py"""
import dataclasses
import json
import math
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)
import numpy as np
import torch
import oracle
from gpu_util import make_plan, oracle_rows, run, sample_rows, to_dev, to_np64
from long_document_sparse_amd import lwattn as lw, workloads

def round_store(a, dt):
    if dt == "bf16": return workloads.round_to_bf16(a)
    if dt == "f16": return workloads.round_to_f16(a)
    return a

res = []
for name in workloads.NAMES:
    base = workloads.named(name)
    dts = [base.dtype] + (["f16"] if base.dtype == "bf16" else [])
    for dt in dts:
        spec = dataclasses.replace(base, dtype=dt)
        for strong in (False, True):
            x = workloads.generate(spec, strong=strong)
            ts, lm, gm = to_dev(x)
            plan = make_plan(spec)
            out, st = run(plan, ts, lm, gm)
            assert st == lw.OK
            rows = sample_rows(x, 600, seed=5) if name != "tiny" else np.arange(spec.B * spec.H * spec.n)
            want = oracle_rows(x, rows)
            got = to_np64(out.reshape(-1, spec.d)[torch.from_numpy(rows).to(out.device)])
            amax = float(np.abs(want).max())
            err = float(np.abs(got - want).max())
            rec = {"workload": name, "dtype": dt, "inputs": "strong" if strong else "scaled",
                   "max_abs_err": err, "max_abs_O": amax, "rel_err": err / amax, "rows": int(rows.size)}
            if dt != "f32":
                c = spec.scale * math.log2(math.e)
                Q, K, V, Qg, Kg, Vg = x.tensors()
                Qs = (round_store(Q * np.float32(c), dt) / np.float32(c)).astype(np.float32)
                Qgs = (round_store(Qg * np.float32(c), dt) / np.float32(c)).astype(np.float32)
                w2 = oracle.rows(Qs, K, V, Qgs, Kg, Vg, x.lmask, x.gmask, spec.window, rows, spec.dilation, spec.scale)
                d = float(np.abs(w2 - want).max())
                rec["scale_q_abs"] = d
                rec["scale_q_rel"] = d / amax
            print(json.dumps(rec), flush=True)
            res.append(rec)
            plan.close()
os.makedirs("gpurun_out", exist_ok=True)
with open("gpurun_out/precision.json", "w") as f:
    json.dump(res, f, indent=1)
