#!/usr/bin/env python3
"""Benchmark of the Longformer window + global attention forward on one MI355X.

One step = one lwattn_forward, a single kernel launch (global-index
compaction, band rows, global rows and the merge of their key slices), over
one batch of seeded synthetic input that is already resident in device
memory.  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload base]
                  [--no-cpu-baseline] [--no-timing] [--copy-probe MIB]
                  [--pass forward|backward]

The default workload is "base": B=1, H=12, n=4096, d=64, w=512 (+-256), no
dilation, one global token at position 0, bf16 storage, fp32 accumulation.

Timing is "warm": forwards run back to back, so inputs that fit the 256 MB
last-level cache stay there between steps.  After the timed loop, a "cold"
pass (--cold-steps) writes 1 GiB between forwards, so every forward starts
with its inputs in HBM only, and reports that kernel time beside the warm one.
The line also carries on-device peaks measured by the library's probes (a
matrix-core loop, an HBM read stream) and a plain copy, and the roofline
fraction against them beside the published peak.  Kernel durations come from HIP
events that the dispatch of the attention kernel itself records at the start
and the end of its execution, on every fourth forward of the timed loop
(recording them on every forward would make the host, not the GPU, set the
pace of the loop).

--pass backward times lwattn_backward instead (dQ, dK, dV, dQg, dKg, dVg of a
seeded dO, after one forward for O) and prints its own line: the whole call
is timed with events on the stream around the timed loop, and each of its
kernels with the events its dispatch records; the roofline is that of the
longest kernel (bf16 storage: its matrix FLOPs against the bf16 matrix-core
peak; fp32 storage: the whole call against the fp32 vector-ALU peak), and the
CPU baseline is the oracle's backward.

--copy-probe runs, after the timed loop, a plain device-to-device copy of the
given size a few times; a counter pass over the same command then gives the
ratio between what FETCH_SIZE / WRITE_SIZE report and the bytes a copy of
known size must move.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}     # MI355X dense MFMA
PEAK_FP32_VECTOR = 157.3                          # MI355X fp32 vector ALU, TFLOP/s
PEAK_BF16_MFMA = 2500.0                           # MI355X dense bf16 matrix cores, TFLOP/s
PEAK_HBM_GBS = 8000.0
TIMING_EVERY = 4
METRIC = "window+global attn fwd tokens/s & TFLOP/s (% bf16 MFMA peak), n=4096 w=512"
METRIC_BWD = "window+global attn bwd tokens/s, n=4096 w=512"
KERNEL_SOURCES = ("long_document_sparse_amd/csrc/kernels.hpp",
                  "long_document_sparse_amd/csrc/lwattn.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_kernel_traffic.txt")


def describe(spec):
    glob = (f"{spec.n_global} global tokens " +
            ("at the start" if spec.global_mode == "first" else "at random positions"))
    pad = {"none": "no padding",
           "per_batch": f"padded tail U{{{spec.pad_lo}..{spec.pad_hi}}} per sequence",
           "one_seq": f"one sequence with a padded tail U{{{spec.pad_lo}..{spec.pad_hi}}}",
           "scatter": f"U{{{spec.pad_lo}..{spec.pad_hi}}} padded positions anywhere"}[spec.pad_mode]
    dil = sorted(set(spec.dilation))
    return (f"{spec.name}: B={spec.B} H={spec.H} n={spec.n} d={spec.d} w={spec.window} "
            f"dilation {dil} {spec.dtype}; {glob}; {pad}")


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, dtype: str = "bf16"):
    """HBM bytes per attn_kernel launch from the committed counter summary, or
    None when there is none for this workload or the kernels changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    want = source_hash()
    for line in lines:
        if not line.startswith("{"):
            continue
        rec = json.loads(line)
        if rec.get("workload") == workload and rec.get("source_sha256") == want and \
                rec.get("dtype", "bf16") == dtype:
            return rec
    return None


def host_cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measure_peaks(lib, dev):
    """What this GPU delivers, measured with the library's probes and a plain
    copy (each timed with events over 3 launches after one warm-up):
    bf16 matrix-core rate, HBM read rate over 2 GiB, device-to-device copy
    rate over 1 GiB (read + write bytes)."""
    import ctypes
    import torch
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = torch.empty(4096, dtype=torch.float32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    iters = 2048
    t = timed(lambda: lib.lwattn_probe_mfma(iters, ctypes.c_void_p(out.data_ptr()), stream))
    mfma = 512 * 4 * iters * 8 * 32768 / t / 1e12
    nread = 2 << 30
    buf = torch.empty(nread, dtype=torch.uint8, device=dev)
    buf.fill_(3)
    t = timed(lambda: lib.lwattn_probe_read(ctypes.c_void_p(buf.data_ptr()), nread,
                                            ctypes.c_void_p(out.data_ptr()), stream))
    read = nread / t / 1e9
    del buf
    ncopy = 1 << 30
    a = torch.empty(ncopy, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    t = timed(lambda: b.copy_(a))
    copy = 2 * ncopy / t / 1e9
    del a, b
    return {"mfma_bf16_tflops": round(mfma, 1), "hbm_read_gbs": round(read, 1),
            "hbm_copy_gbs": round(copy, 1),
            "how": "lwattn_probe_mfma (8 chains of v_mfma_f32_32x32x16_bf16 per wave, 2 waves/SIMD), "
                   "lwattn_probe_read over 2 GiB, torch copy of 1 GiB (read + write bytes)"}


def time_cold(step, plan, steps, dev):
    """Kernel time with the last-level cache emptied before every forward: a
    1 GiB scratch buffer is written between calls (outside the timed kernel);
    the duration comes from the events the dispatch records."""
    import torch
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    plan.timing_enable(steps, every=1)
    for i in range(steps):
        scratch.fill_(i & 255)
        step()
    torch.cuda.synchronize()
    tot, calls = plan.timing_read()
    plan.timing_disable()
    del scratch
    return tot["attention"] / calls * 1e-3


def cpu_baseline(x, budget_s=12.0):
    """The oracle, as it is, on the host cores over a bounded sample of the workload."""
    import numpy as np
    import oracle
    spec = x.spec
    threads = oracle.default_threads()
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit() and int(omp) > 0:
        threads = min(threads, int(omp))
    n, H, B = spec.n, spec.H, spec.B
    total_heads = B * H
    args = (*x.tensors(), x.lmask, x.gmask, spec.window)

    def run_heads(k):
        rows = np.arange(k * n, dtype=np.int64)       # all rows of the first k (b, h) pairs
        t0 = time.perf_counter()
        oracle.rows(*args, rows, spec.dilation, spec.scale, threads=threads)
        return time.perf_counter() - t0

    t1 = run_heads(1)
    if t1 * total_heads <= budget_s / 2:
        # the whole forward is cheap: repeat it until the budget is used
        reps, t = 0, 0.0
        while t < budget_s:
            t0 = time.perf_counter()
            oracle.forward(*args, spec.dilation, spec.scale, threads=threads)
            t += time.perf_counter() - t0
            reps += 1
        value = B * n * reps / t
        sample = f"the whole forward, repeated {reps} times ({t:.2f} s)"
    else:
        k = int(max(1, min(total_heads, budget_s / max(t1, 1e-6))))
        t = run_heads(k) if k > 1 else t1
        value = B * n / (t * total_heads / k)
        sample = (f"every query row of {k} of the {total_heads} (batch, head) pairs "
                  f"({k * n} rows, {t:.2f} s), scaled to the full workload")
    return {"value": round(value, 3), "unit": "tokens/s", "cores": threads, "cpu_model": host_cpu_model(), "kind": "oracle",
            "sample": sample}


def cpu_baseline_backward(x, go, budget_s=12.0):
    """The oracle's backward, as it is, on the host cores, repeated over the
    whole problem for about budget_s seconds."""
    import oracle
    spec = x.spec
    threads = oracle.default_threads()
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit() and int(omp) > 0:
        threads = min(threads, int(omp))
    args = (*x.tensors(), x.lmask, x.gmask, go, spec.window, spec.dilation, spec.scale)
    reps, t = 0, 0.0
    while t < budget_s:
        t0 = time.perf_counter()
        oracle.backward(*args, threads=threads)
        t += time.perf_counter() - t0
        reps += 1
    value = spec.B * spec.n * reps / t
    return {"value": round(value, 3), "unit": "tokens/s", "cores": threads, "cpu_model": host_cpu_model(), "kind": "oracle",
            "sample": f"the whole backward, repeated {reps} times ({t:.2f} s)"}


def cpu_baseline_causal(x, budget_s=12.0):
    """The oracle's causal forward, as it is, on the host cores, repeated over
    the whole problem for about budget_s seconds."""
    import oracle
    spec = x.spec
    threads = oracle.default_threads()
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit() and int(omp) > 0:
        threads = min(threads, int(omp))
    reps, t = 0, 0.0
    while t < budget_s:
        t0 = time.perf_counter()
        oracle.forward_causal(x.Q, x.K, x.V, x.lmask, spec.window, spec.dilation, spec.scale,
                              threads=threads)
        t += time.perf_counter() - t0
        reps += 1
    value = spec.B * spec.n * reps / t
    return {"value": round(value, 3), "unit": "tokens/s", "cores": threads, "cpu_model": host_cpu_model(), "kind": "oracle",
            "sample": f"the whole causal forward, repeated {reps} times ({t:.2f} s)"}


def cpu_baseline_causal_backward(x, budget_s=12.0):
    """The oracle's causal backward, as it is, on the host cores, over whole
    (batch row, head) slices in turn for about budget_s seconds (heads are
    independent, so a slice is a fair sample of the work)."""
    import numpy as np
    import oracle
    spec = x.spec
    threads = oracle.default_threads()
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit() and int(omp) > 0:
        threads = min(threads, int(omp))
    rng = np.random.default_rng(5)
    do = (rng.standard_normal(x.Q.shape[2:]) / 8).astype(np.float32)
    dil = list(spec.dilation)
    heads, t = 0, 0.0
    while t < budget_s:
        b, h = divmod(heads % (spec.B * spec.H), spec.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        t0 = time.perf_counter()
        oracle.backward_causal(x.Q[sl], x.K[sl], x.V[sl], x.lmask[b:b + 1], do[None, None], spec.window,
                               [dil[h]], spec.scale, threads=threads)
        t += time.perf_counter() - t0
        heads += 1
    value = spec.n * heads / spec.H / t          # a token is one row of every head
    return {"value": round(value, 3), "unit": "tokens/s", "cores": threads, "cpu_model": host_cpu_model(), "kind": "oracle",
            "sample": f"{heads} whole (batch row, head) slices of the causal backward ({t:.2f} s), "
                      f"scaled by the {spec.H} heads of a token"}


def run_causal_backward(args, spec, x, ts, lm, plan):
    """--pass causal_backward: one JSON line for lwattn_backward_causal (two
    kernels a call: dQ with the rows' statistics, then dK/dV)."""
    import ctypes
    import torch
    from long_document_sparse_amd import flops as fl
    from long_document_sparse_amd import lwattn
    if spec.dtype not in ("bf16", "f16"):
        raise SystemExit("the causal variant's backward runs on 16-bit storage (bf16 or f16)")
    q, k, v = ts[0], ts[1], ts[2]
    g = torch.Generator().manual_seed(5)
    do = (torch.randn(q.shape, generator=g) / 8).to(q.device).to(torch.bfloat16)
    o = plan.forward_causal(q, k, v, lm)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    fn = plan.lib.lwattn_backward_causal
    cargs = (plan.handle,) + tuple(ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, lm, o, do, dq, dk, dv)) + (None,)

    def step():
        st = fn(*cargs)
        if st != lwattn.OK:
            raise SystemExit(f"causal backward failed: {lwattn.strerror(st)}")

    for _ in range(args.warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    t_call = e0.elapsed_time(e1) * 1e-3 / args.steps        # s per call (both kernels), on the stream
    pairs = fl.causal_pairs(x.lmask, spec.window, spec.dilation)
    # S, dP, dQ, dK, dV: five products of 2 d flops per pair (recomputation not counted)
    flop = 10 * spec.d * pairs
    achieved = flop / t_call / 1e12
    tokens = spec.B * spec.n
    res = {
        "metric": "causal dilated window attn bwd tokens/s, n=8192 w=512",
        "value": round(tokens / (elapsed / args.steps), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded, N(0,1)/sqrt(d) inputs; no dataset)",
        "config": {"workload": describe(spec) + "; causal backward", "global_batch": spec.B, "seq_len": spec.n,
                   "heads": spec.H, "head_dim": spec.d, "window": spec.window,
                   "parallelism": "single GPU", "timing": "warm (back to back)"},
        "us_per_call_on_stream": round(t_call * 1e6, 2),
        "algorithmic_pairs": pairs,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_MFMA,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_MFMA, 4), "traffic": None,
                     "kernel": "causal_dq_kernel + causal_dkv_kernel (one call)", "algorithmic_flop": flop,
                     "source_sha256": source_hash()},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_causal_backward(x)
    plan.close()
    print(json.dumps(res), flush=True)


def run_causal(args, spec, x, ts, lm, plan):
    """--pass causal: one JSON line for lwattn_forward_causal (one kernel a call)."""
    import ctypes
    import torch
    from long_document_sparse_amd import flops as fl
    from long_document_sparse_amd import lwattn
    if spec.dtype not in ("bf16", "f16"):
        raise SystemExit("the causal variant runs on 16-bit storage (bf16 or f16)")
    q, k, v = ts[0], ts[1], ts[2]
    o = torch.empty_like(q)
    plan.forward_causal(q, k, v, lm, out=o)
    fn = plan.lib.lwattn_forward_causal
    cargs = (plan.handle,) + tuple(ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, lm, o)) + (None,)

    def step():
        st = fn(*cargs)
        if st != lwattn.OK:
            raise SystemExit(f"causal forward failed: {lwattn.strerror(st)}")

    for _ in range(args.warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    t_call = e0.elapsed_time(e1) * 1e-3 / args.steps        # s per launch, on the stream
    pairs = fl.causal_pairs(x.lmask, spec.window, spec.dilation)
    flop = 4 * spec.d * pairs                                 # S and P V, 2 d per product and pair
    achieved = flop / t_call / 1e12
    tokens = spec.B * spec.n
    res = {
        "metric": "causal dilated window attn fwd tokens/s, n=8192 w=512",
        "value": round(tokens / (elapsed / args.steps), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded, N(0,1)/sqrt(d) inputs; no dataset)",
        "config": {"workload": describe(spec) + "; causal", "global_batch": spec.B, "seq_len": spec.n,
                   "heads": spec.H, "head_dim": spec.d, "window": spec.window,
                   "parallelism": "single GPU", "timing": "warm (back to back)"},
        "us_per_launch_on_stream": round(t_call * 1e6, 2),
        "algorithmic_pairs": pairs,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_MFMA,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_MFMA, 4), "traffic": None,
                     "kernel": "causal_kernel", "algorithmic_flop": flop,
                     "source_sha256": source_hash()},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_causal(x)
    plan.close()
    print(json.dumps(res), flush=True)


def cpu_baseline_blocksparse(x, layout, causal, budget_s=12.0):
    """The oracle's block-sparse rows, as they are, on the host cores: a
    random sample of rows, grown until about budget_s seconds, scaled to
    tokens/s (a token is all H heads' rows)."""
    import numpy as np
    import oracle
    spec = x.spec
    threads = oracle.default_threads()
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit() and int(omp) > 0:
        threads = min(threads, int(omp))
    rng = np.random.default_rng(0)
    total = spec.B * spec.H * spec.n
    count, t, rows = 2048, 0.0, 0
    while t < budget_s:
        idx = rng.choice(total, min(count, total), replace=False)
        t0 = time.perf_counter()
        oracle.rows_blocksparse(x.Q, x.K, x.V, x.lmask, layout, idx, causal, spec.scale, threads=threads)
        t += time.perf_counter() - t0
        rows += idx.size
        count *= 2
    value = rows / spec.H / t
    return {"value": round(value, 3), "unit": "tokens/s", "cores": threads, "cpu_model": host_cpu_model(), "kind": "oracle",
            "sample": f"{rows} random rows of all heads ({t:.2f} s), scaled by 1/H to tokens"}


def run_blocksparse(args, spec, x, ts, lm, plan):
    """--pass blocksparse: one JSON line for lwattn_forward_blocksparse."""
    import ctypes
    import torch
    from long_document_sparse_amd import flops as fl
    from long_document_sparse_amd import lwattn, workloads
    if spec.dtype not in ("bf16", "f16"):
        raise SystemExit("block-sparse attention runs on 16-bit storage (bf16 or f16)")
    kw = workloads.BSPARSE_LAYOUT
    layout = workloads.blocksparse_layout(spec.H, spec.n, seed=spec.seed, **kw)
    rowptr, cols = workloads.layout_csr(layout)
    rp = torch.from_numpy(rowptr).to(ts[0].device)
    cl = torch.from_numpy(cols).to(ts[0].device)
    q, k, v = ts[0], ts[1], ts[2]
    o = torch.empty_like(q)
    plan.forward_blocksparse(q, k, v, lm, rp, cl, causal=kw["causal"], out=o)
    fn = plan.lib.lwattn_forward_blocksparse
    cargs = (plan.handle,) + tuple(ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, lm, rp, cl)) + \
        (int(cl.numel()), int(kw["causal"]), ctypes.c_void_p(o.data_ptr()), None)

    def step():
        st = fn(*cargs)
        if st != lwattn.OK:
            raise SystemExit(f"block-sparse forward failed: {lwattn.strerror(st)}")

    for _ in range(args.warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    t_call = e0.elapsed_time(e1) * 1e-3 / args.steps
    pairs = fl.blocksparse_pairs(x.lmask, layout, kw["causal"])
    flop = 4 * spec.d * pairs
    achieved = flop / t_call / 1e12
    tokens = spec.B * spec.n
    res = {
        "metric": "block-sparse (64-block layout) attn fwd tokens/s, n=16384",
        "value": round(tokens / (elapsed / args.steps), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded, N(0,1)/sqrt(d) inputs, seeded layout; no dataset)",
        "config": {"workload": (f"{spec.name}: B={spec.B} H={spec.H} n={spec.n} d={spec.d} bf16; layout "
                                f"own + {kw['local'] - 1} previous + {kw['extra']} drawn key blocks per query "
                                f"block{' (causal)' if kw['causal'] else ''}; {cols.size} blocks listed"),
                   "global_batch": spec.B, "seq_len": spec.n, "heads": spec.H, "head_dim": spec.d,
                   "parallelism": "single GPU", "timing": "warm (back to back)"},
        "us_per_launch_on_stream": round(t_call * 1e6, 2),
        "algorithmic_pairs": pairs,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_MFMA,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_MFMA, 4), "traffic": None,
                     "kernel": "blocksparse_kernel", "algorithmic_flop": flop,
                     "source_sha256": source_hash()},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_blocksparse(x, layout, kw["causal"])
    plan.close()
    print(json.dumps(res), flush=True)


def cpu_baseline_layer(x, X, w, inter, budget_s=12.0):
    """The oracle's layer, as it is, on the host cores, over a prefix of the
    rows' batch row grown until about budget_s seconds; scaled to tokens/s."""
    import oracle
    spec = x.spec
    threads = oracle.default_threads()
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit() and int(omp) > 0:
        threads = min(threads, int(omp))
    t0 = time.perf_counter()
    oracle.layer_forward(X.reshape(spec.B, spec.n, -1), w, x.lmask, x.gmask, spec.window, spec.dilation,
                         spec.H, 1e-5, threads=threads)
    t = time.perf_counter() - t0
    return {"value": round(spec.B * spec.n / t, 3), "unit": "tokens/s", "cores": threads, "cpu_model": host_cpu_model(), "kind": "oracle",
            "sample": f"the whole layer once ({t:.2f} s; float64 numpy GEMMs, the attention oracle in C)"}


def run_layer(args, spec, x, lm, gm, plan):
    """--pass layer: one JSON line for lwattn_layer_forward (one encoder layer)."""
    import math
    import numpy as np
    import torch
    from long_document_sparse_amd import flops as fl
    from long_document_sparse_amd import lwattn, workloads
    inter = workloads.FTLAYER_INTER
    layer = lwattn.Layer(plan, inter, 1e-5)
    dev = lm.device
    rng = np.random.default_rng(spec.seed + 7)
    w_np = {}
    for name, shape in layer.shapes().items():
        if name.startswith("ln") and name.endswith("_g"):
            a = 1.0 + 0.1 * rng.standard_normal(shape)
        elif len(shape) == 2:
            a = rng.standard_normal(shape) / math.sqrt(shape[0])
        else:
            a = 0.1 * rng.standard_normal(shape)
        w_np[name] = a.astype(np.float32)
    tdt = lwattn.torch_dtype(spec.dtype)
    w = {k: torch.from_numpy(a).to(dev).to(tdt) for k, a in w_np.items()}
    hid = spec.H * spec.d
    X_np = rng.standard_normal((spec.B * spec.n, hid)).astype(np.float32)
    X = torch.from_numpy(X_np).to(dev).to(tdt)
    Y = torch.empty_like(X)
    layer.forward(X, w, lm, gm, out=Y)
    for _ in range(args.warmup):
        layer.forward(X, w, lm, gm, out=Y)
    st = plan.sync_status()
    if st != lwattn.OK:
        raise SystemExit(f"layer failed: {lwattn.strerror(st)}")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        layer.forward(X, w, lm, gm, out=Y)
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    t_call = e0.elapsed_time(e1) * 1e-3 / args.steps
    M = spec.B * spec.n
    # Q, K, V and Kg, Vg for every row, Qg for the global tokens' rows only
    # (the layer projects no other row of it), output projection, FFN
    n_glob = int(((x.lmask != 0) & (x.gmask != 0)).sum())
    gemm = (2 * M * hid * (3 * hid) + 2 * M * hid * (2 * hid) + 2 * n_glob * hid * hid
            + 2 * M * hid * hid + 2 * 2 * M * hid * inter)
    attn = fl.flops(x.lmask, x.gmask, spec.window, spec.dilation, spec.d)
    flop = gemm + attn
    achieved = flop / t_call / 1e12
    res = {
        "metric": "Longformer encoder layer tokens/s (one layer), n=4096 H=16 inter=4096 w=512",
        "value": round(M / (elapsed / args.steps), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded inputs and weights; no dataset, no trained weights)",
        "config": {"workload": describe(spec) + f"; encoder layer, hidden {hid}, intermediate {inter}",
                   "global_batch": spec.B, "seq_len": spec.n, "heads": spec.H, "head_dim": spec.d,
                   "window": spec.window, "parallelism": "single GPU", "timing": "warm (back to back)"},
        "us_per_layer_on_stream": round(t_call * 1e6, 2),
        "ms_for_24_layers": round(t_call * 24 * 1e3, 3),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_MFMA, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_MFMA, 4), "traffic": None,
                     "kernel": "whole layer (rocBLAS GEMMs and the library's kernels)",
                     "algorithmic_flop": flop, "gemm_flop": gemm, "attention_flop": attn,
                     "source_sha256": source_hash()},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_layer(x, X.float().cpu().numpy(),
                                                 {k: t.float().cpu().numpy() for k, t in w.items()}, inter)
    layer.close()
    plan.close()
    print(json.dumps(res), flush=True)


def run_backward(args, spec, x, ts, lm, gm, plan):
    """--pass backward: one JSON line for lwattn_backward."""
    import numpy as np
    import torch
    from long_document_sparse_amd import flops as fl
    from long_document_sparse_amd import lwattn
    dev = ts[0].device
    o = torch.empty_like(ts[0])
    plan(*ts, lm, gm, out=o)
    go_np = np.random.default_rng(spec.seed + 101).standard_normal(ts[0].shape).astype(np.float32)
    go = torch.from_numpy(go_np).to(dev).to(ts[0].dtype)
    grads = tuple(torch.empty_like(ts[0]) for _ in range(6))
    step = plan.bind_backward(*ts, lm, gm, o, go, grads)
    for _ in range(args.warmup):
        step()
    st = plan.sync_status()
    if st != lwattn.OK:
        raise SystemExit(f"backward failed: {lwattn.strerror(st)}")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if not args.no_timing:
        # per-kernel events recorded by the dispatches themselves, every
        # TIMING_EVERY-th backward of the timed loop
        plan.timing_enable(args.steps, every=TIMING_EVERY)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    st = plan.sync_status()
    if st != lwattn.OK:
        raise SystemExit(f"backward failed: {lwattn.strerror(st)}")
    t_call = e0.elapsed_time(e1) * 1e-3 / args.steps        # s per backward, on the stream
    flop = fl.backward_flops(x.lmask, x.gmask, spec.window, spec.dilation, spec.d)
    nbytes = fl.backward_bytes(x.lmask, x.gmask, spec.H, spec.d, 4 if spec.dtype == "f32" else 2)
    roofline = None
    if not args.no_timing:
        tot, calls = plan.timing_read_backward()
        plan.timing_disable()
        kflop = fl.backward_kernel_flops(x.lmask, x.gmask, spec.window, spec.dilation, spec.d)
        per = {k: v / max(calls, 1) * 1e-3 for k, v in tot.items()}     # s per launch
        dom = max(per, key=per.get)
        if spec.dtype != "f32":
            # the contractions run on the 16-bit matrix cores
            achieved = kflop[dom] / per[dom] / 1e12
            roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_MFMA,
                        "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_MFMA, 4), "traffic": None}
        else:
            # fp32 storage: the contractions run on the fp32 vector ALUs
            achieved = flop / t_call / 1e12
            roofline = {"bound": "alu", "achieved": round(achieved, 2), "peak": PEAK_FP32_VECTOR,
                        "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_VECTOR, 4), "traffic": None}
        roofline.update({"kernel": dom if spec.dtype != "f32" else "backward (all kernels)",
                         "algorithmic_flop": kflop[dom] if spec.dtype != "f32" else flop,
                         "kernel_us": {k: round(v * 1e6, 2) for k, v in per.items() if v > 0},
                         "timed_calls": calls, "source_sha256": source_hash()})
    tokens = spec.B * spec.n
    res = {
        "metric": METRIC_BWD,
        "value": round(tokens / (elapsed / args.steps), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded, N(0,1)/sqrt(d) inputs, N(0,1) dO; no dataset)",
        "config": {"workload": describe(spec) + "; backward", "global_batch": spec.B,
                   "seq_len": spec.n, "heads": spec.H, "head_dim": spec.d, "window": spec.window,
                   "parallelism": "single GPU", "timing": "warm (back to back)"},
        "tflops_per_s": round(flop / (elapsed / args.steps) / 1e12, 2),
        "algorithmic_flop": flop,
        "algorithmic_bytes": nbytes,
        "us_per_backward_on_stream": round(t_call * 1e6, 2),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_backward(x, go_np.astype(np.float32) if spec.dtype == "f32"
                                                    else go.float().cpu().numpy())
    plan.close()
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None,
                    help="named workload (default: base; charlm for --pass causal)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dtype", choices=("bf16", "f16", "f32"), default=None,
                    help="storage type in place of the workload's own (forward and layer passes)")
    ap.add_argument("--no-timing", action="store_true",
                    help="do not record per-kernel HIP events (roofline fields become null)")
    ap.add_argument("--pass", dest="which", choices=("forward", "backward", "causal", "causal_backward", "blocksparse", "layer"), default="forward",
                    help="time the forward (default) or the backward")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="forwards timed cold (1 GiB written between calls); 0 skips the cold mode")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the on-device peak probes (matrix-core loop, HBM read, copy)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="after timing, copy MIB MiB device to device 5 times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported here "
              "(the path would shard over (batch, head) pairs with no communication).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from long_document_sparse_amd import flops as fl
    from long_document_sparse_amd import lwattn, workloads

    if args.workload is None:
        args.workload = {"causal": "charlm", "causal_backward": "charlm", "blocksparse": "bsparse", "layer": "ftlayer"}.get(args.which, "base")
    spec = workloads.named(args.workload)
    if args.dtype is not None:
        if args.which == "causal_backward" and args.dtype == "f32":
            raise SystemExit("the causal variant runs on 16-bit storage (bf16 or f16)")
        import dataclasses
        spec = dataclasses.replace(spec, dtype=args.dtype)
    x = workloads.generate(spec)
    dev = torch.device("cuda", 0)
    tdt = lwattn.torch_dtype(spec.dtype)
    ts = [torch.from_numpy(a).to(dev).to(tdt) for a in x.tensors()]
    lm = torch.from_numpy(x.lmask).to(dev)
    gm = torch.from_numpy(x.gmask).to(dev)
    out = torch.empty_like(ts[0])
    plan = lwattn.Plan(spec.B, spec.H, spec.n, spec.d, spec.window, spec.dilation,
                       spec.max_global, spec.scale, spec.dtype)
    if args.which == "backward":
        run_backward(args, spec, x, ts, lm, gm, plan)
        return
    if args.which == "causal":
        run_causal(args, spec, x, ts, lm, plan)
        return
    if args.which == "causal_backward":
        run_causal_backward(args, spec, x, ts, lm, plan)
        return
    if args.which == "blocksparse":
        run_blocksparse(args, spec, x, ts, lm, plan)
        return
    if args.which == "layer":
        run_layer(args, spec, x, lm, gm, plan)
        return

    # the buffers are validated and the call marshalled once; every step
    # below is one lwattn_forward
    step = plan.bind(*ts, lm, gm, out=out)
    for _ in range(args.warmup):
        step()
    st = plan.sync_status()
    if st != lwattn.OK:
        raise SystemExit(f"forward failed: {lwattn.strerror(st)}")

    if not args.no_timing:
        # per-kernel events on every TIMING_EVERY-th forward of the timed loop
        plan.timing_enable(args.steps, every=TIMING_EVERY)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    st = plan.sync_status()
    if st != lwattn.OK:
        raise SystemExit(f"forward failed: {lwattn.strerror(st)}")

    if args.copy_probe > 0:
        src = torch.empty(args.copy_probe << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ms_step = elapsed * 1e3 / args.steps
    tokens = spec.B * spec.n
    value = tokens / (elapsed / args.steps)
    flop = fl.flops(x.lmask, x.gmask, spec.window, spec.dilation, spec.d)
    nbytes = fl.hbm_bytes(x.lmask, x.gmask, spec.H, spec.d, 4 if spec.dtype == "f32" else 2)
    peak = PEAK_TFLOPS[spec.dtype]

    roofline = None
    kernels = None
    tot, calls = plan.timing_read() if not args.no_timing else ({}, 0)
    plan.timing_disable()
    # cold mode and the on-device peaks, after the warm events are read
    cold = None
    if args.cold_steps > 0:
        t_cold = time_cold(step, plan, args.cold_steps, dev)
        st = plan.sync_status()
        if st != lwattn.OK:
            raise SystemExit(f"forward failed: {lwattn.strerror(st)}")
    peaks = None if args.no_peaks else measure_peaks(plan.lib, dev)
    if not args.no_timing:
        kernels = {k: round(v * 1e3 / calls, 3) for k, v in tot.items()}   # us per launch
        t_attn = tot["attention"] / calls * 1e-3                            # s per launch
        tflops = flop / t_attn / 1e12
        gbs = nbytes / t_attn / 1e9
        # the bound is the roof whose ideal time is longer at this arithmetic intensity
        hbm_bound = nbytes / (PEAK_HBM_GBS * 1e9) > flop / (peak * 1e12)
        tr = measured_traffic(spec.name, spec.dtype)
        traffic = tr["traffic_bytes"] if tr else None
        if hbm_bound:
            roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
        else:
            roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                        "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "traffic": traffic}
        if peaks:
            # the same achieved figure against what the probes measured on this GPU
            meas = peaks["hbm_read_gbs"] if hbm_bound else peaks["mfma_bf16_tflops"]
            if hbm_bound or spec.dtype != "f32":
                roofline["frac_of_measured_peak"] = round(roofline["achieved"] / meas, 4)
                roofline["measured_peak"] = meas
        roofline.update({
            "kernel": "attn_kernel",
            "algorithmic_flop": flop, "algorithmic_bytes": nbytes,
            "mfma_view": {"achieved_tflops": round(tflops, 2), "peak": peak,
                          "frac": round(tflops / peak, 4)},
            "hbm_view": {"achieved_gbs": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "frac": round(gbs / PEAK_HBM_GBS, 4)},
            "source_sha256": source_hash(),
        })

    if args.cold_steps > 0:
        cold = {"steps": args.cold_steps, "us_per_launch": round(t_cold * 1e6, 2),
                "tokens_per_s": round(tokens / t_cold, 1),
                "tflops": round(flop / t_cold / 1e12, 2), "mfma_frac": round(flop / t_cold / 1e12 / peak, 4),
                "hbm_gbs": round(nbytes / t_cold / 1e9, 1),
                "hbm_frac": round(nbytes / t_cold / 1e9 / PEAK_HBM_GBS, 4),
                "how": "1 GiB written between forwards (outside the timed kernel); kernel time from the "
                       "events its dispatch records, every forward"}
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded, N(0,1)/sqrt(d) inputs; no dataset)",
        "config": {"workload": describe(spec), "global_batch": spec.B, "seq_len": spec.n,
                   "heads": spec.H, "head_dim": spec.d, "window": spec.window,
                   "parallelism": "single GPU", "timing": "warm (back to back)"},
        "tflops_per_s": round(flop / (elapsed / args.steps) / 1e12, 2),
        "pct_mfma_peak": round(100 * flop / (elapsed / args.steps) / 1e12 / peak, 2),
        "kernel_us": kernels,
        "roofline": roofline,
        "cold": cold,
        "measured_peaks": peaks,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(x)
    plan.close()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
