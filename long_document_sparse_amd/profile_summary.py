"""Summaries of rocprofv3 output for the attention path (kernel durations and
memory counters), printed as short text.

  python -m long_document_sparse_amd.profile_summary trace DIR
      per-kernel count / average / min / max duration from a --kernel-trace run
  python -m long_document_sparse_amd.profile_summary counters DIR [DIR ...]
      per-kernel average of every collected counter from --pmc runs
  python -m long_document_sparse_amd.profile_summary traffic FETCH_DIR WRITE_DIR WORKLOAD COPY_MIB
      HBM bytes per attention-kernel launch: FETCH_SIZE and WRITE_SIZE (KiB
      per dispatch) of attn_kernel, each scaled by the ratio between the bytes
      a device-to-device copy of COPY_MIB MiB must move and what the same
      counter reads for that copy; prints one JSON record

The rocprofv3 output is a SQLite database (its "kernels" view for the trace,
"counters_collection" for the counters).
"""
from __future__ import annotations

import collections
import glob
import hashlib
import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = ("long_document_sparse_amd/csrc/kernels.hpp",
                  "long_document_sparse_amd/csrc/lwattn.hip")


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _dbs(d):
    found = glob.glob(os.path.join(d, "**", "*.db"), recursive=True)
    if not found:
        raise SystemExit(f"no rocprofv3 database under {d}")
    return found


def _short(name: str) -> str:
    name = name.split("(")[0]
    return name[:60]


def trace(d):
    rows = []
    for db in _dbs(d):
        c = sqlite3.connect(db)
        q = ("select name, count(*), avg(end-start), min(end-start), max(end-start), "
             "sum(end-start) from kernels group by name order by sum(end-start) desc")
        rows += c.execute(q).fetchall()
    total = sum(r[5] for r in rows) or 1
    print(f"{'kernel':60s} {'calls':>6s} {'avg us':>9s} {'min us':>9s} {'max us':>9s} {'share':>6s}")
    for name, n, avg, mn, mx, tot in rows:
        print(f"{_short(name):60s} {n:6d} {avg / 1e3:9.2f} {mn / 1e3:9.2f} {mx / 1e3:9.2f} "
              f"{100 * tot / total:5.1f}%")


def counter_table(dirs):
    """{kernel: {counter: average value per dispatch}}"""
    out = collections.defaultdict(dict)
    for d in dirs:
        for db in _dbs(d):
            c = sqlite3.connect(db)
            try:
                rows = c.execute("select kernel_name, dispatch_id, counter_name, value "
                                 "from counters_collection").fetchall()
            except sqlite3.Error:
                rows = []
            if not rows:
                continue
            per = collections.defaultdict(float)
            names = {}
            for kname, disp, cname, v in rows:
                per[(disp, cname)] += v
                names[disp] = kname
            agg = collections.defaultdict(list)
            for (disp, cname), v in per.items():
                agg[(_short(names[disp]), cname)].append(v)
            for (k, cname), vs in agg.items():
                out[k][cname] = sum(vs) / len(vs)
    return out


def counters(dirs):
    tab = counter_table(dirs)
    for k, cs in sorted(tab.items()):
        print(k)
        for cname, v in sorted(cs.items()):
            print(f"    {cname:28s} {v:16.1f}")


def _dispatch_values(d, kernel_key, counter):
    vals = []
    for db in _dbs(d):
        c = sqlite3.connect(db)
        q = ("select kernel_name, dispatch_id, sum(value) from counters_collection "
             "where counter_name = ? group by dispatch_id")
        for kname, _, v in c.execute(q, (counter,)):
            if kernel_key in kname:
                vals.append(v)
    if not vals:
        raise SystemExit(f"no {counter} for a kernel matching {kernel_key!r} under {d}")
    return vals


def traffic(fetch_dir, write_dir, workload, copy_mib):
    copy_bytes = float(copy_mib) * (1 << 20)

    def mean(v):
        return sum(v) / len(v)

    def copy_reading(d, counter):
        # the copy probe's dispatches are the largest copyBuffer ones (smaller
        # copies of the run are host uploads)
        v = _dispatch_values(d, "copyBuffer", counter)
        top = max(v)
        return mean([x for x in v if x >= 0.5 * top])

    attn_f = mean(_dispatch_values(fetch_dir, "attn_kernel", "FETCH_SIZE"))
    attn_w = mean(_dispatch_values(write_dir, "attn_kernel", "WRITE_SIZE"))
    copy_f = copy_reading(fetch_dir, "FETCH_SIZE")
    copy_w = copy_reading(write_dir, "WRITE_SIZE")
    kf = copy_bytes / (copy_f * 1024.0)
    kw = copy_bytes / (copy_w * 1024.0)
    rec = {
        "kernel": "attn_kernel", "workload": workload, "source_sha256": source_hash(),
        "fetch_kib_per_dispatch": round(attn_f, 1), "write_kib_per_dispatch": round(attn_w, 1),
        "copy_mib": copy_mib, "copy_fetch_kib": round(copy_f, 1), "copy_write_kib": round(copy_w, 1),
        "fetch_scale": round(kf, 4), "write_scale": round(kw, 4),
        "traffic_bytes": int(round(attn_f * 1024.0 * kf + attn_w * 1024.0 * kw)),
    }
    print(json.dumps(rec))


def main(argv):
    if len(argv) < 2:
        raise SystemExit(__doc__)
    cmd = argv[1]
    if cmd == "trace":
        trace(argv[2])
    elif cmd == "counters":
        counters(argv[2:])
    elif cmd == "traffic":
        traffic(argv[2], argv[3], argv[4], int(argv[5]))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv)
