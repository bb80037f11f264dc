"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

  python -m transformer_megakernel_amd.profile_summary stats DIR OUT.txt -- CMD...
      kernel-trace statistics (rocprofv3 --kernel-trace --stats --output-format csv -d DIR)

  python -m transformer_megakernel_amd.profile_summary traffic WORKLOAD KERNEL \\
      FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR COPY_BYTES OUT.json -- CMD...
      HBM bytes per launch of KERNEL from one FETCH_SIZE and one WRITE_SIZE run, each scaled
      by what the same counter read for an elementwise copy of COPY_BYTES bytes.

  python -m transformer_megakernel_amd.profile_summary per_op DIR OUT.json -- CMD...
      from a kernel trace (rocprofv3 --kernel-trace --output-format csv -d DIR) of
      bench.py --per-op-baseline: the kernels of one replayed per-operation step (those
      between two launches of the marker kernel), their count, busy time and the gaps
      between consecutive kernels -- the article's launch cost and memory-pipeline
      bubbles (Megakernel article, section "Why are traditional inference methods so
      inefficient?").

The traffic file records a hash of the kernel sources; bench.py reports the figure only
while the sources are unchanged.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[-1]


def _rows(path: str):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def counter_per_dispatch(d: str, counter: str) -> dict:
    """{kernel name: [value per dispatch]} of one counter (summed over instances)."""
    per = defaultdict(float)
    names = {}
    for r in _rows(_find(d, "counter_collection.csv")):
        if r.get("Counter_Name") != counter:
            continue
        key = r["Dispatch_Id"]
        per[key] += float(r["Counter_Value"])
        names[key] = r["Kernel_Name"]
    out = defaultdict(list)
    for k in sorted(per, key=int):
        out[names[k]].append(per[k])
    return out


def _pick(per: dict, pattern: str) -> list:
    for name, vals in per.items():
        if pattern in name:
            return vals
    raise SystemExit(f"no kernel matching {pattern!r} in {sorted(per)}")


def cmd_stats(d: str, out: str, cmd: str) -> None:
    rows = _rows(_find(d, "kernel_stats.csv"))
    lines = [f"# rocprofv3 kernel-trace statistics", f"# command: {cmd}", "",
             f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    for r in rows:
        name = r["Name"][:60]
        lines.append(f"{name:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                     f"{float(r['Percentage']):6.2f}")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_traffic(workload, kernel, fdir, wdir, cfdir, cwdir, copy_bytes, out, cmd) -> None:
    copy_bytes = int(copy_bytes)
    kf = _pick(counter_per_dispatch(fdir, "FETCH_SIZE"), kernel)
    kw = _pick(counter_per_dispatch(wdir, "WRITE_SIZE"), kernel)
    cf = _pick(counter_per_dispatch(cfdir, "FETCH_SIZE"), "neg_kernel")
    cw = _pick(counter_per_dispatch(cwdir, "WRITE_SIZE"), "neg_kernel")
    # counters are KiB per dispatch; the first dispatch of each run is a cold warm-up
    med = lambda v: sorted(v)[len(v) // 2]
    fetch_scale = copy_bytes / (med(cf) * 1024.0)
    write_scale = copy_bytes / (med(cw) * 1024.0)
    fetch = med(kf[1:] if len(kf) > 1 else kf) * 1024.0 * fetch_scale
    write = med(kw[1:] if len(kw) > 1 else kw) * 1024.0 * write_scale
    res = dict(workload=workload, kernel=kernel, kernel_source_hash=kernel_source_hash(),
               fetch_bytes_per_launch=round(fetch), write_bytes_per_launch=round(write),
               hbm_bytes_per_launch=round(fetch + write),
               copy_calibration=dict(bytes=copy_bytes, fetch_kib=med(cf), write_kib=med(cw),
                                     fetch_scale=round(fetch_scale, 4), write_scale=round(write_scale, 4)),
               raw_kib_per_dispatch=dict(fetch=kf, write=kw), command=cmd)
    json.dump(res, open(out, "w"), indent=1)
    print(json.dumps(res, indent=1))


def cmd_per_op(d: str, out: str, cmd: str, marker: str = "stream_read_kernel") -> None:
    rows = _rows(_find(d, "kernel_trace.csv"))
    ks = sorted(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]) for r in rows))
    marks = [i for i, k in enumerate(ks) if marker in k[2]]
    steps = []
    for a, b in zip(marks, marks[1:]):
        seg = ks[a + 1:b]
        if not seg:
            continue
        busy = sum(e - s0 for s0, e, _ in seg)
        gaps = [seg[j + 1][0] - seg[j][1] for j in range(len(seg) - 1)]
        steps.append(dict(kernels=len(seg), span_us=(seg[-1][1] - seg[0][0]) / 1e3, busy_us=busy / 1e3,
                          mean_gap_us=(sum(gaps) / len(gaps) / 1e3) if gaps else 0.0,
                          max_gap_us=(max(gaps) / 1e3) if gaps else 0.0,
                          mean_kernel_us=busy / len(seg) / 1e3))
    if not steps:
        raise SystemExit("no marked steps in the kernel trace")
    med = lambda key: sorted(x[key] for x in steps)[len(steps) // 2]
    res = dict(steps_traced=len(steps), kernels_per_step=med("kernels"), step_span_us=round(med("span_us"), 1),
               kernel_busy_us=round(med("busy_us"), 1), mean_kernel_us=round(med("mean_kernel_us"), 2),
               mean_gap_between_kernels_us=round(med("mean_gap_us"), 3),
               max_gap_between_kernels_us=round(med("max_gap_us"), 3),
               idle_fraction=round(1 - med("busy_us") / med("span_us"), 4), per_step=steps, command=cmd)
    json.dump(res, open(out, "w"), indent=1)
    print(json.dumps({k: v for k, v in res.items() if k != "per_step"}, indent=1))


def main(argv):
    if "--" in argv:
        i = argv.index("--")
        args, cmd = argv[:i], " ".join(argv[i + 1:])
    else:
        args, cmd = argv, ""
    if args and args[0] == "stats" and len(args) == 3:
        cmd_stats(args[1], args[2], cmd)
    elif args and args[0] == "traffic" and len(args) == 9:
        cmd_traffic(*args[1:], cmd=cmd)
    elif args and args[0] == "per_op" and len(args) == 3:
        cmd_per_op(args[1], args[2], cmd)
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
