"""Summarise rocprofv3 runs of bench.py into a short text profile.

Three runs of the same bench.py arguments feed one summary:

  trace   rocprofv3 --kernel-trace --stats -d D/prof_trace_T -o run --output-format csv -- python bench.py ARGS
          (its stdout, with bench.py's JSON line, saved as D/prof_trace_T.log)
  fetch   rocprofv3 --pmc FETCH_SIZE -d D/prof_fetch_T -o run --output-format csv -- python bench.py ARGS
  write   rocprofv3 --pmc WRITE_SIZE -d D/prof_write_T -o run --output-format csv -- python bench.py ARGS

The summary gives the kernel's average launch duration from the trace, and
its HBM bytes per launch from the two counters (KiB per dispatch), each
scaled by what the same counter reads for the plain copy kernel of known size
that bench.py runs (torch's bitwise_not over int16). It records a hash of the
kernel's generated gfx950 code (build.device_code_sha), so that a reader can
tell when the profile is stale.

    python -m lossless_bf16_weight_afx_amd.profsum --kernel afx_decode_kernel \\
        --dir D --tag T --bench-args "--workload layer --steps 20 --warmup 3 --no-cpu-baseline"

A second mode, `profsum counters`, keeps the median per dispatch of any
counters (e.g. SQ instruction and LDS counters, two passes of 8) that
rocprofv3 --pmc runs recorded for one kernel.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def _pmc(path, kernel, stat=statistics.median):
    per = collections.defaultdict(list)
    for r in _rows(path):
        per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    mine = [k for k in per if kernel in k]
    copy = [k for k in per if "bitwise_not" in k]
    if not mine or not copy:
        raise SystemExit(f"{path}: no dispatches of {kernel} or of the copy kernel")
    return stat(sum((per[k] for k in mine), [])), statistics.median(sum((per[k] for k in copy), []))


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--kernel", required=True, help="kernel name (a substring of rocprofv3's kernel names)")
    ap.add_argument("--dir", required=True, help="directory that holds the three runs' outputs")
    ap.add_argument("--tag", required=True, help="suffix of the run directories")
    ap.add_argument("--bench-args", required=True, help="bench.py arguments of the trace run")
    ap.add_argument("--pmc-bench-args", default=None, help="bench.py arguments of the counter runs, if others")
    ap.add_argument("--stat", choices=["median", "mean"], default="median",
                    help="statistic of the kernel's counters over its dispatches: the median for launches of one "
                         "size, the mean for a pass of launches of different sizes (the whole model)")
    args = ap.parse_args(argv)
    stat = statistics.mean if args.stat == "mean" else statistics.median
    sys.path.insert(0, ROOT)
    import bench

    d, t, k = args.dir, args.tag, args.kernel
    stats = [r for r in _rows(os.path.join(d, f"prof_trace_{t}", "run_kernel_stats.csv")) if k in r["Name"]]
    if len(stats) != 1:
        raise SystemExit(f"expected one kernel named like {k} in the trace, found {len(stats)}")
    st = stats[0]
    trace = _rows(os.path.join(d, f"prof_trace_{t}", "run_kernel_trace.csv"))
    durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in trace if k in r["Kernel_Name"]]
    with open(os.path.join(d, f"prof_trace_{t}.log")) as f:
        line = [json.loads(s) for s in f if s.startswith('{"metric"')][0]
    roof = line["roofline"]
    alg = int(roof["algorithmic_bytes_per_launch"])
    copy_bytes = int(roof.get("calib_copy_bytes_each_way") or (alg // 4) * 2)
    f_k, f_c = _pmc(os.path.join(d, f"prof_fetch_{t}", "run_counter_collection.csv"), k, stat)
    w_k, w_c = _pmc(os.path.join(d, f"prof_write_{t}", "run_counter_collection.csv"), k, stat)
    fs, ws = copy_bytes / (f_c * 1024), copy_bytes / (w_c * 1024)
    rd, wr = f_k * 1024 * fs, w_k * 1024 * ws
    workload = line["config"]["workload"]
    pargs = args.pmc_bench_args or args.bench_args
    cmd_t = f"rocprofv3 --kernel-trace --stats -d {d}/prof_trace_{t} -o run --output-format csv -- python bench.py {args.bench_args}"
    cmd_f = f"rocprofv3 --pmc FETCH_SIZE -d {d}/prof_fetch_{t} -o run --output-format csv -- python bench.py {pargs}"
    cmd_w = cmd_f.replace("FETCH_SIZE", "WRITE_SIZE").replace("prof_fetch", "prof_write")
    avg = float(st["AverageNs"])
    txt = f"""# {k} on {workload}: rocprofv3 summary
# (MI355X, gfx950; run from the repository root, TMPDIR=/tmp)
#
# trace:  {cmd_t}
# fetch:  {cmd_f}
# write:  {cmd_w}
# summary: python -m lossless_bf16_weight_afx_amd.profsum --kernel {k} --dir {d} --tag {t} --bench-args "{args.bench_args}"{f' --pmc-bench-args "{args.pmc_bench_args}"' if args.pmc_bench_args else ''}{' --stat mean' if args.stat == 'mean' else ''}
#
# Kernel trace ({st['Calls']} dispatches of {k} in the run)
kernel = {k}
kernel_sha = {bench.kernel_sha(k)}
avg_duration_ns = {avg:.0f}
median_duration_ns = {statistics.median(durs):.0f}
min_duration_ns = {int(st['MinNs'])}
max_duration_ns = {int(st['MaxNs'])}
bench_ms_per_step = {line['ms_per_step']}
bench_kernel_ms = {roof.get('kernel_ms')}
#
# HBM bytes per dispatch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch, {args.stat} over the kernel's dispatches),
# each scaled by what the same counter reads for torch's elementwise
# bitwise_not over int16 (a plain copy kernel: {copy_bytes} B read, {copy_bytes} B written)
fetch_kib_raw = {f_k:.1f}
write_kib_raw = {w_k:.1f}
copy_fetch_kib_raw = {f_c:.1f}
copy_write_kib_raw = {w_c:.1f}
fetch_scale = {fs:.4f}
write_scale = {ws:.4f}
hbm_read_bytes_per_launch = {rd:.0f}
hbm_write_bytes_per_launch = {wr:.0f}
hbm_bytes_per_launch = {rd + wr:.0f}
algorithmic_bytes_per_launch = {alg}
traffic_over_algorithmic = {(rd + wr) / alg:.4f}
achieved_GBps_from_trace = {alg / avg:.1f}
"""
    out = os.path.join(ROOT, "profiles", f"{k}_{workload}_pmc.txt")
    with open(out, "w") as f:
        f.write(txt)
    print(txt)
    return 0


def counters_main(argv) -> int:
    """`counters` mode: the median per dispatch of every counter that
    rocprofv3 --pmc runs recorded for one kernel (several runs, e.g. two
    passes of 8 SQ counters), written to profiles/<kernel>_<workload>_<name>.txt."""
    ap = argparse.ArgumentParser(prog="profsum counters")
    ap.add_argument("--kernel", required=True)
    ap.add_argument("--workload", required=True, help="workload name for the file name and header")
    ap.add_argument("--name", default="sq", help="suffix of the summary's file name")
    ap.add_argument("--dirs", nargs="+", required=True, help="rocprofv3 -d directories of the runs")
    ap.add_argument("--commands", nargs="+", required=True, help="the rocprofv3 command of each run")
    args = ap.parse_args(argv)
    sys.path.insert(0, ROOT)
    import bench

    vals = {}
    for d in args.dirs:
        found = False
        for root, _, files in os.walk(d):
            for fn in files:
                if not fn.endswith("counter_collection.csv"):
                    continue
                found = True
                per = collections.defaultdict(list)
                for r in _rows(os.path.join(root, fn)):
                    if args.kernel in r["Kernel_Name"]:
                        per[r["Counter_Name"]].append(float(r["Counter_Value"]))
                for k, v in per.items():
                    vals[k] = statistics.median(v)
        if not found:
            raise SystemExit(f"{d}: no counter_collection.csv")
    lines = [f"# {args.kernel} on {args.workload}: rocprofv3 counters (median per dispatch)",
             "# (MI355X, gfx950; run from the repository root, TMPDIR=/tmp)", "#"]
    lines += [f"# run:  {c}" for c in args.commands]
    lines += [f"# summary: python -m lossless_bf16_weight_afx_amd.profsum counters --kernel {args.kernel} "
              f"--workload {args.workload} --name {args.name} --dirs ... --commands ...", "#",
              f"kernel = {args.kernel}", f"kernel_sha = {bench.kernel_sha(args.kernel)}"]
    lines += [f"{k} = {vals[k]:.6g}" for k in sorted(vals)]
    txt = "\n".join(lines) + "\n"
    with open(os.path.join(ROOT, "profiles", f"{args.kernel}_{args.workload}_{args.name}.txt"), "w") as f:
        f.write(txt)
    print(txt)
    return 0


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "counters":
        raise SystemExit(counters_main(sys.argv[2:]))
    raise SystemExit(main())
