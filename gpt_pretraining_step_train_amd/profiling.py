"""Summaries of rocprofv3 output for the step's kernels.

python -m gpt_pretraining_step_train_amd.profiling stats TRACE_DIR STEPS "COMMAND" > summary.md
python -m gpt_pretraining_step_train_amd.profiling steps TRACE_DIR "COMMAND" > summary.md
python -m gpt_pretraining_step_train_amd.profiling traffic --kernel REGEX --fetch DIR --write DIR \
    --copy-fetch DIR --copy-write DIR --copy-bytes N --name NAME --command "..." > traffic.md

`stats` turns a `rocprofv3 --kernel-trace --stats` directory into a per-step
table (totals over every dispatch); `steps` does the same from the kernel trace with
the model's set-up kernels excluded.  `traffic` turns two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of a
program, and the same two counters over a plain device copy of known size, into
calibrated HBM bytes per launch of one kernel; the result block carries a hash
of the kernel sources so that `bench.py` reports it only while they are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
GEMM_SOURCES = ("csrc/gemm.hip", "csrc/common.h")
GEMM_ARGS = ("csrc/kernels.h", "struct GemmArgs {", "\n};\n")  # the GEMM's argument block only
BEGIN, END = "<!-- traffic-record", "-->"


def sources_hash(files=GEMM_SOURCES, args=GEMM_ARGS) -> str:
    """Hash of the GEMM kernel sources: its own files and the GemmArgs definition (the
    rest of kernels.h declares other kernels and does not change the GEMM)."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(PKG, f), "rb") as fh:
            h.update(fh.read())
    text = open(os.path.join(PKG, args[0])).read()
    i = text.index(args[1])
    h.update(text[i:text.index(args[2], i) + len(args[2])].encode())
    return h.hexdigest()[:16]


def _one(d: str, pattern: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no {pattern} under {d}")
    return hits[0]


def _short(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return n[: n.find("(")] if "(" in n else n


def stats_table(trace_dir: str, steps: int, command: str, top: int = 24) -> str:
    rows = list(csv.DictReader(open(_one(trace_dir, "*kernel_stats.csv"))))
    out = []
    total = 0.0
    for r in rows:
        t = float(r["TotalDurationNs"]) / 1e6 / steps
        total += t
        out.append((t, _short(r["Name"]), int(r["Calls"]) / steps, float(r["AverageNs"]) / 1e3))
    out.sort(reverse=True)
    lines = [f"Command: `{command}`", "",
             f"Kernel time per step (totals divided by {steps} step calls, warm-up included).", "",
             "| kernel | launches/step | avg us | ms/step | share |", "|---|---|---|---|---|"]
    for t, n, c, a in out[:top]:
        lines.append(f"| `{n}` | {c:.0f} | {a:.1f} | {t:.2f} | {100 * t / total:.1f}% |")
    lines.append(f"| (all kernels) | | | {total:.1f} | 100% |")
    return "\n".join(lines) + "\n"


# the first kernel of every gpt_step (the token-embedding gather) and its one-per-step
# kernel (the fused cross-entropy): the model's set-up kernels run before the first
STEP_FIRST = "embed_gather"
STEP_MARK = re.compile(r"::ce_(generic_|stream_)?kernel<")  # the cross-entropy kernel, once per step


def step_table(trace_dir: str, command: str, top: int = 28) -> str:
    """Per-step kernel time from a `--kernel-trace` CSV: only dispatches from the first
    step's first kernel on (gpt_init's weight fill, zeroing and casts excluded), divided
    by the number of steps (cross-entropy dispatches)."""
    rows = list(csv.DictReader(open(_one(trace_dir, "*kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    first = next(i for i, r in enumerate(rows) if STEP_FIRST in r["Kernel_Name"])
    rows = rows[first:]
    steps = sum(1 for r in rows if STEP_MARK.search(r["Kernel_Name"]))
    agg = {}
    for r in rows:
        n = _short(r["Kernel_Name"])
        t = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
        c, s_ = agg.get(n, (0, 0.0))
        agg[n] = (c + 1, s_ + t)
    total = sum(v[1] for v in agg.values()) / steps
    # the time some kernel is running (union of the dispatch intervals): kernels on the
    # backward's side stream overlap the main stream's, so the summed time can exceed it
    busy, end = 0, None
    for a, b in sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows):
        if end is None or a > end:
            busy += b - a
            end = b
        elif b > end:
            busy += b - end
            end = b
    out = sorted(((s_ / steps, n, c / steps, 1e3 * s_ / c) for n, (c, s_) in agg.items()), reverse=True)
    lines = [f"Command: `{command}`", "",
             f"Kernel time per step over {steps} steps (every dispatch from the first step's first kernel on;",
             "the model's set-up kernels excluded).  Some kernel is running "
             f"{busy / 1e6 / steps:.1f} ms per step (union of the dispatch intervals; the summed kernel time "
             "below can exceed it where the two streams of the backward overlap).", "",
             "| kernel | launches/step | avg us | ms/step | share |", "|---|---|---|---|---|"]
    for t, n, c, a in out[:top]:
        lines.append(f"| `{n}` | {c:.0f} | {a:.1f} | {t:.2f} | {100 * t / total:.1f}% |")
    lines.append(f"| (all kernels) | | | {total:.1f} | 100% |")
    return "\n".join(lines) + "\n"


def counter_mean(run_dir: str, counter: str, kernel_re: str):
    """Mean per-dispatch value of one counter over the dispatches whose kernel
    name matches kernel_re (summed over the counter's instances)."""
    per = {}
    for r in csv.DictReader(open(_one(run_dir, "*counter_collection.csv"))):
        if r["Counter_Name"] != counter or not re.search(kernel_re, r["Kernel_Name"]):
            continue
        per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise ValueError(f"no {counter} rows for {kernel_re} in {run_dir}")
    return sum(per.values()) / len(per), len(per)


def traffic_block(args) -> str:
    fetch, nf = counter_mean(args.fetch, "FETCH_SIZE", args.kernel)
    write, nw = counter_mean(args.write, "WRITE_SIZE", args.kernel)
    cf, _ = counter_mean(args.copy_fetch, "FETCH_SIZE", args.copy_kernel)
    cw, _ = counter_mean(args.copy_write, "WRITE_SIZE", args.copy_kernel)
    # the counters read KiB per dispatch; a copy of N bytes fetches and writes N bytes
    kf = args.copy_bytes / (cf * 1024.0)
    kw = args.copy_bytes / (cw * 1024.0)
    rec = {
        "name": args.name, "kernel_regex": args.kernel, "sources_sha": sources_hash(),
        "fetch_bytes_per_launch": fetch * 1024.0 * kf, "write_bytes_per_launch": write * 1024.0 * kw,
        "launches_fetch": nf, "launches_write": nw,
        "raw_fetch_kib": fetch, "raw_write_kib": write,
        "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_bytes": args.copy_bytes,
        "scale_fetch": kf, "scale_write": kw,
    }
    rec["bytes_per_launch"] = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    lines = [f"Command: `{args.command}`", "",
             f"HBM traffic of `{args.name}` per launch (mean over {nf} dispatches), from FETCH_SIZE and",
             "WRITE_SIZE (KiB per dispatch) scaled by the same counters over a plain device copy of",
             f"{args.copy_bytes / 2**20:.0f} MiB (fetch x{kf:.4f}, write x{kw:.4f}).", "",
             "| | raw KiB | calibrated MB |", "|---|---|---|",
             f"| fetch | {fetch:.0f} | {rec['fetch_bytes_per_launch'] / 1e6:.1f} |",
             f"| write | {write:.0f} | {rec['write_bytes_per_launch'] / 1e6:.1f} |",
             f"| total | | {rec['bytes_per_launch'] / 1e6:.1f} |", "",
             BEGIN, json.dumps(rec, indent=1), END, ""]
    return "\n".join(lines)


def read_traffic(path: str):
    """The traffic record of a summary file, or None when it is missing or the
    kernel sources have changed since the counters were taken."""
    try:
        text = open(path).read()
    except OSError:
        return None
    i, j = text.find(BEGIN), text.rfind(END)
    if i < 0 or j < i:
        return None
    rec = json.loads(text[i + len(BEGIN): j])
    return rec if rec.get("sources_sha") == sources_hash() else None


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("trace_dir")
    s.add_argument("steps", type=int)
    s.add_argument("command")
    q = sub.add_parser("steps")
    q.add_argument("trace_dir")
    q.add_argument("command")
    t = sub.add_parser("traffic")
    for k in ("--kernel", "--fetch", "--write", "--copy-fetch", "--copy-write", "--name", "--command"):
        t.add_argument(k, required=True)
    # the probe's torch.mul (the tensor fill before it reads nothing and must not count)
    t.add_argument("--copy-kernel", default="AUnaryFunctor")
    t.add_argument("--copy-bytes", type=float, required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        sys.stdout.write(stats_table(a.trace_dir, a.steps, a.command))
    elif a.cmd == "steps":
        sys.stdout.write(step_table(a.trace_dir, a.command))
    else:
        sys.stdout.write(traffic_block(a))
    return 0


if __name__ == "__main__":
    sys.exit(main())
