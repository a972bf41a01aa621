"""Summaries of rocprofv3 output for the measurements the benchmark reports.

    python -m latent_mixture_experts_amd.profiling stats KERNEL_STATS_CSV TITLE COMMAND
        -> markdown table of the layer's kernels (average/min/max duration)

    python -m latent_mixture_experts_amd.profiling traffic --stage gateup \\
        --workload decode_t1 --kernel-regex 'stream_kernel<1, 1,' \\
        --fetch FETCH_CSV --write WRITE_CSV --copy-bytes N --alg-bytes A \\
        --source gemm_skinny.hip --command '...'
        -> profiles/traffic_<stage>_<workload>.json and .md

The traffic figures come from two counter runs (FETCH_SIZE, then WRITE_SIZE,
in KiB per dispatch). Each counter is scaled by what it reads for a plain
elementwise copy of known size in the same run (the copy reads N bytes and
writes N bytes), so that the result is in bytes. The JSON records the SHA-256
of the source files that decide the kernel's traffic (--source, comma
separated: the kernel's own, and for instance the grouping that orders its
work): the benchmark reports the figure only while they are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "latent_mixture_experts_amd", "csrc")


def _short(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "")
    cut = n.find("(moe::")
    if cut < 0:
        cut = n.find("(")
    return n[:cut] if cut > 0 else n


def stats_markdown(path: str, title: str, command: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = [f"# {title}", "", "Command (run from /tmp with TMPDIR=/tmp; $R is the repository root):",
           "", "```", command, "```", "",
           "rocprofv3 kernel statistics of the layer's kernels (input generation and "
           "other torch kernels of the run are omitted).", "",
           "| kernel | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
    for r in rows:
        if "moe::" not in r["Name"]:
            continue
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    return "\n".join(out) + "\n"


def _per_dispatch(path: str, counter: str, pattern: str) -> list[float]:
    rx = re.compile(pattern)
    vals = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter or not rx.search(r["Kernel_Name"]):
            continue
        key = r["Dispatch_Id"]
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return list(vals.values())


def sources_sha256(sources: str) -> str:
    """SHA-256 over the bytes of the comma-separated csrc files, in order."""
    h = hashlib.sha256()
    for name in sources.split(","):
        h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()


def traffic(args) -> dict:
    res = {}
    for counter, path in (("FETCH_SIZE", args.fetch), ("WRITE_SIZE", args.write)):
        kern = _per_dispatch(path, counter, args.kernel_regex)
        copy = _per_dispatch(path, counter, args.copy_regex)
        if not kern or not copy:
            raise SystemExit(f"{path}: no {counter} dispatches for the kernel or the copy")
        # the largest copy dispatches are the probe (torch may copy small tensors too)
        copy_kib = statistics.median(sorted(copy)[-3:])
        factor = args.copy_bytes / (copy_kib * 1024.0)
        res[counter] = dict(kernel_kib_median=statistics.median(kern), dispatches=len(kern),
                            copy_kib=copy_kib, factor=factor,
                            bytes_per_launch=statistics.median(kern) * 1024.0 * factor)
    total = res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"]
    digest = sources_sha256(args.source)
    rec = dict(stage=args.stage, workload=args.workload, kernel_regex=args.kernel_regex,
               source=args.source,
               source_sha256=digest,
               hbm_bytes_per_launch=int(round(total)),
               fetch_bytes_per_launch=int(round(res["FETCH_SIZE"]["bytes_per_launch"])),
               write_bytes_per_launch=int(round(res["WRITE_SIZE"]["bytes_per_launch"])),
               algorithmic_bytes_per_launch=args.alg_bytes,
               ratio_to_algorithmic=round(total / args.alg_bytes, 4) if args.alg_bytes else None,
               counters=res, copy_bytes=args.copy_bytes, command=args.command)
    return rec


def traffic_markdown(rec: dict) -> str:
    f, w = rec["counters"]["FETCH_SIZE"], rec["counters"]["WRITE_SIZE"]
    lines = [f"# HBM traffic of the {rec['stage']} kernel, workload {rec['workload']}", "",
             "Two rocprofv3 counter runs of the benchmark (one counter each); $R is the "
             "repository root, CTR is FETCH_SIZE in the first run and WRITE_SIZE in the second:",
             "", "```", rec["command"], "```", "",
             f"Kernel dispatches matched by `{rec['kernel_regex']}`; the calibration copy (copy_kernel of libmoe_peaks.so) is a plain copy "
             f"kernel that reads and writes {rec['copy_bytes']} bytes.", "",
             "| counter | kernel, median KiB per dispatch | dispatches | copy KiB | bytes per KiB read | bytes per launch |",
             "|---|---|---|---|---|---|",
             f"| FETCH_SIZE | {f['kernel_kib_median']:.0f} | {f['dispatches']} | {f['copy_kib']:.0f} | "
             f"{f['factor'] * 1024:.1f} | {f['bytes_per_launch']:.4g} |",
             f"| WRITE_SIZE | {w['kernel_kib_median']:.0f} | {w['dispatches']} | {w['copy_kib']:.0f} | "
             f"{w['factor'] * 1024:.1f} | {w['bytes_per_launch']:.4g} |", "",
             f"Total {rec['hbm_bytes_per_launch']:.4g} B per launch against "
             f"{rec['algorithmic_bytes_per_launch']:.4g} algorithmic bytes "
             f"(ratio {rec['ratio_to_algorithmic']}).",
             f"Sources `{rec['source']}` (comma separated), SHA-256 of their bytes in that order "
             f"`{rec['source_sha256']}`.", ""]
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("title")
    s.add_argument("command")
    t = sub.add_parser("traffic")
    t.add_argument("--stage", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--kernel-regex", required=True)
    t.add_argument("--copy-regex", default="copy_kernel")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--alg-bytes", type=int, required=True)
    t.add_argument("--source", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args()
    if a.cmd == "stats":
        print(stats_markdown(a.csv, a.title, a.command), end="")
        return
    rec = traffic(a)
    base = os.path.join(a.out_dir, f"traffic_{a.stage}_{a.workload}")
    with open(base + ".json", "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    with open(base + ".md", "w") as fh:
        fh.write(traffic_markdown(rec))
    print(json.dumps({k: rec[k] for k in ("hbm_bytes_per_launch", "algorithmic_bytes_per_launch",
                                          "ratio_to_algorithmic")}))


if __name__ == "__main__":
    main()
