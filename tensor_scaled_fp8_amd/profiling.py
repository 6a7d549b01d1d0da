"""Summaries of rocprofv3 output for the benchmark (no GPU needed).

    python -m tensor_scaled_fp8_amd.profiling stats DIR [--out FILE.md]
        per-kernel count / total / average duration from a
        `rocprofv3 --kernel-trace --stats --output-format csv` directory.
    python -m tensor_scaled_fp8_amd.profiling traffic --fetch DIR --write DIR
            --kernel SUBSTR --copy-bytes N [--out FILE.json]
        HBM bytes per dispatch of the kernels whose name contains SUBSTR,
        from one `--pmc FETCH_SIZE` run and one `--pmc WRITE_SIZE` run of
        the same command. Each counter (KiB per dispatch) is scaled by what
        it reads for the plain device copy of N bytes that the benchmark
        performs (`bench.py --calibration-copy N`): factor = N / (KiB * 1024).
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
from collections import defaultdict


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def kernel_stats(d: str) -> dict:
    rows = list(csv.DictReader(open(_find(d, "kernel_trace.csv"))))
    agg = defaultdict(lambda: [0, 0])
    for r in rows:
        dt = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        a = agg[r["Kernel_Name"]]
        a[0] += 1
        a[1] += dt
    return {k: {"count": c, "total_us": t / 1e3, "avg_us": t / 1e3 / c} for k, (c, t) in agg.items()}


def _short(name: str) -> str:
    for key in ("gemm_nt_kernel<0, 0>", "gemm_nt_kernel<1, 0>", "gemm_nt_kernel<0, 1>", "gemm_nt_kernel<1, 1>"):
        if key in name:
            return key
    for key in ("amax_finish_kernel", "amax_kernel", "cast_kernel<0>", "cast_kernel<1>", "scale_kernel",
                "copyBuffer"):
        if key in name:
            return key
    return name[:60]


def stats_markdown(d: str, title: str, command: str) -> str:
    st = kernel_stats(d)
    tot = sum(v["total_us"] for v in st.values())
    lines = [f"# {title}", "", "Command:", "", "```", command, "```", "",
             "| kernel | calls | total us | avg us | share |", "|---|---:|---:|---:|---:|"]
    for k, v in sorted(st.items(), key=lambda kv: -kv[1]["total_us"]):
        lines.append(f"| `{_short(k)}` | {v['count']} | {v['total_us']:.1f} | {v['avg_us']:.2f} | "
                     f"{100 * v['total_us'] / tot:.1f}% |")
    return "\n".join(lines) + "\n"


def _pmc(d: str, counter: str) -> dict:
    rows = list(csv.DictReader(open(_find(d, "counter_collection.csv"))))
    per = defaultdict(float)
    names = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        per[r["Dispatch_Id"]] += float(r["Counter_Value"])
        names[r["Dispatch_Id"]] = r["Kernel_Name"]
    return {k: (names[k], v) for k, v in per.items()}


def traffic(fetch_dir: str, write_dir: str, kernel: str, copy_bytes: int) -> dict:
    out = {}
    for key, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        per = _pmc(d, counter)
        copies = [v for n, v in per.values() if "copyBuffer" in n]
        if not copies:
            raise RuntimeError(f"no copy dispatch in {d}")
        factor = copy_bytes / (max(copies) * 1024.0)
        vals = [v for n, v in per.values() if kernel in n]
        if not vals:
            raise RuntimeError(f"no dispatch of {kernel} in {d}")
        out[f"{key}_kib_per_dispatch_raw"] = sum(vals) / len(vals)
        out[f"{key}_scale"] = factor
        out[f"{key}_bytes_per_dispatch"] = sum(vals) / len(vals) * 1024.0 * factor
        out[f"{key}_dispatches"] = len(vals)
    out["gemm_bytes_per_launch"] = out["fetch_bytes_per_dispatch"] + out["write_bytes_per_dispatch"]
    out["kernel"] = kernel
    out["copy_bytes"] = copy_bytes
    import hashlib
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "gemm.hip")
    with open(src, "rb") as f:
        out["gemm_source_sha256"] = hashlib.sha256(f.read()).hexdigest()
    return out


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("dir")
    a.add_argument("--title", default="rocprofv3 kernel statistics")
    a.add_argument("--command", default="")
    a.add_argument("--out")
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--kernel", default="gemm_nt_kernel")
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--out")
    args = ap.parse_args()
    if args.cmd == "stats":
        text = stats_markdown(args.dir, args.title, args.command)
    else:
        text = json.dumps(traffic(args.fetch, args.write, args.kernel, args.copy_bytes), indent=1) + "\n"
    if getattr(args, "out", None):
        with open(args.out, "w") as f:
            f.write(text)
    print(text, end="")


if __name__ == "__main__":
    main()
