"""Summaries of rocprofv3 output for the benchmark (no GPU needed).

    python -m tensor_scaled_fp8_amd.profiling stats DIR [--out FILE.md]
        per-kernel count / total / average duration from a
        `rocprofv3 --kernel-trace --stats --output-format csv` directory.
    python -m tensor_scaled_fp8_amd.profiling traffic --fetch DIR --write DIR
            --kernel SUBSTR --copy-bytes N [--command CMD] [--out FILE.json]
        HBM bytes per dispatch of the kernels whose name contains SUBSTR,
        from one `--pmc FETCH_SIZE` run and one `--pmc WRITE_SIZE` run of
        the same command. Each counter (KiB per dispatch) is scaled by what
        it reads for the plain device copy of N bytes that the benchmark
        performs (`bench.py --calibration-copy N`): factor = N / (KiB * 1024).
    python -m tensor_scaled_fp8_amd.profiling quant-traffic --fetch DIR --write DIR
            --copy-bytes N [--command CMD] [--out FILE.md]
        The same counters for the cast kernels (128 x 128 tiles of 256
        threads, so elements = work-items * 64) and the amax kernels, next
        to the algorithmic bytes (cast: 2 read + 1 per FP8 copy written;
        amax: 2 read).
    python -m tensor_scaled_fp8_amd.profiling mfma DIR [--command CMD] [--out FILE.md]
        Per GEMM dispatch shape, from one run with --pmc
        SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F8
        SQ_INSTS_VALU_MFMA_MOPS_F6F4 SQ_BUSY_CYCLES: the FP8 MFMA flops
        counted, the average shader clock over the dispatch, the MFMA busy
        fraction at that clock and the dense FP8 peak at that clock
        (256 CUs x 8192 flops per clock).
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
    """Kernel name without namespaces and parameter list; template arguments
    kept (they select formats, layouts and variants)."""
    for key in ("gemm_nt_kernel<", "gemm_pair_kernel<", "cast_kernel<"):
        if key in name:
            return name[name.index(key):].split(">")[0] + ">"
    base = name.replace("(anonymous namespace)::", "")
    if base.startswith("void "):
        base = base[5:]
    base = base.split("(")[0].split("<")[0]
    return base.split("::")[-1][:60]


def stats_markdown(d: str, title: str, command: str, dominant: str = "", flop_per_launch: float = 0.0,
                   peak_tflops: float = 5000.0) -> str:
    st = kernel_stats(d)
    tot = sum(v["total_us"] for v in st.values())
    lines = [f"# {title}", "", "Command:", "", "```", command, "```", "",
             "| kernel | calls | total us | avg us | share |", "|---|---:|---:|---:|---:|"]
    for k, v in sorted(st.items(), key=lambda kv: -kv[1]["total_us"]):
        lines.append(f"| `{_short(k)}` | {v['count']} | {v['total_us']:.1f} | {v['avg_us']:.2f} | "
                     f"{100 * v['total_us'] / tot:.1f}% |")
    if dominant and flop_per_launch:
        hits = [v for k, v in st.items() if dominant in k]
        if hits:
            calls = sum(v["count"] for v in hits)
            avg = sum(v["total_us"] for v in hits) / calls
            tf = flop_per_launch / (avg * 1e-6) / 1e12
            lines += ["", f"Roofline of the dominant kernel `{dominant}`: {flop_per_launch:.6g} algorithmic "
                      f"FLOP per launch (mean over the step's launches) / {avg:.2f} us average duration = "
                      f"{tf:.1f} TFLOP/s, {tf / peak_tflops:.4f} of {peak_tflops:.0f} TFLOP/s."]
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


def traffic(fetch_dir: str, write_dir: str, kernel: str, copy_bytes: int, workload: str = "") -> dict:
    out = {}
    for key, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        per = _pmc(d, counter)
        copies = [v for n, v in per.values() if "copyBuffer" in n]
        if not copies:
            raise RuntimeError(f"no copy dispatch in {d}")
        factor = copy_bytes / (max(copies) * 1024.0)
        vals = [v for n, v in per.values() if any(k in n for k in kernel.split(","))]
        if not vals:
            raise RuntimeError(f"no dispatch of {kernel} in {d}")
        out[f"{key}_kib_per_dispatch_raw"] = sum(vals) / len(vals)
        out[f"{key}_scale"] = factor
        out[f"{key}_bytes_per_dispatch"] = sum(vals) / len(vals) * 1024.0 * factor
        out[f"{key}_dispatches"] = len(vals)
    out["gemm_bytes_per_launch"] = out["fetch_bytes_per_dispatch"] + out["write_bytes_per_dispatch"]
    out["kernel"] = kernel
    out["workload"] = workload
    out["copy_bytes"] = copy_bytes
    out["gemm_code_sha256"] = gemm_code_sha256()
    return out


def gemm_code_sha256() -> str:
    """sha256 of csrc/gemm.hip with // comments and blank lines removed, so
    the stamp changes with the code and not with its comments."""
    import hashlib
    import re
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "gemm.hip")
    with open(src) as f:
        lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in f]
    return hashlib.sha256("\n".join(ln for ln in lines if ln).encode()).hexdigest()


def _pmc_rows(d: str) -> dict:
    """Dispatch id -> {"name", "grid", "ns", counter: summed value, ...}."""
    out = {}
    for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
        e = out.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"], "grid": int(r["Grid_Size"]),
                                                "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _copy_factor(rows: dict, counter: str, copy_bytes: int) -> float:
    copies = [e[counter] for e in rows.values() if "copyBuffer" in e["name"] and counter in e]
    if not copies:
        raise RuntimeError("no copy dispatch")
    return copy_bytes / (max(copies) * 1024.0)


def quant_traffic_markdown(fetch_dir: str, write_dir: str, copy_bytes: int, command: str,
                           layer: str = "GPT-175B-style layer") -> str:
    fe, wr = _pmc_rows(fetch_dir), _pmc_rows(write_dir)
    ff, wf = _copy_factor(fe, "FETCH_SIZE", copy_bytes), _copy_factor(wr, "WRITE_SIZE", copy_bytes)
    fk, wk = sorted(fe, key=int), sorted(wr, key=int)
    if len(fk) != len(wk):
        raise RuntimeError("the two runs dispatched different kernels")
    groups = defaultdict(list)
    pairs = list(zip(fk, wk))
    for i, (a, b) in enumerate(pairs):
        ea, eb = fe[a], wr[b]
        if ea["name"] != eb["name"]:
            raise RuntimeError("the two runs dispatched different kernels")
        name = ea["name"]
        fb, wb = ea["FETCH_SIZE"] * 1024 * ff, eb["WRITE_SIZE"] * 1024 * wf
        if "cast_kernel<" in name:
            tmpl = name[name.index("cast_kernel<"):].split(">")[0] + ">"
            groups[(tmpl, ea["grid"] * 64)].append((fb, wb))
        elif "cast_batch_kernel" in name:   # the tiles of all the batch's tensors
            groups[("cast_batch_kernel", ea["grid"] * 64)].append((fb, wb))
        elif "amax_gen_kernel" in name or "amax_batch_kernel" in name:
            # in fp8_quantize(_batch) the cast of the same tensors is the next dispatch
            key = "amax_gen_kernel" if "amax_gen_kernel" in name else "amax_batch_kernel"
            nxt = fe[pairs[i + 1][0]] if i + 1 < len(pairs) else None
            if nxt is not None and ("cast_kernel<" in nxt["name"] or "cast_batch_kernel" in nxt["name"]):
                groups[(key, nxt["grid"] * 64)].append((fb, wb))
            else:
                groups[(key, None)].append((fb, wb))
    lines = [f"# HBM traffic of the quantise kernels (amax and cast), {layer}", "",
             "Commands (FETCH_SIZE and WRITE_SIZE in separate runs; counters scaled by a plain "
             f"{copy_bytes}-byte device copy in the same run: fetch x{ff:.3f}, write x{wf:.3f}):", "",
             "```", command, "```", "",
             "Cast: elements = work-items x 64 (one 128 x 128 tile per 256 threads); algorithmic "
             "read 2 B/element, write 1 B per FP8 copy (2 copies when the transpose is written, "
             "template flags <fmt, derive, count>; cast_batch_kernel: all tensors of one "
             "fp8_quantize_batch call). amax: algorithmic read = 2 B/element. A write "
             "figure below the algorithmic one means lines were still dirty in the L2 when the "
             "dispatch ended; they reach HBM later, inside another dispatch's count.", "",
             "| kernel | elements | dispatches | HBM read MB | alg. read MB | read/alg | HBM write MB | "
             "write/elements (B) |", "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for (k, n), v in sorted(groups.items(), key=lambda kv: (kv[0][0], kv[0][1] or 0)):
        if k in ("amax_gen_kernel", "amax_batch_kernel") and n is None:
            continue  # not followed by a cast: size unknown from the counters alone
        f = sum(x[0] for x in v) / len(v)
        w = sum(x[1] for x in v) / len(v)
        lines.append(f"| `{k}` | {n} | {len(v)} | {f / 1e6:.1f} | {2 * n / 1e6:.1f} | {f / (2 * n):.3f} | "
                     f"{w / 1e6:.1f} | {w / n:.3f} |")
    return "\n".join(lines) + "\n"


def mfma_markdown(d: str, command: str, layer: str = "GPT-175B-style layer") -> str:
    rows = _pmc_rows(d)
    groups = defaultdict(list)
    for e in rows.values():
        key = next((k for k in ("gemm_nt_kernel<", "gemm_pair_kernel<") if k in e["name"]), None)
        if key is None:
            continue
        tmpl = e["name"][e["name"].index(key):].split(">")[0] + ">"
        groups[(tmpl, e["grid"] // 256)].append(e)
    lines = [f"# FP8 MFMA utilisation and shader clock of the GEMM kernel, {layer}", "",
             "Command:", "", "```", command, "```", "",
             "flops = 512 x (SQ_INSTS_VALU_MFMA_MOPS_F8 + SQ_INSTS_VALU_MFMA_MOPS_F6F4); MFMA cycles = "
             "SQ_VALU_MFMA_BUSY_CYCLES per SIMD (1024 SIMDs), which the hardware counts as 64 per "
             "32x32x64 and 32 per 16x16x128 FP8 MFMA (2048 flops per SIMD cycle either way), so it "
             "equals flops / (1024 x 2048) when no MFMA work is wasted; "
             "clock = SQ_BUSY_CYCLES per shader engine (32 of them) / dispatch duration (waves are "
             "present for the whole GEMM); MFMA busy = MFMA cycles / (clock x duration); peak at "
             "clock = 256 CUs x 8192 FP8 flops per clock x clock. Kernels run one at a time under "
             "counter collection.", "",
             "| kernel | tiles | dispatches | GFLOP | MFMA cycles / ideal | TFLOP/s | clock GHz | MFMA busy | "
             "peak at clock | of 5.0 PF |", "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for (k, tiles), v in sorted(groups.items()):
        n = len(v)
        busy = sum(e.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for e in v) / n / 1024
        fl = sum(512 * (e.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0) + e.get("SQ_INSTS_VALU_MFMA_MOPS_F6F4", 0.0))
                 for e in v) / n
        ns = sum(e["ns"] for e in v) / n
        se = sum(e.get("SQ_BUSY_CYCLES", 0.0) for e in v) / n / 32
        ghz = se / ns if se else float("nan")
        tf = fl / ns / 1e3
        peak = 256 * 8192 * ghz / 1e3
        ideal = fl / (1024 * 2048)
        lines.append(f"| `{k}` | {tiles} | {n} | {fl / 1e9:.1f} | {busy / ideal:.3f} | {tf:.0f} | {ghz:.3f} | "
                     f"{busy / (ghz * ns):.3f} | {peak:.0f} | {tf / 5000:.3f} |")
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("dir")
    a.add_argument("--title", default="rocprofv3 kernel statistics")
    a.add_argument("--command", default="")
    a.add_argument("--dominant", default="", help="kernel name part of the dominant kernel")
    a.add_argument("--flop-per-launch", type=float, default=0.0,
                   help="its algorithmic FLOP per launch (bench.py prints it as roofline.flop_per_launch)")
    a.add_argument("--out")
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--kernel", default="gemm_pair_kernel",
                   help="comma-separated kernel name parts; dispatches of any of them are averaged")
    b.add_argument("--workload", default="", help="workload name recorded with the figures")
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--command", default="")
    b.add_argument("--out")
    c = sub.add_parser("quant-traffic")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--command", default="")
    c.add_argument("--layer", default="GPT-175B-style layer")
    c.add_argument("--out")
    m = sub.add_parser("mfma")
    m.add_argument("dir")
    m.add_argument("--command", default="")
    m.add_argument("--layer", default="GPT-175B-style layer")
    m.add_argument("--out")
    args = ap.parse_args()
    if args.cmd == "stats":
        text = stats_markdown(args.dir, args.title, args.command, args.dominant, args.flop_per_launch)
    elif args.cmd == "quant-traffic":
        text = quant_traffic_markdown(args.fetch, args.write, args.copy_bytes, args.command, args.layer)
    elif args.cmd == "mfma":
        text = mfma_markdown(args.dir, args.command, args.layer)
    else:
        t = traffic(args.fetch, args.write, args.kernel, args.copy_bytes, args.workload)
        if args.command:
            t["command"] = args.command
        text = json.dumps(t, indent=1) + "\n"
    if getattr(args, "out", None):
        with open(args.out, "w") as f:
            f.write(text)
    print(text, end="")


if __name__ == "__main__":
    main()
