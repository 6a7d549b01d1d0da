#!/usr/bin/env python3
"""Benchmark: one per-tensor dynamically scaled FP8 transformer layer's
linears, forward + backward, on one MI355X.

A step runs, for every linear of the layer (default: the GPT-7B-style
layer, 4096 tokens, hidden 4096: qkv 4096->12288, proj 4096->4096,
up 4096->16384, down 16384->4096):
    amax+scale(X), amax+scale(W)        (E4M3)
    cast+transpose(X), cast+transpose(W)
    Y  = FP8 GEMM (x8, w8t)
    amax+scale(dY)                       (E5M2)
    cast+transpose(dY)
    dX = FP8 GEMM (dy8, w8),  dW = FP8 GEMM (x8t, dy8t)
through the C ABI of libfp8lin.so, with inputs resident in HBM.

Prints ONE JSON line: value = sum over linears of 6*M*K*N / step time
(TFLOP/s). HIP events around every kernel launch of the timed steps give
the per-kernel durations; `roofline` reports the FP8 GEMM kernel (the
dominant one) against the dense FP8 MFMA peak, and `kernels` the amax and
cast kernels against HBM bandwidth. `cpu_baseline` times the oracle on a
bounded token sample of the same layer on the host cores."""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "FP8 linear fwd+bwd TFLOP/s and % of FP8 MFMA peak; amax+cast GB/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2, help="layer workload index (1-5)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=512, help="token rows of the CPU oracle sample")
    ap.add_argument("--cpu-cols", type=int, default=6144, help="output features of the CPU oracle sample")
    ap.add_argument("--check", action="store_true", help="check sampled outputs against the oracle")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "gemm_traffic_gpt7b-layer.json"),
                    help="JSON file with measured per-launch HBM bytes of the GEMM kernel")
    ap.add_argument("--calibration-copy", type=int, default=0,
                    help="bytes of one plain device copy run before timing (PMC calibration)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import tensor_scaled_fp8_amd as tsf
    from workloads import linear_inputs, workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tsf.load()
    wl = workload(args.workload)

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    lin = []
    t_gen = time.perf_counter()
    for li, L in enumerate(wl.linears):
        X, W, dY = linear_inputs(wl, li)
        d = dict(L=L, X=up(X), W=up(W), dY=up(dY))
        del X, W, dY
        d["ws"] = tsf.LinearWorkspace(L.M, L.K, L.N, dev)
        d["Y"] = torch.empty((L.M, L.N), dtype=torch.bfloat16, device=dev)
        d["dX"] = torch.empty((L.M, L.K), dtype=torch.bfloat16, device=dev)
        d["dW"] = torch.empty((L.K, L.N), dtype=torch.bfloat16, device=dev)
        lin.append(d)
    t_gen = time.perf_counter() - t_gen
    margin, mu = wl.margin, wl.mu_log2

    # kernel-level step: the same launches fp8_linear_fwd/bwd make, with an
    # event pair around each so per-kernel durations come from the timed run
    events = []

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def step(record: bool):
        for d in lin:
            L, ws = d["L"], d["ws"]
            seq = [
                ("amax", 2 * L.M * L.K, 0, lambda: tsf.fp8_amax_scale(d["X"], "e4m3", ws.sx, margin)),
                ("amax", 2 * L.K * L.N, 0, lambda: tsf.fp8_amax_scale(d["W"], "e4m3", ws.sw, margin)),
                ("cast", 4 * L.M * L.K, 0, lambda: tsf.fp8_cast(d["X"], "e4m3", ws.sx, ws.x8, ws.x8t)),
                ("cast", 4 * L.K * L.N, 0, lambda: tsf.fp8_cast(d["W"], "e4m3", ws.sw, ws.w8, ws.w8t)),
                ("gemm", 0, 2 * L.M * L.N * L.K,
                 lambda: tsf.fp8_gemm_nt(ws.x8, "e4m3", ws.sx, ws.w8t, "e4m3", ws.sw, d["Y"])),
                ("amax", 2 * L.M * L.N, 0,
                 lambda: tsf.fp8_amax_scale(d["dY"], "e5m2", ws.sdy, margin, mu)),
                ("cast", 4 * L.M * L.N, 0, lambda: tsf.fp8_cast(d["dY"], "e5m2", ws.sdy, ws.dy8, ws.dy8t)),
                ("gemm", 0, 2 * L.M * L.K * L.N,
                 lambda: tsf.fp8_gemm_nt(ws.dy8, "e5m2", ws.sdy, ws.w8, "e4m3", ws.sw, d["dX"])),
                ("gemm", 0, 2 * L.K * L.N * L.M,
                 lambda: tsf.fp8_gemm_nt(ws.x8t, "e4m3", ws.sx, ws.dy8t, "e5m2", ws.sdy, d["dW"])),
            ]
            for kind, nbytes, flops, fn in seq:
                if record:
                    e0 = ev()
                    fn()
                    events.append((kind, nbytes, flops, e0, ev()))
                else:
                    fn()

    if args.calibration_copy:
        n = args.calibration_copy
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    flops = wl.flops_fwd_bwd()
    value = flops / (ms * 1e-3) / 1e12

    agg = {}
    for kind, nbytes, fl, e0, e1 in events:
        a = agg.setdefault(kind, {"ms": 0.0, "bytes": 0, "flops": 0, "n": 0})
        a["ms"] += e0.elapsed_time(e1)
        a["bytes"] += nbytes
        a["flops"] += fl
        a["n"] += 1
    g = agg["gemm"]
    gemm_tflops = g["flops"] / (g["ms"] * 1e-3) / 1e12
    traffic = gemm_traffic(args.traffic)
    roofline = {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4), "traffic": traffic,
                "kernel": "gemm_nt_kernel (FP8 MFMA)",
                "avg_launch_us": round(g["ms"] * 1e3 / g["n"], 2)}
    kernels = {}
    for kind in ("amax", "cast"):
        a = agg[kind]
        gbs = a["bytes"] / (a["ms"] * 1e-3) / 1e9
        kernels[kind] = {"GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                         "ms_per_step": round(a["ms"] / args.steps, 4),
                         "avg_launch_us": round(a["ms"] * 1e3 / a["n"], 2)}
    qa = agg["amax"]["bytes"] + agg["cast"]["bytes"]
    qms = agg["amax"]["ms"] + agg["cast"]["ms"]
    kernels["amax+cast"] = {"GB/s": round(qa / (qms * 1e-3) / 1e9, 1),
                            "frac_hbm": round(qa / (qms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    kernels["gemm"] = {"TFLOP/s": round(gemm_tflops, 1), "ms_per_step": round(g["ms"] / args.steps, 4)}

    check = None
    if args.check:
        check = sampled_check(lin, wl, margin, mu)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_rows, args.cpu_cols)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 (E4M3 X/W, E5M2 dY; fp32 accumulate; bf16 in/out)", "data": "synthetic",
        "config": {"workload": wl.name, "tokens": wl.linears[0].M,
                   "linears": {L.name: [L.M, L.K, L.N] for L in wl.linears},
                   "margin": margin, "mu_log2": mu, "flops_per_step": flops,
                   "quant_bytes_per_step": wl.quant_bytes()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "frac_fp8_peak_step": round(value / PEAK_FP8_TFLOPS, 4),
        "input_gen_s": round(t_gen, 1),
    }
    if check is not None:
        out["check"] = check
    print(json.dumps(out), flush=True)


def gemm_traffic(path):
    """Measured HBM bytes per GEMM launch from a committed counter summary,
    reported only while the GEMM source is the one the counters were taken
    on (sha256 of gemm.hip recorded in the summary)."""
    import hashlib
    if not path or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    src = os.path.join(ROOT, "tensor_scaled_fp8_amd", "csrc", "gemm.hip")
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if rec.get("gemm_source_sha256") != sha:
        return None
    return round(rec["gemm_bytes_per_launch"])


def sampled_check(lin, wl, margin, mu):
    """Bit-exact scale records + sampled GEMM outputs against the oracle."""
    import numpy as np
    import oracle
    import tensor_scaled_fp8_amd as tsf
    from workloads import linear_inputs
    bad = 0
    g = np.random.Generator(np.random.PCG64(0))
    for li, d in enumerate(lin):
        L, ws = d["L"], d["ws"]
        X, W, dY = linear_inputs(wl, li)
        for key, bits, fmt, mm in (("sx", X, oracle.E4M3, 0), ("sw", W, oracle.E4M3, 0),
                                   ("sdy", dY, oracle.E5M2, mu)):
            r = tsf.read_scale(getattr(ws, key))
            ref = oracle.scale_record(bits, fmt, margin, mm)
            bad += int((r["bias"], r["flags"]) != (ref["bias"], ref["flags"]))
        sx, sw, sdy = (tsf.read_scale(s)["bias"] for s in (ws.sx, ws.sw, ws.sdy))
        x8, _ = oracle.cast(X, oracle.E4M3, sx)
        w8, w8t = oracle.cast(W, oracle.E4M3, sw)
        dy8, _ = oracle.cast(dY, oracle.E5M2, sdy)
        for name, A, fa, ba, B, fb, bb, out in (
                ("Y", x8, oracle.E4M3, sx, w8t, oracle.E4M3, sw, d["Y"]),
                ("dX", dy8, oracle.E5M2, sdy, w8, oracle.E4M3, sw, d["dX"]),
                ("dW", x8.T, oracle.E4M3, sx, dy8.T, oracle.E5M2, sdy, d["dW"])):
            M, N = out.shape
            rows, cols = g.integers(0, M, 64), g.integers(0, N, 64)
            rb, r64, tol = oracle.gemm_nt_rows(A, fa, ba, B, fb, bb, rows, cols)
            got = out.cpu().view(__import__("torch").int16).numpy().view(np.uint16)[rows, cols]
            err = np.abs(oracle.bf16_to_f64(got) - oracle.bf16_to_f64(rb))
            bad += int(np.count_nonzero(~(err <= tol)))
    return {"mismatches": bad}


def cpu_baseline(wl, rows, cols):
    """The oracle, as it stands, on a bounded sample of the same layer: the
    first `rows` tokens and the first `cols` output features of every
    linear (X [rows, K], W [K, cols], dY [rows, cols]): amax, bias, cast,
    three fp64 GEMMs."""
    import numpy as np
    import oracle
    from workloads import linear_inputs
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    flops = 0
    t = 0.0
    for li, L in enumerate(wl.linears):
        X, W, dY = linear_inputs(wl, li, rows_x=rows)
        n = min(cols, L.N)
        W = np.ascontiguousarray(W[:, :n])
        dY = np.ascontiguousarray(dY[:, :n])
        t0 = time.perf_counter()
        oracle.linear_fwd_bwd(X, W, dY, wl.margin, wl.mu_log2, with_tolerance=False)
        t += time.perf_counter() - t0
        flops += 6 * X.shape[0] * L.K * n
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{wl.name}: first {rows} tokens x first {cols} output features of each "
                      f"linear, fwd+bwd "
                      f"({flops / 1e9:.1f} GFLOP) in {t:.1f} s; BLAS threads = cores, "
                      "elementwise numpy steps single-threaded"}


if __name__ == "__main__":
    main()
