#!/usr/bin/env python3
"""Benchmark: one per-tensor dynamically scaled FP8 transformer layer's
linears, forward + backward, on one MI355X.

A step runs, for every linear of the layer (default: the GPT-175B-style
layer at full width, 2048 tokens, hidden 12288: qkv 12288->36864,
proj 12288->12288, up 12288->49152, down 49152->12288, the largest of the
layer workloads):
    quantize(X), quantize(W)   amax + scale + cast to row-major FP8 (E4M3),
                               both tensors in one launch pair (fp8_quantize_batch)
    Y  = FP8 GEMM (x8, w8 read reduction-major; a last wave at most half
         full is split into reduction halves over the workspace)
    quantize(dY)               (E5M2)
    dX = FP8 GEMM (dy8, w8) and dW = FP8 GEMM (x8, dy8 both read
    reduction-major), both in one launch (fp8_gemm_pair)
through the C ABI of libfp8lin.so (the launches fp8_linear_fwd/bwd make),
with inputs resident in HBM.

Prints ONE JSON line: value = sum over linears of 6*M*K*N / step time
(TFLOP/s). HIP events (fence-free) around every GEMM launch of the timed
steps give the GEMM durations: `roofline` reports the dominant kernel, the
backward pair (gemm_pair_kernel: a linear's dgrad + wgrad in one launch),
against the dense FP8 MFMA peak; `kernels.gemm` has all GEMM launches and
the forward kernel. A short extra pass with events around every launch
gives the amax and cast figures (`kernels`, against HBM bandwidth).
`other_workloads` repeats the step, GEMM and amax+cast figures on the
GPT-7B-style layer. `cpu_baseline` times the oracle on a bounded sample of
the same layer on the host cores."""
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
    ap.add_argument("--workload", type=int, default=4,
                    help="layer workload index (1-5); default 4, the GPT-175B-style layer (the largest)")
    ap.add_argument("--side-workloads", default="2",
                    help="comma-separated workloads also measured (step, GEMM and amax+cast) under "
                         "'other_workloads'; empty for none")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=512, help="token rows of the CPU oracle sample")
    ap.add_argument("--cpu-cols", type=int, default=3072, help="output features of the CPU oracle sample")
    ap.add_argument("--check", action="store_true", help="check sampled outputs against the oracle")
    ap.add_argument("--breakdown-steps", type=int, default=5,
                    help="extra steps with events around every launch (amax/cast figures)")
    ap.add_argument("--traffic-dir", default=os.path.join(ROOT, "profiles"),
                    help="directory of gemm_traffic_<workload>.json counter summaries")
    ap.add_argument("--calibration-copy", type=int, default=0,
                    help="bytes of one plain device copy run before timing (PMC calibration)")
    ap.add_argument("--step-only", action="store_true",
                    help="only the warm-up and timed steps (for profiler runs): no breakdown, side "
                         "workloads, inference, FP8 weight-gradient, Adam or cold-cache passes")
    return ap.parse_args()


DOMINANT = "gemm_pair_kernel"   # dgrad + wgrad in one launch: the kernel with the largest share of the step


class Layer:
    """Device tensors of one layer workload and its step (the launches
    fp8_linear_fwd / fp8_linear_bwd make, through the primitive entry
    points), with HIP events around the GEMM launches (or every launch)."""

    def __init__(self, tsf, torch, np, wl, dev, hip, cpu_rows=0, cpu_cols=0):
        from workloads import linear_inputs
        self.tsf, self.torch, self.wl, self.hip = tsf, torch, wl, hip
        self.margin, self.mu = wl.margin, wl.mu_log2
        self.events = []
        self.sample = []   # host slices for the CPU oracle sample

        def up(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

        self.lin = []
        t = time.perf_counter()
        for li, L in enumerate(wl.linears):
            X, W, dY = linear_inputs(wl, li)
            if cpu_rows:
                n = min(cpu_cols, L.N)
                self.sample.append((np.ascontiguousarray(X[:cpu_rows]), np.ascontiguousarray(W[:, :n]),
                                    np.ascontiguousarray(dY[:cpu_rows, :n])))
            d = dict(L=L, X=up(X), W=up(W), dY=up(dY))
            del X, W, dY
            d["ws"] = tsf.LinearWorkspace(L.M, L.K, L.N, dev)
            d["Y"] = torch.empty((L.M, L.N), dtype=torch.bfloat16, device=dev)
            d["dX"] = torch.empty((L.M, L.K), dtype=torch.bfloat16, device=dev)
            d["dW"] = torch.empty((L.K, L.N), dtype=torch.bfloat16, device=dev)
            self.lin.append(d)
        self.gen_s = time.perf_counter() - t

    def step(self, instrument, spec=False):
        """instrument: None, "gemm" (events around the GEMM launches) or "all".
        spec: quantise X, W and dY with fp8_quantize_spec (one pass with the
        bias the record kept, a recast only if it changed) instead."""
        tsf, margin, mu, hip = self.tsf, self.margin, self.mu, self.hip
        for d in self.lin:
            L, ws = d["L"], d["ws"]
            n = L.name
            # amax + cast to the row-major FP8 copy (2 B read twice, 1 B written);
            # the GEMMs read those copies, reduction-major where needed
            if spec:
                qxw = lambda: (tsf.fp8_quantize_spec(d["X"], "e4m3", ws.sx, margin, 0, ws.x8),
                               tsf.fp8_quantize_spec(d["W"], "e4m3", ws.sw, margin, 0, ws.w8))
                qdy = lambda: tsf.fp8_quantize_spec(d["dY"], "e5m2", ws.sdy, margin, mu, ws.dy8)
            else:
                qxw = lambda: tsf.fp8_quantize_batch([
                    dict(x=d["X"], fmt="e4m3", s=ws.sx, margin=margin, out_row=ws.x8, transposed=False),
                    dict(x=d["W"], fmt="e4m3", s=ws.sw, margin=margin, out_row=ws.w8, transposed=False)])
                qdy = lambda: tsf.fp8_quantize(d["dY"], "e5m2", ws.sdy, margin, mu, ws.dy8, transposed=False)
            seq = [
                ("quant", f"{n}.X+W", 5 * (L.M * L.K + L.K * L.N), 0, qxw),
                ("fwd", f"{n}.fwd {L.M}x{L.N}x{L.K}", 0, 2 * L.M * L.N * L.K,
                 lambda: tsf.fp8_gemm(ws.x8, "e4m3", ws.sx, ws.w8, "e4m3", ws.sw, d["Y"], "rows", "cols",
                                      workspace=ws.scratch)),
                ("quant", f"{n}.dY", 5 * L.M * L.N, 0, qdy),
                ("pair", f"{n}.bwd dgrad {L.M}x{L.K}x{L.N} + wgrad {L.K}x{L.N}x{L.M}", 0, 4 * L.M * L.K * L.N,
                 lambda: tsf.fp8_gemm_pair(
                     dict(a=ws.dy8, fa="e5m2", sa=ws.sdy, b=ws.w8, fb="e4m3", sb=ws.sw, out=d["dX"]),
                     dict(a=ws.x8, fa="e4m3", sa=ws.sx, b=ws.dy8, fb="e5m2", sb=ws.sdy, out=d["dW"],
                          a_layout="cols", b_layout="cols"))),
            ]
            for kind, label, nbytes, flops, fn in seq:
                if instrument == "all" or (instrument == "gemm" and kind != "quant"):
                    e0 = hip.record()
                    fn()
                    self.events.append((kind, label, nbytes, flops, e0, hip.record()))
                else:
                    fn()

    def collect(self):
        rows = [(k, lb, b, f, self.hip.elapsed_ms(e0, e1)) for k, lb, b, f, e0, e1 in self.events]
        self.events.clear()
        return rows

    def timed(self, steps, warmup):
        """warmup untimed steps, then steps timed (events around the GEMMs)."""
        torch = self.torch
        for _ in range(warmup):
            self.step(None)
        self.hip.reserve(self.hip.next + 2 * 2 * len(self.lin) * steps + 64)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step("gemm")
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        return ms, self.collect()

    def quant_breakdown(self, steps):
        """Steps with events around every launch: median per quantise call."""
        import statistics
        for _ in range(steps):
            self.step("all")
        self.torch.cuda.synchronize()
        qcalls = {}
        for kind, label, nbytes, _, t in self.collect():
            if kind == "quant":
                qcalls.setdefault(label, [nbytes, []])[1].append(t)
        q_ms = sum(statistics.median(ts) for _, ts in qcalls.values())
        q_bytes = sum(nb for nb, _ in qcalls.values())
        gbs = q_bytes / (q_ms * 1e-3) / 1e9
        agg = {"GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "ms_per_step": round(q_ms, 4),
               "avg_call_us": round(q_ms * 1e3 / len(qcalls), 2),
               "bytes": "5 per element: amax read 2, cast read 2, row-major FP8 copy 1",
               "timing": f"median per call over {steps} steps"}
        per = {lb: {"us": round(statistics.median(ts) * 1e3, 1),
                    "GB/s": round(nb / (statistics.median(ts) * 1e-3) / 1e9, 1)} for lb, (nb, ts) in qcalls.items()}
        return agg, per


def gemm_figures(timed, steps):
    """GEMM aggregates from the timed steps' events: all GEMM launches, the
    dominant kernel (the backward pair) and the forward, per launch and per
    linear."""
    def agg(kinds):
        ms = sum(t for k, _, _, _, t in timed if k in kinds)
        fl = sum(f for k, _, _, f, _ in timed if k in kinds)
        n = sum(1 for k, *_ in timed if k in kinds)
        return ms, fl, n
    out = {}
    for key, kinds in (("all", ("fwd", "pair")), ("pair", ("pair",)), ("fwd", ("fwd",))):
        ms, fl, n = agg(kinds)
        out[key] = {"TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1), "ms_per_step": round(ms / steps, 4),
                    "launches_per_step": n // steps, "avg_launch_us": round(ms * 1e3 / n, 2),
                    "flop_per_launch": fl // n}
    per = {}
    for kind, label, _, fl, t in timed:
        if kind != "quant":
            p = per.setdefault(label, [0.0, 0, fl])
            p[0] += t
            p[1] += 1
    out["by_launch"] = {lb: {"us": round(t * 1e3 / n, 1), "TFLOP/s": round(fl / (t / n * 1e-3) / 1e12, 1)}
                        for lb, (t, n, fl) in per.items()}
    lt = {}
    for kind, label, _, fl, t in timed:
        if kind != "quant":
            e = lt.setdefault(label.split(".")[0], [0.0, 0.0])
            e[0] += t
            e[1] += fl
    out["by_linear"] = {n: {"us_per_step": round(t * 1e3 / steps, 1), "TFLOP/s": round(f / (t * 1e-3) / 1e12, 1)}
                        for n, (t, f) in lt.items()}
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import tensor_scaled_fp8_amd as tsf
    from workloads import workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tsf.load()
    wl = workload(args.workload)

    # Timing events are HIP events created once, without the system-scope
    # fence on record (a fenced timing event writes back and invalidates the
    # caches and measurably slows the kernels around it).
    hip = HipEvents(torch.cuda.current_stream(dev).cuda_stream)
    want_cpu = not args.no_cpu_baseline
    layer = Layer(tsf, torch, np, wl, dev, hip, args.cpu_rows if want_cpu else 0, args.cpu_cols)

    if args.calibration_copy:
        n = args.calibration_copy
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # timed region: K whole steps bracketed by synchronisation; events
    # bracket every GEMM launch
    ms, timed = layer.timed(args.steps, args.warmup)
    flops = wl.flops_fwd_bwd()
    value = flops / (ms * 1e-3) / 1e12
    g = gemm_figures(timed, args.steps)
    dom = g["pair"]
    traffic = gemm_traffic(os.path.join(args.traffic_dir, f"gemm_traffic_{wl.name}.json"), wl.name)
    roofline = {"bound": "mfma", "achieved": dom["TFLOP/s"], "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(dom["TFLOP/s"] / PEAK_FP8_TFLOPS, 4), "traffic": traffic,
                "kernel": f"{DOMINANT} (a linear's dgrad + wgrad in one launch, FP8 MFMA)",
                "avg_launch_us": dom["avg_launch_us"], "flop_per_launch": dom["flop_per_launch"],
                "note": "achieved = mean algorithmic FLOP per launch (4*M*K*N over the layer's linears) / "
                        "mean launch duration (fence-free HIP events around each launch in the timed steps); "
                        "the rocprofv3 average of the same kernel gives the same ratio"}
    kernels = {"gemm": {"TFLOP/s": g["all"]["TFLOP/s"], "ms_per_step": g["all"]["ms_per_step"],
                        "forward_gemm_nt": g["fwd"], "backward_pair": g["pair"]},
               "gemm_by_launch": g["by_launch"], "gemm_by_linear": g["by_linear"]}
    infer = fp8dw = o2 = spec = None
    side = {}
    if not args.step_only:
        qa, qper = layer.quant_breakdown(args.breakdown_steps)
        kernels["amax+cast"] = qa
        kernels["amax+cast_by_tensor"] = qper
        spec = spec_pass(tsf, torch, layer.lin, layer.margin, layer.mu, hip, layer.step, args.steps, flops, wl)
        infer = inference_pass(tsf, torch, layer.lin, layer.margin, args.steps, args.warmup)
        fp8dw = fp8_dw_pass(tsf, torch, layer.lin, layer.margin, layer.mu, args.steps, args.warmup)
        o2 = adam_pass(tsf, torch, layer.lin, layer.margin, layer.mu, args.steps, args.warmup)
        kernels["amax+cast_cold"] = quantize_cold(tsf, torch, layer.lin, layer.margin, layer.mu, hip)
        kernels["note"] = ("gemm: events in the timed region; amax+cast (fp8_quantize / fp8_quantize_batch: "
                           f"amax pass + cast kernel): a separate pass of {args.breakdown_steps} steps with "
                           "events around every call, median per call")
        for w in [int(x) for x in args.side_workloads.split(",") if x.strip()]:
            if w == args.workload:
                continue
            other = Layer(tsf, torch, np, workload(w), dev, hip)
            oms, otimed = other.timed(args.steps, args.warmup)
            og = gemm_figures(otimed, args.steps)
            oq, _ = other.quant_breakdown(args.breakdown_steps)
            oflops = other.wl.flops_fwd_bwd()
            side[other.wl.name] = {
                "value": round(oflops / (oms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms_per_step": round(oms, 4),
                "tokens": other.lin[0]["L"].M, "linears": {L.name: [L.M, L.K, L.N] for L in other.wl.linears},
                "gemm": {"TFLOP/s": og["all"]["TFLOP/s"], "frac": round(og["all"]["TFLOP/s"] / PEAK_FP8_TFLOPS, 4),
                         "backward_pair": og["pair"]["TFLOP/s"], "forward_gemm_nt": og["fwd"]["TFLOP/s"]},
                "amax+cast": oq}
            del other
            torch.cuda.synchronize()

    check = None
    if args.check:
        check = sampled_check(layer.lin, wl, layer.margin, layer.mu)

    cpu = None
    if want_cpu:
        cpu = cpu_baseline(wl, layer.sample, args.cpu_rows, args.cpu_cols)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 (E4M3 X/W, E5M2 dY; fp32 accumulate; bf16 in/out)", "data": "synthetic",
        "config": {"workload": wl.name, "tokens": wl.linears[0].M,
                   "linears": {L.name: [L.M, L.K, L.N] for L in wl.linears},
                   "margin": layer.margin, "mu_log2": layer.mu, "flops_per_step": flops,
                   "quant_bytes_per_step": wl.quant_bytes()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "frac_fp8_peak_step": round(value / PEAK_FP8_TFLOPS, 4),
        "other_workloads": side or None,
        "inference": infer,
        "fp8_weight_gradient": fp8dw,
        "o2_adam": o2,
        "quantize_speculative": spec,
        "input_gen_s": round(layer.gen_s, 1),
    }
    if check is not None:
        out["check"] = check
    print(json.dumps(out), flush=True)


def quantize_cold(tsf, torch, lin, margin, mu, hip, reps=3):
    """fp8_quantize of every tensor of the step with the caches cold: a
    512 MB fill runs before each timed call (the 256 MB MALL would otherwise
    hold part of the tensor). Median of reps; 5 B per element."""
    import statistics
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=lin[0]["X"].device)
    out = {}
    for d in lin:
        ws, n = d["ws"], d["L"].name
        for label, x, fmt, s, q, m in ((f"{n}.X", d["X"], "e4m3", ws.sx, ws.x8, 0),
                                       (f"{n}.W", d["W"], "e4m3", ws.sw, ws.w8, 0),
                                       (f"{n}.dY", d["dY"], "e5m2", ws.sdy, ws.dy8, mu)):
            ts = []
            for r in range(reps):
                scratch.fill_(r)
                e0 = hip.record()
                tsf.fp8_quantize(x, fmt, s, margin, m, q, transposed=False)
                e1 = hip.record()
                torch.cuda.synchronize()
                ts.append(hip.elapsed_ms(e0, e1))
            t = statistics.median(ts)
            out[label] = {"us": round(t * 1e3, 1), "GB/s": round(5 * x.numel() / (t * 1e-3) / 1e9, 1)}
    del scratch
    return out


def spec_pass(tsf, torch, lin, margin, mu, hip, step, steps, flops, wl):
    """fp8_quantize_spec (one pass casting with the bias the record kept,
    then a check that recasts only if the tensor's own amax gives another
    bias; same bytes and records as fp8_quantize) on every tensor of the
    step: per-call time when the guess holds ("hit": 2 B read + 1 B
    written per element) and when it is wrong ("miss", forced by presetting
    a wrong bias outside the timed calls: 4 B read + 2 B written), against
    the two-pass fp8_quantize (5 B). Plus the whole step with speculative
    quantisation; the benchmark's inputs are the same every step, so there
    every guess holds: it is the best case, reported beside the step, not
    as it."""
    import statistics
    tensors = []
    for d in lin:
        ws, n = d["ws"], d["L"].name
        tensors += [(f"{n}.X", d["X"], "e4m3", ws.sx, ws.x8, 0), (f"{n}.W", d["W"], "e4m3", ws.sw, ws.w8, 0),
                    (f"{n}.dY", d["dY"], "e5m2", ws.sdy, ws.dy8, mu)]
    miss_rec = tsf.new_scale(len(tensors))
    biases = [tsf.read_scale(s)["bias"] for _, _, _, s, _, _ in tensors]
    out = {}
    for mode in ("two_pass", "hit", "miss"):
        per, elems = [], 0
        for i, (label, x, fmt, s, q, m) in enumerate(tensors):
            ts = []
            for _ in range(3):
                if mode == "miss":
                    tsf.fp8_scale_fixed(miss_rec[i], biases[i] + 5 if biases[i] < 100 else biases[i] - 5)
                e0 = hip.record()
                if mode == "two_pass":
                    tsf.fp8_quantize(x, fmt, s, margin, m, q, transposed=False)
                elif mode == "hit":
                    tsf.fp8_quantize_spec(x, fmt, s, margin, m, q)
                else:
                    tsf.fp8_quantize_spec(x, fmt, miss_rec[i], margin, m, q)
                e1 = hip.record()
                torch.cuda.synchronize()
                ts.append(hip.elapsed_ms(e0, e1))
            per.append(statistics.median(ts))
            elems += x.numel()
        t = sum(per)
        moved = {"two_pass": 5, "hit": 3, "miss": 6}[mode]
        out[mode] = {"ms_per_step": round(t, 4), "bytes_moved_per_element": moved,
                     "GB/s_moved": round(moved * elems / (t * 1e-3) / 1e9, 1),
                     "elements_per_ns": round(elems / (t * 1e6), 2)}
    for _ in range(2):
        step(None, spec=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(None, spec=True)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    out["step_guess_holds"] = {"ms_per_step": round(ms, 4), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1)}
    # does the guess hold for a new batch? Independent N(0, sigma) draws of
    # every tensor (normal workloads only), each quantised with the record
    # its predecessor left: a hit when the derived bias equals the guess
    if not wl.x_outliers and not wl.dy_log_uniform:
        g = torch.Generator(device=lin[0]["X"].device)
        g.manual_seed(20261)
        sig = {"X": 1.0, "W": wl.sigma_w, "dY": wl.sigma_dy}
        hits = 0
        for label, x, fmt, s, q, m in tensors:
            x2 = (torch.randn(x.shape, generator=g, device=x.device) * sig[label.split(".")[1]]).to(torch.bfloat16)
            tsf.fp8_quantize_spec(x2, fmt, s, margin, m, q)
            w = s.cpu()
            hits += int(w[1] == w[6])          # bias == the guess it replaced
            tsf.fp8_quantize(x, fmt, s, margin, m, q, transposed=False)   # back to this input's record
            del x2
        out["independent_draws"] = {"tensors": len(tensors), "guess_held": hits}
        out["stream"] = spec_stream(tsf, torch, lin, margin, mu, step, steps, flops, g, sig)
    out["note"] = ("one call per tensor with events around it (median of 3); miss = the record's bias preset "
                   "wrong; step_guess_holds = the whole step with fp8_quantize_spec for X, W and dY on the "
                   "benchmark's fixed inputs (every guess holds: the best case, not the headline)")
    return out


def spec_stream(tsf, torch, lin, margin, mu, step, steps, flops, g, sig):
    """The step over a stream of distinct batches: the inputs rotate through
    three sets (the benchmark's own and two independent N(0, sigma) draws of
    every tensor), timed with the two-pass quantise and with the speculative
    one; then an untimed pass over the same rotation counts the speculative
    calls whose guess held."""
    sets = [[(d["X"], d["W"], d["dY"]) for d in lin]]
    for _ in range(2):
        sets.append([tuple((torch.randn(t.shape, generator=g, device=t.device) * sig[k]).to(torch.bfloat16)
                           for t, k in zip((d["X"], d["W"], d["dY"]), ("X", "W", "dY"))) for d in lin])

    def use(i):
        for d, (x, w, dy) in zip(lin, sets[i % len(sets)]):
            d["X"], d["W"], d["dY"] = x, w, dy

    out = {"sets": len(sets)}
    for name, spec in (("two_pass", False), ("speculative", True)):
        for i in range(len(sets)):
            use(i)
            step(None, spec=spec)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            use(i)
            step(None, spec=spec)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        out[name] = {"ms_per_step": round(ms, 4), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1)}
    calls = held = 0
    for i in range(2 * len(sets)):
        use(i)
        for d in lin:
            ws = d["ws"]
            for x, fmt, s, q, m in ((d["X"], "e4m3", ws.sx, ws.x8, 0), (d["W"], "e4m3", ws.sw, ws.w8, 0),
                                    (d["dY"], "e5m2", ws.sdy, ws.dy8, mu)):
                tsf.fp8_quantize_spec(x, fmt, s, margin, m, q)
                w = s.cpu()
                calls += 1
                held += int(w[1] == w[6])
    out["calls"], out["guess_held"] = calls, held
    use(0)
    for d in lin:   # leave each record as its own input's
        ws = d["ws"]
        tsf.fp8_quantize(d["X"], "e4m3", ws.sx, margin, 0, ws.x8, transposed=False)
        tsf.fp8_quantize(d["W"], "e4m3", ws.sw, margin, 0, ws.w8, transposed=False)
        tsf.fp8_quantize(d["dY"], "e5m2", ws.sdy, margin, mu, ws.dy8, transposed=False)
    del sets
    torch.cuda.synchronize()
    return out


def inference_pass(tsf, torch, lin, margin, steps, warmup):
    """Forward-only inference on weights cast once (post-training
    quantisation): per linear, fp8_linear_fwd_cached = X quantised (amax
    rule, or a fixed FP8-CSCALE bias) + the forward GEMM on the cached
    row-major w8 (read reduction-major, as in training).
    Reported beside the training step, not part of its value."""
    out = {}
    flops = sum(2 * d["L"].M * d["L"].K * d["L"].N for d in lin)
    recs = tsf.new_scale(len(lin), lin[0]["X"].device)
    # weights cast once (post-training quantisation), outside the timing
    prepared = [tsf.prepare_weight(d["W"], margin) for d in lin]
    for mode in ("amax", "fixed"):
        if mode == "fixed":
            for i, d in enumerate(lin):   # the bias the amax rule chose, now held fixed
                recs[i].copy_(d["ws"].sx)

        def fwd():
            for i, d in enumerate(lin):
                w8, sw = prepared[i]
                tsf.fp8_linear_fwd_cached(d["X"], w8, sw, d["ws"].x8, recs[i], margin, mode, Y=d["Y"])
        for _ in range(warmup):
            fwd()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fwd()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        out[mode] = {"ms_per_forward": round(ms, 4), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1)}
    out["note"] = ("forward only, weights cast once (prepare_weight): X scaled from its "
                   "amax per call, or with a fixed bias (FP8-CSCALE); 2*M*K*N per linear")
    return out


def fp8_dw_pass(tsf, torch, lin, margin, mu, steps, warmup):
    """FP8 weight gradient per linear: fp8_wgrad_fp8 (wgrad GEMM whose
    epilogue also takes max |dW|, then the E5M2 cast) against the unfused
    wgrad GEMM + fp8_quantize(dW). Reported beside the training step."""
    bufs = []
    for d in lin:
        L = d["L"]
        bufs.append(dict(dw8=torch.empty((L.K, L.N), dtype=torch.uint8, device=d["dW"].device),
                         s=tsf.new_scale(2, d["dW"].device)))
    flops = sum(2 * d["L"].M * d["L"].K * d["L"].N for d in lin)
    q_bytes = sum(3 * d["L"].K * d["L"].N for d in lin)   # E5M2 cast of dW: 2 B read + 1 B write

    def fused():
        for d, b in zip(lin, bufs):
            ws = d["ws"]
            tsf.fp8_wgrad_fp8(ws.x8, ws.sx, ws.dy8, ws.sdy, margin, mu, dW=d["dW"], s_dw=b["s"][0], dw8=b["dw8"],
                              x_layout="cols", dy_layout="cols")

    def unfused():
        for d, b in zip(lin, bufs):
            ws = d["ws"]
            tsf.fp8_gemm(ws.x8, "e4m3", ws.sx, ws.dy8, "e5m2", ws.sdy, d["dW"], "cols", "cols")
            tsf.fp8_quantize(d["dW"], "e5m2", b["s"][1], margin, mu, out_row=b["dw8"], transposed=False)

    out = {}
    for name, fn in (("fused", fused), ("unfused", unfused)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        out[name] = {"ms_per_step": round(ms, 4), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1)}
    out["saved_ms"] = round(out["unfused"]["ms_per_step"] - out["fused"]["ms_per_step"], 4)
    out["note"] = ("all linears' dW in E5M2 per step: wgrad GEMM + cast (fused amax) vs wgrad GEMM + "
                   f"fp8_quantize(dW); the cast moves {q_bytes} bytes per step")
    return out


def adam_pass(tsf, torch, lin, margin, mu, steps, warmup):
    """O2 Adam step over every weight of the layer (FP8 E4M3 first moment,
    scaled FP16 second moment and master weights), fed by the FP8 weight
    gradients of fp8_wgrad_fp8; the new bf16 weights are written too.
    Algorithmic HBM bytes per parameter (the one-pass minimum): gradient
    (1), m1 (1), m2 (2), master (2) read, m1, m2, master and bf16 weights
    written (7): 13. The kernels move 19: the new scales need the new
    tensors' maxima before anything is stored, so a first pass reads the
    6 bytes once more."""
    states = []
    for d in lin:
        ws = d["ws"]
        _, dw8, _, s_dw = tsf.fp8_wgrad_fp8(ws.x8, ws.sx, ws.dy8, ws.sdy, margin, mu, x_layout="cols",
                                            dy_layout="cols")
        st = tsf.AdamState(d["W"])
        states.append((st, dw8.reshape(-1), s_dw, torch.empty(st.n, dtype=torch.bfloat16, device=dw8.device)))
    n = sum(st.n for st, _, _, _ in states)

    def run():
        for st, g8, s_g, wout in states:
            tsf.fp8_adam_step(st, g8, s_g, 1e-4, 0.9, 0.95, 1e-8, 0.1, w_bf16=wout)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    gbs = 13 * n / (ms * 1e-3) / 1e9
    moved = 19 * n / (ms * 1e-3) / 1e9
    grads = [(g8, s_g, wout) for _, g8, s_g, wout in states]
    del states
    out = {"params": n, "ms_per_step": round(ms, 4), "GB/s": round(gbs, 1),
           "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "GB/s_moved": round(moved, 1),
           "note": "fp8_adam_step on all weights of the layer (3 launches each); GB/s at the one-pass "
                   "minimum of 13 bytes/param, GB/s_moved at the 19 bytes/param the two passes move"}
    # the one-pass step (fp8_adam_step_spec) from fresh states, same gradients
    spec = [(tsf.AdamState(d["W"]), g8, s_g, wout, torch.zeros(steps, dtype=torch.int32, device=g8.device))
            for d, (g8, s_g, wout) in zip(lin, grads)]
    warm = torch.zeros(1, dtype=torch.int32, device=grads[0][0].device)

    def run_spec(k=None):
        for st, g8, s_g, wout, miss in spec:
            tsf.fp8_adam_step_spec(st, g8, s_g, 1e-4, 0.9, 0.95, 1e-8, 0.1, w_bf16=wout,
                                   missed=warm if k is None else miss[k:k + 1])
    spec_warmup = max(warmup, 40)   # the moments settle (with one gradient they grow for tens of steps)
    for _ in range(spec_warmup):
        run_spec()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        run_spec(k)
    torch.cuda.synchronize()
    ms1 = (time.perf_counter() - t0) * 1e3 / steps
    recomputed = int(sum(int((miss != 0).sum()) for *_, miss in spec))
    gbs1 = 13 * n / (ms1 * 1e-3) / 1e9
    del spec
    out["one_pass"] = {
        "ms_per_step": round(ms1, 4), "GB/s": round(gbs1, 1), "frac_hbm": round(gbs1 / PEAK_HBM_GBS, 4),
        "tensor_steps_recomputed": f"{recomputed} of {steps * len(lin)}", "warmup_steps": spec_warmup,
        "note": "fp8_adam_step_spec (out of place, 3 launches each): 13 bytes/param when no scale changes, "
                "24 when one does (its second kernel recomputes); the same gradient every step, so the "
                "moments grow toward their limits and some tensor-steps move a max across a power of two "
                "(counted over the timed steps)"}
    return out


class HipEvents:
    """Timing events of the HIP runtime the process already uses, created
    with hipEventDisableSystemFence, recorded on one stream."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, stream: int):
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("HIP runtime not loaded")
        self.ct = ctypes
        self.lib = ctypes.CDLL(path)   # already loaded: same runtime instance
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.stream = ctypes.c_void_p(stream)
        self.pool = []
        self.next = 0

    def reserve(self, n):
        while len(self.pool) < n:
            e = self.ct.c_void_p()
            if self.lib.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.pool.append(e)

    def record(self):
        if self.next >= len(self.pool):
            self.reserve(self.next + 64)
        e = self.pool[self.next]
        self.next += 1
        if self.lib.hipEventRecord(e, self.stream) != 0:
            raise RuntimeError("hipEventRecord failed")
        return e

    def elapsed_ms(self, e0, e1):
        t = self.ct.c_float()
        if self.lib.hipEventElapsedTime(self.ct.byref(t), e0, e1) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return t.value


def gemm_traffic(path, workload_name):
    """Measured HBM bytes per launch of the dominant GEMM kernel from a
    committed counter summary of this workload, reported only while the
    GEMM code is the one the counters were taken on (sha256 of gemm.hip
    without comments, recorded in the summary)."""
    from tensor_scaled_fp8_amd.profiling import gemm_code_sha256
    if not path or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("gemm_code_sha256") != gemm_code_sha256() or rec.get("workload") != workload_name:
        return None
    if DOMINANT not in rec.get("kernel", ""):
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


def cpu_baseline(wl, sample, rows, cols):
    """The oracle, as it stands, on a bounded sample of the same layer: the
    first `rows` tokens and the first `cols` output features of every
    linear (X [rows, K], W [K, cols], dY [rows, cols], sliced from the
    benchmark's own inputs): amax, bias, cast, three fp64 GEMMs."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    flops = 0
    t = 0.0
    for (X, W, dY), L in zip(sample, wl.linears):
        n = W.shape[1]
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
