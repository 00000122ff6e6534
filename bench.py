"""Benchmark of the W4A16 quantized linear path on one MI355X.

Default workload: the 7B-style MLP decode batch -- M = 16 tokens through
gate [11008 x 4096], up [11008 x 4096] and down [4096 x 11008] INT4 layers
(group 128, fp16 scale, 4-bit zero point), fp16 activations.  One step is the
three dequant-GEMV calls.  Weights are quantized on the GPU once (offline
step, outside the timed region) and replicated into enough distinct copies
(>= 512 MB) that every step reads weights the 256 MB Infinity Cache has not
just served; inputs are resident in HBM when timing starts.

Reported value: effective HBM GB/s = algorithmic bytes of one step (packed
codes + fp16 scales + 4-bit zeros + x + y, each read or written once) / step
time.  The "roofline" object covers the dominant kernel (the decode GEMV),
timed per call with HIP events recorded on the stream the library launches
on; "cpu_baseline" times the CPU oracle on a bounded sample of the same
layers.

Other workloads (--workload): decode_m1 (M = 1, 4096 x 4096), prefill
(M = 2048 through q, k, v, o and up; TFLOP/s), nf4_m1 / nf4_m512 (NF4 14336 x
4096, bf16), int8_70b (LLM.int8 at 28672 x 8192, M = 256).
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA16_PEAK_TFLOPS = 2500.0
ROTATE_BYTES = 512 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------- workloads
class Workload:
    """One step = a list of library calls; bytes/flops are algorithmic."""

    name = ""
    unit = "GB/s"
    metric = "W4A16 g128 linear: effective HBM GB/s (M=1) and TFLOP/s (M=2048), % roofline"
    dtype = "f16"

    def setup(self):
        raise NotImplementedError

    def calls(self, step):
        raise NotImplementedError


def _int4_layer(wq, torch, w_np):
    n, k = w_np.shape
    qw = wq.alloc_int4(n, k)
    wq.wq_quantize_groupwise(torch.from_numpy(w_np).cuda(), 4, 128, 0, qw.codes, qw.scales, qw.zeros)
    return qw


def _ws(wq, torch, m, qw):
    need = wq.wq_linear_w4a16_workspace(m, qw)
    return torch.empty((need,), dtype=torch.uint8, device="cuda") if need else None


def _copies(qw_list, per_copy_bytes):
    reps = max(1, -(-ROTATE_BYTES // max(1, per_copy_bytes)))
    out = [qw_list]
    for _ in range(reps - 1):
        out.append([q.clone() for q in qw_list])
    return out


class W4Layers(Workload):
    """A sequence of INT4 layers applied to their own inputs (decode or prefill)."""

    def __init__(self, name, layers, unit):
        self.name = name
        self.layers_np = layers          # list of (layer name, x, w)
        self.unit = unit

    def setup(self):
        import torch
        import bit_quantized_linear_int4_amd as wq
        self.wq = wq
        base = []
        self.xs, self.ys, self.wss = [], [], []
        self.bytes_per_call, self.flops_per_call = [], []
        for name, x, w in self.layers_np:
            qw = _int4_layer(wq, torch, w)
            base.append(qw)
            m, n, k = x.shape[0], w.shape[0], w.shape[1]
            self.xs.append(torch.from_numpy(x).cuda())
            self.ys.append(torch.empty((m, n), dtype=torch.float16, device="cuda"))
            self.wss.append(_ws(wq, torch, m, qw))
            self.bytes_per_call.append(qw.nbytes() + x.size * 2 + m * n * 2)
            self.flops_per_call.append(2 * m * n * k)
        torch.cuda.synchronize()
        self.copies = _copies(base, sum(q.nbytes() for q in base))
        torch.cuda.synchronize()
        self.m = [x.shape[0] for _, x, _ in self.layers_np]

    def calls(self, step):
        wq = self.wq
        ws = self.copies[step % len(self.copies)]
        return [(lambda i=i: wq.wq_linear_w4a16(self.xs[i], ws[i], self.ys[i], self.wss[i]))
                for i in range(len(ws))]

    def work_per_step(self):
        return sum(self.bytes_per_call) if self.unit == "GB/s" else sum(self.flops_per_call)

    def dominant(self):
        if self.unit == "GB/s":
            return ("w4a16 skinny dequant-GEMV (HIP events per call)",
                    sum(self.bytes_per_call) / len(self.bytes_per_call), "hbm")
        return ("w4a16 dequant-GEMM (HIP events per call)",
                sum(self.flops_per_call) / len(self.flops_per_call), "mfma")

    def cpu_sample(self):
        """Oracle: dequantize + fp64 product on the first rows of every layer."""
        import numpy as np
        from oracle import int4, linear
        layers = []
        for name, x, w in self.layers_np:
            rows = max(16, w.shape[0] // 32)
            layers.append((x, w[:rows]))
        pre = [(x, int4.quantize(w)) + (w.shape,) for x, w in layers]

        def run():
            for x, (q, s, z), shp in pre:
                wh = int4.dequantize(q, s, z, shp[1])
                linear.reference(x.astype(np.float32), wh)
        work = 0
        for x, (q, s, z), shp in pre:
            m, n, k = x.shape[0], shp[0], shp[1]
            if self.unit == "GB/s":
                work += q.nbytes + s.nbytes + z.nbytes + x.size * 2 + m * n * 2
            else:
                work += 2 * m * n * k
        desc = ", ".join(f"{nm} first {max(16, w.shape[0] // 32)} rows"
                         for nm, x, w in self.layers_np)
        return run, work, desc

    def config(self):
        return {"workload": self.name,
                "layers": [{"name": nm, "m": int(x.shape[0]), "n": int(w.shape[0]),
                            "k": int(w.shape[1])} for nm, x, w in self.layers_np],
                "format": "INT4 asymmetric, group 128, fp16 scale, 4-bit zero",
                "weight_copies": len(self.copies)}


def make_workload(name):
    import workloads
    if name == "mlp_decode":
        return W4Layers("mlp_decode_m16_7b", workloads.mlp_decode(), "GB/s")
    if name == "decode_m1":
        d = workloads.decode_m1()
        return W4Layers("decode_m1_4096x4096", [("proj", d["x"], d["w"])], "GB/s")
    if name == "prefill":
        return W4Layers("prefill_m2048_7b", workloads.prefill(), "TFLOP/s")
    raise SystemExit(f"unknown workload {name}")


# ------------------------------------------------------------------- timing
def time_workload(wl, steps, warmup):
    import torch
    for s in range(warmup):
        for c in wl.calls(s):
            c()
    torch.cuda.synchronize()
    ncalls = len(wl.calls(0))
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps * ncalls)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps * ncalls)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    for s in range(steps):
        for c in wl.calls(warmup + s):
            starts[i].record()
            c()
            ends[i].record()
            i += 1
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per_call = [starts[j].elapsed_time(ends[j]) for j in range(i)]  # ms
    return (t1 - t0) / steps * 1e3, sum(per_call) / len(per_call)


def cpu_baseline(wl, unit, budget_s=15.0):
    try:
        import threadpoolctl
        limiter = threadpoolctl.threadpool_limits
    except Exception:  # pragma: no cover
        limiter = None
    cores = os.cpu_count() or 1
    run, work, desc = wl.cpu_sample()
    ctx = limiter(limits=cores) if limiter else None
    reps, t = 0, 0.0
    if ctx:
        ctx.__enter__()
    try:
        t0 = time.perf_counter()
        while True:
            run()
            reps += 1
            t = time.perf_counter() - t0
            if t > budget_s or reps >= 50:
                break
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    scale = 1e9 if unit == "GB/s" else 1e12
    return {"value": round(work * reps / t / scale, 4), "unit": unit, "cores": cores,
            "kind": "oracle",
            "sample": f"{desc}; dequantize + fp64 product, {reps} repetitions in {t:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mlp_decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); this library's path is "
              "single-GPU. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    wl = make_workload(args.workload)
    log(f"[bench] setting up {wl.name}")
    wl.setup()
    log(f"[bench] timing {args.steps} steps after {args.warmup} warmup")
    ms_step, ms_call = time_workload(wl, args.steps, args.warmup)
    work = wl.work_per_step()
    scale = 1e9 if wl.unit == "GB/s" else 1e12
    value = work / (ms_step * 1e-3) / scale
    kname, per_call_work, bound = wl.dominant()
    achieved = per_call_work / (ms_call * 1e-3) / scale
    peak = HBM_PEAK_GBS if bound == "hbm" else MFMA16_PEAK_TFLOPS
    out = {
        "metric": wl.metric,
        "value": round(value, 3),
        "unit": wl.unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations with fixed outlier channels)",
        "config": wl.config(),
        "roofline": {"bound": bound, "achieved": round(achieved, 3), "peak": peak,
                     "unit": wl.unit, "frac": round(achieved / peak, 4), "traffic": None,
                     "kernel": kname, "avg_call_us": round(ms_call * 1e3, 3),
                     "work_per_call": per_call_work},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle sample")
        out["cpu_baseline"] = cpu_baseline(wl, wl.unit, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
