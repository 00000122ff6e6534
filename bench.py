"""Benchmark of the quantized linear path on one MI355X.

Default (--workload metric): the two shapes the metric is quoted on, in one
JSON line.
  * value: the single W4A16 layer at M = 1 -- W [4096 x 4096] INT4 (group
    128, fp16 scale, 4-bit zero point), x fp16 [1 x 4096], y fp16; one step
    is one dequant-GEMV call; effective HBM GB/s.
  * secondary: the 7B-style prefill at M = 2048 -- q, k, v, o [4096 x 4096]
    and up [11008 x 4096], one step is the five dequant-GEMM calls; TFLOP/s.
Each carries the roofline of its dominant kernel.  Weights are quantized on
the GPU once (offline step, outside the timed region) and replicated into
enough distinct copies (>= 512 MB) that successive steps read weights the
256 MB Infinity Cache has not just served; inputs are resident in HBM when
timing starts.

Timing.  The K timed steps are captured into one HIP graph and replayed
once between two HIP events on the capture stream (warmup: W eager steps,
then one untimed replay that also uploads the graph).  The dominant kernel
is timed the same way in a region of its own: K launches of it alone, back
to back, so its average launch duration is comparable with the
rocprofv3 kernel trace of the same command.

Reported value: effective HBM GB/s = algorithmic bytes of one step (packed
codes + scales + zero points + x + y, each read or written once) / step time
(TFLOP/s = 2*M*N*K / step time for the GEMM workloads).

Other workloads (--workload), one per line: decode_m1, prefill, mlp_decode
(M = 16 through gate + up as one pair call and down [4096 x 11008]),
decode_m1_actorder (the M = 1 layer quantized in a synthetic act-order: each
call gathers x into that order first), nf4_m1 / nf4_m512 (NF4 14336 x 4096,
bf16), int8_70b (LLM.int8 at 28672 x 8192, M = 256).
"""

import argparse
import hashlib
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
METRIC = "W4A16 g128 linear: effective HBM GB/s (M=1) and TFLOP/s (M=2048), % roofline"
KERNEL_SOURCES = {
    "stream": "bit_quantized_linear_int4_amd/csrc/w4a16.hip",
    "gemm": "bit_quantized_linear_int4_amd/csrc/w4a16.hip",
    "int8": "bit_quantized_linear_int4_amd/csrc/int8.hip",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _copies_needed(per_copy_bytes):
    return max(1, -(-ROTATE_BYTES // max(1, per_copy_bytes)))


class Workload:
    """One step = a list of calls.  Work (bytes or flops) is algorithmic:
    what the method has to move or compute, not what the kernels do."""

    unit = "GB/s"
    dtype = "f16"
    kernel = "stream"        # family of the dominant kernel
    kernel_desc = ""

    def __init__(self, name, layers, unit):
        self.name = name
        self.layers_np = layers
        self.unit = unit

    # to be provided: setup(), step_calls(copy), dominant_calls(copy),
    # work_per_step(), dominant_work(), cpu_stages(), config(), release()


def _int4_weight(wq, torch, w_np):
    n, k = w_np.shape
    qw = wq.alloc_int4(n, k)
    wq.wq_quantize_groupwise(torch.from_numpy(w_np).cuda(), 4, 128, 0, qw.codes, qw.scales,
                             qw.zeros)
    return qw


class W4Layers(Workload):
    """INT4 layers, each applied to its own seeded input (decode or prefill).
    A gate projection followed by an up projection of the same input runs
    as one pair call (the activations are read once for both)."""

    act_order = None   # seed of a synthetic act-order for every layer, or None

    def setup(self):
        import torch
        import bit_quantized_linear_int4_amd as wq
        self.wq = wq
        base, self.xs, self.ys, self.wss = [], [], [], []
        bytes_, flops = [], []
        for _, x, w in self.layers_np:
            if self.act_order is None:
                qw = _int4_weight(wq, torch, w)
            else:
                # columns stored in quantization order; every call gathers x
                import workloads
                perm = torch.from_numpy(workloads.act_order_perm(w.shape[1], self.act_order)).cuda()
                wp = torch.empty(w.shape, dtype=torch.float16, device="cuda")
                wq.wq_permute_columns(torch.from_numpy(w).cuda(), perm, wp)
                n, k = w.shape
                qw = wq.alloc_int4(n, k)
                wq.wq_quantize_groupwise(wp, 4, 128, 0, qw.codes, qw.scales, qw.zeros)
                qw.perm = perm
                del wp
            base.append(qw)
            m, n, k = x.shape[0], w.shape[0], w.shape[1]
            self.xs.append(torch.from_numpy(x).cuda())
            self.ys.append(torch.empty((m, n), dtype=torch.float16, device="cuda"))
            # (an act-order weight also reads its permutation, 4 bytes a channel)
            bytes_.append(qw.nbytes() + (4 * k if qw.perm is not None else 0) + x.size * 2
                          + m * n * 2)
            flops.append(2 * m * n * k)
            # the workspace the call needs: act-order's gathered x, else none
            need = wq.wq_linear_w4a16_workspace(m, qw)
            self.wss.append(torch.empty((need,), dtype=torch.uint8, device="cuda") if need else None)
        torch.cuda.synchronize()
        reps = _copies_needed(sum(q.nbytes() for q in base))
        self.copies = [base] + [[q.clone() for q in base] for _ in range(reps - 1)]
        torch.cuda.synchronize()
        # call units: (i,) one layer; (i, j) a gate/up pair sharing x
        names = [nm for nm, _, _ in self.layers_np]
        self.units, i = [], 0
        while i < len(names):
            if (i + 1 < len(names) and names[i] == "gate" and names[i + 1] == "up"
                    and self.layers_np[i][1] is self.layers_np[i + 1][1]):
                self.units.append((i, i + 1))
                i += 2
            else:
                self.units.append((i,))
                i += 1
        # algorithmic work of a unit (a pair reads x once)
        self.ubytes = [sum(bytes_[j] for j in u) - (len(u) - 1) * self.layers_np[u[0]][1].size * 2
                       for u in self.units]
        self.uflops = [sum(flops[j] for j in u) for u in self.units]
        # dominant kernel: the unit shape whose launches take most of the step
        groups = {}
        for ui, u in enumerate(self.units):
            key = tuple((self.layers_np[j][1].shape[0],) + self.layers_np[j][2].shape for j in u)
            groups.setdefault(key, []).append(ui)
        per = self.ubytes if self.unit == "GB/s" else self.uflops
        self.dom = max(groups.values(), key=lambda idx: (sum(per[ui] for ui in idx), -idx[0]))
        u0 = self.units[self.dom[0]]
        m, n, k = self.layers_np[u0[0]][1].shape[0], *self.layers_np[u0[0]][2].shape
        fam = "stream dequant-GEMV" if m <= 16 else "dequant-GEMM"
        self.kernel = "stream" if m <= 16 else "gemm"
        names_dom = "/".join("+".join(self.layers_np[j][0] for j in self.units[ui])
                             for ui in self.dom)
        pair = " pair" if len(u0) == 2 else ""
        act = ", act-order: x gathered first" if self.act_order is not None else ""
        self.kernel_desc = f"w4a16 {fam}{pair} ({names_dom}: M={m}, N={n}, K={k}{act})"

    def _call(self, copy, ui):
        wq, ws = self.wq, self.copies[copy % len(self.copies)]
        u = self.units[ui]
        if len(u) == 2:
            i, j = u
            return lambda: wq.wq_linear_w4a16_gate_up(self.xs[i], ws[i], ws[j], self.ys[i],
                                                      self.ys[j], act=0)
        i = u[0]
        return lambda: wq.wq_linear_w4a16(self.xs[i], ws[i], self.ys[i], self.wss[i])

    def step_calls(self, copy):
        return [self._call(copy, ui) for ui in range(len(self.units))]

    def dominant_calls(self, copy):
        return [self._call(copy, ui) for ui in self.dom]

    def work_per_step(self):
        return sum(self.ubytes) if self.unit == "GB/s" else sum(self.uflops)

    def dominant_work(self):
        per = self.ubytes if self.unit == "GB/s" else self.uflops
        return per[self.dom[0]]

    def cpu_stages(self):
        """The oracle's stages on the first layer (its first 4096 rows):
        quantize + pack, dequantize, fp64 reference product."""
        import numpy as np
        from oracle import int4, linear
        nm, x, w = self.layers_np[0]
        w = w[:4096]
        m, n, k = x.shape[0], w.shape[0], w.shape[1]
        st = {}

        def quant():
            st["q"] = int4.quantize(w)

        def deq():
            st["wh"] = int4.dequantize(*st["q"], k)

        def ref():
            linear.reference(x.astype(np.float32), st["wh"])
        g = k // 128
        work = (n * k // 2 + n * g * 2 + n * ((g + 1) // 2) + m * k * 2 + m * n * 2
                if self.unit == "GB/s" else 2 * m * n * k)
        desc = f"{nm} layer, rows 0..{n - 1} of {self.layers_np[0][2].shape[0]}, M={m}, K={k}"
        return [("quantize_pack", quant), ("dequantize", deq), ("reference_linear_fp64", ref)], \
            work, desc

    def release(self):
        self.copies = self.xs = self.ys = self.wss = None

    def config(self):
        return {"workload": self.name,
                "layers": [{"name": nm, "m": int(x.shape[0]), "n": int(w.shape[0]),
                            "k": int(w.shape[1])} for nm, x, w in self.layers_np],
                "format": "INT4 asymmetric, group 128, fp16 scale, 4-bit zero"
                          + (", act-order (seeded synthetic channel order)"
                             if self.act_order is not None else ""),
                "calls": ["+".join(self.layers_np[j][0] for j in u) for u in self.units],
                "weight_copies": len(self.copies)}


class NF4Layer(Workload):
    dtype = "bf16"

    def setup(self):
        import torch
        import bit_quantized_linear_int4_amd as wq
        self.wq = wq
        (_, x, w), = self.layers_np
        n, k = w.shape
        m = x.shape[0]
        wd = torch.from_numpy(w.view("uint16").astype("int16")).cuda().view(torch.bfloat16)
        qw = wq.alloc_nf4(n, k, double_quant=True)
        wq.wq_pack_nf4(wd, 64, True, 256, qw.codes, qw.scales, qw.scales2)
        self.x = torch.from_numpy(x.view("uint16").astype("int16")).cuda().view(torch.bfloat16)
        self.y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        reps = _copies_needed(qw.nbytes())
        self.copies = [qw] + [qw.clone() for _ in range(reps - 1)]
        self.nbytes = qw.nbytes() + m * k * 2 + m * n * 2
        self.nflops = 2 * m * n * k
        self.kernel = "stream" if m <= 16 else "gemm"
        fam = "stream dequant-GEMV" if m <= 16 else "dequant-GEMM"
        self.kernel_desc = f"nf4 {fam} (M={m}, N={n}, K={k})"

    def step_calls(self, copy):
        qw = self.copies[copy % len(self.copies)]
        return [lambda: self.wq.wq_linear_w4a16(self.x, qw, self.y, None)]

    dominant_calls = step_calls

    def work_per_step(self):
        return self.nbytes if self.unit == "GB/s" else self.nflops

    dominant_work = work_per_step

    def cpu_stages(self):
        import numpy as np
        from oracle import nf4, linear, numerics
        (_, x, w), = self.layers_np
        rows = 4096 if self.unit == "GB/s" else 1024
        ws = numerics.bf16_bits_to_f32(w[:rows])
        xs = numerics.bf16_bits_to_f32(x)
        st = {}

        def quant():
            st["q"] = nf4.quantize(ws, double_quant=True)

        def deq():
            st["wh"] = nf4.dequantize(*st["q"], ws.shape, out_dtype="bf16")

        def ref():
            linear.reference(xs, st["wh"])
        m, k = x.shape
        work = (rows * k // 2 + rows * k // 64 + m * k * 2 + m * rows * 2
                if self.unit == "GB/s" else 2 * m * rows * k)
        return [("quantize_pack", quant), ("dequantize", deq), ("reference_linear_fp64", ref)], \
            work, f"rows 0..{rows - 1} of {w.shape[0]}, M={m}, K={k}"

    def release(self):
        self.copies = self.x = self.y = None

    def config(self):
        (_, x, w), = self.layers_np
        return {"workload": self.name, "m": int(x.shape[0]), "n": int(w.shape[0]),
                "k": int(w.shape[1]),
                "format": "NF4 block 64, int8 double-quantized absmax (block 256)",
                "weight_copies": len(self.copies)}


class Int8Layer(Workload):
    kernel = "int8"

    def setup(self):
        import torch
        import bit_quantized_linear_int4_amd as wq
        self.wq = wq
        (_, x, w), = self.layers_np
        n, k = w.shape
        m = x.shape[0]
        qw = wq.alloc_int8(n, k)
        wq.wq_quantize_groupwise(torch.from_numpy(w).cuda(), 8, k, 1, qw.codes, qw.scales)
        self.x = torch.from_numpy(x).cuda()
        self.y = torch.empty((m, n), dtype=torch.float16, device="cuda")
        need = wq.wq_linear_int8_decomp_workspace(m, k)
        self.ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        reps = _copies_needed(qw.nbytes())
        self.copies = [qw] + [qw.clone() for _ in range(reps - 1)]
        self.nbytes = qw.nbytes() + m * k * 2 + m * n * 2
        self.kernel_desc = f"LLM.int8 decomposition (M={m}, N={n}, K={k})"

    def step_calls(self, copy):
        qw = self.copies[copy % len(self.copies)]
        return [lambda: self.wq.wq_linear_int8_decomp(self.x, qw, 6.0, self.y, self.ws)]

    dominant_calls = step_calls

    def work_per_step(self):
        return self.nbytes

    dominant_work = work_per_step

    def cpu_stages(self):
        from oracle import llm_int8
        (_, x, w), = self.layers_np
        rows = 1024
        wsub = w[:rows]
        st = {}

        def quant():
            st["q"] = llm_int8.quantize_rows(wsub)

        def lin():
            llm_int8.linear(x, *st["q"], 6.0)
        m, k = x.shape
        work = rows * k + rows * 4 + m * k * 2 + m * rows * 2
        return [("quantize_rows", quant), ("decomposition_fp64", lin)], \
            work, f"rows 0..{rows - 1} of {w.shape[0]}, M={m}, K={k}"

    def release(self):
        self.copies = self.x = self.y = self.ws = None

    def config(self):
        (_, x, w), = self.layers_np
        return {"workload": self.name, "m": int(x.shape[0]), "n": int(w.shape[0]),
                "k": int(w.shape[1]), "threshold": 6.0,
                "format": "int8 per output row (absmax/127), fp16 outlier columns",
                "weight_copies": len(self.copies)}


def make_workload(name):
    import workloads
    if name == "mlp_decode":
        return W4Layers("mlp_decode_m16_7b", workloads.mlp_decode(), "GB/s")
    if name == "decode_m1":
        d = workloads.decode_m1()
        return W4Layers("decode_m1_4096x4096", [("proj", d["x"], d["w"])], "GB/s")
    if name == "decode_m1_actorder":
        d = workloads.decode_m1()
        wl = W4Layers("decode_m1_actorder_4096x4096", [("proj", d["x"], d["w"])], "GB/s")
        wl.act_order = workloads.SEEDS["decode_m1"]
        return wl
    if name == "prefill":
        return W4Layers("prefill_m2048_7b", workloads.prefill(), "TFLOP/s")
    if name in ("nf4_m1", "nf4_m512"):
        d = workloads.nf4_layer()
        m = 1 if name == "nf4_m1" else 512
        return NF4Layer(f"nf4_8b_m{m}", [("w", d["x"][m], d["w"])],
                        "GB/s" if m == 1 else "TFLOP/s")
    if name == "int8_70b":
        d = workloads.int8_70b()
        return Int8Layer("llm_int8_70b_m256", [("w", d["x"], d["w"])], "GB/s")
    raise SystemExit(f"unknown workload {name}")


# ------------------------------------------------------------------- timing
def timed_graph(calls_for_step, count, warm_eager):
    """Capture `count` steps into one graph; run `warm_eager` eager steps
    and one untimed replay; return the replay time in ms (HIP events on the
    capture stream)."""
    import torch
    for s in range(warm_eager):
        for c in calls_for_step(s):
            c()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for s in range(count):
            for c in calls_for_step(s):
                c()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def traffic_from_profile(wl):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{wl.name}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            fields[k.strip()] = v.strip()
    src = os.path.join(ROOT, KERNEL_SOURCES[wl.kernel])
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("source_sha256") != sha:
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_threads():
    """Threads for the all-cores setting: the cores this process may run on,
    at most 16 (the host CPU share of one GPU on the measurement boxes)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def oracle_stage_times(wl, threads, budget_s=5.0, min_reps=3):
    """Median wall time of each oracle stage at `threads` BLAS/OpenMP
    threads: the whole path (every stage once) repeated at least `min_reps`
    times and until `budget_s` seconds of CPU work have run.  Returns the
    medians, the work of one pass, the sample's description and the count
    of repetitions."""
    import statistics
    import threadpoolctl
    stages, work, desc = wl.cpu_stages()
    med = {}
    reps = 0
    t_start = time.perf_counter()
    with threadpoolctl.threadpool_limits(limits=threads):
        while reps < min_reps or time.perf_counter() - t_start < budget_s:
            for name, fn in stages:
                t0 = time.perf_counter()
                fn()
                med.setdefault(name, []).append(time.perf_counter() - t0)
            reps += 1
    med = {k: statistics.median(v) for k, v in med.items()}
    return med, work, desc, reps


def cpu_baseline(wls):
    """The oracle (as it stands) on the host cores: every stage of the first
    workload timed at 1 thread and at all threads (medians over a bounded
    number of repetitions), the whole
    path's rate on the sample as `value`; the same for the secondary
    workload."""
    allc = cpu_threads()
    out = {}
    for i, wl in enumerate(wls):
        one, work, desc, reps1 = oracle_stage_times(wl, 1)
        many, _, _, repsn = oracle_stage_times(wl, allc)
        scale = 1e9 if wl.unit == "GB/s" else 1e12
        rec = {"value": round(work / sum(many.values()) / scale, 6), "unit": wl.unit,
               "cores": allc, "kind": "oracle",
               "sample": f"{wl.name}: {desc}; every stage once per repetition, medians over "
                         f"{reps1} repetitions at 1 thread and {repsn} at {allc} threads "
                         "(at least 3, and at least 5 s of work per setting)",
               "value_1_thread": round(work / sum(one.values()) / scale, 6),
               "stages_s_1_thread": {k: round(v, 4) for k, v in one.items()},
               f"stages_s_{allc}_threads": {k: round(v, 4) for k, v in many.items()}}
        if i == 0:
            out.update(rec)
            out.update({"nproc": os.cpu_count(), "cpu_model": cpu_model(),
                        "threads_note": "NumPy elementwise stages run on one thread in both "
                                        "settings; only the fp64 BLAS product uses more"})
        else:
            out["secondary"] = rec
    return out


# The pages' own figures, all on NVIDIA GPUs and all end-to-end model numbers
# (no page gives a kernel-level figure for this path): context only.
PAGES_CONTEXT = [
    {"figure": "LLM.int8 generation speed relative to FP16", "value": "about 1.05-1.1x",
     "hardware": "A100 80G", "workload": "13B model",
     "page": "LLM quantization selection: five mainstream schemes compared, section 2.2"},
    {"figure": "4-bit weights of a 7B model", "value": "about 3.5 GB (14 GB in FP16)",
     "page": "the quantization-concepts article, opening"},
    {"figure": "LLaMA-2-7B decode throughput", "value":
     "FP16 95 tok/s, GPTQ-4bit 110, AWQ-4bit 125, bitsandbytes NF4 70",
     "hardware": "A100 80G",
     "page": "Inference & deployment 05: quantized deployment compared, section 9.2"},
    {"figure": "group size 32 against 128", "value": "about 8% slower generation",
     "hardware": "RTX 3060", "workload": "7B, 4-bit",
     "page": "Open-source model quantization guide: GGUF, GPTQ, AWQ, section 4.3"},
]


def copy_probe(mib):
    """A plain device copy of known size (reads and writes `mib` MiB per
    launch), run 5 times: the reference dispatch for scaling the rocprofv3
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    a = torch.ones((mib << 20) // 2, dtype=torch.float16, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()


def summarize_pmc(fetch_csv, write_csv, kernel_substr, copy_mib, out_path, command):
    """Write the traffic summary of the dominant kernel from two rocprofv3
    --pmc runs (FETCH_SIZE, then WRITE_SIZE), each counter scaled by what it
    reads for the plain copy of `copy_mib` MiB."""
    import csv
    import statistics

    # "NAME@THREADS" selects the dispatches of NAME whose grid has THREADS
    # work-items (one instantiation can serve several layer shapes)
    name_substr, _, grid = kernel_substr.partition("@")

    def per_dispatch(path, counter):
        rows = {}
        for r in csv.DictReader(open(path)):
            if r.get("Counter_Name") != counter:
                continue
            if grid and name_substr in r["Kernel_Name"] and r["Grid_Size"] != grid:
                continue
            rows.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return rows

    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = per_dispatch(path, counter)
        copy = [v for k, vs in rows.items() if "copy" in k.lower() or "elementwise" in k.lower()
                for v in vs]
        copy = sorted(copy)[-5:]                  # the five probe copies (largest dispatches)
        factor = statistics.median(copy) / (copy_mib * 1024.0)   # counter units per KiB moved
        kern = [v for k, vs in rows.items() if name_substr in k for v in vs]
        res[counter] = (statistics.mean(kern) / factor * 1024.0, factor, len(kern))
    fetch, write = res["FETCH_SIZE"][0], res["WRITE_SIZE"][0]
    src = os.path.join(ROOT, KERNEL_SOURCES["stream" if "stream" in name_substr else
                                            ("int8" if "int8" in name_substr else "gemm")])
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    with open(out_path, "w") as f:
        f.write(f"# HBM traffic of one launch of the kernels matching '{kernel_substr}',\n")
        f.write("# from two rocprofv3 --pmc runs, each counter scaled by its reading for a\n")
        f.write(f"# plain device copy of {copy_mib} MiB (reads and writes {copy_mib} MiB).\n")
        f.write(f"# command: {command}\n")
        f.write(f"fetch_factor_per_kib={res['FETCH_SIZE'][1]:.6f}\n")
        f.write(f"write_factor_per_kib={res['WRITE_SIZE'][1]:.6f}\n")
        f.write(f"dispatches={res['FETCH_SIZE'][2]}\n")
        f.write(f"fetch_bytes_per_launch={fetch:.0f}\n")
        f.write(f"write_bytes_per_launch={write:.0f}\n")
        f.write(f"hbm_bytes_per_launch={fetch + write:.0f}\n")
        f.write(f"source={os.path.relpath(src, ROOT)}\n")
        f.write(f"source_sha256={sha}\n")
    print(open(out_path).read())


def summarize_counters(csv_paths, kernel_substr, avg_ns, out_path, command):
    """Write the mean per-dispatch value of every counter in one or more
    rocprofv3 --pmc runs for the kernels matching NAME[@GRID_WORK_ITEMS],
    with the matrix-core busy share derived from them.  avg_ns is the
    kernel's average duration (from the kernel trace of the same command),
    used for the effective clock."""
    import csv
    import statistics
    name_substr, _, grid = kernel_substr.partition("@")
    vals = {}
    for path in csv_paths:
        for r in csv.DictReader(open(path)):
            if name_substr not in r["Kernel_Name"] or (grid and r["Grid_Size"] != grid):
                continue
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    mean = {k: statistics.mean(v) for k, v in vals.items()}
    with open(out_path, "w") as f:
        f.write(f"# rocprofv3 counters, mean per dispatch, kernels matching '{kernel_substr}'\n")
        f.write(f"# command: {command}\n")
        for k in sorted(mean):
            f.write(f"{k}={mean[k]:.6g}  # {len(vals[k])} dispatches\n")
        if "GRBM_GUI_ACTIVE" in mean and avg_ns > 0:
            # GRBM_GUI_ACTIVE is summed over the 8 XCDs; SQ_* counters over
            # every CU (256) and SIMD (4 per CU)
            cyc = mean["GRBM_GUI_ACTIVE"] / 8.0
            ghz = cyc / avg_ns
            if ghz <= 2.4:
                f.write(f"# derived: active cycles per XCD {cyc:.0f} (GRBM_GUI_ACTIVE / 8); over the "
                        f"traced {avg_ns / 1e3:.2f} us dispatch that is {ghz:.3f} GHz, an upper "
                        "bound on the clock (counter runs lengthen dispatches)\n")
            else:
                f.write(f"# derived: active cycles per XCD {cyc:.0f} (GRBM_GUI_ACTIVE / 8), "
                        f"{cyc / 2.4e3:.2f} us at 2.4 GHz against the traced {avg_ns / 1e3:.2f} us: "
                        "the counter run stretches a dispatch this short, so the shares below "
                        "are taken over that longer window and understate the kernel's own\n")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
                f.write(f"mfma_busy_share={mean['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024.0 * cyc):.4f}"
                        "  # SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x active cycles)\n")
            if "SQ_LDS_BANK_CONFLICT" in mean:
                f.write(f"lds_bank_conflict_share={mean['SQ_LDS_BANK_CONFLICT'] / (256.0 * cyc):.4f}"
                        "  # SQ_LDS_BANK_CONFLICT / (256 CUs x active cycles)\n")
            if "TCP_PENDING_STALL_CYCLES" in mean:
                f.write(f"l1_pending_stall_share={mean['TCP_PENDING_STALL_CYCLES'] / (256.0 * cyc):.4f}"
                        "  # TCP_PENDING_STALL_CYCLES / (256 CUs x active cycles)\n")
        if "TCP_TCC_READ_REQ" in mean and "TCP_TCC_READ_REQ_LATENCY" in mean:
            f.write(f"l1_to_l2_read_latency_cycles="
                    f"{mean['TCP_TCC_READ_REQ_LATENCY'] / mean['TCP_TCC_READ_REQ']:.1f}\n")
        if "TCC_HIT" in mean and "TCC_MISS" in mean:
            f.write(f"l2_hit_rate={mean['TCC_HIT'] / (mean['TCC_HIT'] + mean['TCC_MISS']):.4f}\n")
    print(open(out_path).read())


def summarize_trace(prof_dir, bench_json, title, out_path, command):
    """Write a rocprofv3 --kernel-trace --stats summary: per kernel and
    launch grid (one grid per layer shape), the calls and the average /
    min / max duration of the dispatches, with the bench line of the same
    run."""
    import csv
    import statistics
    per = {}
    order = []   # (start, key, duration) of every dispatch
    for r in csv.DictReader(open(os.path.join(prof_dir, "run_kernel_trace.csv"))):
        grid = tuple(int(r[f"Grid_Size_{a}"]) // max(1, int(r[f"Workgroup_Size_{a}"]))
                     for a in "XYZ")
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        per.setdefault((r["Kernel_Name"], grid), []).append(dur)
        order.append((int(r["Start_Timestamp"]), (r["Kernel_Name"], grid), dur))
    order.sort()
    total = sum(sum(v) for v in per.values())
    rows = sorted(per.items(), key=lambda kv: -sum(kv[1]))
    with open(out_path, "w") as f:
        f.write(f"# rocprofv3 kernel-trace summary: {title}\n")
        f.write("# command (repository root, on one MI355X):\n")
        f.write(f"#   {command}\n")
        f.write("# columns: calls, average ns, min ns, max ns, share of GPU time, "
                "workgroups (x,y,z), kernel\n")
        for (name, grid), v in rows:
            f.write(f"{len(v):6d} {statistics.mean(v):12.1f} {min(v):9d} {max(v):9d} "
                    f"{100.0 * sum(v) / total:6.2f}%  {grid}  {name[:140]}\n")
        if bench_json and os.path.exists(bench_json):
            d = json.load(open(bench_json))
            rf = d.get("roofline", {})
            f.write("\n# bench.py line of the same run (graph-replayed; kernel time from HIP events):\n")
            f.write(f"#   value {d['value']} {d['unit']}, ms_per_step {d['ms_per_step']}, "
                    f"dominant kernel avg_launch_us {rf.get('avg_launch_us')} "
                    f"({rf.get('kernel')})\n")
            # bench.py times the dominant kernel last, in a region of its own:
            # the last `launches` dispatches of the last kernel shape traced
            n = int(rf.get("launches") or 0)
            work = [o for o in order if "copy" not in o[1][0].lower()
                    and "elementwise" not in o[1][0]]
            if n > 0 and work:
                key = work[-1][1]
                tail = [o[2] for o in work if o[1] == key][-n:]
                f.write(f"# traced average of that region ({len(tail)} dispatches of "
                        f"{key[0][:60]}..., {key[1]}): {statistics.mean(tail):.1f} ns; the "
                        "table's average also holds the warmup and the full steps\n")
    print(open(out_path).read())


def measure(wl, steps, warmup):
    """Graph-replayed step time and the dominant kernel's average launch
    time of a set-up workload, as the bench line's value / roofline fields."""
    log(f"[bench] timing {steps} steps of {wl.name} after {warmup} warmup")
    ms = timed_graph(wl.step_calls, steps, warmup)
    ms_step = ms / steps
    log(f"[bench] timing the dominant kernel: {wl.kernel_desc}")
    ndom = len(wl.dominant_calls(0))
    ms_dom = timed_graph(wl.dominant_calls, steps, 2)
    launches = steps * ndom
    us_launch = ms_dom * 1e3 / launches
    scale = 1e9 if wl.unit == "GB/s" else 1e12
    value = wl.work_per_step() / (ms_step * 1e-3) / scale
    achieved = wl.dominant_work() / (us_launch * 1e-6) / scale
    bound = "hbm" if wl.unit == "GB/s" else "mfma"
    peak = HBM_PEAK_GBS if bound == "hbm" else MFMA16_PEAK_TFLOPS
    return {
        "value": round(value, 3),
        "unit": wl.unit,
        "ms_per_step": round(ms_step, 5),
        "dtype": wl.dtype,
        "config": wl.config(),
        "roofline": {"bound": bound, "achieved": round(achieved, 3), "peak": peak,
                     "unit": wl.unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic_from_profile(wl),
                     "kernel": wl.kernel_desc, "avg_launch_us": round(us_launch, 3),
                     "work_per_launch": wl.dominant_work(), "launches": launches},
    }


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-trace":
        # --summarize-trace PROF_DIR BENCH_JSON TITLE OUT "COMMAND"
        a = sys.argv[2:]
        summarize_trace(a[0], a[1], a[2], a[3], a[4])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-pmc":
        # --summarize-pmc FETCH_CSV WRITE_CSV KERNEL_SUBSTR COPY_MIB OUT "COMMAND"
        a = sys.argv[2:]
        summarize_pmc(a[0], a[1], a[2], int(a[3]), a[4], a[5])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-counters":
        # --summarize-counters KERNEL[@GRID] AVG_NS OUT "COMMAND" CSV [CSV ...]
        a = sys.argv[2:]
        summarize_counters(a[4:], a[0], float(a[1]), a[2], a[3])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="metric",
                    choices=["metric", "mlp_decode", "decode_m1", "decode_m1_actorder", "prefill",
                             "nf4_m1", "nf4_m512", "int8_70b"],
                    help="metric (default): the M = 1 decode layer as the value, with the "
                         "M = 2048 prefill step as the secondary figure in the same line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB five times (the reference "
                         "dispatch for scaling rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}): the quantized linear "
              "path here is single-GPU; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(args.copy_probe)
    names = ["decode_m1", "prefill"] if args.workload == "metric" else [args.workload]
    results, wls = [], []
    for name in names:
        wl = make_workload(name)
        log(f"[bench] setting up {wl.name}")
        wl.setup()
        results.append(measure(wl, args.steps, args.warmup))
        wls.append(wl)
        wl.release()
        torch.cuda.empty_cache()
    head = results[0]
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic: seeded N(0,0.02) weights, N(0,1) activations (fixed outlier "
                "channels where the workload has them), random-init layers of the 7B/8B/70B "
                "shapes",
        "config": head["config"],
        "roofline": head["roofline"],
    }
    if len(results) > 1:
        sec = dict(results[1])
        sec["metric"] = "W4A16 g128 prefill dequant-GEMM TFLOP/s (M=2048)"
        out["secondary"] = sec
    out["context"] = PAGES_CONTEXT
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(wls)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
