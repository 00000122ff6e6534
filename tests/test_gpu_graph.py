"""The library's calls captured into a HIP graph (as bench.py times them)
and replayed: every replay must reproduce the eager results bit for bit
(every kernel sums in a fixed order).  Between the replays the outputs are
cleared and other eager work runs on the same stream."""

import numpy as np
import pytest
import torch

import bit_quantized_linear_int4_amd as wq
import workloads
from gpu_util import dev, dev_f16, say

pytestmark = pytest.mark.gpu


def _int4(n, k, seed, dtype="f16"):
    w = workloads.weights(n, k, seed, 1, dtype=dtype)
    qw = wq.alloc_int4(n, k)
    wq.wq_quantize_groupwise(dev(w, dtype), 4, 128, 0, qw.codes, qw.scales, qw.zeros)
    return qw


def test_graph_replay_matches_eager():
    say("graph replay: gate/up pair, down decode, INT4 and NF4 GEMMs, LLM.int8")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        gate, up = _int4(1024, 1024, 900), _int4(1024, 1024, 901)
        down = _int4(512, 2048, 902)
        wnf = workloads.weights(512, 1024, 903, 1, dtype="bf16")
        qnf = wq.alloc_nf4(512, 1024, double_quant=True)
        wq.wq_pack_nf4(dev(wnf, "bf16"), 64, 1, 256, qnf.codes, qnf.scales, qnf.scales2)
        w8 = workloads.weights(256, 1024, 904, 1)
        q8 = wq.alloc_int8(256, 1024)
        wq.wq_quantize_groupwise(dev_f16(w8), 8, 1024, 1, q8.codes, q8.scales)

        x16 = dev_f16(workloads.activations(16, 1024, 905, 0, outliers=(3, 20.0, 80.0))[0])
        xd = dev_f16(workloads.activations(16, 2048, 906, 0)[0])
        xp = dev_f16(workloads.activations(64, 1024, 907, 0)[0])
        xb = dev(workloads.activations(40, 1024, 908, 0, dtype="bf16")[0], "bf16")
        x8 = dev_f16(workloads.activations(64, 1024, 909, 0, outliers=(4, 20.0, 100.0))[0])

        outs = {
            "pair": torch.empty((16, 1024), dtype=torch.float32, device="cuda"),
            "down": torch.empty((16, 512), dtype=torch.float16, device="cuda"),
            "gemm": torch.empty((64, 1024), dtype=torch.float32, device="cuda"),
            "nf4": torch.empty((40, 512), dtype=torch.float32, device="cuda"),
            "int8": torch.empty((64, 256), dtype=torch.float32, device="cuda"),
            "count": torch.empty((1,), dtype=torch.int32, device="cuda"),
        }
        ws = torch.empty((wq.wq_linear_int8_decomp_workspace(64, 1024),), dtype=torch.uint8,
                         device="cuda")

        def calls():
            wq.wq_linear_w4a16_gate_up(x16, gate, up, outs["pair"], None, act=1)
            wq.wq_linear_w4a16(xd, down, outs["down"])
            wq.wq_linear_w4a16(xp, gate, outs["gemm"])
            wq.wq_linear_w4a16(xb, qnf, outs["nf4"])
            wq.wq_linear_int8_decomp(x8, q8, 6.0, outs["int8"], ws, outs["count"])

        calls()
        s.synchronize()
        ref = {k: v.clone() for k, v in outs.items()}
        s.synchronize()
        assert int(ref["count"].item()) == 4

        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            calls()
        other = torch.empty((16, 1024), dtype=torch.float32, device="cuda")
        for rep in range(3):
            for v in outs.values():
                v.zero_()
            s.synchronize()
            g.replay()
            s.synchronize()
            for name, v in outs.items():
                assert torch.equal(v, ref[name]), f"replay {rep}: {name} differs from eager"
            # unrelated eager work on the same stream between replays
            wq.wq_linear_w4a16(x16, up, other)
            s.synchronize()
        say("  3 replays equal to eager")
