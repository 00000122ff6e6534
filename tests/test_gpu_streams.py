"""Calls on two streams at once: the library keeps no state between calls
(every scratch byte comes from the caller's workspace), so independent calls
issued concurrently on two streams must give the same bits as the same calls
run one after another on one stream.  Covers the decode GEMV (M = 1 and the
gate/up pair), the prefill GEMM, NF4 and the LLM.int8 decomposition, each
stream with its own weights, inputs, outputs and workspaces."""

import numpy as np
import pytest
import torch

import bit_quantized_linear_int4_amd as wq
import workloads
from gpu_util import dev, dev_f16, say

pytestmark = pytest.mark.gpu


def _int4(n, k, seed):
    w = workloads.weights(n, k, seed, 1)
    qw = wq.alloc_int4(n, k)
    wq.wq_quantize_groupwise(dev_f16(w), 4, 128, 0, qw.codes, qw.scales, qw.zeros)
    return qw


def _setup(seed):
    """One stream's work: weights, inputs, outputs, workspaces and the calls."""
    t = {}
    t["w1"] = _int4(4096, 4096, seed)
    t["g"], t["u"] = _int4(2048, 1024, seed + 1), _int4(2048, 1024, seed + 2)
    t["wp"] = _int4(1024, 2048, seed + 3)
    wnf = workloads.weights(1024, 1024, seed + 4, 1, dtype="bf16")
    t["nf"] = wq.alloc_nf4(1024, 1024, double_quant=True)
    wq.wq_pack_nf4(dev(wnf, "bf16"), 64, 1, 256, t["nf"].codes, t["nf"].scales, t["nf"].scales2)
    w8 = workloads.weights(512, 2048, seed + 5, 1)
    t["q8"] = wq.alloc_int8(512, 2048)
    wq.wq_quantize_groupwise(dev_f16(w8), 8, 2048, 1, t["q8"].codes, t["q8"].scales)
    t["x1"] = dev_f16(workloads.activations(1, 4096, seed + 6, 0)[0])
    t["x16"] = dev_f16(workloads.activations(16, 1024, seed + 7, 0, outliers=(3, 20.0, 80.0))[0])
    t["xp"] = dev_f16(workloads.activations(96, 2048, seed + 8, 0)[0])
    t["xn"] = dev(workloads.activations(1, 1024, seed + 9, 0, dtype="bf16")[0], "bf16")
    t["x8"] = dev_f16(workloads.activations(64, 2048, seed + 10, 0, outliers=(4, 20.0, 80.0))[0])
    t["y1"] = torch.empty((1, 4096), dtype=torch.float32, device="cuda")
    t["yg"] = torch.empty((16, 2048), dtype=torch.float16, device="cuda")
    t["yu"] = torch.empty_like(t["yg"])
    t["yp"] = torch.empty((96, 1024), dtype=torch.float32, device="cuda")
    t["yn"] = torch.empty((1, 1024), dtype=torch.bfloat16, device="cuda")
    t["y8"] = torch.empty((64, 512), dtype=torch.float32, device="cuda")
    t["ws8"] = torch.empty((wq.wq_linear_int8_decomp_workspace(64, 2048),), dtype=torch.uint8,
                           device="cuda")
    return t


def _outputs(t):
    return ("y1", "yg", "yu", "yp", "yn", "y8")


def _issue(t, s):
    """Every call of one stream's work, three times over, on stream s."""
    for _ in range(3):
        wq.wq_linear_w4a16(t["x1"], t["w1"], t["y1"], stream=s)
        wq.wq_linear_w4a16_gate_up(t["x16"], t["g"], t["u"], t["yg"], t["yu"], act=0, stream=s)
        wq.wq_linear_w4a16(t["xp"], t["wp"], t["yp"], stream=s)
        wq.wq_linear_w4a16(t["xn"], t["nf"], t["yn"], stream=s)
        wq.wq_linear_int8_decomp(t["x8"], t["q8"], 6.0, t["y8"], t["ws8"], stream=s)


def test_two_streams_match_one_stream():
    say("two streams: independent calls interleaved, against the same calls on one stream")
    a, b = _setup(1000), _setup(2000)
    torch.cuda.synchronize()
    s0 = torch.cuda.current_stream()
    _issue(a, s0)
    _issue(b, s0)
    torch.cuda.synchronize()
    ref = {(tag, k): t[k].float().cpu().numpy().copy()
           for tag, t in (("a", a), ("b", b)) for k in _outputs(t)}
    for t in (a, b):
        for k in _outputs(t):
            t[k].fill_(float("nan"))
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(2):
        _issue(a, sa)
        _issue(b, sb)
    torch.cuda.synchronize()
    for tag, t in (("a", a), ("b", b)):
        for k in _outputs(t):
            got = t[k].float().cpu().numpy()
            assert np.array_equal(got, ref[(tag, k)]), f"stream {tag}: {k} differs"
