"""GPU parity of the NF4 path (blockwise absmax, double quantization, bf16
compute) against the CPU oracle, through the C ABI.

Codes, first-level int8 absmax codes and second-level scales are bit-exact;
the dequantized weights are bit-exact; float outputs are judged on fp32
output (a bf16 output's own rounding is close to the 2e-3 budget) and, for
bf16 outputs, with the output rounding added to the bound.
"""

import numpy as np
import pytest
import torch

import bit_quantized_linear_int4_amd as wq
import workloads
from oracle import fp4, linear, nf4
from gpu_util import check_close, dev, host16, say, to_np, torch_dtype

pytestmark = pytest.mark.gpu


def gpu_pack(w_dev, double_quant=True):
    n, k = w_dev.shape
    qw = wq.alloc_nf4(n, k, double_quant=double_quant)
    wq.wq_pack_nf4(w_dev, 64, double_quant, 256, qw.codes, qw.scales, qw.scales2)
    return qw


@pytest.mark.parametrize("n,k,dtype,dq", [
    (64, 512, "bf16", True),
    (37, 640, "bf16", True),       # numel not a multiple of 256 blocks
    (37, 640, "f16", False),
    (14336, 4096, "bf16", True),   # the 8B-shaped layer
])
def test_pack_nf4_bitexact(n, k, dtype, dq):
    say(f"pack_nf4 n={n} k={k} dtype={dtype} dq={dq}")
    w = workloads.weights(n, k, 40 + n, 1, dtype=dtype)
    if n == 64:
        wv = host16(w, dtype).copy()
        wv[0, :64] = 0                      # all-zero block -> code 7
        wv[1, :64] = np.linspace(-1, 1, 64)  # exact +-absmax present
        w = workloads.to_bf16_bits(wv) if dtype == "bf16" else wv.astype(np.float16)
    qw = gpu_pack(dev(w, dtype), dq)
    torch.cuda.synchronize()
    ref_codes, ref_a, ref_c2 = nf4.quantize(host16(w, dtype), double_quant=dq)
    assert np.array_equal(qw.codes.cpu().numpy(), ref_codes)
    if dq:
        assert np.array_equal(qw.scales.cpu().numpy(), ref_a)
        assert np.array_equal(qw.scales2.cpu().numpy(), ref_c2)
    else:
        assert np.array_equal(qw.scales.cpu().numpy(), ref_a)


@pytest.mark.parametrize("dq,odt", [(True, "bf16"), (False, "bf16"), (True, "f16")])
def test_dequantize_nf4_bitexact(dq, odt):
    say(f"dequantize_nf4 dq={dq} odt={odt}")
    n, k = 40, 1024
    w = workloads.weights(n, k, 77, 1, dtype="bf16")
    qw = gpu_pack(dev(w, "bf16"), dq)
    out = torch.empty((n, k), dtype=torch_dtype(odt), device="cuda")
    wq.wq_dequantize(qw, out)
    torch.cuda.synchronize()
    c, a, c2 = nf4.quantize(host16(w, "bf16"), double_quant=dq)
    ref = nf4.dequantize(c, a, c2, (n, k), out_dtype=odt)
    assert np.array_equal(to_np(out), ref)


def oracle_y(x, w, xdt, dq=True, rows=None):
    n, k = w.shape
    c, a, c2 = nf4.quantize(host16(w, xdt), double_quant=dq)
    wh = nf4.dequantize(c, a, c2, (n, k), out_dtype=xdt)
    xs = host16(x, xdt)
    return linear.reference(xs if rows is None else xs[rows], wh)


def run(x, w, xdt, ydt, dq=True, qw=None):
    m = x.shape[0]
    n = w.shape[0]
    if qw is None:
        qw = gpu_pack(dev(w, xdt), dq)
    y = torch.empty((m, n), dtype=torch_dtype(ydt), device="cuda")
    need = wq.wq_linear_w4a16_workspace(m, qw)
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda") if need else None
    wq.wq_linear_w4a16(dev(x, xdt), qw, y, ws)
    torch.cuda.synchronize()
    return to_np(y), qw


@pytest.mark.parametrize("m,n,k,xdt,ydt,dq", [
    (1, 300, 1152, "bf16", "f32", True),
    (1, 1000, 4096, "bf16", "bf16", True),
    (4, 272, 640, "f16", "f32", False),
    (16, 512, 2048, "bf16", "f32", True),
    (1, 208, 11008, "bf16", "f32", True),
    (9, 160, 5120, "bf16", "f32", False),
    (40, 300, 1152, "bf16", "f32", True),   # absmax not stageable: the generic GEMM
    (512, 1024, 4096, "bf16", "f32", True),
    (40, 296, 1152, "bf16", "f32", True),   # staged absmax, ragged m and n tiles
    (64, 256, 2048, "f16", "bf16", True),   # fp16 activations
    (24, 128, 8192, "bf16", "f32", True),   # 32 KB of staged absmax codes: the limit
    (20, 160, 8320, "bf16", "f32", True),   # past it: the generic GEMM
    (40, 296, 1152, "bf16", "f32", False),  # fp32 absmax: the generic GEMM
])
def test_linear_nf4_parity(m, n, k, xdt, ydt, dq):
    say(f"linear_nf4 m={m} n={n} k={k} x={xdt} y={ydt} dq={dq}")
    seed = 300 + m + n
    x, _ = workloads.activations(m, k, seed, 0, dtype=xdt)
    w = workloads.weights(n, k, seed, 1, dtype=xdt)
    y, _ = run(x, w, xdt, ydt, dq)
    rel = check_close(y, oracle_y(x, w, xdt, dq), ydt)
    say(f"  max-rel {rel:.2e}")


def test_linear_nf4_full_layer(record_margin):
    """The 8B-shaped layer (14336 x 4096) at M = 1 (all outputs) and M = 512
    (32 sampled rows), fp32 output."""
    say("linear_nf4_full n=14336 k=4096")
    d = workloads.nf4_layer()
    qw = None
    for m in (1, 512):
        y, qw = run(d["x"][m], d["w"], "bf16", "f32", True, qw)
        rows = None if m == 1 else np.random.default_rng(1).choice(m, 32, replace=False)
        ref = oracle_y(d["x"][m], d["w"], "bf16", True, rows)
        rel = check_close(y if rows is None else y[rows], ref, "f32")
        say(f"  m={m} max-rel {rel:.2e}")
        record_margin(f"NF4 14336x4096 M={m}" + ("" if rows is None else " (32 rows sampled)"),
                      rel)


@pytest.mark.parametrize("m,n,k", [(2048, 11008, 1024), (2048, 4296, 1024)])
def test_linear_nf4_wide_prefill(m, n, k):
    """NF4 prefill at M = 2048 over 11008 columns (three rounds of 256-wide
    tiles) and 4296 columns (seven-wave 224-wide tiles: 320 against 272
    tiles, both two rounds); 24 sampled rows, the last among them, against
    the oracle, every column."""
    say(f"linear_nf4_wide m={m} n={n} k={k}")
    seed = 900 + n
    x, _ = workloads.activations(m, k, seed, 0, dtype="bf16")
    w = workloads.weights(n, k, seed, 1, dtype="bf16")
    y, _ = run(x, w, "bf16", "bf16", True)
    rows = np.random.default_rng(n).choice(m, 24, replace=False)
    rows[0] = m - 1
    rel = check_close(y[rows], oracle_y(x, w, "bf16", True, rows), "bf16")
    say(f"  max-rel {rel:.2e}")


# ---------------------------------------------------------------- FP4 (E2M1)

def gpu_pack_fp4(w_dev, double_quant=True):
    n, k = w_dev.shape
    qw = wq.alloc_fp4(n, k, double_quant=double_quant)
    wq.wq_pack_fp4(w_dev, 64, double_quant, 256, qw.codes, qw.scales, qw.scales2)
    return qw


@pytest.mark.parametrize("n,k,dtype,dq", [
    (64, 512, "bf16", True),
    (37, 640, "f16", False),       # numel not a multiple of 256 blocks
    (14336, 4096, "bf16", True),   # the 8B-shaped layer
])
def test_pack_fp4_bitexact(n, k, dtype, dq):
    say(f"pack_fp4 n={n} k={k} dtype={dtype} dq={dq}")
    w = workloads.weights(n, k, 50 + n, 1, dtype=dtype)
    if n == 64:
        wv = host16(w, dtype).copy()
        wv[0, :64] = 0                        # all-zero block -> code 0
        wv[1, :64] = np.linspace(-1, 1, 64)    # exact +-absmax -> codes 15, 7
        w = workloads.to_bf16_bits(wv) if dtype == "bf16" else wv.astype(np.float16)
    qw = gpu_pack_fp4(dev(w, dtype), dq)
    torch.cuda.synchronize()
    ref_codes, ref_a, ref_c2 = fp4.quantize(host16(w, dtype), double_quant=dq)
    assert np.array_equal(qw.codes.cpu().numpy(), ref_codes)
    assert np.array_equal(qw.scales.cpu().numpy(), ref_a)
    if dq:
        assert np.array_equal(qw.scales2.cpu().numpy(), ref_c2)


@pytest.mark.parametrize("dq,odt", [(True, "bf16"), (False, "f16")])
def test_dequantize_fp4_bitexact(dq, odt):
    say(f"dequantize_fp4 dq={dq} odt={odt}")
    n, k = 40, 1024
    w = workloads.weights(n, k, 78, 1, dtype="bf16")
    qw = gpu_pack_fp4(dev(w, "bf16"), dq)
    out = torch.empty((n, k), dtype=torch_dtype(odt), device="cuda")
    wq.wq_dequantize(qw, out)
    torch.cuda.synchronize()
    c, a, c2 = fp4.quantize(host16(w, "bf16"), double_quant=dq)
    assert np.array_equal(to_np(out), fp4.dequantize(c, a, c2, (n, k), out_dtype=odt))


@pytest.mark.parametrize("m,n,k,xdt,ydt,dq", [
    (1, 300, 1152, "bf16", "f32", True),
    (4, 272, 640, "f16", "f32", False),
    (16, 512, 2048, "bf16", "f32", True),
    (40, 300, 1152, "bf16", "f32", True),
    (512, 1024, 4096, "bf16", "f32", True),
    (40, 296, 1152, "bf16", "f32", True),   # staged absmax, ragged m and n tiles
    (72, 512, 2048, "f16", "f32", True),    # fp16 activations
])
def test_linear_fp4_parity(m, n, k, xdt, ydt, dq):
    say(f"linear_fp4 m={m} n={n} k={k} x={xdt} y={ydt} dq={dq}")
    seed = 500 + m + n
    x, _ = workloads.activations(m, k, seed, 0, dtype=xdt)
    w = workloads.weights(n, k, seed, 1, dtype=xdt)
    qw = gpu_pack_fp4(dev(w, xdt), dq)
    y = torch.empty((m, n), dtype=torch_dtype(ydt), device="cuda")
    wq.wq_linear_w4a16(dev(x, xdt), qw, y, None)
    torch.cuda.synchronize()
    c, a, c2 = fp4.quantize(host16(w, xdt), double_quant=dq)
    wh = fp4.dequantize(c, a, c2, (n, k), out_dtype=xdt)
    rel = check_close(to_np(y), linear.reference(host16(x, xdt), wh), ydt)
    say(f"  max-rel {rel:.2e}")


# ------------------------------------------------ NF4 / FP4 gate/up pairs

def _fmt_oracle(fmt, w, xdt, dq):
    mod = nf4 if fmt == "nf4" else fp4
    c, a, c2 = mod.quantize(host16(w, xdt), double_quant=dq)
    return mod.dequantize(c, a, c2, w.shape, out_dtype=xdt)


@pytest.mark.parametrize("fmt,m,n,k,xdt,ydt,dq", [
    ("nf4", 1, 14336, 4096, "bf16", "f32", True),   # the 8B gate/up shape, one token
    ("nf4", 1, 300, 1152, "bf16", "bf16", True),    # ragged n, odd unit count
    ("nf4", 4, 1000, 2048, "bf16", "f32", True),
    ("nf4", 16, 14336, 4096, "bf16", "f32", True),  # four tiles of each matrix
    ("nf4", 16, 4100, 1024, "f16", "f32", False),   # fp32 absmax: loaded per unit
    ("nf4", 16, 14336, 1024, "bf16", "f32", False), # fp32 absmax, 896 tiles: two per matrix
    ("nf4", 40, 300, 1152, "bf16", "f32", True),    # prefill rows: two GEMMs
    ("fp4", 1, 1000, 2048, "bf16", "f32", True),
    ("fp4", 16, 5120, 1024, "f16", "bf16", False),
])
def test_gate_up_pair_nf4_fp4(fmt, m, n, k, xdt, ydt, dq):
    """Both outputs of an NF4 / FP4 pair against the oracle, and equal bit
    for bit to the two single-matrix calls (the pair runs the same per-tile
    schedule)."""
    say(f"gate_up {fmt} m={m} n={n} k={k} x={xdt} y={ydt} dq={dq}")
    seed = 600 + m + n
    x_np, _ = workloads.activations(m, k, seed, 0, dtype=xdt)
    wg_np = workloads.weights(n, k, seed, 1, dtype=xdt)
    wu_np = workloads.weights(n, k, seed, 2, dtype=xdt)
    pack = gpu_pack if fmt == "nf4" else gpu_pack_fp4
    qg, qu = pack(dev(wg_np, xdt), dq), pack(dev(wu_np, xdt), dq)
    x = dev(x_np, xdt)
    yg = torch.empty((m, n), dtype=torch_dtype(ydt), device="cuda")
    yu = torch.empty_like(yg)
    wq.wq_linear_w4a16_gate_up(x, qg, qu, yg, yu, act=0)
    g1 = torch.empty_like(yg)
    u1 = torch.empty_like(yg)
    wq.wq_linear_w4a16(x, qg, g1, None)
    wq.wq_linear_w4a16(x, qu, u1, None)
    torch.cuda.synchronize()
    xs = host16(x_np, xdt)
    rg = check_close(to_np(yg), linear.reference(xs, _fmt_oracle(fmt, wg_np, xdt, dq)), ydt)
    ru = check_close(to_np(yu), linear.reference(xs, _fmt_oracle(fmt, wu_np, xdt, dq)), ydt)
    say(f"  max-rel gate {rg:.2e} up {ru:.2e}")
    assert np.array_equal(to_np(yg), to_np(g1)) and np.array_equal(to_np(yu), to_np(u1))


@pytest.mark.parametrize("m,n,k", [(1, 1000, 2048), (16, 5120, 1024), (96, 1000, 2048)])
def test_gate_up_nf4_swiglu(m, n, k):
    """silu(gate) * up of an NF4 pair against the oracle's product of its own
    fp64 projections (past 16 rows the two GEMMs store fp32 gate and up, so
    the product is still formed from fp32 sums)."""
    say(f"gate_up_swiglu nf4 m={m} n={n} k={k}")
    seed = 700 + m + n
    x_np, _ = workloads.activations(m, k, seed, 0, dtype="bf16")
    wg_np = workloads.weights(n, k, seed, 1, dtype="bf16")
    wu_np = workloads.weights(n, k, seed, 2, dtype="bf16")
    qg, qu = gpu_pack(dev(wg_np, "bf16")), gpu_pack(dev(wu_np, "bf16"))
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    yu = torch.empty_like(y) if m > 16 else None
    wq.wq_linear_w4a16_gate_up(dev(x_np, "bf16"), qg, qu, y, yu, act=1)
    torch.cuda.synchronize()
    xs = host16(x_np, "bf16")
    ref = linear.silu_gated(linear.reference(xs, _fmt_oracle("nf4", wg_np, "bf16", True)),
                            linear.reference(xs, _fmt_oracle("nf4", wu_np, "bf16", True)))
    rel = check_close(to_np(y), ref, "f32")
    say(f"  max-rel {rel:.2e}")
