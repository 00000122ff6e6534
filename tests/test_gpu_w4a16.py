"""GPU parity of the INT4 path against the CPU oracle, through the C ABI.

Codes, scales and zero points must match bit for bit; float outputs must be
within max|y - y_ref| / max|y_ref| <= 2e-3 of the fp64 oracle computed on the
oracle's own dequantized weights.  Inputs come from the seeded workload
generators; the oracle never sees a value produced by the GPU.
"""

import numpy as np
import pytest
import torch

import bit_quantized_linear_int4_amd as wq
import workloads
from oracle import int4, llm_int8, linear
from gpu_util import check_close, dev, dev_f16, host16, say, to_np, torch_dtype

pytestmark = pytest.mark.gpu


def edge_weights(n, k, seed, dtype="f16"):
    """N(0, 0.02) weights with degenerate groups planted in the first rows."""
    w = host16(workloads.weights(n, k, seed, 1, dtype=dtype), dtype).copy()
    if n >= 6 and k >= 128:
        w[0, :128] = 0
        w[1, :128] = 0.01
        w[2, :128] = np.abs(w[2, :128]) + 1
        w[3, :128] = -np.abs(w[3, :128]) - 2
        w[4, :128] *= 1e-4
        w[5, :128] *= 1000
    if dtype == "bf16":
        return workloads.to_bf16_bits(w)
    return w.astype(np.float16)


def gpu_quantize_int4(w_dev, group=128):
    n, k = w_dev.shape
    qw = wq.alloc_int4(n, k, group)
    wq.wq_quantize_groupwise(w_dev, 4, group, 0, qw.codes, qw.scales, qw.zeros)
    return qw


@pytest.mark.parametrize("n,k,group,dtype", [
    (64, 512, 128, "f16"),
    (37, 1152, 128, "f16"),       # ragged rows, odd group count
    (37, 1152, 128, "bf16"),
    (16, 640, 64, "f16"),
    (16, 640, 32, "bf16"),
    (4096, 4096, 128, "f16"),     # the single-layer decode shape
    (4096, 11008, 128, "f16"),    # the down-projection shape (86 groups)
])
def test_quantize_int4_bitexact(n, k, group, dtype):
    say(f"quantize_int4 n={n} k={k} group={group} dtype={dtype}")
    w = edge_weights(n, k, seed=n + k + group, dtype=dtype)
    qw = gpu_quantize_int4(dev(w, dtype), group)
    torch.cuda.synchronize()
    ref_q, ref_s, ref_z = int4.quantize(host16(w, dtype), group)
    assert np.array_equal(qw.codes.cpu().numpy().view(np.uint32), ref_q)
    assert np.array_equal(qw.scales.cpu().numpy().view(np.uint16), ref_s.view(np.uint16))
    assert np.array_equal(qw.zeros.cpu().numpy(), ref_z)


@pytest.mark.parametrize("n,k,dtype", [(33, 512, "f16"), (64, 8192, "f16"), (8, 256, "bf16")])
def test_quantize_int8_rows_bitexact(n, k, dtype):
    say(f"quantize_int8 n={n} k={k} dtype={dtype}")
    w = edge_weights(n, k, seed=7 + n, dtype=dtype)
    wd = dev(w, dtype)
    qw = wq.alloc_int8(n, k)
    wq.wq_quantize_groupwise(wd, 8, k, 1, qw.codes, qw.scales)
    torch.cuda.synchronize()
    ref_q, ref_s = llm_int8.quantize_rows(host16(w, dtype))
    assert np.array_equal(qw.codes.cpu().numpy(), ref_q)
    assert np.array_equal(qw.scales.cpu().numpy(), ref_s)


@pytest.mark.parametrize("odt", ["f16", "bf16"])
def test_dequantize_int4_bitexact(odt):
    say(f"dequantize_int4 odt={odt}")
    w = edge_weights(48, 1152, seed=3)
    qw = gpu_quantize_int4(dev_f16(w))
    out = torch.empty((48, 1152), dtype=torch_dtype(odt), device="cuda")
    wq.wq_dequantize(qw, out)
    torch.cuda.synchronize()
    ref = int4.dequantize(*int4.quantize(w.astype(np.float32)), 1152, out_dtype=odt)
    assert np.array_equal(to_np(out), ref)


def run_linear(x_np, w_np, xdt, ydt, qw=None):
    """GPU path: quantize (unless given) + linear, through the ABI."""
    n, k = w_np.shape
    m = x_np.shape[0]
    if qw is None:
        qw = gpu_quantize_int4(dev(w_np, xdt))
    x = dev(x_np, xdt)
    y = torch.empty((m, n), dtype=torch_dtype(ydt), device="cuda")
    need = wq.wq_linear_w4a16_workspace(m, qw)
    ws = torch.empty((max(need, 1),), dtype=torch.uint8, device="cuda") if need else None
    wq.wq_linear_w4a16(x, qw, y, ws)
    torch.cuda.synchronize()
    return to_np(y), qw


def oracle_linear(x_np, w_np, xdt, rows=None, group=128):
    n, k = w_np.shape
    wh = int4.dequantize(*int4.quantize(host16(w_np, xdt), group), k, group=group, out_dtype=xdt)
    xs = host16(x_np, xdt)
    if rows is not None:
        xs = xs[rows]
    return linear.reference(xs, wh)


@pytest.mark.parametrize("m,n,k,xdt,ydt", [
    (1, 300, 1152, "f16", "f32"),     # ragged n, odd G (9 groups over 16 waves)
    (1, 4096, 4096, "f16", "f32"),    # full single-layer decode shape (sixteen waves)
    (1, 4096, 4096, "f16", "f16"),
    (1, 1000, 2048, "bf16", "bf16"),  # sixteen-wave m = 1 schedule, bf16 (exact decoder)
    (3, 257, 640, "bf16", "f32"),
    (5, 520, 2048, "f16", "bf16"),
    (16, 1000, 2048, "f16", "f32"),
    (16, 4096, 11008, "f16", "f32"),  # full down-projection shape at M = 16
    (16, 11008, 4096, "f16", "f16"),  # full gate/up shape at M = 16
    (16, 5120, 4096, "f16", "f32"),   # two row tiles per workgroup, four phases
    (9, 6001, 4096, "f16", "bf16"),   # two row tiles per workgroup, ragged last tile
    (16, 14336, 4096, "f16", "f32"),  # four row tiles per workgroup (8B MLP width)
    (16, 777, 1024, "bf16", "f32"),
    (1, 520, 11008, "f16", "f32"),    # three activation phases at m = 1
    (2, 300, 11008, "f16", "f16"),    # four staged rows, three phases
    (7, 200, 13824, "f16", "f32"),    # 108 groups: many phases per wave
    (16, 96, 5120, "bf16", "f32"),    # double-buffered phases, exact bf16 dequant
    (8, 1000, 11008, "bf16", "bf16"), # 86 groups, one tile: four waves, whole-line code loads
    (1, 300, 11008, "bf16", "f32"),   # m = 1, groups in pairs (whole lines), ragged n
])
def test_linear_skinny_parity(m, n, k, xdt, ydt):
    say(f"linear_skinny m={m} n={n} k={k} x={xdt} y={ydt}")
    seed = 100 + m + n
    x, _ = workloads.activations(m, k, seed, 0, dtype=xdt, outliers=(min(6, k // 128), 20.0, 80.0))
    w = workloads.weights(n, k, seed, 1, dtype=xdt)
    y, _ = run_linear(x, w, xdt, ydt)
    rel = check_close(y, oracle_linear(x, w, xdt), ydt)
    say(f"  max-rel {rel:.2e}")


@pytest.mark.parametrize("m,n,k,xdt,ydt", [
    (17, 300, 1152, "f16", "f32"),    # smallest GEMM-path m, ragged tiles
    (130, 129, 256, "f16", "bf16"),
    (200, 520, 1024, "bf16", "f32"),
    (256, 1024, 4096, "f16", "f16"),
    (130, 272, 1024, "f16", "f32"),   # staged-scale GEMM: ragged m and n tiles
    (40, 4096, 4096, "f16", "bf16"),  # one partial m tile, full n tiles
    (300, 11008, 4096, "f16", "f32"), # the up-projection rows, three m tiles
    (64, 520, 11008, "f16", "f32"),   # 86 groups, past the staged GEMM's 64: the generic GEMM
])
def test_linear_gemm_parity(m, n, k, xdt, ydt):
    say(f"linear_gemm m={m} n={n} k={k} x={xdt} y={ydt}")
    seed = 200 + m + n
    x, _ = workloads.activations(m, k, seed, 0, dtype=xdt)
    w = workloads.weights(n, k, seed, 1, dtype=xdt)
    y, _ = run_linear(x, w, xdt, ydt)
    rel = check_close(y, oracle_linear(x, w, xdt), ydt)
    say(f"  max-rel {rel:.2e}")


@pytest.mark.parametrize("m,n,k,xdt,ydt", [
    (1, 300, 1152, "f16", "f32"),     # ragged n, odd G, one tile per matrix
    (1, 11008, 4096, "f16", "f16"),   # m = 1 with the single call's schedule: bit-equal
    (3, 257, 640, "bf16", "f32"),     # bf16 activations, ragged last tile
    (4, 11008, 4096, "f16", "f16"),
    (9, 1000, 2048, "f16", "bf16"),   # one row tile per matrix, 16 staged rows
    (16, 5120, 4096, "f16", "f32"),   # two row tiles per matrix
    (16, 11008, 4096, "f16", "f16"),  # the full gate/up shape: three row tiles per matrix
    (12, 11008, 2048, "bf16", "f32"), # three row tiles per matrix, bf16 (exact decoder)
    (16, 14336, 4096, "f16", "f32"),  # four row tiles per matrix
    (1, 4096, 11008, "f16", "f32"),   # 86 groups
    (40, 520, 1024, "f16", "f32"),    # prefill rows: two GEMMs
])
def test_gate_up_pair_parity(m, n, k, xdt, ydt):
    """Both outputs of the pair against the oracle, and equal to the two
    single-matrix calls bit for bit where the schedules match (every case
    but m = 1, where the single call takes two groups per wave for 64 or
    more groups, and sixteen waves for at most 256 row tiles)."""
    say(f"gate_up m={m} n={n} k={k} x={xdt} y={ydt}")
    seed = 300 + m + n
    x_np, _ = workloads.activations(m, k, seed, 0, dtype=xdt, outliers=(min(6, k // 128), 20.0, 80.0))
    wg_np = workloads.weights(n, k, seed, 1, dtype=xdt)
    wu_np = workloads.weights(n, k, seed, 2, dtype=xdt)
    qg, qu = gpu_quantize_int4(dev(wg_np, xdt)), gpu_quantize_int4(dev(wu_np, xdt))
    x = dev(x_np, xdt)
    yg = torch.empty((m, n), dtype=torch_dtype(ydt), device="cuda")
    yu = torch.empty_like(yg)
    wq.wq_linear_w4a16_gate_up(x, qg, qu, yg, yu, act=0)
    torch.cuda.synchronize()
    g, u = to_np(yg), to_np(yu)
    check_close(g, oracle_linear(x_np, wg_np, xdt), ydt)
    check_close(u, oracle_linear(x_np, wu_np, xdt), ydt)
    if not (m == 1 and (k // 128 >= 64 or (n + 15) // 16 <= 256)):
        g1, _ = run_linear(x_np, wg_np, xdt, ydt, qw=qg)
        u1, _ = run_linear(x_np, wu_np, xdt, ydt, qw=qu)
        assert np.array_equal(g, g1) and np.array_equal(u, u1)


@pytest.mark.parametrize("m,n,k,ydt", [
    (1, 300, 1152, "f32"),
    (5, 520, 2048, "bf16"),
    (16, 11008, 4096, "f16"),         # the full gate/up shape
    (16, 5120, 4096, "f32"),
])
def test_gate_up_swiglu_parity(m, n, k, ydt):
    """silu(gate) * up against the oracle's fp64 product of its own fp64
    projections."""
    say(f"gate_up_swiglu m={m} n={n} k={k} y={ydt}")
    seed = 400 + m + n
    x_np, _ = workloads.activations(m, k, seed, 0, outliers=(min(6, k // 128), 20.0, 80.0))
    wg_np = workloads.weights(n, k, seed, 1)
    wu_np = workloads.weights(n, k, seed, 2)
    qg, qu = gpu_quantize_int4(dev_f16(wg_np)), gpu_quantize_int4(dev_f16(wu_np))
    y = torch.empty((m, n), dtype=torch_dtype(ydt), device="cuda")
    wq.wq_linear_w4a16_gate_up(dev_f16(x_np), qg, qu, y, None, act=1)
    torch.cuda.synchronize()
    ref = linear.silu_gated(oracle_linear(x_np, wg_np, "f16"), oracle_linear(x_np, wu_np, "f16"))
    rel = check_close(to_np(y), ref, ydt)
    say(f"  max-rel {rel:.2e}")


@pytest.mark.parametrize("m,n,k,xdt,ydt", [
    (17, 300, 1152, "f16", "f32"),      # the first row count past the decode pass
    (64, 520, 2048, "f16", "f16"),
    (200, 1000, 1024, "bf16", "bf16"),  # ragged tiles, bf16 throughout
    (512, 11008, 4096, "f16", "f16"),   # the full MLP block at prefill
])
def test_gate_up_swiglu_prefill(m, n, k, xdt, ydt):
    """silu(gate) * up past 16 rows: two GEMMs store gate and up in the output
    type, then the product is taken on those stored values.  Checked two ways:
    within one output ulp of silu(g) * u formed in fp32 from the act 0 outputs
    of the same call (the same GEMMs, so the same g and u), and against the
    oracle's fp64 product.  There three roundings to the output type (g, u and
    the result, each within 2^-9 relative in bf16 and 2^-11 in fp16, with
    silu's relative sensitivity to g under 1.3 where silu is not small) add at
    most 3.3 such terms: under 2^-7 |y| in bf16 and within the plain bound in
    fp16."""
    say(f"gate_up_swiglu prefill m={m} n={n} k={k} x={xdt} y={ydt}")
    seed = 450 + m + n
    x_np, _ = workloads.activations(m, k, seed, 0, dtype=xdt, outliers=(min(6, k // 128), 20.0, 80.0))
    wg_np = workloads.weights(n, k, seed, 1, dtype=xdt)
    wu_np = workloads.weights(n, k, seed, 2, dtype=xdt)
    qg, qu = gpu_quantize_int4(dev(wg_np, xdt)), gpu_quantize_int4(dev(wu_np, xdt))
    x = dev(x_np, xdt)
    y = torch.empty((m, n), dtype=torch_dtype(ydt), device="cuda")
    yu = torch.empty_like(y)
    g0, u0 = torch.empty_like(y), torch.empty_like(y)
    wq.wq_linear_w4a16_gate_up(x, qg, qu, g0, u0, act=0)
    wq.wq_linear_w4a16_gate_up(x, qg, qu, y, yu, act=1)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(yu), to_np(u0)), "y_up holds the up projection"
    g, u = to_np(g0).astype(np.float32), to_np(u0).astype(np.float32)
    near = (g / (np.float32(1) + np.exp(-g)) * u).astype(np.float64)
    # host and device exp differ by a few fp32 ulps; 2^-24 covers fp16 subnormals
    ulp = {"f32": 2.0 ** -20, "f16": 2.0 ** -10, "bf16": 2.0 ** -7}[ydt]
    got = to_np(y).astype(np.float64)
    assert (np.abs(got - near) <= ulp * np.abs(near) + 2.0 ** -24).all()
    ref = linear.silu_gated(oracle_linear(x_np, wg_np, xdt), oracle_linear(x_np, wu_np, xdt))
    if ydt == "bf16":
        den = np.abs(ref).max()
        err = np.abs(got - ref)
        assert (err <= 2e-3 * den + 2.0 ** -7 * np.abs(ref)).all()
        rel = float(err.max() / den)
    else:
        rel = check_close(got, ref, ydt)
    say(f"  max-rel {rel:.2e}")


@pytest.mark.parametrize("m,n,k,xdt,ydt,group", [
    (1, 300, 1152, "f16", "f32", 64),     # scales not stageable (n * zb % 16 != 0)
    (1, 4096, 4096, "f16", "f16", 32),
    (4, 11008, 4096, "f16", "f32", 64),
    (16, 11008, 4096, "f16", "f16", 32),  # three row tiles, staged scales
    (16, 4096, 11008, "f16", "f32", 64),  # 172 groups per row
    (3, 257, 640, "bf16", "f32", 32),     # bf16: the exact per-word decoder
    (9, 1000, 2048, "bf16", "bf16", 64),
    (40, 520, 1024, "f16", "f32", 64),    # GEMM with staged scales (16 groups)
    (300, 1024, 2048, "f16", "f16", 32),  # GEMM, 64 groups: the staging limit
    (130, 272, 4096, "f16", "f32", 32),   # 128 groups: the generic GEMM
    (200, 520, 1024, "bf16", "f32", 64),
    (130, 264, 2048, "bf16", "bf16", 32),  # bf16 GEMM, four groups per unit, ragged tiles
])
def test_linear_group_sizes(m, n, k, xdt, ydt, group):
    """Groups of 64 and 32 ([P5] 2.2 group-wise granularity, the group-size
    knob): every decode and GEMM path against the oracle with the same
    groups."""
    say(f"linear_group m={m} n={n} k={k} x={xdt} y={ydt} group={group}")
    seed = 600 + m + n + group
    x, _ = workloads.activations(m, k, seed, 0, dtype=xdt, outliers=(min(6, k // 128), 20.0, 80.0))
    w = workloads.weights(n, k, seed, 1, dtype=xdt)
    qw = gpu_quantize_int4(dev(w, xdt), group)
    y, _ = run_linear(x, w, xdt, ydt, qw=qw)
    rel = check_close(y, oracle_linear(x, w, xdt, group=group), ydt)
    say(f"  max-rel {rel:.2e}")


@pytest.mark.parametrize("m,n,k,group,act", [(16, 5120, 4096, 64, 0), (1, 300, 1152, 32, 1),
                                             (16, 11008, 2048, 32, 1)])
def test_gate_up_group_sizes(m, n, k, group, act):
    say(f"gate_up_group m={m} n={n} k={k} group={group} act={act}")
    seed = 700 + m + n
    x_np, _ = workloads.activations(m, k, seed, 0)
    wg_np, wu_np = workloads.weights(n, k, seed, 1), workloads.weights(n, k, seed, 2)
    qg = gpu_quantize_int4(dev_f16(wg_np), group)
    qu = gpu_quantize_int4(dev_f16(wu_np), group)
    yg = torch.empty((m, n), dtype=torch.float32, device="cuda")
    yu = torch.empty_like(yg)
    wq.wq_linear_w4a16_gate_up(dev_f16(x_np), qg, qu, yg, yu if act == 0 else None, act=act)
    torch.cuda.synchronize()
    g = oracle_linear(x_np, wg_np, "f16", group=group)
    u = oracle_linear(x_np, wu_np, "f16", group=group)
    if act == 0:
        check_close(to_np(yg), g, "f32")
        check_close(to_np(yu), u, "f32")
    else:
        check_close(to_np(yg), linear.silu_gated(g, u), "f32")


@pytest.mark.parametrize("xdt,ydt,group", [("bf16", "bf16", 128), ("f16", "f16", 64),
                                           ("f16", "f32", 32)])
def test_gemm_up_shape(xdt, ydt, group):
    """The up-projection width at M = 2048 (688 tiles of 128 x 256, three
    rounds of 256 workgroups, the last one partly filled) with the exact bf16
    decoder and groups of 64 and 32; 24 sampled rows, the last among them,
    against the oracle, every column."""
    m, n, k = 2048, 11008, 1024
    say(f"gemm_up_shape m={m} n={n} k={k} x={xdt} y={ydt} group={group}")
    seed = 800 + group
    x, _ = workloads.activations(m, k, seed, 0, dtype=xdt)
    w = workloads.weights(n, k, seed, 1, dtype=xdt)
    qw = gpu_quantize_int4(dev(w, xdt), group)
    y, _ = run_linear(x, w, xdt, ydt, qw=qw)
    rows = np.random.default_rng(seed).choice(m, 24, replace=False)
    rows[0] = m - 1
    rel = check_close(y[rows], oracle_linear(x, w, xdt, rows=rows, group=group), ydt)
    say(f"  max-rel {rel:.2e}")


def _act_order_perm(k, seed):
    """A synthetic act-order: channels by decreasing seeded importance."""
    return np.argsort(-np.random.default_rng(seed).random(k), kind="stable").astype(np.int32)


@pytest.mark.parametrize("rows,k,dt", [(37, 1152, "f16"), (5, 4096, "bf16"), (2048, 4096, "f16")])
def test_permute_columns_bitexact(rows, k, dt):
    say(f"permute_columns rows={rows} k={k} dt={dt}")
    src = workloads.weights(rows, k, rows + k, 1, dtype=dt)
    perm = _act_order_perm(k, rows)
    out = torch.empty((rows, k), dtype=torch_dtype(dt), device="cuda")
    wq.wq_permute_columns(dev(src, dt), torch.from_numpy(perm).cuda(), out)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(out), host16(src, dt)[:, perm].astype(np.float32))


@pytest.mark.parametrize("m,n,k,group", [
    (1, 300, 1152, 128), (16, 4096, 4096, 128), (16, 1000, 2048, 64), (300, 520, 4096, 128),
])
def test_act_order_linear_parity(m, n, k, group):
    """Act-order weights (columns stored in quantization order) against the
    oracle's original-order g_idx definition; the stored codes, scales and
    zeros bit for bit against the oracle's act-order packing."""
    say(f"act_order m={m} n={n} k={k} group={group}")
    seed = 800 + m + n
    x, _ = workloads.activations(m, k, seed, 0, outliers=(min(6, k // 128), 20.0, 80.0))
    w = workloads.weights(n, k, seed, 1)
    perm = _act_order_perm(k, seed)
    perm_d = torch.from_numpy(perm).cuda()
    w_perm = torch.empty((n, k), dtype=torch.float16, device="cuda")
    wq.wq_permute_columns(dev_f16(w), perm_d, w_perm)
    qw = gpu_quantize_int4(w_perm, group)
    qw.perm = perm_d
    torch.cuda.synchronize()
    rq, rs, rz = int4.quantize_act_order(w, perm, group)
    assert np.array_equal(qw.codes.cpu().numpy().view(np.uint32), rq)
    assert np.array_equal(qw.scales.cpu().numpy().view(np.uint16), rs.view(np.uint16))
    assert np.array_equal(qw.zeros.cpu().numpy(), rz)
    y, _ = run_linear(x, w, "f16", "f32", qw=qw)
    ref = linear.reference(host16(x, "f16"), int4.dequantize_act_order(w, perm, group))
    rel = check_close(y, ref, "f32")
    say(f"  max-rel {rel:.2e}")


def test_linear_prefill_full_shape_sampled():
    """The prefill layer at full size (M = 2048, up-projection 11008 x 4096):
    every output column of 64 sampled token rows against the oracle."""
    say("linear_prefill_full m=2048 n=11008 k=4096")
    layers = workloads.prefill(layers=("up",))
    name, x, w = layers[0]
    y, _ = run_linear(x, w, "f16", "f32")
    rows = np.random.default_rng(0).choice(2048, size=64, replace=False)
    rel = check_close(y[rows], oracle_linear(x, w, "f16", rows=rows), "f32")
    say(f"  max-rel {rel:.2e}")


def test_linear_with_oracle_packed_weights():
    """The linear kernels on weights packed by the oracle (isolates them from
    the quantize kernel)."""
    say("linear_oracle_packed")
    m_list = (1, 16, 64)
    n, k = 272, 1408
    w = workloads.weights(n, k, 9, 1)
    q, s, z = int4.quantize(w.astype(np.float32))
    qw = wq.QuantizedWeight(
        wq.FMT_INT4_ASYM, n, k, 128,
        torch.from_numpy(q.view(np.int32)).cuda(),
        torch.from_numpy(s).cuda(),
        torch.from_numpy(z).cuda())
    for m in m_list:
        x, _ = workloads.activations(m, k, 9, 2)
        y, _ = run_linear(x, w, "f16", "f32", qw=qw)
        check_close(y, oracle_linear(x, w, "f16"), "f32")


def test_deterministic_repeats():
    say("determinism")
    x, _ = workloads.activations(16, 4096, 5, 0)
    w = workloads.weights(4096, 4096, 5, 1)
    y1, qw = run_linear(x, w, "f16", "f32")
    y2, _ = run_linear(x, w, "f16", "f32", qw=qw)
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("case", ["decode_m1", "mlp_gate_up_pair", "mlp_down", "prefill_q",
                                  "prefill_up"])
def test_workload_full_shape_margins(case, record_margin):
    """The benchmarked layers at full size and with the benchmark's own
    seeded inputs (fp32 outputs): single-layer decode at M = 1, the MLP
    decode step at M = 16 (gate + up as one pair call, down at K = 11008,
    both with the fixed outlier channels), and the prefill q and up layers at
    M = 2048 (64 sampled token rows, every output column).  The max-relative
    error of each is recorded and printed at the end of the run."""
    say(f"workload_margin {case}")
    if case == "decode_m1":
        d = workloads.decode_m1()
        y, _ = run_linear(d["x"], d["w"], "f16", "f32")
        rel = check_close(y, oracle_linear(d["x"], d["w"], "f16"), "f32")
        record_margin("decode M=1 4096x4096 (fp16 fast path)", rel)
    elif case == "mlp_gate_up_pair":
        (_, x_np, wg_np), (_, _, wu_np) = workloads.mlp_decode(layers=("gate", "up"))
        qg, qu = gpu_quantize_int4(dev_f16(wg_np)), gpu_quantize_int4(dev_f16(wu_np))
        yg = torch.empty((16, 11008), dtype=torch.float32, device="cuda")
        yu = torch.empty_like(yg)
        wq.wq_linear_w4a16_gate_up(dev_f16(x_np), qg, qu, yg, yu, act=0)
        torch.cuda.synchronize()
        rg = check_close(to_np(yg), oracle_linear(x_np, wg_np, "f16"), "f32")
        ru = check_close(to_np(yu), oracle_linear(x_np, wu_np, "f16"), "f32")
        record_margin("MLP gate (pair) M=16 11008x4096, outliers", rg)
        record_margin("MLP up (pair) M=16 11008x4096, outliers", ru)
        rel = max(rg, ru)
    elif case == "mlp_down":
        _, x_np, w_np = workloads.mlp_decode()[2]
        y, _ = run_linear(x_np, w_np, "f16", "f32")
        rel = check_close(y, oracle_linear(x_np, w_np, "f16"), "f32")
        record_margin("MLP down M=16 4096x11008, outliers", rel)
    else:
        (_, x_np, w_np), = workloads.prefill(layers=(case.split("_")[1],))
        y, _ = run_linear(x_np, w_np, "f16", "f32")
        rows = np.random.default_rng(1).choice(2048, size=64, replace=False)
        rel = check_close(y[rows], oracle_linear(x_np, w_np, "f16", rows=rows), "f32")
        record_margin(f"prefill {case.split('_')[1]} M=2048 (64 rows sampled)", rel)
    say(f"  max-rel {rel:.2e}")
