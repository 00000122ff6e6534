"""GPU parity of the LLM.int8() decomposition against the CPU oracle, through
the C ABI: outlier set, per-token int8 activations and scales, and the int32
accumulators are bit-exact; the output is within 2e-3 max-relative error."""

import numpy as np
import pytest
import torch

import bit_quantized_linear_int4_amd as wq
import workloads
from oracle import llm_int8
from gpu_util import check_close, dev_f16, say, to_np, torch_dtype

pytestmark = pytest.mark.gpu


def prepare(x_np, thr):
    m, k = x_np.shape
    x = dev_f16(x_np)
    mask = torch.empty((k,), dtype=torch.uint8, device="cuda")
    idx = torch.full((k,), -1, dtype=torch.int32, device="cuda")
    cnt = torch.empty((1,), dtype=torch.int32, device="cuda")
    qx = torch.empty((m, k), dtype=torch.int8, device="cuda")
    sx = torch.empty((m,), dtype=torch.float32, device="cuda")
    wq.wq_int8_prepare_activations(x, thr, mask, idx, cnt, qx, sx)
    torch.cuda.synchronize()
    return mask.cpu().numpy(), idx.cpu().numpy(), int(cnt.item()), qx.cpu().numpy(), sx.cpu().numpy()


@pytest.mark.parametrize("m,k,n_out,thr", [
    (8, 256, 3, 6.0),
    (70, 1024, 8, 6.0),       # two 64-row chunks
    (256, 8192, 8, 6.0),      # the 70B-layer activation shape
    (5, 512, 0, 6.0),         # no injected outliers
    (4, 256, 2, float("inf")),
    (4, 256, 2, 0.0),         # every non-zero column is an outlier
])
def test_prepare_activations_bitexact(m, k, n_out, thr):
    say(f"int8_prepare m={m} k={k} outliers={n_out} thr={thr}")
    x, chans = workloads.activations(m, k, 500 + m, 0, outliers=(n_out, 20.0, 100.0) if n_out else None)
    mask, idx, cnt, qx, sx = prepare(x, thr)
    ref_o = llm_int8.outlier_columns(x, thr)
    ref_qx, ref_sx = llm_int8.quantize_activations(x, ref_o)
    assert cnt == ref_o.size
    assert np.array_equal(idx[:cnt], ref_o)
    assert np.array_equal(np.nonzero(mask)[0], ref_o)
    assert np.array_equal(qx, ref_qx)
    assert np.array_equal(sx, ref_sx)
    if thr == 6.0 and n_out:
        assert np.array_equal(ref_o, chans)


def run_decomp(x_np, w_np, thr, ydt):
    m, k = x_np.shape
    n = w_np.shape[0]
    qw = wq.alloc_int8(n, k)
    wq.wq_quantize_groupwise(dev_f16(w_np), 8, k, 1, qw.codes, qw.scales)
    y = torch.empty((m, n), dtype=torch_dtype(ydt), device="cuda")
    acc = torch.empty((m, n), dtype=torch.int32, device="cuda")
    cnt = torch.empty((1,), dtype=torch.int32, device="cuda")
    ws = torch.empty((wq.wq_linear_int8_decomp_workspace(m, k),), dtype=torch.uint8, device="cuda")
    wq.wq_linear_int8_decomp(dev_f16(x_np), qw, thr, y, ws, cnt, acc)
    torch.cuda.synchronize()
    return to_np(y), acc.cpu().numpy(), int(cnt.item())


@pytest.mark.parametrize("m,n,k,n_out,thr,ydt", [
    (8, 130, 256, 3, 6.0, "f32"),
    (70, 300, 1024, 8, 6.0, "f16"),
    (70, 300, 1024, 8, 6.0, "bf16"),
    (256, 512, 2048, 40, 6.0, "f32"),     # more than one 32-column outlier chunk
    (300, 200, 512, 5, 6.0, "f32"),       # two 256-row tiles
    (16, 256, 1024, 4, float("inf"), "f32"),
    (16, 128, 256, 2, 0.0, "f32"),
    (512, 1000, 640, 3, 6.0, "f32"),      # two full 256-row tiles, 112-wide column tiles, ragged n
    (16, 28688, 256, 2, 6.0, "f16"),      # 128-wide column tiles (112 would need a second round)
    (256, 224, 8192, 40, 6.0, "f32"),     # 64 K steps: outlier weights copied from the stream
    (8, 200, 8320, 3, 6.0, "f16"),        # 65 K steps: outlier weights gathered instead
])
def test_decomp_parity(m, n, k, n_out, thr, ydt):
    say(f"int8_decomp m={m} n={n} k={k} outliers={n_out} thr={thr} y={ydt}")
    seed = 600 + m + n
    x, _ = workloads.activations(m, k, seed, 0, outliers=(n_out, 20.0, 100.0))
    w = workloads.weights(n, k, seed, 1)
    y, acc, cnt = run_decomp(x, w, thr, ydt)
    qw, sw = llm_int8.quantize_rows(w)
    y_ref, outl, qx, sx, acc_ref = llm_int8.linear(x, qw, sw, thr)
    assert cnt == outl.size
    assert np.array_equal(acc, acc_ref)
    rel = check_close(y, y_ref, ydt)
    say(f"  max-rel {rel:.2e}")


def test_decomp_70b_shape_sampled(record_margin):
    """The 70B layer at full size: 28672 x 8192 int8 weights, 256 tokens with
    8 outlier channels; int32 accumulators and outputs of 2048 sampled output
    features against the oracle."""
    say("int8_decomp_full m=256 n=28672 k=8192")
    d = workloads.int8_70b()
    y, acc, cnt = run_decomp(d["x"], d["w"], 6.0, "f32")
    assert cnt == 8
    cols = np.sort(np.random.default_rng(2).choice(28672, 2048, replace=False))
    qw, sw = llm_int8.quantize_rows(d["w"][cols])
    y_ref, outl, qx, sx, acc_ref = llm_int8.linear(d["x"], qw, sw)
    assert np.array_equal(outl, d["outlier_channels"])
    assert np.array_equal(acc[:, cols], acc_ref)
    rel = check_close(y[:, cols], y_ref, "f32")
    say(f"  max-rel {rel:.2e}")
    record_margin("LLM.int8 70B layer M=256 (2048 columns sampled)", rel)


# ---------------------------------------------------- SmoothQuant-style W8A8

@pytest.mark.parametrize("rows,k,dt", [(37, 1024, "f16"), (8, 512, "bf16")])
def test_scale_columns_bitexact(rows, k, dt):
    say(f"scale_columns rows={rows} k={k} dt={dt}")
    from gpu_util import dev, host16
    a = workloads.weights(rows, k, rows + k, 1, dtype=dt)
    sc = np.random.default_rng(rows).uniform(0.05, 20.0, k).astype(np.float32)
    out = torch.empty((rows, k), dtype=torch_dtype(dt), device="cuda")
    wq.wq_scale_columns(dev(a, dt), torch.from_numpy(sc).cuda(), out)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(out), llm_int8.scale_columns(host16(a, dt), sc, dt))


@pytest.mark.parametrize("m,n,k", [(16, 256, 1024), (256, 512, 2048)])
def test_smoothed_w8a8_parity(m, n, k):
    """Smoothing (alpha = 0.5, synthetic calibration maxima from the inputs
    themselves) folded into the weights, activations divided on the GPU,
    then the INT8 product with no outlier columns: int32 accumulators bit
    for bit and y against the oracle on the same smoothed inputs.  The
    smoothing must also cut the error against the unquantized product."""
    say(f"smoothed_w8a8 m={m} n={n} k={k}")
    seed = 900 + m + n
    x, _ = workloads.activations(m, k, seed, 0, outliers=(8, 20.0, 100.0))
    w = workloads.weights(n, k, seed, 1)
    s = llm_int8.smooth_factors(np.abs(x.astype(np.float32)).max(axis=0),
                                np.abs(w.astype(np.float32)).max(axis=0), 0.5)
    inv = (np.float32(1) / s).astype(np.float32)
    xs = torch.empty((m, k), dtype=torch.float16, device="cuda")
    ws_ = torch.empty((n, k), dtype=torch.float16, device="cuda")
    wq.wq_scale_columns(dev_f16(x), torch.from_numpy(inv).cuda(), xs)
    wq.wq_scale_columns(dev_f16(w), torch.from_numpy(s).cuda(), ws_)
    torch.cuda.synchronize()
    x_ref = llm_int8.scale_columns(x, inv, "f16").astype(np.float16)
    w_ref = llm_int8.scale_columns(w, s, "f16").astype(np.float16)
    assert np.array_equal(xs.cpu().numpy(), x_ref) and np.array_equal(ws_.cpu().numpy(), w_ref)
    y, acc, cnt = run_decomp(x_ref, w_ref, float("inf"), "f32")
    qw, sw = llm_int8.quantize_rows(w_ref)
    y_ref, outl, qx, sx, acc_ref = llm_int8.linear(x_ref, qw, sw, float("inf"))
    assert cnt == 0 and np.array_equal(acc, acc_ref)
    check_close(y, y_ref, "f32")
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    y_plain, _, _ = run_decomp(x, w, float("inf"), "f32")
    err_s = np.abs(y - exact).max() / np.abs(exact).max()
    err_p = np.abs(y_plain - exact).max() / np.abs(exact).max()
    say(f"  W8A8 error vs fp64: smoothed {err_s:.2e}, plain {err_p:.2e}")
    assert err_s < err_p
