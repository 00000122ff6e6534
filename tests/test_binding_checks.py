"""The Python binding's size and layout checks (CPU only, no library call).

The C entry points take pointers and the sizes passed with them; the binding
derives those sizes from the tensors and checks every tensor against them
first, so a tensor smaller than the sizes say never reaches a kernel.  These
calls use CPU tensors: a shape or layout mismatch must raise
WqError(WQ_ERR_SHAPE) before anything else, and correctly shaped CPU tensors
must raise WqError(WQ_ERR_UNSUPPORTED) (they are not GPU tensors) -- in
neither case is the library loaded or called."""

import pytest
import torch

import bit_quantized_linear_int4_amd as wq

SHAPE, UNSUP = 2, 4


def status(fn, *a, **kw):
    with pytest.raises(wq.WqError) as e:
        fn(*a, **kw)
    return e.value.status


def int4(n=32, k=256, group=128):
    return wq.alloc_int4(n, k, group, device="cpu")


def test_linear_checks():
    w = int4()
    x = torch.zeros((4, 256), dtype=torch.float16)
    y = torch.zeros((4, 32), dtype=torch.float16)
    assert status(wq.wq_linear_w4a16, x, w, y) == UNSUP            # well formed, not on a GPU
    assert status(wq.wq_linear_w4a16, x[0], w, y) == SHAPE         # 1-D x
    assert status(wq.wq_linear_w4a16, x[:, :128], w, y[:, :]) == SHAPE   # k mismatch
    assert status(wq.wq_linear_w4a16, x, w, y[:3]) == SHAPE        # y rows
    assert status(wq.wq_linear_w4a16, torch.zeros((256, 4), dtype=torch.float16).t(), w, y) == SHAPE
    assert status(wq.wq_linear_w4a16, x, w, torch.zeros((32, 4), dtype=torch.float16).t()) == SHAPE
    bad = int4()
    bad.codes = bad.codes[:16]                                      # fewer rows than n
    assert status(wq.wq_linear_w4a16, x, bad, y) == SHAPE
    bad = int4()
    bad.scales = torch.zeros((32, 4), dtype=torch.float16)           # groups of 64 stored
    assert status(wq.wq_linear_w4a16, x, bad, y) == SHAPE
    bad = int4()
    bad.zeros = bad.zeros[:, :0]
    assert status(wq.wq_linear_w4a16, x, bad, y) == SHAPE
    bad = int4()
    bad.perm = torch.zeros((255,), dtype=torch.int32)
    assert status(wq.wq_linear_w4a16, x, bad, y) == SHAPE


def test_gate_up_checks():
    g, u = int4(), int4()
    x = torch.zeros((2, 256), dtype=torch.float16)
    yg = torch.zeros((2, 32), dtype=torch.float16)
    yu = torch.zeros((2, 32), dtype=torch.float16)
    assert status(wq.wq_linear_w4a16_gate_up, x, g, u, yg, yu) == UNSUP
    assert status(wq.wq_linear_w4a16_gate_up, x, g, u, yg, None) == SHAPE    # act = 0 needs y_up
    assert status(wq.wq_linear_w4a16_gate_up, x, g, u, yg, None, act=1) == UNSUP
    assert status(wq.wq_linear_w4a16_gate_up, x, g, int4(k=512), yg, yu) == SHAPE
    assert status(wq.wq_linear_w4a16_gate_up, x, g, u, yg, yu[:1]) == SHAPE


def test_nf4_weight_checks():
    w = wq.alloc_nf4(16, 256, device="cpu")
    x = torch.zeros((1, 256), dtype=torch.bfloat16)
    y = torch.zeros((1, 16), dtype=torch.bfloat16)
    assert status(wq.wq_linear_w4a16, x, w, y) == UNSUP
    w.scales2 = w.scales2[:0]
    assert status(wq.wq_linear_w4a16, x, w, y) == SHAPE
    w = wq.alloc_nf4(16, 256, double_quant=False, device="cpu")
    assert status(wq.wq_linear_w4a16, x, w, y) == UNSUP
    w.scales = torch.zeros((64,), dtype=torch.int8)                  # int8 absmax without scales2
    assert status(wq.wq_linear_w4a16, x, w, y) == SHAPE


def test_quantize_and_pack_checks():
    w = torch.zeros((32, 256), dtype=torch.float16)
    q = int4()
    assert status(wq.wq_quantize_groupwise, w, 4, 128, 0, q.codes, q.scales, q.zeros) == UNSUP
    assert status(wq.wq_quantize_groupwise, w, 4, 128, 0, q.codes[:8], q.scales, q.zeros) == SHAPE
    assert status(wq.wq_quantize_groupwise, w, 4, 96, 0, q.codes, q.scales, q.zeros) == SHAPE
    assert status(wq.wq_quantize_groupwise, w[0], 4, 128, 0, q.codes, q.scales, q.zeros) == SHAPE
    q8 = wq.alloc_int8(32, 256, device="cpu")
    assert status(wq.wq_quantize_groupwise, w, 8, 256, 1, q8.codes, q8.scales) == UNSUP
    assert status(wq.wq_quantize_groupwise, w, 8, 256, 1, q8.codes, q8.scales[:31]) == SHAPE
    nf = wq.alloc_nf4(32, 256, device="cpu")
    wb = w.to(torch.bfloat16)
    assert status(wq.wq_pack_nf4, wb, 64, True, 256, nf.codes, nf.scales, nf.scales2) == UNSUP
    assert status(wq.wq_pack_nf4, wb, 64, True, 256, nf.codes, nf.scales[:1], nf.scales2) == SHAPE
    assert status(wq.wq_pack_fp4, wb, 64, True, 256, nf.codes[:5], nf.scales, nf.scales2) == SHAPE
    assert status(wq.wq_pack_nf4, wb, 64, False, 256, nf.codes, nf.scales, None) == SHAPE


def test_int8_checks():
    w = wq.alloc_int8(48, 256, device="cpu")
    x = torch.zeros((8, 256), dtype=torch.float16)
    y = torch.zeros((8, 48), dtype=torch.float16)
    ws = torch.zeros((1 << 16,), dtype=torch.uint8)
    assert status(wq.wq_linear_int8_decomp, x, w, 6.0, y, ws) == UNSUP
    acc = torch.zeros((8, 47), dtype=torch.int32)
    assert status(wq.wq_linear_int8_decomp, x, w, 6.0, y, ws, acc_out=acc) == SHAPE
    assert status(wq.wq_linear_int8_decomp, x, w, 6.0, y, None) == SHAPE
    assert status(wq.wq_linear_int8_decomp, x, w, 6.0, y[:, :40], ws) == SHAPE
    cnt = torch.zeros((0,), dtype=torch.int32)
    assert status(wq.wq_linear_int8_decomp, x, w, 6.0, y, ws, outlier_count=cnt) == SHAPE
    mask = torch.zeros((256,), dtype=torch.uint8)
    idx = torch.zeros((256,), dtype=torch.int32)
    count = torch.zeros((1,), dtype=torch.int32)
    qx = torch.zeros((8, 256), dtype=torch.int8)
    sx = torch.zeros((8,), dtype=torch.float32)
    f = wq.wq_int8_prepare_activations
    assert status(f, x, 6.0, mask, idx, count, qx, sx) == UNSUP
    assert status(f, x, 6.0, mask[:128], idx, count, qx, sx) == SHAPE
    assert status(f, x, 6.0, mask, idx, count, qx[:4], sx) == SHAPE
    assert status(f, x, 6.0, mask, idx, count, qx, sx[:7]) == SHAPE


def test_column_op_and_dequantize_checks():
    src = torch.zeros((4, 64), dtype=torch.float16)
    perm = torch.arange(64, dtype=torch.int32)
    assert status(wq.wq_permute_columns, src, perm, torch.zeros_like(src)) == UNSUP
    assert status(wq.wq_permute_columns, src, perm[:63], torch.zeros_like(src)) == SHAPE
    assert status(wq.wq_permute_columns, src, perm, torch.zeros((4, 32), dtype=torch.float16)) == SHAPE
    sc = torch.ones((64,), dtype=torch.float32)
    assert status(wq.wq_scale_columns, src, sc, src) == UNSUP
    assert status(wq.wq_scale_columns, src, sc[:32], src) == SHAPE
    w = int4()
    assert status(wq.wq_dequantize, w, torch.zeros((32, 256), dtype=torch.float16)) == UNSUP
    assert status(wq.wq_dequantize, w, torch.zeros((256, 32), dtype=torch.float16)) == SHAPE
