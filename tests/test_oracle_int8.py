"""Pins for the LLM.int8() oracle (CPU only): the pages' worked scale,
the strict outlier threshold, exact integer accumulation by brute force, and
the two special cases that reduce to plain products (no outliers; all
columns outliers)."""

import numpy as np
import torch

from oracle import llm_int8
from oracle.numerics import round_f16
from golden_util import load
import workloads


def test_worked_scale_80_over_127():
    gold = load("int8_worked_example.txt")
    s = llm_int8.symmetric_scale(float(gold["max_abs"]))
    assert abs(float(s) - float(gold["scale_approx"])) < float(gold["scale_tolerance"])
    assert int(np.float32(s).view(np.uint32)) == int(gold["scale_fp32_hex"], 16)
    # and the row quantizer produces that scale for a row whose max |w| is 80
    row = np.zeros((1, 64), dtype=np.float16)
    row[0, 5] = -80
    row[0, 7] = 33
    qw, sw = llm_int8.quantize_rows(row)
    assert sw[0] == s and qw[0, 5] == -127 and qw[0, 7] == round(33 / float(s))


def test_row_quant_bound_and_range():
    r = np.random.default_rng(0)
    w = (r.standard_normal((16, 300)) * 0.02).astype(np.float16)
    w[3] = 0
    qw, sw = llm_int8.quantize_rows(w)
    assert qw.dtype == np.int8 and qw.min() >= -127 and qw.max() <= 127
    assert sw[3] == 1.0 and (qw[3] == 0).all()
    err = np.abs(w.astype(np.float64) - qw.astype(np.float64) * sw[:, None])
    assert (err <= sw[:, None] * 0.5 * (1 + 2.0 ** -20)).all()
    big = np.abs(w.astype(np.float32)).argmax(axis=1)
    for n in range(16):
        if n != 3:
            assert abs(int(qw[n, big[n]])) == 127


def test_outlier_threshold_is_strict():
    x = np.zeros((3, 8), dtype=np.float16)
    x[0, 1] = 6.0          # equal: not an outlier
    x[1, 2] = -6.0039      # exceeds in magnitude
    x[2, 5] = 6.0039
    x[2, 6] = 5.99
    assert llm_int8.outlier_columns(x, 6.0).tolist() == [2, 5]


def test_outliers_found_on_injected_channels():
    d = workloads.int8_70b(m=32, n=16, k=1024, n_outliers=8)
    assert llm_int8.outlier_columns(d["x"]).tolist() == d["outlier_channels"].tolist()


def test_activation_scale_ignores_outlier_columns():
    x = np.array([[1.0, 50.0, -2.0, 0.5], [0.0, 7.0, 0.0, 0.0]], dtype=np.float16)
    outl = llm_int8.outlier_columns(x)
    assert outl.tolist() == [1]
    qx, sx = llm_int8.quantize_activations(x, outl)
    assert sx[0] == np.float32(2.0) / np.float32(127)
    assert sx[1] == 1.0                                 # only an outlier in the row
    assert qx[0].tolist() == [64, 0, -127, 32] and (qx[1] == 0).all()


def test_integer_accumulation_brute_force():
    r = np.random.default_rng(1)
    qx = r.integers(-127, 128, size=(5, 33)).astype(np.int8)
    qw = r.integers(-127, 128, size=(7, 33)).astype(np.int8)
    acc = llm_int8.int_matmul(qx, qw)
    for i in range(5):
        for j in range(7):
            assert int(acc[i, j]) == sum(int(a) * int(b) for a, b in zip(qx[i], qw[j]))
    # the extreme case stays exact: 127*127*K with K = 8192 fits int32
    big = np.full((1, 8192), 127, np.int8)
    assert int(llm_int8.int_matmul(big, big)[0, 0]) == 127 * 127 * 8192


def test_no_outliers_is_plain_w8a8():
    """threshold = +inf: no column is split off, y = acc * sx * sw."""
    d = workloads.int8_70b(m=4, n=6, k=64, n_outliers=2)
    qw, sw = llm_int8.quantize_rows(d["w"])
    y, outl, qx, sx, acc = llm_int8.linear(d["x"], qw, sw, threshold=np.inf)
    assert outl.size == 0
    x = d["x"].astype(np.float64)
    for i in range(4):
        s = np.abs(x[i]).max() / 127.0
        for j in range(6):
            # per-element re-derivation with Python integers
            q = [int(np.clip(np.rint(np.float32(v) / np.float32(sx[i])), -127, 127)) for v in d["x"][i]]
            a = sum(qq * int(ww) for qq, ww in zip(q, qw[j]))
            assert a == int(acc[i, j])
            assert abs(y[i, j] - a * float(sx[i]) * float(sw[j])) <= 1e-12 * max(1.0, abs(y[i, j]))
        assert abs(float(sx[i]) - s) <= 1e-7 * s


def test_all_outliers_is_fp16_matmul():
    """threshold = 0: every (non-zero) column is an outlier, the INT8 part
    vanishes and y is the fp16-weight product, checked against torch's linear."""
    d = workloads.int8_70b(m=3, n=5, k=40, n_outliers=1)
    qw, sw = llm_int8.quantize_rows(d["w"])
    y, outl, qx, sx, acc = llm_int8.linear(d["x"], qw, sw, threshold=0.0)
    assert outl.size == 40 and (acc == 0).all()
    w16 = round_f16(qw.astype(np.float32) * sw[:, None]).astype(np.float64)
    ref = torch.nn.functional.linear(torch.from_numpy(d["x"].astype(np.float64)),
                                     torch.from_numpy(w16)).numpy()
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_decomposition_close_to_float_product():
    """The decomposed product stays close to the unquantized fp64 product:
    the split keeps the large outlier contributions exact in fp16."""
    d = workloads.int8_70b(m=8, n=64, k=2048, n_outliers=8)
    qw, sw = llm_int8.quantize_rows(d["w"])
    y, outl, *_ = llm_int8.linear(d["x"], qw, sw)
    ref = d["x"].astype(np.float64) @ d["w"].astype(np.float64).T
    rel = np.abs(y - ref).max() / np.abs(ref).max()
    assert outl.size == 8 and rel < 0.05
    # without the split (everything through int8) the error is far larger
    y_all, o2, *_ = llm_int8.linear(d["x"], qw, sw, threshold=np.inf)
    rel_all = np.abs(y_all - ref).max() / np.abs(ref).max()
    assert o2.size == 0 and rel_all > 2 * rel


def test_smoothing_is_an_exact_migration():
    """(x / s) . (W * s)^T equals x . W^T before any rounding ([P1] 5.1)."""
    d = workloads.int8_70b(m=8, n=16, k=256, n_outliers=4)
    x, w = d["x"].astype(np.float64), d["w"].astype(np.float64)
    s = llm_int8.smooth_factors(np.abs(x).max(axis=0), np.abs(w).max(axis=0)).astype(np.float64)
    np.testing.assert_allclose((x / s) @ (w * s).T, x @ w.T, rtol=1e-12, atol=1e-12)


def test_smoothing_balances_the_ranges_at_alpha_half():
    """With alpha = 1/2 every channel's activation and weight maxima become
    equal (both sqrt(max|X| max|W|)); alpha = 0 scales every weight column
    to maximum 1, alpha = 1 every activation column."""
    rng = np.random.default_rng(1)
    ax, aw = rng.uniform(0.1, 80, 64), rng.uniform(0.001, 0.1, 64)
    s = llm_int8.smooth_factors(ax, aw, 0.5).astype(np.float64)
    np.testing.assert_allclose(ax / s, aw * s, rtol=1e-6)
    np.testing.assert_allclose(ax / s, np.sqrt(ax * aw), rtol=1e-6)
    s0 = llm_int8.smooth_factors(ax, aw, 0.0).astype(np.float64)
    np.testing.assert_allclose(aw * s0, np.ones(64), rtol=1e-6)
    s1 = llm_int8.smooth_factors(ax, aw, 1.0).astype(np.float64)
    np.testing.assert_allclose(ax / s1, np.ones(64), rtol=1e-6)
    assert llm_int8.smooth_factors([0.0, 2.0], [1.0, 0.0]).tolist() == [1.0, 1.0]


def test_scale_columns_rounds_once():
    a = np.array([[1.0, 3.0, -2.5, 1e-3]], np.float16)
    sc = np.array([0.5, 1.0 / 3.0, 4.0, 7.0], np.float32)
    got = llm_int8.scale_columns(a, sc, "f16")
    ref = (a.astype(np.float32) * sc).astype(np.float16).astype(np.float32)
    np.testing.assert_array_equal(got, ref)
