"""Pins for the reference linear and the rounding helpers (CPU only)."""

import struct

import numpy as np
import pytest

from oracle import int4, linear
from oracle.numerics import round_f16
import workloads


def test_reference_matches_triple_loop():
    r = np.random.default_rng(0)
    x = r.standard_normal((3, 17)).astype(np.float16)
    w = r.standard_normal((5, 17)).astype(np.float16)
    assert np.allclose(linear.reference(x, w), linear.naive(x, w), rtol=1e-13, atol=1e-13)


def test_integer_case_is_exact():
    """Scale 1 and zero point 8 make w_hat = q - 8, an integer; with
    integer-valued activations y is an exact integer."""
    r = np.random.default_rng(1)
    n, k, m = 6, 256, 2
    q = r.integers(0, 16, size=(n, k))
    qweight = int4.pack_codes(q)
    g = k // 128
    scales = np.ones((n, g), dtype=np.float16)
    zeros = int4.pack_zeros(np.full((n, g), 8))
    wh = int4.dequantize(qweight, scales, zeros, k)
    x = r.integers(-20, 21, size=(m, k)).astype(np.float16)
    y = linear.reference(x, wh)
    for i in range(m):
        for j in range(n):
            assert y[i, j] == sum(int(a) * (int(b) - 8) for a, b in zip(x[i].astype(int), q[j]))


def test_max_rel_err():
    assert linear.max_rel_err([1.0, 2.0], [1.0, 2.0]) == 0.0
    assert abs(linear.max_rel_err([1.0, 2.002], [1.0, 2.0]) - 1e-3) < 1e-12


def test_f16_rounding_matches_struct():
    r = np.random.default_rng(2)
    v = (r.standard_normal(5000) * np.exp(r.uniform(-12, 10, 5000))).astype(np.float32)
    mine = round_f16(v)
    ref = np.array([struct.unpack("<e", struct.pack("<e", float(t)))[0] for t in v])
    assert np.array_equal(mine.astype(np.float64), ref)


def test_quantized_layer_error_is_small():
    """End to end on a small decode-shaped layer: the INT4 g128 product stays
    within a few percent of the unquantized fp64 product (4-bit weights keep
    the output, [P2] opening)."""
    d = workloads.decode_m1(n=256, k=1024)
    qw, s, z = int4.quantize(d["w"])
    y = linear.reference(d["x"], int4.dequantize(qw, s, z, 1024))
    ref = linear.reference(d["x"], d["w"])
    assert linear.max_rel_err(y, ref) < 0.1


def test_silu_gated_closed_forms():
    """sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4 give exact values; the
    identity silu(v) - silu(-v) = v (sigmoid(v) + sigmoid(-v) = 1) and the
    two limits pin the sign of the exponent and the factor v."""
    l3 = np.log(3.0)
    assert linear.silu_gated(l3, 1.0) == pytest.approx(0.75 * l3, rel=1e-15)
    assert linear.silu_gated(-l3, 1.0) == pytest.approx(-0.25 * l3, rel=1e-15)
    assert linear.silu_gated(0.0, 5.0) == 0.0
    v = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(linear.silu_gated(v, 1.0) - linear.silu_gated(-v, 1.0), v,
                               rtol=0, atol=1e-12)
    assert linear.silu_gated(40.0, 1.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(linear.silu_gated(-40.0, 1.0)) < 1e-15
    assert linear.silu_gated(-1e4, 2.0) == 0.0          # exp overflow gives -0, not NaN


def test_silu_gated_is_linear_in_up():
    rng = np.random.default_rng(3)
    g, u = rng.standard_normal(50), rng.standard_normal(50)
    np.testing.assert_allclose(linear.silu_gated(g, 2.0 * u), 2.0 * linear.silu_gated(g, u),
                               rtol=1e-15)
    np.testing.assert_array_equal(linear.silu_gated(g, 0.0 * u), 0.0 * u)
