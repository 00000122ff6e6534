"""Pins for the FP4 (E2M1) oracle (CPU only)."""

import numpy as np

from oracle import fp4, nf4


def test_codebook_is_the_e2m1_value_table():
    """The E2M1 values (exponent bias 1, one subnormal step) are the
    well-known set 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives; the
    codebook is that table in code order divided by 6."""
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    lv = fp4.codebook()
    np.testing.assert_array_equal(lv[:8], np.float32(table) / np.float32(6))
    np.testing.assert_array_equal(lv[8:], -np.float32(table) / np.float32(6))
    assert np.signbit(lv[8]) and lv[8] == 0       # code 8 is -0
    assert lv[7] == 1.0 and lv[15] == -1.0


def test_encode_is_the_nearest_value_brute_force():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float16)
    codes, a = fp4.encode(w)
    lv = fp4.codebook().astype(np.float64)
    normed = (w.astype(np.float32).reshape(-1, 64) / a[:, None]).reshape(-1).astype(np.float64)
    dist = np.abs(normed[:, None] - lv[None, :])
    best = dist.min(axis=1)
    # away from midpoints the nearest value is unique up to the sign of 0
    second = np.sort(dist, axis=1)[:, 1]
    clear = (second - best) > 1e-6
    got = lv[codes.astype(np.int64)]
    np.testing.assert_array_equal(np.abs(got[clear] - normed[clear]), best[clear])
    # the sign bit follows the sign of w / a
    assert np.array_equal(codes[normed < 0] >> 3, np.ones(int((normed < 0).sum()), np.uint8))
    assert np.all(codes[normed > 0] < 8)


def test_extremes_zero_block_and_symmetry():
    w = np.zeros((2, 64), np.float16)
    w[1] = np.linspace(-1, 1, 64).astype(np.float16)
    codes, a = fp4.encode(w)
    assert np.all(codes[:64] == 0) and a[0] == 0           # all-zero block
    assert codes[64] == 15 and codes[127] == 7             # -absmax, +absmax
    c_pos, _ = fp4.encode(w[1:])
    c_neg, _ = fp4.encode(-w[1:])
    nz = (c_pos & 7) != 0
    assert np.array_equal(c_neg[nz], c_pos[nz] ^ 8)


def test_ties_go_to_the_lower_magnitude():
    t = fp4.magnitude_thresholds()
    blk = np.zeros(64, np.float32)
    blk[0] = 1.0                                           # absmax 1: normed = w
    blk[1:8] = t                                           # exactly on each midpoint
    codes, _ = fp4.encode(blk.reshape(1, 64))
    assert list(codes[1:8]) == [0, 1, 2, 3, 4, 5, 6]


def test_roundtrip_error_bound():
    """|w - w_hat| <= absmax * (largest half gap = 1/6) + the 16-bit rounding."""
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((32, 512)) * 0.02).astype(np.float16)
    c, a, c2 = fp4.quantize(w, double_quant=False)
    wh = fp4.dequantize(c, a, None, w.shape, out_dtype="f16")
    amax = np.repeat(a, 64).reshape(w.shape)
    err = np.abs(w.astype(np.float64) - wh)
    assert np.all(err <= amax / 6 * (1 + 1e-6) + np.abs(wh) * 2.0 ** -11)


def test_double_quant_matches_the_nf4_second_level():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((8, 4096)) * 0.02).astype(np.float16)
    c, q8, c2 = fp4.quantize(w, double_quant=True)
    codes, a = fp4.encode(w)
    rq8, rc2 = nf4.double_quantize(a)
    assert np.array_equal(q8, rq8) and np.array_equal(c2, rc2)
    assert np.array_equal(c, nf4.pack(codes))
