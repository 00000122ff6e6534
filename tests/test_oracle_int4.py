"""Pins for the INT4 group-quantization oracle (CPU only).

Each test ties the oracle to something other than itself: the round-trip
error bound that the formula implies, exact rational arithmetic on tiny
groups, a grid that must quantize to itself, hand-packed words, and the
memory figures printed on the pages.
"""

import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import int4
import workloads
from golden_util import load


def _groups_with_edges(seed=0, n=64, k=512):
    r = np.random.default_rng(seed)
    w = (r.standard_normal((n, k)) * 0.02).astype(np.float16)
    w[0, :128] = 0                                   # all-zero group
    w[1, :128] = np.float16(0.01)                    # constant positive group
    w[2, :128] = np.abs(w[2, :128]) + np.float16(1)  # all positive, away from 0
    w[3, :128] = -np.abs(w[3, :128]) - np.float16(2) # all negative
    w[4, :128] = (r.standard_normal(128) * 1e-6).astype(np.float16)  # tiny range
    w[5, :128] = (r.standard_normal(128) * 100).astype(np.float16)   # wide range
    return w


def test_roundtrip_error_bound():
    """|w - (q - z) s16| <= s16 (1/2 + 15 * 2^-11) (+ fp32 rounding slack).

    Derivation: unclamped codes round w/s16 to the nearest integer; a code
    clamped at 15 can be off by at most 15 |s32 - s16| more, and the fp16
    scale is within 2^-11 of the fp32 one.
    """
    w = _groups_with_edges()
    q, s16, z = int4.quantize_codes(w)
    s = np.repeat(s16.astype(np.float64), 128, axis=1)
    zz = np.repeat(z, 128, axis=1)
    err = np.abs(w.astype(np.float64) - (q - zz) * s)
    bound = s * (0.5 + 15 * 2.0 ** -11 * 1.001) + 15 * 2.0 ** -25 + np.abs(w.astype(np.float64)) * 2.0 ** -20
    assert (err <= bound).all()
    # the pages' "round to the nearest step": away from the clamp the error is half a step
    inner = (q > 0) & (q < 15)
    assert (err[inner] <= s[inner] * 0.5 * (1 + 2.0 ** -20) + np.abs(w.astype(np.float64))[inner] * 2.0 ** -22).all()


def test_codes_range_and_extremes():
    w = _groups_with_edges(seed=1)
    q, s16, z = int4.quantize_codes(w)
    assert q.min() >= 0 and q.max() <= 15 and z.min() >= 0 and z.max() <= 15
    g = w.astype(np.float32).reshape(w.shape[0], -1, 128)
    qg = q.reshape(g.shape)
    for n in range(g.shape[0]):
        for j in range(g.shape[1]):
            lo, hi = g[n, j].min(), g[n, j].max()
            if lo < 0:
                assert qg[n, j, g[n, j].argmin()] == 0
            if hi > 0 and lo < 0 and s16[n, j] >= 2.0 ** -14:
                # a normal fp16 scale is within 2^-11 of (hi - lo)/15
                assert qg[n, j, g[n, j].argmax()] in (14, 15)
    # 16 levels: an evenly spread group uses every one of them
    spread = np.linspace(-0.03, 0.05, 128).astype(np.float16)[None, :]
    assert np.unique(int4.quantize_codes(spread)[0]).tolist() == list(range(16))


def test_grid_is_a_fixed_point():
    """Weights already on a grid (q - z) s16 with codes 0 and 15 present
    quantize back to exactly that grid (scale, zero and every code)."""
    r = np.random.default_rng(7)
    n, k = 32, 256
    # scales with at most 7 significant bits so (q - z) s16 is exact in fp16
    mant = r.integers(64, 128, size=(n, 2))
    expo = r.integers(-14, -4, size=(n, 2)).astype(np.float64)
    s16 = (mant * 2.0 ** (expo - 6)).astype(np.float16)
    z = r.integers(1, 15, size=(n, 2))
    q = r.integers(0, 16, size=(n, k))
    q[:, 0] = 0
    q[:, 1] = 15
    q[:, 128] = 0
    q[:, 129] = 15
    s = np.repeat(s16.astype(np.float64), 128, axis=1)
    zz = np.repeat(z, 128, axis=1)
    w = ((q - zz) * s).astype(np.float16)
    assert np.array_equal(w.astype(np.float64), (q - zz) * s)  # exact grid
    q2, s2, z2 = int4.quantize_codes(w)
    assert np.array_equal(s2, s16)
    assert np.array_equal(z2, z)
    assert np.array_equal(q2, q)


def _rn16(fr):
    """Exact rational -> nearest fp16 (via the correctly rounded double)."""
    return Fraction(struct.unpack("<e", struct.pack("<e", float(fr)))[0])


def _rne_frac(fr):
    f = fr.numerator // fr.denominator
    rem = fr - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return f


def test_against_exact_rational_arithmetic():
    """Recompute scale, zero and codes with exact rationals (fractions)."""
    w = _groups_with_edges(seed=3, n=12, k=256)
    q, s16, z = int4.quantize_codes(w)
    near_tie = 0
    for n in range(w.shape[0]):
        for g in range(w.shape[1] // 128):
            vals = [Fraction(float(v)) for v in w[n, g * 128:(g + 1) * 128]]
            lo = min(min(vals), Fraction(0))
            hi = max(max(vals), Fraction(0))
            s = _rn16((hi - lo) / 15)
            if s == 0:
                s = Fraction(1)
            assert s == Fraction(float(s16[n, g]))
            zr = min(max(_rne_frac(-lo / s), 0), 15)
            assert zr == z[n, g]
            for t, v in enumerate(vals):
                quo = v / s
                frac = quo - (quo.numerator // quo.denominator)
                if abs(frac - Fraction(1, 2)) < Fraction(1, 2 ** 20) * (1 + abs(quo)):
                    # within fp32 rounding of a tie: either neighbour is right
                    near_tie += 1
                    lo_c = quo.numerator // quo.denominator
                    ok = {min(max(c + zr, 0), 15) for c in (lo_c, lo_c + 1)}
                    assert q[n, g * 128 + t] in ok
                    continue
                qr = min(max(_rne_frac(quo) + zr, 0), 15)
                assert qr == q[n, g * 128 + t], (n, g, t)
    assert near_tie < w.size // 20


def test_exact_ties_round_half_even():
    """w = (j + 1/2) s16 exactly: the code is the even neighbour."""
    s16 = np.float16(2.0 ** -6)
    z = 8
    lo = -z * float(s16)                     # group minimum -> zero point 8
    hi = (15 - z) * float(s16)
    vals = [lo, hi] + [(j + 0.5) * float(s16) for j in range(-7, 6)]
    row = np.zeros(128, dtype=np.float16)
    row[: len(vals)] = np.array(vals, dtype=np.float16)
    q, s, zz = int4.quantize_codes(row[None, :])
    assert s[0, 0] == s16 and zz[0, 0] == z
    for i, j in enumerate(range(-7, 6)):
        expect = j if j % 2 == 0 else j + 1
        assert q[0, 2 + i] == expect + z


def test_packing_hand_example():
    gold = load("int4_pack_example.txt")
    codes = np.array([int(c) for c in gold["codes"].split()], dtype=np.int32)[None, :]
    words = [int(h, 16) for h in gold["words"].split()]
    packed = int4.pack_codes(codes)
    assert packed.tolist() == [words]
    assert np.array_equal(int4.unpack_codes(packed, 16), codes)
    zeros = np.array([int(c) for c in gold["zeros"].split()], dtype=np.int32)[None, :]
    zb = [int(h, 16) for h in gold["zero_bytes"].split()]
    assert int4.pack_zeros(zeros).tolist() == [zb]
    assert np.array_equal(int4.unpack_zeros(int4.pack_zeros(zeros), 3), zeros)


def test_packing_matches_hex_digits():
    """Nibble k%8 of a word is hex digit (7 - k%8) of its 8-digit spelling."""
    r = np.random.default_rng(11)
    q = r.integers(0, 16, size=(5, 64))
    packed = int4.pack_codes(q)
    for n in range(5):
        for wi in range(8):
            digits = format(int(packed[n, wi]), "08x")[::-1]
            assert [int(d, 16) for d in digits] == q[n, wi * 8:(wi + 1) * 8].tolist()


def test_dequantize_single_rounding():
    """w_hat = round16((q - z) s16): check against rational products rounded
    by struct's half-precision conversion."""
    w = _groups_with_edges(seed=5, n=8, k=256)
    qw, s16, zp = int4.quantize(w)
    wh = int4.dequantize(qw, s16, zp, 256)
    q = int4.unpack_codes(qw, 256)
    z = int4.unpack_zeros(zp, 2)
    for n in range(8):
        for t in range(0, 256, 7):
            g = t // 128
            exact = (q[n, t] - z[n, g]) * Fraction(float(s16[n, g]))
            assert Fraction(float(wh[n, t])) == _rn16(exact)


def test_memory_figures_from_the_pages():
    gold = load("memory_accounting.txt")
    p = float(gold["params_7b"])
    # 4 bits per weight: half a byte each
    assert p * 4 / 8 / 1e9 == pytest.approx(float(gold["int4_gb_7b"]))
    assert p * 16 / 8 / 1e9 == pytest.approx(float(gold["fp16_gb_7b"]))
    # one fp16 scale per group of 128: the scale overhead printed for Qwen2-1.5B
    n, k = 1536, 1536
    codes_only = n * k // 2
    zero_bytes = n * ((k // 128 + 1) // 2)
    scale_bytes = int4.packed_bytes(n, k) - codes_only - zero_bytes
    per_param = scale_bytes / (n * k)
    q = float(gold["params_qwen2_1_5b"]) * per_param / 1e9
    assert q == pytest.approx(float(gold["scale_gb_qwen2_1_5b"]), rel=0.03)


def _perm(k, seed):
    """A synthetic act-order: channels by decreasing seeded importance."""
    return np.argsort(-np.random.default_rng(seed).random(k), kind="stable")


def test_act_order_identity_is_plain_quantization():
    w = workloads.weights(24, 512, 4, 1)
    ident = np.arange(512)
    plain = int4.dequantize(*int4.quantize(w), 512)
    np.testing.assert_array_equal(int4.dequantize_act_order(w, ident), plain)
    for a, b in zip(int4.quantize_act_order(w, ident), int4.quantize(w)):
        assert np.array_equal(a, b)


def test_act_order_two_formulations_agree():
    """Storage in quantization order (contiguous groups of W[:, perm]) and
    the original-order g_idx definition give the same dequantized weights
    channel by channel."""
    n, k = 16, 768
    w = workloads.weights(n, k, 5, 1)
    perm = _perm(k, 9)
    stored = int4.dequantize(*int4.quantize_act_order(w, perm), k)
    back = np.empty_like(stored)
    back[:, perm] = stored
    np.testing.assert_array_equal(back, int4.dequantize_act_order(w, perm))
    # and it is not the plain quantization
    assert not np.array_equal(back, int4.dequantize(*int4.quantize(w), k))


def test_act_order_group_membership_brute_force():
    """Tiny case: the group of each channel found by scanning perm."""
    k, group = 256, 128
    perm = _perm(k, 3)
    gi = int4.g_idx(perm, group)
    for c in range(k):
        pos = [j for j in range(k) if perm[j] == c][0]
        assert gi[c] == pos // group
    assert np.bincount(gi).tolist() == [group] * (k // group)
