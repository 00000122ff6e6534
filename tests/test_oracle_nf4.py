"""Pins for the NF4 oracle (CPU only): the codebook's defining properties,
an independent recomputation of the normal quantiles, nearest-level encoding
by brute force, and the double-quantization error bound."""

import math

import numpy as np
import torch

from oracle import nf4
from oracle.numerics import bf16_bits_to_f32


def _phi_inv_bisect(p):
    """Normal quantile by bisection on the complementary error function
    (independent of statistics.NormalDist)."""
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if 0.5 * math.erfc(-mid / math.sqrt(2.0)) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def test_codebook_shape_and_anchors():
    L = nf4.codebook()
    assert L.dtype == np.float32 and L.shape == (16,)
    assert (np.diff(L) > 0).all()
    assert L[7] == 0.0 and L[0] == -1.0 and L[15] == 1.0
    assert (L[:7] < 0).all() and (L[8:] > 0).all()


def test_codebook_independent_quantiles():
    """Same construction, quantiles from bisection on erfc: equal in fp32."""
    pmax = 1 - 1 / 32
    top = _phi_inv_bisect(pmax)
    pos = [_phi_inv_bisect(0.5 + (pmax - 0.5) * i / 8) / top for i in range(1, 9)]
    neg = [-_phi_inv_bisect(0.5 + (pmax - 0.5) * i / 7) / top for i in range(1, 8)]
    ref = np.array(sorted(neg) + [0.0] + pos, dtype=np.float32)
    assert np.array_equal(ref, nf4.codebook())


def test_codebook_equal_probability_bins():
    """Quantile quantization: on each side the levels sit at equally spaced
    probabilities of the normal distribution."""
    L = nf4.codebook().astype(np.float64)
    top = _phi_inv_bisect(1 - 1 / 32)
    cdf = [0.5 * math.erfc(-(v * top) / math.sqrt(2.0)) for v in L]
    dpos = np.diff(cdf[7:])
    dneg = np.diff(cdf[:8])
    assert np.allclose(dpos, dpos[0], rtol=1e-5)
    assert np.allclose(dneg, dneg[0], rtol=1e-5)


def test_codebook_denser_near_zero():
    """Gaps between adjacent levels grow moving away from 0 on both sides."""
    g = np.diff(nf4.codebook())
    assert (np.diff(g[7:]) > 0).all()          # positive side, outward
    assert (np.diff(g[:7]) < 0).all()          # negative side, outward (leftward)


def test_thresholds_are_midpoints():
    L = nf4.codebook()
    T = nf4.thresholds()
    assert T.shape == (15,)
    assert ((T > L[:-1]) & (T < L[1:])).all()


def test_encode_nearest_level_brute_force():
    r = np.random.default_rng(0)
    w = (r.standard_normal((8, 256)) * 0.02).astype(np.float16)
    codes, a = nf4.encode(w)
    L = nf4.codebook().astype(np.float64)
    n = (w.astype(np.float64).reshape(-1, 64) / a[:, None].astype(np.float64)).reshape(-1)
    dist = np.abs(n[:, None] - L[None, :])
    best = dist.argmin(axis=1)
    second = np.sort(dist, axis=1)[:, 1]
    clear = (second - dist.min(axis=1)) > 1e-6
    assert np.array_equal(codes[clear], best[clear])
    # the error never exceeds half the local gap
    gaps = np.diff(L)
    half = 0.5 * np.maximum(np.r_[gaps, 0][codes], np.r_[0, gaps][codes])
    assert (np.abs(n - L[codes]) <= half + 1e-7).all()


def test_encode_extremes_and_zero_block():
    w = np.zeros((2, 128), dtype=np.float32)
    w[0, 3] = 0.5
    w[0, 9] = -0.25
    w[0, 64 + 5] = -0.75
    w[0, 64 + 6] = 0.1
    codes, a = nf4.encode(w.astype(np.float16))
    assert a.tolist()[:2] == [0.5, 0.75] and a[2] == 0 and a[3] == 0
    assert codes[3] == 15 and codes[64 + 5] == 0
    assert codes[0] == 7                       # exact 0 -> the zero level
    assert (codes[128:] == 7).all()            # all-zero blocks


def test_encode_tie_goes_to_lower_level():
    """A normalised value exactly on a midpoint takes the lower level."""
    T = nf4.thresholds()
    w = np.zeros(64, dtype=np.float32)
    w[0] = 1.0                                   # absmax 1: n = w exactly
    w[1:16] = T
    codes, a = nf4.encode(w)
    assert a[0] == 1.0
    assert codes[1:16].tolist() == list(range(15))


def test_pack_nibble_order():
    codes = np.arange(16, dtype=np.uint8)
    p = nf4.pack(codes)
    assert p.tolist() == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert np.array_equal(nf4.unpack(p), codes)


def test_double_quant_bound():
    r = np.random.default_rng(1)
    a = np.abs(r.standard_normal(1000)).astype(np.float32) * 0.05
    q8, c2 = nf4.double_quantize(a, 256)
    assert c2.shape == (4,) and q8.dtype == np.int8
    assert q8.min() >= 0 and q8.max() <= 127
    ah = nf4.absmax_hat(q8, c2)
    c = np.repeat(c2, 256)[:1000].astype(np.float64)
    assert (np.abs(a - ah.astype(np.float64)) <= c * 0.5 * (1 + 2.0 ** -20)).all()
    for j in range(4):
        seg = a[j * 256:(j + 1) * 256]
        assert q8[j * 256 + seg.argmax()] == 127


def test_double_quant_zero_block():
    q8, c2 = nf4.double_quantize(np.zeros(300, np.float32), 256)
    assert (q8 == 0).all() and c2.tolist() == [1.0, 1.0]


def test_dequantize_matches_torch_bf16_rounding():
    r = np.random.default_rng(2)
    w = (r.standard_normal((4, 512)) * 0.02).astype(np.float32)
    packed, q8, c2 = nf4.quantize(w.astype(np.float16))
    wh = nf4.dequantize(packed, q8, c2, (4, 512))
    codes = nf4.unpack(packed)
    prod = nf4.codebook()[codes] * np.repeat(nf4.absmax_hat(q8, c2), 64)
    ref = torch.from_numpy(prod.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(wh.reshape(-1), ref)


def test_bf16_helpers_match_torch():
    r = np.random.default_rng(3)
    v = (r.standard_normal(10000) * np.exp(r.uniform(-20, 20, 10000))).astype(np.float32)
    # exact ties: low 16 bits 0x8000 with both parities of the kept bit
    ties = (r.integers(0x3000, 0x4800, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    v = np.concatenate([v, ties, -ties])
    from oracle.numerics import round_bf16_bits
    mine = bf16_bits_to_f32(round_bf16_bits(v))
    ref = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
    assert np.array_equal(mine, ref)


def test_about_half_the_levels_within_one_sigma():
    """Loose check of the printed claim that about 68% of weights lie within
    +-1 sigma and get 8 of the 16 levels ([P5] section 6.2): with absmax-64
    normalisation of N(0, s^2) weights, sigma of the normalised values is
    about 0.4, and 8 +- 1 levels fall inside +-sigma."""
    r = np.random.default_rng(4)
    w = (r.standard_normal((64, 4096)) * 0.02).astype(np.float32)
    b = w.reshape(-1, 64)
    sig = float((b / np.abs(b).max(axis=1, keepdims=True)).std())
    inside = int((np.abs(nf4.codebook()) <= sig).sum())
    assert 7 <= inside <= 9
