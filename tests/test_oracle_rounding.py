"""Exact-rational pins of the oracle's "fp32 product, then one 16-bit
rounding" steps (CPU only).

Three oracle functions form a 16-bit value from a product that is not exact
in fp32:
  * ``llm_int8.dequant_weight_f16``: the outlier weights w16 = fp16(fp32(q * sw))
    ("LLM quantization selection", section 2.1: outliers stay in FP16; the
    int8 weights are dequantized back, no fp16 copy of W is kept);
  * ``llm_int8.scale_columns``: SmoothQuant's column scaling round16(fp32(a * s))
    (same page, section 5);
  * ``nf4.dequantize``: w_hat = bf16(fp32(L[code] * a_hat)) with
    a_hat = fp32(q8 * c2) (same page, sections 6.1-6.3: dequantize to the
    compute dtype with the double-quantized absmax).

Each is checked against exact rational arithmetic (``tests/exact_fp.py``) on
inputs constructed next to the 16-bit rounding boundaries, where every
plausible slip -- skipping the fp32 rounding, rounding a_hat differently or
multiplying in another order, casting to the wrong 16-bit type, dropping the
16-bit cast -- gives a different value.  Every test first proves on its own
cases that each slip is caught, then requires the oracle to equal the
definition on all of them.  The NF4 round trip is also bounded element by
element.
"""

import itertools
from fractions import Fraction

import numpy as np

from exact_fp import BF16, FP16, FP32, exact, f32, f32_next, rn, ulp
from oracle import llm_int8, nf4


def _midpoints(fmt, rng, count, lo_exp, hi_exp):
    """`count` exact midpoints between adjacent positive values of `fmt`."""
    p, _ = fmt
    out = []
    for _ in range(count):
        e = int(rng.integers(lo_exp, hi_exp))
        sig = int(rng.integers(2 ** (p - 1), 2 ** p - 1))
        h = Fraction(sig) * Fraction(2) ** (e - p + 1)
        out.append(h + ulp(h, fmt) / 2)
    return out


def _search(candidates, correct, alts, need=2, cap=20000):
    """Walk `candidates` (tuples); keep a case when some alternative formula
    disagrees with `correct` on it.  Stops once every alternative has been
    caught `need` times.  Returns the kept cases and the catch counts."""
    kept, caught = [], {k: 0 for k in alts}
    for i, case in enumerate(candidates):
        if i >= cap or all(v >= need for v in caught.values()):
            break
        good = correct(*case)
        hit = False
        for name, f in alts.items():
            if caught[name] < need and f(*case) != good:
                caught[name] += 1
                hit = True
        if hit:
            kept.append(case)
    return kept, caught


def _near(mid, mult, span):
    """fp32 values s with mult * s within a few fp32 steps of `mid`."""
    s0 = f32(mid / mult)
    for j in range(-span, span + 1):
        s = f32_next(s0, j)
        if s > 0:
            yield s


# ------------------------------------------------------ int8 outlier weights
def test_dequant_weight_f16_is_fp32_product_then_fp16():
    rng = np.random.default_rng(11)
    mids = _midpoints(FP16, rng, 40, -8, 0)
    qs = [3, 5, 7, 9, 11, 13, 19, 25, 37, 53, 77, 99, 113, 127]

    def cands():
        for mid, q in itertools.product(mids, qs):
            for s in _near(mid, q, 24):
                yield (q, s)
    correct = lambda q, s: rn(rn(q * exact(s), FP32), FP16)
    alts = {
        "single rounding (no fp32 step)": lambda q, s: rn(q * exact(s), FP16),
        "no fp16 cast": lambda q, s: rn(q * exact(s), FP32),
        "bf16 instead of fp16": lambda q, s: rn(rn(q * exact(s), FP32), BF16),
        "scale rounded to fp16 first": lambda q, s: rn(rn(q * rn(exact(s), FP16), FP32), FP16),
    }
    cases, caught = _search(cands(), correct, alts)
    assert all(v >= 2 for v in caught.values()), caught
    # plus ordinary random cases, both signs
    for _ in range(200):
        cases.append((int(rng.integers(-127, 128)), float(np.float32(rng.uniform(1e-5, 1e-3)))))
    qw = np.zeros((len(cases), 4), np.int8)
    sw = np.zeros(len(cases), np.float32)
    for i, (q, s) in enumerate(cases):
        qw[i, 0], qw[i, 1], sw[i] = q, -q, s
    got = llm_int8.dequant_weight_f16(qw, sw)
    for i, (q, s) in enumerate(cases):
        assert Fraction(float(got[i, 0])) == correct(q, s), (q, s)
        assert Fraction(float(got[i, 1])) == correct(-q, s), (q, s)
        assert got[i, 2] == 0.0


# ----------------------------------------------------- SmoothQuant scaling
def test_scale_columns_is_fp32_product_then_16bit():
    rng = np.random.default_rng(12)
    mults = [3.0, 5.0, 0.75, 1.375, 2.5, 6.125, 0.0234375, 11.0, 13.5, 0.3125]
    for fmt, name in ((FP16, "f16"), (BF16, "bf16")):
        mids = _midpoints(fmt, rng, 30, -10, 2)
        other = BF16 if fmt == FP16 else FP16

        def cands():
            for mid, a in itertools.product(mids, mults):
                for s in _near(mid, Fraction(a), 24):
                    yield (a, s)
        correct = lambda a, s: rn(rn(exact(a) * exact(s), FP32), fmt)
        alts = {
            "single rounding": lambda a, s: rn(exact(a) * exact(s), fmt),
            "no 16-bit cast": lambda a, s: rn(exact(a) * exact(s), FP32),
            "other 16-bit type": lambda a, s: rn(rn(exact(a) * exact(s), FP32), other),
        }
        cases, caught = _search(cands(), correct, alts)
        assert all(v >= 2 for v in caught.values()), (name, caught)
        a16 = np.array([[a for a, _ in cases]], np.float16)
        assert all(float(v) == a for v, (a, _) in zip(a16[0], cases))   # exact in fp16
        sc = np.array([s for _, s in cases], np.float32)
        got = llm_int8.scale_columns(a16, sc, name)
        for i, (a, s) in enumerate(cases):
            assert Fraction(float(got[0, i])) == correct(a, s), (name, a, s)


# ----------------------------------------------------------- NF4 dequantize
def _pack_pairs(codes):
    c = np.asarray(codes, np.uint8).reshape(-1, 2)
    return (c[:, 0] | (c[:, 1] << 4)).astype(np.uint8)


def test_nf4_dequantize_is_level_times_ahat_then_bf16():
    """w_hat = bf16(fp32(L[code] * a_hat)), a_hat = fp32(fp32(q8) * c2)."""
    L = [float(v) for v in nf4.codebook()]
    rng = np.random.default_rng(13)
    mids = _midpoints(BF16, rng, 24, -9, -3)

    def ah(q8, c2):
        return rn(q8 * exact(c2), FP32)

    correct = lambda c, q8, c2: rn(rn(exact(L[c]) * ah(q8, c2), FP32), BF16)
    alts = {
        "single rounding": lambda c, q8, c2: rn(exact(L[c]) * ah(q8, c2), BF16),
        "a_hat not rounded to fp32": lambda c, q8, c2: rn(rn(exact(L[c]) * q8 * exact(c2), FP32), BF16),
        "a_hat rounded to bf16 first": lambda c, q8, c2: rn(rn(exact(L[c]) * rn(ah(q8, c2), BF16), FP32), BF16),
        "(L * q8) * c2 order": lambda c, q8, c2: rn(rn(rn(exact(L[c]) * q8, FP32) * exact(c2), FP32), BF16),
        "no bf16 cast": lambda c, q8, c2: rn(exact(L[c]) * ah(q8, c2), FP32),
        "fp16 instead of bf16": lambda c, q8, c2: rn(rn(exact(L[c]) * ah(q8, c2), FP32), FP16),
    }
    codes = [c for c in range(16) if c != 7]

    def cands():
        for mid, c, q8 in itertools.product(mids, codes, (1, 3, 7, 13, 27, 61, 101, 127)):
            for c2 in _near(mid, abs(exact(L[c])) * q8, 12):
                yield (c, q8, c2)
    cases, caught = _search(cands(), correct, alts)
    assert all(v >= 2 for v in caught.values()), caught
    # one block of 64 per case (block2 = 1: one second-level scale per block);
    # element 0 carries the case, element 1 code 15 - c, the rest the exact
    # zero level
    nb = len(cases)
    codes_arr = np.full((nb, 64), 7, np.uint8)
    q8 = np.zeros(nb, np.int8)
    c2 = np.zeros(nb, np.float32)
    for i, (c, q, s) in enumerate(cases):
        codes_arr[i, 0], codes_arr[i, 1] = c, 15 - c
        q8[i], c2[i] = q, s
    got = nf4.dequantize(_pack_pairs(codes_arr.reshape(-1)), q8, c2, (nb, 64), block=64, block2=1)
    for i, (c, q, s) in enumerate(cases):
        assert Fraction(float(got[i, 0])) == correct(c, q, s), (c, q, s)
        c1 = int(codes_arr[i, 1])
        assert Fraction(float(got[i, 1])) == correct(c1, q, s), (c1, q, s)
        assert (got[i, 2:] == 0).all()


def test_nf4_round_trip_bound():
    """|w - w_hat| <= a * (half the widest level gap) + |a - a_hat| + the fp32
    and bf16 roundings of the product, per element, for N(0, 0.02) bf16
    weights with double-quantized absmax."""
    rng = np.random.default_rng(14)
    w32 = (rng.standard_normal((64, 1024)) * 0.02).astype(np.float32)
    # bf16 weights: keep the top 16 bits (a valid bf16 value, exact in fp32)
    w = (w32.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    packed, q8, c2 = nf4.quantize(w)
    wh = nf4.dequantize(packed, q8, c2, w.shape).astype(np.float64)
    a = np.abs(w.reshape(-1, 64)).max(axis=1).astype(np.float64)
    ahat = q8.astype(np.float64) * np.repeat(c2.astype(np.float64), 256)[: a.size]
    half_gap = 0.5 * np.diff(nf4.codebook().astype(np.float64)).max()
    bound = (np.repeat(a * half_gap + np.abs(a - ahat) * (1 + 2.0 ** -23), 64)
             + (2.0 ** -8 + 2.0 ** -23) * np.abs(wh.reshape(-1)) + 2.0 ** -133)
    err = np.abs(w.reshape(-1).astype(np.float64) - wh.reshape(-1))
    assert (err <= bound).all()
    # and the bound is not slack: the worst element uses most of it
    assert (err / bound).max() > 0.5
