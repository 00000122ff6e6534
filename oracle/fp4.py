"""FP4 (E2M1) blockwise quantization (oracle): the FP4 variant of the NF4 path.

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product.

The pages: bitsandbytes offers FP4 next to NF4 as its second 4-bit format
([P1] section 6.3: NF4 is the more accurate one, FP4 the one closer to
hardware), and an FP4 code is a sign bit, a 2-bit exponent and a 1-bit
mantissa ([P5] section 7.2, the E2M1 layout).

Reading taken (the pages give the layout, not the variant's details): the
same blocks of 64, absmax scaling and double quantization as NF4; the
16 codes are the E2M1 bit patterns s eem with exponent bias 1, so the
magnitudes are 0 and m/2 for e = 0 (subnormal) and 2^(e-1) (1 + m/2) for
e > 0, i.e. {0, 1/2, 1, 3/2, 2, 3, 4, 6}; the codebook divides them by the
largest (6) so that the block absmax maps to code 7 (and -absmax to 15).
Encoding: the sign bit is set for w/a < 0, the magnitude code counts the 7
fp32 midpoints between adjacent magnitudes that |w/a| exceeds (nearest
magnitude, ties to the lower); an all-zero block gives code 0.  Code 8 is
-0 and decodes to 0.  The dequantized weight is the 16-bit rounding of
L[code] * absmax_hat, exactly as for NF4.
"""

import numpy as np

from . import nf4
from .numerics import f32, round_to


def e2m1_value(code):
    """Value of a 4-bit E2M1 code (sign bit 3, exponent bits 2..1, mantissa
    bit 0, exponent bias 1), as a Python float."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return -mag if s else mag


def codebook():
    """The 16 levels indexed by code, fp32: E2M1 value / 6 (code 8 is -0)."""
    return np.array([e2m1_value(c) / 6.0 for c in range(16)], dtype=np.float32)


def magnitude_thresholds():
    """The 7 fp32 midpoints between adjacent magnitudes (codes 0..7)."""
    lv = codebook()[:8]
    return (lv[:-1] + lv[1:]) * np.float32(0.5)


def encode(w, block=64):
    """Blockwise absmax FP4 encode.  Returns ``(codes uint8 [numel]
    unpacked, absmax fp32 [numel/block])``."""
    flat = f32(w).reshape(-1)
    if flat.size % block:
        raise ValueError("numel must be a multiple of the block size")
    b = flat.reshape(-1, block)
    absmax = np.abs(b).max(axis=1)
    safe = np.where(absmax == 0, np.float32(1), absmax)
    normed = b / safe[:, None]                        # fp32 IEEE division
    mag = np.abs(normed)
    codes = np.zeros(b.shape, dtype=np.int32)
    for t in magnitude_thresholds():
        codes += (mag > t)
    codes += np.where(normed < 0, 8, 0)
    codes[absmax == 0, :] = 0
    return codes.reshape(-1).astype(np.uint8), absmax.astype(np.float32)


def quantize(w, block=64, double_quant=True, block2=256):
    """Encode + pack (+ double quantization), the NF4 layout: ``(packed
    codes uint8 [numel/2], absmax, absmax_scale)``."""
    codes, a = encode(w, block)
    if double_quant:
        q8, c2 = nf4.double_quantize(a, block2)
        return nf4.pack(codes), q8, c2
    return nf4.pack(codes), a, None


def dequantize(packed, absmax, absmax_scale, shape, block=64, block2=256, out_dtype="bf16"):
    """w_hat = round_to_dtype(L[code] * absmax_hat) as fp32 [shape]."""
    codes = nf4.unpack(packed)
    if absmax_scale is None:
        a = np.asarray(absmax, dtype=np.float32)
    else:
        a = nf4.absmax_hat(absmax, absmax_scale, block2)
    prod = codebook()[codes] * np.repeat(a, block)   # fp32 product
    return round_to(prod, out_dtype).reshape(shape)
