"""Rounding helpers shared by the oracle modules (oracle-internal).

bf16 values are carried as ``np.uint16`` bit patterns because NumPy has no
bfloat16 dtype; fp16 values use ``np.float16``.

All conversions are IEEE round-to-nearest, ties-to-even.  None of the pages
names a rounding mode; ties-to-even is the IEEE default and the mode every
conversion instruction of the target uses, so it is the reading taken
throughout.
"""

import numpy as np


def rne(a):
    """Round to the nearest integer, ties to even (IEEE default), same dtype."""
    return np.rint(a)


def f32(a):
    """Exact widening of fp16 / fp32 input to fp32 (no rounding involved)."""
    return np.asarray(a, dtype=np.float32)


def round_f16(a32):
    """fp32 -> fp16, round to nearest even (NumPy's cast is IEEE RNE)."""
    return np.asarray(a32, dtype=np.float32).astype(np.float16)


def round_bf16_bits(a32):
    """fp32 -> bf16 bit pattern (uint16), round to nearest even.

    bf16 keeps the top 16 bits of the fp32 encoding.  Adding 0x7FFF plus the
    lowest kept bit before truncating rounds to nearest with ties to even.
    Inputs are finite (NaN handling is not needed by any caller).
    """
    u = np.asarray(a32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """bf16 bit pattern (uint16) -> fp32, exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def round_to(a32, dtype):
    """Round fp32 values to the 16-bit type ``dtype`` and return them as fp32.

    ``dtype`` is ``"f16"`` or ``"bf16"``; the result is the rounded value,
    widened back to fp32 (exactly).
    """
    if dtype == "f16":
        return round_f16(a32).astype(np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(round_bf16_bits(a32))
    raise ValueError(f"unknown 16-bit dtype {dtype!r}")
