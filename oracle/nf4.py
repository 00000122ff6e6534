"""NF4 (4-bit NormalFloat) blockwise quantization with double quantization (oracle).

What the pages fix:
  * NF4 is quantile quantization: 16 values placed at normal-distribution
    quantiles of evenly spaced probabilities, so that every bin is equally
    likely and the levels are densest near 0 ([P1] section 6.1; [P2]
    section 七; [P5] section 6.2).
  * Blockwise: each block of 64 weights shares one scale, the block's
    absolute maximum ([P1] section 6.3).
  * Double quantization quantizes those scales again ([P1] section 6.2;
    [P2] section 七; [P5] section 6.1, ``bnb_4bit_use_double_quant``).
  * Codes are stored two per byte, ``quant_storage = uint8`` ([P5] 6.1), and
    the weights are dequantized to the compute dtype (bf16) before the
    matmul ([P1] section 6.2).

Readings taken where the pages are silent:
  * Levels.  With p_max = 1 - 1/32 (the centre of the outermost of 16 equal
    probability bins, which keeps the quantiles finite), the 8 positive
    levels are PhiInv(p)/PhiInv(p_max) for the 8 probabilities
    evenly spaced in (0.5, p_max], the 7 negative levels are the mirror of
    the 7 evenly spaced in (0.5, p_max], and one level is exactly 0.  The
    table is ascending: index 0 = -1, index 7 = 0, index 15 = +1.  Values are
    computed in double precision and rounded once to fp32.
  * Encode: n = w / absmax (fp32 division); the code is the number of the 15
    fp32 midpoints T_i = (L_i + L_{i+1}) * 0.5 (fp32) that n exceeds -- the
    nearest level, ties going to the lower level.  An all-zero block gets
    code 7 (the exact 0).  Blocks of 64 run over the row-major flattening of
    W; element 2j is the low nibble of byte j (this equals the INT4 nibble
    order inside a little-endian uint32 word).
  * Double quantization: blocks of 256 consecutive absmax values; the second
    level scale is c2 = max(absmax)/127 in fp32 (1.0 if that is 0), and the
    int8 code is clamp(round_half_even(absmax / c2), 0, 127).  The dequantized
    absmax is fp32(code) * c2.
  * Dequantized weight: round_to_dtype(L[code] * absmax_hat), an fp32 product
    rounded once into the activation dtype (bf16 for the NF4 workloads).
"""

import math
import statistics

import numpy as np

from .numerics import f32, rne, round_to

P_MAX = 1.0 - 1.0 / 32.0
ZERO_INDEX = 7


def codebook():
    """The 16 NF4 levels as fp32, ascending, with L[7] == 0 exactly."""
    inv = statistics.NormalDist().inv_cdf
    top = inv(P_MAX)
    pos = [inv(0.5 + (P_MAX - 0.5) * i / 8) / top for i in range(1, 9)]
    neg = [-inv(0.5 + (P_MAX - 0.5) * i / 7) / top for i in range(1, 8)]
    levels = sorted(neg) + [0.0] + pos
    return np.array(levels, dtype=np.float32)


def thresholds(levels=None):
    """The 15 fp32 decision midpoints between adjacent levels."""
    lv = codebook() if levels is None else np.asarray(levels, np.float32)
    return (lv[:-1] + lv[1:]) * np.float32(0.5)


def encode(w, block=64):
    """Blockwise absmax NF4 encode.

    ``w`` is a 16-bit weight matrix (float16, or bf16 widened to fp32).
    Returns ``(codes uint8 [numel] unpacked, absmax fp32 [numel/block])``.
    """
    flat = f32(w).reshape(-1)
    if flat.size % block:
        raise ValueError("numel must be a multiple of the block size")
    b = flat.reshape(-1, block)
    absmax = np.abs(b).max(axis=1)
    safe = np.where(absmax == 0, np.float32(1), absmax)
    normed = b / safe[:, None]                        # fp32 IEEE division
    t = thresholds()
    codes = np.zeros(b.shape, dtype=np.int32)
    for ti in t:
        codes += (normed > ti)
    codes[absmax == 0, :] = ZERO_INDEX
    return codes.reshape(-1).astype(np.uint8), absmax.astype(np.float32)


def pack(codes):
    """Two codes per byte: element 2j -> low nibble of byte j."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1, 2)
    return (c[:, 0] | (c[:, 1] << np.uint8(4))).astype(np.uint8)


def unpack(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.size, 2), dtype=np.uint8)
    out[:, 0] = p & 0xF
    out[:, 1] = p >> 4
    return out.reshape(-1)


def double_quantize(absmax, block2=256):
    """Second-level quantization of the absmax values.

    Returns ``(q8 int8 [nblocks], c2 fp32 [ceil(nblocks/block2)])``.
    """
    a = np.asarray(absmax, dtype=np.float32)
    nb = a.size
    n2 = (nb + block2 - 1) // block2
    q8 = np.empty(nb, dtype=np.int8)
    c2 = np.empty(n2, dtype=np.float32)
    for j in range(n2):
        seg = a[j * block2:(j + 1) * block2]
        c = seg.max() / np.float32(127)               # fp32 IEEE division
        if c == 0:
            c = np.float32(1)
        c2[j] = c
        q8[j * block2:(j + 1) * block2] = np.clip(rne(seg / c), 0, 127).astype(np.int8)
    return q8, c2


def absmax_hat(q8, c2, block2=256):
    """Dequantized absmax: fp32(q8) * c2 (fp32 product)."""
    q = np.asarray(q8, dtype=np.int8).astype(np.float32)
    c = np.repeat(np.asarray(c2, np.float32), block2)[: q.size]
    return q * c


def quantize(w, block=64, double_quant=True, block2=256):
    """Encode + pack (+ double quantization).

    Returns ``(packed codes uint8 [numel/2], absmax, absmax_scale)`` where
    ``absmax`` is int8 codes and ``absmax_scale`` the fp32 second-level scales
    when ``double_quant``; otherwise ``absmax`` is fp32 and ``absmax_scale``
    is ``None``.
    """
    codes, a = encode(w, block)
    if double_quant:
        q8, c2 = double_quantize(a, block2)
        return pack(codes), q8, c2
    return pack(codes), a, None


def dequantize(packed, absmax, absmax_scale, shape, block=64, block2=256,
               out_dtype="bf16"):
    """w_hat = round_to_dtype(L[code] * absmax_hat) as fp32 [shape]."""
    codes = unpack(packed)
    lv = codebook()
    if absmax_scale is None:
        a = np.asarray(absmax, dtype=np.float32)
    else:
        a = absmax_hat(absmax, absmax_scale, block2)
    per_elem = np.repeat(a, block)
    prod = lv[codes] * per_elem                        # fp32 product
    return round_to(prod, out_dtype).reshape(shape)


def packed_bytes(n, k, block=64, double_quant=True, block2=256):
    """HBM bytes of one NF4 layer (codes + first- and second-level scales)."""
    nb = n * k // block
    if double_quant:
        return n * k // 2 + nb + 4 * math.ceil(nb / block2)
    return n * k // 2 + 4 * nb
