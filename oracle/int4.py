"""Asymmetric INT4 group-wise weight quantization (oracle).

What the pages fix:
  * Linear quantization stores integers plus a scale and a zero point; the
    zero point is the integer that stands for float 0, and asymmetric
    quantization shifts it away from 0 ([P2] section 一 "what quantization
    does"; [P4] section 1.1).
  * Asymmetric formula: scale = (max - min) / (2^b - 1),
    zero_point = round(-min / scale), codes in [0, 2^b - 1] ([P5] section 2.3,
    printed there for b = 8 as /255; here b = 4, so /15 and codes 0..15).
  * Per-group granularity, group_size = 128 along the input dimension as the
    usual choice ([P5] section 2.2; [P1] section 3.2; [P2] section 二).
  * INT4 takes half a byte per weight, 16 levels ([P2] opening; [P4] 1.1).
  * W4A16 dequantizes the weights back to 16-bit floats and multiplies in
    16-bit ([P1] section 5 opening; [P2] section 七 / 十一).

Readings taken where the pages are silent (each listed in the design notes):
  * "round" is round-half-to-even; divisions are IEEE fp32 divisions.
  * The scale is rounded to fp16 for storage before any code is computed, and
    codes are computed by dividing by that stored scale, so dequantization is
    consistent with the codes.
  * The quantization range is [min(min w, 0), max(max w, 0)]: the zero point
    must be an integer code that represents float 0, which needs 0 inside the
    range.  For groups that straddle 0 (every group of the synthetic
    N(0, 0.02) layers, with overwhelming probability) this is the printed
    formula unchanged.
  * A scale that is 0 in fp16 (an all-zero group, or a range so small that
    (max - min)/15 underflows fp16) is stored as 1.0.
  * Layout: W is [N][K] (N output features, K input features), groups run
    along K.  Codes: element (n, k) sits in bits 4*(k % 8) .. +3 of uint32
    word (n, k // 8).  Scales: fp16 [N][G], G = K / group.  Zero points: 4-bit,
    two per byte along G, group g in byte (n, g // 2), low nibble when g is
    even; the high nibble of a last odd byte is 0.
"""

import numpy as np

from .numerics import f32, rne, round_f16, round_to

BITS = 4
QMAX = (1 << BITS) - 1  # 15


def group_params(w16, group=128):
    """Per-(row, group) fp16 scale and integer zero point.

    Returns ``(s16, z)``: ``s16`` float16 [N][G], ``z`` int32 [N][G].
    """
    w = f32(w16)
    n, k = w.shape
    if k % group:
        raise ValueError("K must be a multiple of the group size")
    g = w.reshape(n, k // group, group)
    lo = np.minimum(g.min(axis=2), np.float32(0))
    hi = np.maximum(g.max(axis=2), np.float32(0))
    s32 = (hi - lo) / np.float32(QMAX)              # fp32 IEEE division
    s16 = round_f16(s32)                             # stored scale
    s16 = np.where(s16 == 0, np.float16(1), s16)     # degenerate group
    z = rne(-lo / s16.astype(np.float32))            # fp32 IEEE division
    z = np.clip(z, 0, QMAX).astype(np.int32)
    return s16, z


def quantize_codes(w16, group=128):
    """Unpacked INT4 codes [N][K] (int32), scales fp16 [N][G], zeros int32 [N][G]."""
    w = f32(w16)
    n, k = w.shape
    s16, z = group_params(w16, group)
    s = np.repeat(s16.astype(np.float32), group, axis=1)
    zz = np.repeat(z, group, axis=1)
    q = rne(w / s) + zz                              # fp32 IEEE division
    q = np.clip(q, 0, QMAX).astype(np.int32)
    return q, s16, z


def pack_codes(q):
    """Pack 4-bit codes [N][K] into uint32 [N][K/8]; element k -> bits 4*(k%8)."""
    q = np.asarray(q, dtype=np.uint32)
    n, k = q.shape
    if k % 8:
        raise ValueError("K must be a multiple of 8")
    q = q.reshape(n, k // 8, 8)
    out = np.zeros((n, k // 8), dtype=np.uint32)
    for j in range(8):
        out |= q[:, :, j] << np.uint32(4 * j)
    return out


def unpack_codes(words, k):
    """Inverse of :func:`pack_codes`."""
    words = np.asarray(words, dtype=np.uint32)
    n = words.shape[0]
    out = np.empty((n, k // 8, 8), dtype=np.int32)
    for j in range(8):
        out[:, :, j] = (words >> np.uint32(4 * j)) & np.uint32(0xF)
    return out.reshape(n, k)


def pack_zeros(z):
    """Pack 4-bit zero points [N][G] two per byte: group g -> byte g//2,
    low nibble when g is even."""
    z = np.asarray(z, dtype=np.uint8)
    n, g = z.shape
    nb = (g + 1) // 2
    out = np.zeros((n, nb), dtype=np.uint8)
    out |= z[:, 0::2]
    hi = z[:, 1::2]
    out[:, : hi.shape[1]] |= (hi << np.uint8(4)).astype(np.uint8)
    return out


def unpack_zeros(zp, g):
    """Inverse of :func:`pack_zeros`."""
    zp = np.asarray(zp, dtype=np.uint8)
    out = np.empty((zp.shape[0], g), dtype=np.int32)
    out[:, 0::2] = zp[:, : (g + 1) // 2] & 0xF
    out[:, 1::2] = zp[:, : g // 2] >> 4
    return out


def quantize(w16, group=128):
    """The full quantize-and-pack step.

    Returns ``(qweight uint32 [N][K/8], scales fp16 [N][G], zeros uint8 [N][ceil(G/2)])``.
    """
    q, s16, z = quantize_codes(w16, group)
    return pack_codes(q), s16, pack_zeros(z)


def dequantize(qweight, scales, zeros, k, group=128, out_dtype="f16"):
    """w_hat = round16((q - z) * s16), returned as fp32 holding 16-bit values.

    (q - z) * s16 is exact in fp32 (a 5-bit integer times an 11-bit
    significand), so this is a single rounding into the activation dtype
    ``out_dtype`` ("f16" or "bf16").
    """
    q = unpack_codes(qweight, k)
    g = k // group
    z = unpack_zeros(zeros, g)
    s = np.repeat(np.asarray(scales, np.float16).astype(np.float32), group, axis=1)
    zz = np.repeat(z, group, axis=1)
    prod = (q - zz).astype(np.float32) * s
    return round_to(prod, out_dtype)


def packed_bytes(n, k, group=128):
    """HBM bytes of one packed layer: codes + fp16 scales + 4-bit zeros."""
    g = k // group
    return n * k // 2 + n * g * 2 + n * ((g + 1) // 2)


# ------------------------------------------------------------------ act-order
#
# Act-order (GPTQ's desc_act): the input channels are quantized in an order
# set by activation importance, so the groups of 128 run along that order,
# not along k; inference then has to reorder ([P1] section 3.2; [P4]
# section 3.2; [P5] section 3.4 on the slower inference).  Reading taken:
# the order is a permutation ``perm`` of 0..K-1 given by the caller
# (choosing it needs calibration data, which is out of scope); position j of
# the quantization order is input channel perm[j]; the group of channel c is
# g_idx[c] = (position of c in perm) // group.

def g_idx(perm, group=128):
    """Group of every original input channel: g_idx[perm[j]] = j // group."""
    perm = np.asarray(perm, dtype=np.int64)
    g = np.empty(perm.size, dtype=np.int64)
    g[perm] = np.arange(perm.size) // group
    return g


def dequantize_act_order(w16, perm, group=128, out_dtype="f16"):
    """The act-order dequantized weight in the ORIGINAL channel order.

    The group statistics are taken over the channels each group holds
    (those c with g_idx[c] == g), then every weight is encoded with its own
    group's scale and zero point and dequantized:
    w_hat[n][c] = round16((q[n][c] - z[n][g_idx[c]]) * s16[n][g_idx[c]]).
    """
    w = f32(w16)
    n, k = w.shape
    gi = g_idx(perm, group)
    G = k // group
    out = np.empty((n, k), dtype=np.float32)
    for g in range(G):
        cols = np.nonzero(gi == g)[0]
        s16, z = group_params(np.asarray(w16)[:, cols], group=cols.size)
        s = s16.astype(np.float32)                    # [n][1]
        q = np.clip(rne(w[:, cols] / s) + z, 0, QMAX)
        out[:, cols] = round_to((q - z).astype(np.float32) * s, out_dtype)
    return out


def quantize_act_order(w16, perm, group=128):
    """Act-order storage: the weight with its columns in quantization order,
    W[:, perm], quantized with contiguous groups -- ``(qweight, scales,
    zeros)`` exactly as :func:`quantize` packs them.  Dequantizing it and
    scattering the columns back (column j to channel perm[j]) gives
    :func:`dequantize_act_order`; x[:, perm] times it gives the same y."""
    return quantize(np.asarray(w16)[:, np.asarray(perm)], group)
