"""LLM.int8() vector-wise INT8 with mixed-precision outlier decomposition (oracle).

What the pages fix:
  * Vector-wise quantization: one scale per output feature of the weight
    matrix ([P1] section 2.1, first layer of the design).
  * Symmetric INT8: scale = max|w| / 127, codes in [-127, 127] ([P5]
    section 2.3); worked example: a maximum of 80 gives 80/127 ~ 0.63
    ([P1] section 1).
  * Mixed-precision decomposition: feature dimensions whose activations
    exceed 6.0 in absolute value are outliers; the outlier sub-matrices of
    the activations and the weights are multiplied in FP16, the rest in INT8,
    and the two results are summed ([P1] section 2.1, second layer;
    ``llm_int8_threshold=6.0`` in [P5] section 6.1).
  * Outliers must stay in FP16; they cannot be dropped or crudely quantized
    ([P1] section 2.1).

Readings taken where the pages are silent:
  * W is [N][K]; "one scale per output feature" is one fp32 scale per row n:
    sw[n] = fp32(max_k |W[n,k]|) / 127 (fp32 division; 1.0 for an all-zero
    row); qw = clamp(round_half_even(w / sw), -127, 127).
  * A column k is an outlier when |x[m,k]| > threshold for at least one row
    m (strict ">": "exceeds").  The outlier set is reported as the ascending
    list of such k.
  * Activations are quantized per token (row of x) over the non-outlier
    columns ([P5] section 2.2 names per-token granularity for activations):
    sx[m] = max_{k not outlier} |x[m,k]| / 127 (1.0 when that is 0);
    qx = clamp(round_half_even(x / sx), -127, 127), and 0 in outlier columns.
  * The FP16 part multiplies the outlier activations by the int8 weights
    dequantized to fp16, w16 = round_f16(fp32(qw) * sw) (``has_fp16_weight``
    false: no fp16 copy of W is kept, [P5] section 6.1).
  * y = acc * sx[m] * sw[n] + x[:, O] . w16[:, O]^T, with acc the exact int32
    product of the int8 codes; the reference evaluates y in fp64.
"""

import numpy as np

from .numerics import f32, rne, round_f16, round_to

QMAX = 127


def quantize_rows(w16):
    """Row-wise symmetric int8: returns ``(qw int8 [N][K], sw fp32 [N])``."""
    w = f32(w16)
    sw = np.abs(w).max(axis=1) / np.float32(QMAX)     # fp32 IEEE division
    sw = np.where(sw == 0, np.float32(1), sw).astype(np.float32)
    qw = np.clip(rne(w / sw[:, None]), -QMAX, QMAX).astype(np.int8)
    return qw, sw


def symmetric_scale(max_abs):
    """The symmetric INT8 scale of a tensor whose largest magnitude is ``max_abs``."""
    return np.float32(max_abs) / np.float32(QMAX)


def outlier_columns(x16, threshold=6.0):
    """Ascending int32 list of columns k with any |x[m,k]| > threshold."""
    x = f32(x16)
    flag = (np.abs(x) > np.float32(threshold)).any(axis=0)
    return np.nonzero(flag)[0].astype(np.int32)


def quantize_activations(x16, outliers):
    """Per-token int8 over the non-outlier columns.

    Returns ``(qx int8 [M][K] with zeros in outlier columns, sx fp32 [M])``.
    """
    x = f32(x16)
    keep = np.ones(x.shape[1], dtype=bool)
    keep[np.asarray(outliers, dtype=np.int64)] = False
    ax = np.where(keep[None, :], np.abs(x), np.float32(0))
    sx = ax.max(axis=1) / np.float32(QMAX)            # fp32 IEEE division
    sx = np.where(sx == 0, np.float32(1), sx).astype(np.float32)
    qx = np.clip(rne(x / sx[:, None]), -QMAX, QMAX)
    qx = np.where(keep[None, :], qx, 0).astype(np.int8)
    return qx, sx


def int_matmul(qx, qw):
    """acc[m,n] = sum_k qx[m,k] * qw[n,k], exact.

    Every partial sum is an integer of magnitude <= 127*127*K < 2^53, so fp64
    BLAS evaluates it exactly whatever its summation order.
    """
    acc = np.asarray(qx, np.float64) @ np.asarray(qw, np.float64).T
    if np.abs(acc).max(initial=0) >= 2 ** 31:
        raise OverflowError("int32 accumulator overflow")
    return acc.astype(np.int32)


def dequant_weight_f16(qw, sw):
    """w16 = round_f16(fp32(qw) * sw): the fp16 weights used for outliers."""
    prod = np.asarray(qw, np.int8).astype(np.float32) * np.asarray(sw, np.float32)[:, None]
    return round_f16(prod).astype(np.float32)


def linear(x16, qw, sw, threshold=6.0):
    """The decomposed product in fp64.

    Returns ``(y fp64 [M][N], outliers, qx, sx, acc)``.
    """
    outl = outlier_columns(x16, threshold)
    qx, sx = quantize_activations(x16, outl)
    acc = int_matmul(qx, qw)
    y = acc.astype(np.float64) * sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]
    if outl.size:
        xo = f32(x16)[:, outl].astype(np.float64)
        wo = dequant_weight_f16(qw[:, outl], sw).astype(np.float64)
        y = y + xo @ wo.T
    return y, outl, qx, sx, acc


# --------------------------------------------------------- SmoothQuant W8A8
#
# W8A8 with smoothing ([P1] section 5): Wx = (W diag(s)^-1)(diag(s) x) holds
# exactly, so part of the activations' range is moved into the weights;
# alpha (about 0.5) sets how much; the scaling is folded into the weights
# offline, which are then stored as INT8 and multiplied by INT8 activations
# (the decomposition above with no outlier columns, threshold = +inf).
# Reading taken (the pages print no formula for s): per input channel c,
# s_c = max|X_c|^alpha / max|W_c|^(1 - alpha) from calibration maxima
# (given by the caller; here synthetic), activations divided by s and weight
# columns multiplied by s, each product in fp32 and rounded once to the
# 16-bit type.

def smooth_factors(x_absmax, w_absmax, alpha=0.5):
    """s_c = max|X_c|^alpha / max|W_c|^(1 - alpha) in fp64, returned as fp32
    (channels with a zero maximum get s = 1)."""
    ax = np.asarray(x_absmax, np.float64)
    aw = np.asarray(w_absmax, np.float64)
    s = np.where((ax > 0) & (aw > 0), ax ** alpha / np.where(aw > 0, aw, 1.0) ** (1.0 - alpha), 1.0)
    return s.astype(np.float32)


def scale_columns(a16, scale, out_dtype="f16"):
    """round16(a[r][c] * scale[c]): fp32 product, one rounding."""
    prod = f32(a16) * np.asarray(scale, np.float32)[None, :]
    return round_to(prod, out_dtype)
