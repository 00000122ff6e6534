"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, reports its codebook, and rejects bad arguments before any
HIP call (the header promises that an error other than WQ_ERR_HIP enqueued
nothing, so these calls never reach the device)."""

import ctypes
import os
import re

import numpy as np
import pytest

import bit_quantized_linear_int4_amd as wq
from oracle import fp4, nf4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(wq.library_path()),
                                reason="libwq.so not built")

OK, NULL, SHAPE, ALIGN, UNSUP, WS = 0, 1, 2, 3, 4, 5


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wq_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_documented_surface():
    names = declared_functions()
    for required in ("wq_quantize_groupwise", "wq_pack_nf4", "wq_linear_w4a16",
                     "wq_linear_int8_decomp"):
        assert required in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(wq.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for s in range(7):
        assert wq.wq_status_string(s).startswith("WQ_")
    assert "unknown" in wq.wq_status_string(99)


def test_library_codebook_matches_oracle():
    """The library derives the NF4 levels with its own quantile routine;
    they must equal the oracle's in fp32."""
    lib_levels = np.array(wq.wq_nf4_codebook(), dtype=np.float32)
    assert np.array_equal(lib_levels, nf4.codebook())


def test_library_fp4_codebook_matches_oracle():
    """The library's FP4 table (E2M1 values / 6, by code) equals the
    oracle's in fp32, including the sign of code 8's zero."""
    lib_levels = np.array(wq.wq_fp4_codebook(), dtype=np.float32)
    ref = fp4.codebook()
    assert np.array_equal(lib_levels, ref)
    assert np.array_equal(np.signbit(lib_levels), np.signbit(ref))


# fake device addresses: never dereferenced, because validation fails first
A16 = 0x10000
ODD = 0x10001


def _lib():
    return wq._load()


def test_quantize_argument_errors():
    q = _lib().wq_quantize_groupwise
    args = dict(w=A16, wdt=wq.F16, n=4, k=256, bits=4, group=128, sym=0,
                codes=A16, scales=A16, zeros=A16)

    def call(**kw):
        a = dict(args, **kw)
        return q(a["w"], a["wdt"], a["n"], a["k"], a["bits"], a["group"], a["sym"],
                 a["codes"], a["scales"], a["zeros"], None)

    assert call(w=None) == NULL
    assert call(zeros=None) == NULL
    assert call(k=100) == SHAPE
    assert call(k=192) == SHAPE            # not a multiple of the group
    assert call(n=0) == SHAPE
    assert call(n=-3) == SHAPE
    assert call(w=ODD) == ALIGN
    assert call(codes=A16 + 4) == ALIGN
    assert call(group=96) == UNSUP
    assert call(bits=3) == UNSUP
    assert call(wdt=wq.F32) == UNSUP
    assert call(bits=8, sym=1, group=256, zeros=None, scales=A16 + 2) == ALIGN
    assert call(bits=8, sym=1, group=128, zeros=None) == UNSUP
    assert call(bits=8, sym=1, group=256) == UNSUP  # zeros must be NULL


@pytest.mark.parametrize("entry", ["wq_pack_nf4", "wq_pack_fp4"])
def test_pack_nf4_argument_errors(entry):
    p = getattr(_lib(), entry)

    def call(w=A16, wdt=wq.BF16, n=4, k=256, block=64, dq=1, block2=256, codes=A16,
             absmax=A16, scale2=A16):
        return p(w, wdt, n, k, block, dq, block2, codes, absmax, scale2, None)

    assert call(codes=None) == NULL
    assert call(scale2=None) == NULL
    assert call(block=32) == UNSUP
    assert call(block2=128) == UNSUP
    assert call(dq=0) == UNSUP              # second-level scale given without double quant
    assert call(n=1, k=40) == SHAPE
    assert call(w=ODD) == ALIGN


def _weight(fmt=wq.FMT_INT4_ASYM, n=64, k=256, group=128, codes=A16, scales=A16, zeros=A16,
            scales2=None, group2=0, perm=None):
    d = wq._Weight()
    d.fmt, d.group, d.n, d.k = fmt, group, n, k
    d.codes, d.scales, d.zeros, d.scales2 = codes, scales, zeros, scales2
    d.perm = perm
    d.group2 = group2
    return d


def test_act_order_argument_errors():
    f = _lib().wq_linear_w4a16
    ws_q = _lib().wq_linear_w4a16_workspace

    def call(w, ws=None, wsb=0):
        return f(A16, wq.F16, 16, ctypes.byref(w), A16, wq.F32, ws, wsb, None)

    ao = _weight(n=64, k=256, perm=A16)
    # the gathered activations: 16 x 256 x 2 bytes, rounded to 256
    assert ws_q(16, ctypes.byref(ao)) == 8192
    assert ws_q(16, ctypes.byref(_weight())) == 0
    assert call(ao) == WS                                # no workspace for the gather
    assert call(ao, A16, 4096) == WS                     # too small
    assert call(ao, A16 + 16, 8192) == ALIGN             # 256-byte workspace alignment
    assert call(_weight(perm=A16 + 2)) == ALIGN
    nf4w = _weight(fmt=wq.FMT_NF4, group=64, zeros=None, perm=A16)
    assert call(nf4w) == UNSUP                           # act-order is INT4 only
    g = _lib().wq_linear_w4a16_gate_up
    assert g(A16, wq.F16, 1, ctypes.byref(ao), ctypes.byref(_weight()), 0, A16, A16, wq.F32,
             None) == UNSUP
    p = _lib().wq_permute_columns
    assert p(None, wq.F16, 4, 64, A16, A16 + 4096, None) == NULL
    assert p(A16, wq.F16, 4, 64, None, A16 + 4096, None) == NULL
    assert p(A16, wq.F32, 4, 64, A16, A16 + 4096, None) == UNSUP
    assert p(A16, wq.F16, 4, 64, A16, A16, None) == UNSUP   # not in place
    assert p(A16, wq.F16, 4, 60, A16, A16 + 4096, None) == SHAPE
    assert p(A16, wq.F16, 0, 64, A16, A16 + 4096, None) == SHAPE
    assert p(A16, wq.F16, 4, 64, A16, A16 + 4104, None) == ALIGN
    assert p(A16, wq.F16, 4, 64, A16 + 2, A16 + 4096, None) == ALIGN


def test_scale_columns_argument_errors():
    f = _lib().wq_scale_columns
    assert f(None, wq.F16, 4, 64, A16, A16, None) == NULL
    assert f(A16, wq.F16, 4, 64, None, A16, None) == NULL
    assert f(A16, wq.F32, 4, 64, A16, A16, None) == UNSUP
    assert f(A16, wq.F16, 4, 60, A16, A16, None) == SHAPE
    assert f(A16, wq.F16, 4, 64, A16, A16 + 8, None) == ALIGN
    assert f(A16, wq.F16, 4, 64, A16 + 2, A16, None) == ALIGN


def test_gate_up_argument_errors():
    f = _lib().wq_linear_w4a16_gate_up

    def call(x=A16, xdt=wq.F16, m=1, wg=None, wu=None, act=0, yg=A16, yu=A16, ydt=wq.F32):
        wg = _weight() if wg is None else wg
        wu = _weight() if wu is None else wu
        return f(x, xdt, m, ctypes.byref(wg), ctypes.byref(wu), act, yg, yu, ydt, None)

    assert call(x=None) == NULL
    assert call(yg=None) == NULL
    assert call(yu=None) == NULL                      # act 0 writes both outputs
    assert call(wu=_weight(zeros=None)) == NULL
    assert call(act=2) == UNSUP
    assert call(act=1, m=17, yu=None) == NULL         # prefill SiLU keeps up in y_up
    assert call(act=1, m=17, yu=ODD) == ALIGN
    assert call(act=1, m=16, yu=ODD, x=ODD) == ALIGN  # decode: y_up unused, x checked
    assert call(wu=_weight(n=128)) == SHAPE           # the pair shares n and k
    assert call(wu=_weight(k=384)) == SHAPE
    assert call(wu=_weight(group=64)) == SHAPE        # and the group size
    assert call(m=0) == SHAPE
    assert call(m=1 << 23) == SHAPE
    assert call(wg=_weight(fmt=wq.FMT_NF4, group=64, zeros=None)) == UNSUP   # mixed formats
    nf4 = dict(fmt=wq.FMT_NF4, group=64, zeros=None)
    assert call(wg=_weight(**nf4, scales2=A16, group2=256),
                wu=_weight(**nf4)) == UNSUP           # double quantization on one only
    int8 = dict(fmt=wq.FMT_INT8_SYM_ROW, group=256, zeros=None)
    assert call(wg=_weight(**int8), wu=_weight(**int8)) == UNSUP
    assert call(xdt=wq.F32) == UNSUP
    assert call(x=ODD) == ALIGN
    assert call(yu=ODD, act=0) == ALIGN


def test_linear_w4a16_argument_errors():
    f = _lib().wq_linear_w4a16

    def call(x=A16, xdt=wq.F16, m=1, w=None, y=A16, ydt=wq.F32, ws=None, wsb=0):
        w = _weight() if w is None else w
        return f(x, xdt, m, ctypes.byref(w), y, ydt, ws, wsb, None)

    assert call(x=None) == NULL
    assert call(w=_weight(codes=None)) == NULL
    assert call(w=_weight(zeros=None)) == NULL
    assert call(m=0) == SHAPE
    assert call(w=_weight(k=200, group=8)) == UNSUP
    assert call(w=_weight(group=16)) == UNSUP     # groups of 128, 64 or 32
    assert call(w=_weight(k=136)) == SHAPE
    assert call(x=ODD) == ALIGN
    assert call(w=_weight(codes=A16 + 8)) == ALIGN
    assert call(xdt=wq.F32) == UNSUP
    assert call(ydt=7) == UNSUP
    assert call(w=_weight(fmt=wq.FMT_INT8_SYM_ROW, group=256)) == UNSUP
    assert call(w=_weight(fmt=wq.FMT_NF4, group=64, zeros=None, scales2=A16, group2=128)) == UNSUP
    # size limits: every dimension below 2^23, every matrix at most 2^34 elements
    assert call(m=1 << 23) == SHAPE
    assert call(w=_weight(n=1 << 23, k=128)) == SHAPE
    assert call(w=_weight(n=(1 << 21) + 16, k=8192)) == SHAPE     # n * k > 2^34
    assert call(m=(1 << 21) + 1, w=_weight(n=4096, k=8192)) == SHAPE   # m * k > 2^34
    assert _lib().wq_linear_w4a16_workspace(1 << 23, ctypes.byref(_weight())) == 0
    # no decode or GEMM schedule needs scratch: NULL workspace is accepted
    big = _weight(n=4096, k=16384)
    assert _lib().wq_linear_w4a16_workspace(16, ctypes.byref(big)) == 0


def test_workspace_queries():
    lib = _lib()
    d = _weight(n=4096, k=11008)
    assert lib.wq_linear_w4a16_workspace(0, ctypes.byref(d)) == 0
    assert lib.wq_linear_w4a16_workspace(2048, ctypes.byref(d)) == 0   # GEMM path: none
    assert lib.wq_linear_int8_decomp_workspace(256, 8192) >= 256 * 8192 + 8192 * 5
    assert lib.wq_linear_int8_decomp_workspace(0, 8192) == 0


def test_int8_argument_errors():
    f = _lib().wq_linear_int8_decomp
    w = _weight(fmt=wq.FMT_INT8_SYM_ROW, n=64, k=256, group=256, zeros=None)
    need = _lib().wq_linear_int8_decomp_workspace(4, 256)

    def call(x=A16, m=4, w=w, thr=6.0, y=A16, ydt=wq.F16, ws=A16, wsb=None):
        return f(x, m, ctypes.byref(w), thr, y, ydt, ws, need if wsb is None else wsb,
                 None, None, None)

    assert call(x=None) == NULL
    assert call(ws=None) == WS
    assert call(wsb=need - 1) == WS
    assert call(ydt=7) == UNSUP
    assert call(ydt=wq.BF16, ws=None) == WS          # bf16 output passes the type check
    assert call(thr=-1.0) == SHAPE
    assert call(thr=float("nan")) == SHAPE
    assert call(ws=A16 + 16) == ALIGN
    w2 = _weight(fmt=wq.FMT_INT8_SYM_ROW, n=64, k=200, group=200, zeros=None)
    assert call(w=w2) == SHAPE
    # the int32 accumulator holds 127 * 127 * k only up to k = 133,143: the
    # largest multiple of 128 below passes the shape check, the next fails
    big_ws = _lib().wq_linear_int8_decomp_workspace(1, 133248)
    for k, want in ((133120, WS), (133248, SHAPE)):
        wk = _weight(fmt=wq.FMT_INT8_SYM_ROW, n=64, k=k, group=k, zeros=None)
        assert f(A16, 1, ctypes.byref(wk), 6.0, A16, wq.F16, None, big_ws, None, None,
                 None) == want, k
    p = _lib().wq_int8_prepare_activations
    assert p(A16, 4, 256, 6.0, A16, A16, A16, None, A16, None) == NULL
    assert p(A16, 4, 250, 6.0, A16, A16, A16, A16, A16, None) == SHAPE
    assert p(A16, 4, 256, 6.0, A16 + 4, A16, A16, A16, A16, None) == ALIGN


def test_int8_noalloc_argument_errors():
    """The no-allocation entry point checks its arguments like the workspace
    one, and rejects sizes whose scratch exceeds the library's fixed array
    (before any HIP call)."""
    f = _lib().wq_linear_int8_decomp_noalloc
    w = _weight(fmt=wq.FMT_INT8_SYM_ROW, n=64, k=8192, group=8192, zeros=None)
    limit = 8 << 20

    def call(x=A16, m=4, thr=6.0, y=A16, ydt=wq.F16):
        return f(x, m, ctypes.byref(w), thr, y, ydt, None, None, None)

    assert call(x=None) == NULL
    assert call(ydt=7) == UNSUP
    assert call(thr=-1.0) == SHAPE
    assert call(y=ODD) == ALIGN
    # the 70B layer's 256 tokens fit; 1024 tokens of k = 8192 do not
    assert _lib().wq_linear_int8_decomp_workspace(256, 8192) <= limit
    assert _lib().wq_linear_int8_decomp_workspace(1024, 8192) > limit
    assert call(m=1024) == WS


def test_dequantize_argument_errors():
    f = _lib().wq_dequantize
    assert f(ctypes.byref(_weight()), None, wq.F16, None) == NULL
    assert f(ctypes.byref(_weight()), A16, wq.F32, None) == UNSUP
    assert f(ctypes.byref(_weight()), ODD, wq.F16, None) == ALIGN
    assert f(None, A16, wq.F16, None) == NULL
