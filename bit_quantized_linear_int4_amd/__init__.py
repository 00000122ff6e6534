"""Python binding of libwq, the MI355X group-wise low-bit quantized linear library.

Argument marshalling only: every function below forwards to the C entry point
of the same name in ``libwq.so`` (declared in ``include/wq.h``), passing device
pointers of torch tensors and the current HIP stream.  All computation happens
in the library's HIP kernels; there is no fallback path.  If ``libwq.so`` has
not been built, importing works but the first call raises ``WqError``.

Tensors are torch CUDA (HIP) tensors; dtypes map as float16 -> WQ_F16,
bfloat16 -> WQ_BF16, float32 -> WQ_F32.  Outputs are caller-allocated (the
``alloc_*`` helpers allocate the documented shapes).
"""

import ctypes
import os

__all__ = [
    "WqError", "QuantizedWeight", "F16", "BF16", "F32",
    "FMT_INT4_ASYM", "FMT_NF4", "FMT_INT8_SYM_ROW",
    "wq_quantize_groupwise", "wq_pack_nf4", "wq_nf4_codebook", "wq_pack_fp4", "wq_fp4_codebook",
    "wq_linear_w4a16_workspace", "wq_linear_w4a16", "wq_linear_w4a16_gate_up",
    "wq_permute_columns", "wq_scale_columns",
    "wq_int8_prepare_activations", "wq_linear_int8_decomp_workspace",
    "wq_linear_int8_decomp", "wq_linear_int8_decomp_noalloc", "wq_dequantize",
    "wq_status_string",
    "alloc_int4", "alloc_nf4", "alloc_fp4", "alloc_int8", "library_path", "FMT_FP4",
]

F16, BF16, F32 = 0, 1, 2
FMT_INT4_ASYM, FMT_NF4, FMT_INT8_SYM_ROW, FMT_FP4 = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
# WQ_LIBRARY names another build of the same library (for example one whose
# host code carries sanitizers); by default the in-tree libwq.so
_LIB_PATH = os.environ.get("WQ_LIBRARY") or os.path.join(_HERE, "libwq.so")
_lib = None


class WqError(RuntimeError):
    """A libwq call returned a non-zero wq_status (or the library is missing)."""

    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


class _Weight(ctypes.Structure):
    _fields_ = [
        ("fmt", ctypes.c_int32), ("group", ctypes.c_int32),
        ("n", ctypes.c_int64), ("k", ctypes.c_int64),
        ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
        ("zeros", ctypes.c_void_p), ("scales2", ctypes.c_void_p),
        ("group2", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("perm", ctypes.c_void_p),
    ]


def library_path():
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise WqError(-1, f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                          "or python -m bit_quantized_linear_int4_amd._build")
    lib = ctypes.CDLL(_LIB_PATH)
    c_i32, c_i64, c_vp, c_f = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    wp = ctypes.POINTER(_Weight)
    sig = {
        "wq_quantize_groupwise": (c_i32, [c_vp, c_i32, c_i64, c_i64, c_i32, c_i32, c_i32,
                                          c_vp, c_vp, c_vp, c_vp]),
        "wq_pack_nf4": (c_i32, [c_vp, c_i32, c_i64, c_i64, c_i32, c_i32, c_i32,
                                c_vp, c_vp, c_vp, c_vp]),
        "wq_nf4_codebook": (c_i32, [ctypes.POINTER(ctypes.c_float)]),
        "wq_pack_fp4": (c_i32, [c_vp, c_i32, c_i64, c_i64, c_i32, c_i32, c_i32,
                                c_vp, c_vp, c_vp, c_vp]),
        "wq_fp4_codebook": (c_i32, [ctypes.POINTER(ctypes.c_float)]),
        "wq_linear_w4a16_workspace": (ctypes.c_size_t, [c_i64, wp]),
        "wq_linear_w4a16": (c_i32, [c_vp, c_i32, c_i64, wp, c_vp, c_i32, c_vp,
                                    ctypes.c_size_t, c_vp]),
        "wq_linear_w4a16_gate_up": (c_i32, [c_vp, c_i32, c_i64, wp, wp, c_i32, c_vp, c_vp,
                                            c_i32, c_vp]),
        "wq_int8_prepare_activations": (c_i32, [c_vp, c_i64, c_i64, c_f, c_vp, c_vp, c_vp,
                                                c_vp, c_vp, c_vp]),
        "wq_linear_int8_decomp_workspace": (ctypes.c_size_t, [c_i64, c_i64]),
        "wq_linear_int8_decomp": (c_i32, [c_vp, c_i64, wp, c_f, c_vp, c_i32, c_vp,
                                          ctypes.c_size_t, c_vp, c_vp, c_vp]),
        "wq_linear_int8_decomp_noalloc": (c_i32, [c_vp, c_i64, wp, c_f, c_vp, c_i32, c_vp, c_vp,
                                                  c_vp]),
        "wq_dequantize": (c_i32, [wp, c_vp, c_i32, c_vp]),
        "wq_permute_columns": (c_i32, [c_vp, c_i32, c_i64, c_i64, c_vp, c_vp, c_vp]),
        "wq_scale_columns": (c_i32, [c_vp, c_i32, c_i64, c_i64, c_vp, c_vp, c_vp]),
        "wq_status_string": (ctypes.c_char_p, [c_i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def wq_status_string(status):
    return _load().wq_status_string(int(status)).decode()


def _check(status, what):
    if status != 0:
        raise WqError(status, f"{what}: {wq_status_string(status)}")


def _dt(t):
    import torch
    m = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}
    if t.dtype not in m:
        raise WqError(4, f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, t):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


# ------------------------------------------------------------ validation
# Sizes and layouts are checked here, before the C call: the C layer sees
# only pointers and the sizes passed to it, so a tensor smaller than the
# sizes say would be read or written out of bounds on the device.  Shape and
# layout mismatches raise WqError(WQ_ERR_SHAPE); tensors that are not GPU
# tensors raise WqError(WQ_ERR_UNSUPPORTED).
_ERR_SHAPE, _ERR_UNSUP = 2, 4


def _fail(what, msg, status=_ERR_SHAPE):
    raise WqError(status, f"{what}: {msg}")


def _nbytes(t):
    return t.numel() * t.element_size()


def _dense(what, name, t, nbytes=None, shape=None):
    """`t` is contiguous, with `shape` (if given) and exactly `nbytes` bytes
    (if given)."""
    if t is None:
        _fail(what, f"{name} is required")
    if shape is not None and tuple(t.shape) != tuple(shape):
        _fail(what, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        _fail(what, f"{name} is not contiguous")
    if nbytes is not None and _nbytes(t) != nbytes:
        _fail(what, f"{name} holds {_nbytes(t)} bytes, expected {nbytes}")


def _on_gpu(what, *ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            _fail(what, "tensors must be GPU tensors", _ERR_UNSUP)
        if dev is None:
            dev = t.device
        elif t.device != dev:
            _fail(what, "tensors are on different devices", _ERR_UNSUP)


def _matrix(what, name, t):
    if t is None or t.dim() != 2:
        _fail(what, f"{name} must be a 2-D [rows][k] tensor")
    _dense(what, name, t)
    return int(t.shape[0]), int(t.shape[1])


def _weight_tensors(what, w):
    """The tensors of a QuantizedWeight against the sizes its descriptor
    states (layouts as in wq_weight)."""
    n, k, g = w.n, w.k, w.group
    if n < 1 or k < 1 or g < 1 or k % 8:
        _fail(what, f"weight sizes n={n} k={k} group={g} are invalid")
    if w.fmt == FMT_INT4_ASYM:
        if k % g:
            _fail(what, f"k={k} is not a multiple of the group {g}")
        ng = k // g
        _dense(what, "codes", w.codes, n * k // 2)
        _dense(what, "scales", w.scales, 2 * n * ng)
        _dense(what, "zeros", w.zeros, n * ((ng + 1) // 2))
        if w.perm is not None:
            _dense(what, "perm", w.perm, 4 * k)
    elif w.fmt in (FMT_NF4, FMT_FP4):
        if (n * k) % g:
            _fail(what, f"n*k={n * k} is not a multiple of the block {g}")
        nb = n * k // g
        _dense(what, "codes", w.codes, n * k // 2)
        if w.scales2 is not None:
            if w.group2 < 1:
                _fail(what, f"group2={w.group2} is invalid")
            _dense(what, "absmax", w.scales, nb)
            _dense(what, "absmax_scale", w.scales2, 4 * (-(-nb // w.group2)))
        else:
            _dense(what, "absmax", w.scales, 4 * nb)
        if w.perm is not None:
            _dense(what, "perm", w.perm, 4 * k)
    elif w.fmt == FMT_INT8_SYM_ROW:
        _dense(what, "codes", w.codes, n * k)
        _dense(what, "scales", w.scales, 4 * n)
    else:
        _fail(what, f"unknown weight format {w.fmt}", _ERR_UNSUP)
    return [w.codes, w.scales, w.zeros, w.scales2, w.perm]


class QuantizedWeight:
    """Device tensors of one quantized weight plus its wq_weight descriptor."""

    def __init__(self, fmt, n, k, group, codes, scales, zeros=None, scales2=None, group2=0,
                 perm=None):
        self.fmt, self.n, self.k, self.group = fmt, int(n), int(k), int(group)
        self.codes, self.scales, self.zeros, self.scales2 = codes, scales, zeros, scales2
        self.group2 = int(group2)
        self.perm = perm          # INT4 act-order: device int32 [k], or None

    def descriptor(self):
        d = _Weight()
        d.fmt, d.group, d.n, d.k = self.fmt, self.group, self.n, self.k
        d.codes = self.codes.data_ptr()
        d.scales = self.scales.data_ptr()
        d.zeros = self.zeros.data_ptr() if self.zeros is not None else None
        d.scales2 = self.scales2.data_ptr() if self.scales2 is not None else None
        d.group2 = self.group2
        d.reserved = 0
        d.perm = self.perm.data_ptr() if self.perm is not None else None
        return d

    def nbytes(self):
        return sum(t.numel() * t.element_size()
                   for t in (self.codes, self.scales, self.zeros, self.scales2) if t is not None)

    def clone(self):
        c = lambda t: None if t is None else t.clone()
        return QuantizedWeight(self.fmt, self.n, self.k, self.group, c(self.codes),
                               c(self.scales), c(self.zeros), c(self.scales2), self.group2,
                               c(self.perm))


def alloc_int4(n, k, group=128, device="cuda"):
    import torch
    g = k // group
    return QuantizedWeight(
        FMT_INT4_ASYM, n, k, group,
        torch.empty((n, k // 8), dtype=torch.int32, device=device),
        torch.empty((n, g), dtype=torch.float16, device=device),
        torch.empty((n, (g + 1) // 2), dtype=torch.uint8, device=device))


def alloc_nf4(n, k, block=64, double_quant=True, block2=256, device="cuda", fmt=FMT_NF4):
    import torch
    nb = n * k // block
    codes = torch.empty((n * k // 2,), dtype=torch.uint8, device=device)
    if double_quant:
        return QuantizedWeight(fmt, n, k, block, codes,
                               torch.empty((nb,), dtype=torch.int8, device=device),
                               None, torch.empty(((nb + block2 - 1) // block2,),
                                                 dtype=torch.float32, device=device), block2)
    return QuantizedWeight(fmt, n, k, block, codes,
                           torch.empty((nb,), dtype=torch.float32, device=device))


def alloc_fp4(n, k, block=64, double_quant=True, block2=256, device="cuda"):
    return alloc_nf4(n, k, block, double_quant, block2, device, fmt=FMT_FP4)


def alloc_int8(n, k, device="cuda"):
    import torch
    return QuantizedWeight(FMT_INT8_SYM_ROW, n, k, k,
                           torch.empty((n, k), dtype=torch.int8, device=device),
                           torch.empty((n,), dtype=torch.float32, device=device))


def wq_quantize_groupwise(w, bits, group, symmetric, codes, scales, zeros=None, stream=None):
    what = "wq_quantize_groupwise"
    n, k = _matrix(what, "w", w)
    if bits == 4:
        if group < 1 or k % group:
            _fail(what, f"k={k} is not a multiple of the group {group}")
        ng = k // group
        _dense(what, "codes", codes, n * k // 2)
        _dense(what, "scales", scales, 2 * n * ng)
        _dense(what, "zeros", zeros, n * ((ng + 1) // 2))
    elif bits == 8:
        _dense(what, "codes", codes, n * k)
        _dense(what, "scales", scales, 4 * n)
        if zeros is not None:
            _fail(what, "zeros must be None for 8-bit symmetric codes", _ERR_UNSUP)
    else:
        _fail(what, f"bits={bits} group={group} do not fit k={k}", _ERR_UNSUP)
    _on_gpu(what, w, codes, scales, zeros)
    st = _load().wq_quantize_groupwise(_ptr(w), _dt(w), n, k, bits, group, symmetric,
                                       _ptr(codes), _ptr(scales), _ptr(zeros), _stream(stream, w))
    _check(st, "wq_quantize_groupwise")


def _check_pack(what, w, block, double_quant, block2, codes, absmax, absmax_scale):
    n, k = _matrix(what, "w", w)
    if block < 1 or (n * k) % block or (double_quant and block2 < 1):
        _fail(what, f"block={block} block2={block2} do not fit n*k={n * k}")
    nb = n * k // block
    _dense(what, "codes", codes, n * k // 2)
    if double_quant:
        _dense(what, "absmax", absmax, nb)
        _dense(what, "absmax_scale", absmax_scale, 4 * (-(-nb // block2)))
    else:
        _dense(what, "absmax", absmax, 4 * nb)
        if absmax_scale is not None:
            _fail(what, "absmax_scale must be None without double quantization", _ERR_UNSUP)
    _on_gpu(what, w, codes, absmax, absmax_scale)
    return n, k


def wq_pack_nf4(w, block, double_quant, block2, codes, absmax, absmax_scale=None, stream=None):
    n, k = _check_pack("wq_pack_nf4", w, block, double_quant, block2, codes, absmax,
                       absmax_scale)
    st = _load().wq_pack_nf4(_ptr(w), _dt(w), n, k, block, 1 if double_quant else 0, block2,
                             _ptr(codes), _ptr(absmax), _ptr(absmax_scale), _stream(stream, w))
    _check(st, "wq_pack_nf4")


def wq_pack_fp4(w, block, double_quant, block2, codes, absmax, absmax_scale=None, stream=None):
    n, k = _check_pack("wq_pack_fp4", w, block, double_quant, block2, codes, absmax,
                       absmax_scale)
    st = _load().wq_pack_fp4(_ptr(w), _dt(w), n, k, block, 1 if double_quant else 0, block2,
                             _ptr(codes), _ptr(absmax), _ptr(absmax_scale), _stream(stream, w))
    _check(st, "wq_pack_fp4")


def wq_fp4_codebook():
    out = (ctypes.c_float * 16)()
    _check(_load().wq_fp4_codebook(out), "wq_fp4_codebook")
    return [float(v) for v in out]


def wq_nf4_codebook():
    out = (ctypes.c_float * 16)()
    _check(_load().wq_nf4_codebook(out), "wq_nf4_codebook")
    return [float(v) for v in out]


def wq_linear_w4a16_workspace(m, weight):
    d = weight.descriptor()
    return int(_load().wq_linear_w4a16_workspace(int(m), ctypes.byref(d)))


def _check_linear(what, x, weight, ys):
    m, k = _matrix(what, "x", x)
    if k != weight.k:
        _fail(what, f"x has k={k}, the weight k={weight.k}")
    wt = _weight_tensors(what, weight)
    for name, y in ys:
        _dense(what, name, y, shape=(m, weight.n))
    return m, [x] + wt + [y for _, y in ys]


def wq_linear_w4a16(x, weight, y, workspace=None, stream=None):
    what = "wq_linear_w4a16"
    _, ts = _check_linear(what, x, weight, [("y", y)])
    if workspace is not None:
        _dense(what, "workspace", workspace)
    _on_gpu(what, workspace, *ts)
    d = weight.descriptor()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _load().wq_linear_w4a16(_ptr(x), _dt(x), x.shape[0], ctypes.byref(d), _ptr(y), _dt(y),
                                 _ptr(workspace), ws_bytes, _stream(stream, x))
    _check(st, "wq_linear_w4a16")


def wq_linear_w4a16_gate_up(x, w_gate, w_up, y_gate, y_up=None, act=0, stream=None):
    what = "wq_linear_w4a16_gate_up"
    # y_up receives the up projection for act 0, and for act 1 once m > 16
    # (the two-GEMM path keeps it there before the SiLU product)
    up_out = act == 0 or x.shape[0] > 16
    _, tg = _check_linear(what, x, w_gate,
                          [("y_gate", y_gate)] + ([("y_up", y_up)] if up_out else []))
    _, tu = _check_linear(what, x, w_up, [])
    _on_gpu(what, *tg, *tu)
    dg, du = w_gate.descriptor(), w_up.descriptor()
    st = _load().wq_linear_w4a16_gate_up(_ptr(x), _dt(x), x.shape[0], ctypes.byref(dg),
                                         ctypes.byref(du), int(act), _ptr(y_gate), _ptr(y_up),
                                         _dt(y_gate), _stream(stream, x))
    _check(st, "wq_linear_w4a16_gate_up")


def wq_int8_prepare_activations(x, threshold, mask, idx, count, qx, sx, stream=None):
    what = "wq_int8_prepare_activations"
    m, k = _matrix(what, "x", x)
    _dense(what, "mask", mask, k)
    _dense(what, "idx", idx, 4 * k)
    _dense(what, "count", count, 4)
    _dense(what, "qx", qx, m * k)
    _dense(what, "sx", sx, 4 * m)
    _on_gpu(what, x, mask, idx, count, qx, sx)
    st = _load().wq_int8_prepare_activations(_ptr(x), m, k, float(threshold), _ptr(mask),
                                             _ptr(idx), _ptr(count), _ptr(qx), _ptr(sx),
                                             _stream(stream, x))
    _check(st, "wq_int8_prepare_activations")


def wq_linear_int8_decomp_workspace(m, k):
    return int(_load().wq_linear_int8_decomp_workspace(int(m), int(k)))


def wq_linear_int8_decomp(x, weight, threshold, y, workspace, outlier_count=None, acc_out=None,
                          stream=None):
    what = "wq_linear_int8_decomp"
    m, ts = _check_linear(what, x, weight, [("y", y)])
    _dense(what, "workspace", workspace)
    if outlier_count is not None:
        _dense(what, "outlier_count", outlier_count, 4)
    if acc_out is not None:
        _dense(what, "acc_out", acc_out, 4 * m * weight.n)
    _on_gpu(what, workspace, outlier_count, acc_out, *ts)
    d = weight.descriptor()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _load().wq_linear_int8_decomp(_ptr(x), x.shape[0], ctypes.byref(d), float(threshold),
                                       _ptr(y), _dt(y), _ptr(workspace), ws_bytes,
                                       _ptr(outlier_count), _ptr(acc_out), _stream(stream, x))
    _check(st, "wq_linear_int8_decomp")


def wq_linear_int8_decomp_noalloc(x, weight, threshold, y, outlier_count=None, acc_out=None,
                                  stream=None):
    what = "wq_linear_int8_decomp_noalloc"
    m, ts = _check_linear(what, x, weight, [("y", y)])
    if outlier_count is not None:
        _dense(what, "outlier_count", outlier_count, 4)
    if acc_out is not None:
        _dense(what, "acc_out", acc_out, 4 * m * weight.n)
    _on_gpu(what, outlier_count, acc_out, *ts)
    d = weight.descriptor()
    st = _load().wq_linear_int8_decomp_noalloc(_ptr(x), m, ctypes.byref(d), float(threshold),
                                               _ptr(y), _dt(y), _ptr(outlier_count),
                                               _ptr(acc_out), _stream(stream, x))
    _check(st, what)


def wq_permute_columns(src, perm, dst, stream=None):
    what = "wq_permute_columns"
    rows, k = _matrix(what, "src", src)
    _dense(what, "perm", perm, 4 * k)
    _dense(what, "dst", dst, _nbytes(src), shape=(rows, k))
    _on_gpu(what, src, perm, dst)
    st = _load().wq_permute_columns(_ptr(src), _dt(src), rows, k, _ptr(perm), _ptr(dst),
                                    _stream(stream, src))
    _check(st, "wq_permute_columns")


def wq_scale_columns(src, scale, dst, stream=None):
    what = "wq_scale_columns"
    rows, k = _matrix(what, "src", src)
    _dense(what, "scale", scale, 4 * k)
    _dense(what, "dst", dst, _nbytes(src), shape=(rows, k))
    _on_gpu(what, src, scale, dst)
    st = _load().wq_scale_columns(_ptr(src), _dt(src), rows, k, _ptr(scale), _ptr(dst),
                                  _stream(stream, src))
    _check(st, "wq_scale_columns")


def wq_dequantize(weight, out, stream=None):
    what = "wq_dequantize"
    wt = _weight_tensors(what, weight)
    _dense(what, "out", out, shape=(weight.n, weight.k))
    _on_gpu(what, out, *wt)
    d = weight.descriptor()
    st = _load().wq_dequantize(ctypes.byref(d), _ptr(out), _dt(out), _stream(stream, out))
    _check(st, "wq_dequantize")
