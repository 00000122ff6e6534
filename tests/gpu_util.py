"""Helpers for the GPU parity tests: host <-> device conversion of the
workload arrays and the float acceptance check."""

import sys

import numpy as np
import torch

TOL = 2e-3          # max|y - y_ref| / max|y_ref| for fp32 / fp16 outputs
BF16_ULP = 2.0 ** -8


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_f16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).cuda()


def dev_bf16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev(a, dtype):
    return dev_bf16(a) if dtype == "bf16" else dev_f16(a)


def host16(a, dtype):
    """Workload array -> fp32 NumPy values (exact)."""
    if dtype == "bf16":
        return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32)
    return np.asarray(a, np.float16).astype(np.float32)


def to_np(t):
    """Device tensor -> NumPy (fp32 for float tensors, raw bits otherwise)."""
    t = t.detach().cpu()
    if t.dtype in (torch.float16, torch.bfloat16, torch.float32):
        return t.float().numpy()
    if t.dtype == torch.int32:
        return t.numpy()
    return t.numpy()


def torch_dtype(name):
    return {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[name]


def check_close(y, y_ref, ydt, tol=TOL):
    """Float acceptance: max-relative error against the fp64 oracle.

    For bf16 outputs the output rounding alone can reach 2^-8 |y|, so the bound
    adds that term per element; fp32 and fp16 outputs use the plain bound.
    """
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    den = np.abs(y_ref).max()
    err = np.abs(y - y_ref)
    if ydt == "bf16":
        ok = err <= tol * den + BF16_ULP * np.abs(y_ref)
        rel = float((err - BF16_ULP * np.abs(y_ref)).max() / den)
    else:
        ok = err <= tol * den
        rel = float(err.max() / den)
    assert ok.all(), f"max-rel error {rel:.3e} exceeds {tol:.1e}"
    return rel
