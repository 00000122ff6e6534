"""Seeded synthetic inputs for the quantized-linear workloads.

This module only draws random numbers and casts them to 16-bit storage
types; it holds none of the quantization arithmetic.  Both the CPU oracle
(through the tests) and the HIP library (through the tests and the bench)
consume what it returns, as NumPy arrays:

  * fp16 tensors as ``np.float16``;
  * bf16 tensors as ``np.uint16`` bit patterns (NumPy has no bf16), produced
    by torch's round-to-nearest-even fp32 -> bf16 cast.

Every tensor is drawn from its own PCG64 stream,
``np.random.default_rng([seed, tensor_id])``, in fp32, then cast.

Workload shapes (the pages give no trained weights and no datasets; these
synthetic layers stand in for the 7B / 8B / 70B layers they discuss):

  decode_m1     W fp16 [4096 x 4096] ~ N(0, 0.02); x fp16 [1 x 4096] ~ N(0, 1);
                seed 0.
  mlp_decode    M = 16 tokens; x fp16 ~ N(0, 1) with 6 fixed channels whose
                magnitudes are U[20, 80] with random signs; gate and up
                W [11008 x 4096], down W [4096 x 11008], all ~ N(0, 0.02).
                The down layer's input is its own seeded [16 x 11008] tensor
                with the same outlier structure.
  prefill       M = 2048; x fp16 [2048 x 4096] ~ N(0, 1); q, k, v, o
                W [4096 x 4096] and up W [11008 x 4096], ~ N(0, 0.02).
  nf4_layer     W bf16 [14336 x 4096] ~ N(0, 0.02); x bf16 [1 x 4096] and
                [512 x 4096] ~ N(0, 1).
  int8_70b      W fp16 [28672 x 8192] ~ N(0, 0.02); x fp16 [256 x 8192]
                ~ N(0, 1) with 8 fixed outlier channels, |x| ~ U[20, 100].
  act_order_perm  a synthetic act-order over k input channels: the channels
                by decreasing seeded U[0, 1) importance (choosing the real
                order needs calibration data).
"""

import numpy as np

SEEDS = {"decode_m1": 0, "mlp_decode": 2, "prefill": 3, "nf4_layer": 4, "int8_70b": 5}


def _rng(seed, tid):
    return np.random.default_rng([int(seed), int(tid)])


def to_bf16_bits(a32):
    """fp32 -> bf16 bit patterns via torch's RNE cast (CPU)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _cast(a32, dtype):
    if dtype == "f16":
        return a32.astype(np.float16)
    if dtype == "bf16":
        return to_bf16_bits(a32)
    raise ValueError(dtype)


def weights(n, k, seed, tid, dtype="f16", std=0.02):
    """W [n x k] ~ N(0, std^2), cast to ``dtype``."""
    a = _rng(seed, tid).standard_normal((n, k), dtype=np.float32) * np.float32(std)
    return _cast(a, dtype)


def activations(m, k, seed, tid, dtype="f16", outliers=None):
    """x [m x k] ~ N(0, 1); ``outliers = (count, lo, hi)`` overwrites ``count``
    distinct channels (chosen once, shared by all rows) with magnitudes
    U[lo, hi] and an independent random sign per element.

    Returns ``(x, channels)`` where ``channels`` is the sorted int array of
    overwritten columns (empty when ``outliers`` is None).
    """
    r = _rng(seed, tid)
    a = r.standard_normal((m, k), dtype=np.float32)
    chans = np.zeros(0, dtype=np.int64)
    if outliers:
        count, lo, hi = outliers
        chans = np.sort(r.choice(k, size=count, replace=False))
        mag = r.uniform(lo, hi, size=(m, count)).astype(np.float32)
        sign = np.where(r.random((m, count)) < 0.5, -1.0, 1.0).astype(np.float32)
        a[:, chans] = mag * sign
    return _cast(a, dtype), chans


def decode_m1(n=4096, k=4096, seed=SEEDS["decode_m1"]):
    """Single W4A16 layer at M = 1."""
    x, _ = activations(1, k, seed, 0)
    return {"x": x, "w": weights(n, k, seed, 1)}


def mlp_decode(m=16, hidden=4096, inter=11008, seed=SEEDS["mlp_decode"], layers=("gate", "up", "down")):
    """7B-style MLP decode batch: list of (name, x, w) for three independent layers."""
    out = []
    x_in, _ = activations(m, hidden, seed, 0, outliers=(6, 20.0, 80.0))
    for i, name in enumerate(layers):
        if name == "down":
            xd, _ = activations(m, inter, seed, 10, outliers=(6, 20.0, 80.0))
            out.append((name, xd, weights(hidden, inter, seed, 1 + i)))
        else:
            out.append((name, x_in, weights(inter, hidden, seed, 1 + i)))
    return out


def prefill(m=2048, hidden=4096, inter=11008, seed=SEEDS["prefill"], layers=("q", "k", "v", "o", "up")):
    """7B-style prefill: list of (name, x, w); x is shared by all layers."""
    x, _ = activations(m, hidden, seed, 0)
    out = []
    for i, name in enumerate(layers):
        n = inter if name == "up" else hidden
        out.append((name, x, weights(n, hidden, seed, 1 + i)))
    return out


def nf4_layer(n=14336, k=4096, ms=(1, 512), seed=SEEDS["nf4_layer"]):
    """NF4 8B-shaped layer: bf16 weights and bf16 activations at each M."""
    w = weights(n, k, seed, 1, dtype="bf16")
    xs = {m: activations(m, k, seed, 10 + m, dtype="bf16")[0] for m in ms}
    return {"w": w, "x": xs}


def int8_70b(m=256, n=28672, k=8192, n_outliers=8, seed=SEEDS["int8_70b"]):
    """LLM.int8 layer: fp16 W, fp16 x with fixed outlier channels."""
    x, chans = activations(m, k, seed, 0, outliers=(n_outliers, 20.0, 100.0))
    return {"x": x, "w": weights(n, k, seed, 1), "outlier_channels": chans}


def act_order_perm(k, seed, tid=7):
    """A synthetic act-order: the k channels by decreasing seeded importance
    (int32 [k], a permutation)."""
    imp = _rng(seed, tid).random(k)
    return np.argsort(-imp, kind="stable").astype(np.int32)
