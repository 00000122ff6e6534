"""The no-allocation LLM.int8 entry point against the workspace one.

wq_linear_int8_decomp_noalloc runs the same kernels as wq_linear_int8_decomp
with the library's own per-GPU scratch array instead of a caller workspace.
Two calls in a row, the second on a smaller input (so the scratch still
holds the first call's larger contents), each compared with the workspace
entry point on the same inputs: outlier count and int32 accumulators bit for
bit, outputs bit for bit (same kernels, same summation order), and the
accumulators against the oracle."""

import numpy as np
import pytest
import torch

import bit_quantized_linear_int4_amd as wq
import workloads
from gpu_util import dev_f16, say, torch_dtype
from oracle import llm_int8

pytestmark = pytest.mark.gpu


def _outputs(x, qw, thr, ydt, noalloc):
    m, n = x.shape[0], qw.n
    y = torch.full((m, n), float("nan"), dtype=torch_dtype(ydt), device="cuda")
    acc = torch.full((m, n), -1, dtype=torch.int32, device="cuda")
    cnt = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    if noalloc:
        wq.wq_linear_int8_decomp_noalloc(x, qw, thr, y, cnt, acc)
    else:
        ws = torch.empty((wq.wq_linear_int8_decomp_workspace(m, qw.k),), dtype=torch.uint8,
                         device="cuda")
        wq.wq_linear_int8_decomp(x, qw, thr, y, ws, cnt, acc)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), acc.cpu().numpy(), int(cnt.item())


@pytest.mark.parametrize("ydt", ["f16", "f32"])
def test_noalloc_equals_workspace_call_twice(ydt):
    for m, n, k, n_out in ((256, 2048, 8192, 8), (37, 300, 1024, 3)):
        say(f"int8_decomp_noalloc m={m} n={n} k={k} outliers={n_out} y={ydt}")
        x_np, chans = workloads.activations(m, k, 950 + m, 0, outliers=(n_out, 20.0, 100.0))
        w_np = workloads.weights(n, k, 950 + m, 1)
        qw = wq.alloc_int8(n, k)
        wq.wq_quantize_groupwise(dev_f16(w_np), 8, k, 1, qw.codes, qw.scales)
        x = dev_f16(x_np)
        y_na, acc_na, cnt_na = _outputs(x, qw, 6.0, ydt, True)
        y_ws, acc_ws, cnt_ws = _outputs(x, qw, 6.0, ydt, False)
        assert cnt_na == cnt_ws == n_out
        assert np.array_equal(acc_na, acc_ws)
        assert np.array_equal(y_na, y_ws)
        q_ref, s_ref = llm_int8.quantize_rows(w_np)
        _, outl, _, _, acc_ref = llm_int8.linear(x_np, q_ref, s_ref, 6.0)
        assert np.array_equal(outl, chans)
        assert np.array_equal(acc_na, acc_ref)
