"""The forward that keeps each row's gate and up products, and the backward
that takes them instead of recomputing them ("Triton MoE Kernels & Memory
Checkpointing", Part A section 8: the autograd contract recomputes g = v W1
and u = v W3; keeping them trades storage for that recompute).

Checked on the GPU through the C ABI:
  * forward_save_gu's y is bitwise moe_ffn_forward's y;
  * its gu rows match the fp64 oracle's gate and up products (the permuted
    oracle path with_gu) within the bf16 output tolerance, and are bitwise
    the [g | u] rows the backward's own recompute stores in its workspace;
  * the cached backward returns bitwise the gradients of the recomputing
    one, on every forward path that writes gu (the small-chunk up GEMM with
    and without the sort inside it, the 256-row engine on half and on whole
    tiles), with invalid ids, empty experts and no shared expert;
  * fp32 and the fused variant are refused with MOE_ERR_UNSUPPORTED.
"""
import ctypes

import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from gpu_util import check_close, dev, device_inputs, host_shared, make_case, oracle_threads, say

pytestmark = pytest.mark.gpu

GRADS = ("dx", "dW1", "dW3", "dW2", "dWs1", "dWs3", "dWs2", "dtopk_w")

CASES = [
    # T, D, F, E, k, shared, routing, what it exercises
    (512, 256, 512, 8, 2, False, "uniform"),    # small chunks, the sort inside the up GEMM
    (300, 128, 256, 8, 2, True, "uniform"),     # the same with a shared expert
    (3000, 64, 128, 40, 2, True, "uniform"),    # small chunks, permute launch before the up GEMM
    (2500, 128, 256, 8, 2, True, "zipf"),       # 256-row engine, half tiles
    (1111, 64, 128, 16, 4, False, "zipf"),      # empty / tiny experts
]


def _sorted_rows(inp):
    """(valid routed rows, total rows R): gu is written for sorted rows
    0 .. valid-1 and the shared rows S .. R-1."""
    w = inp["workload"]
    idx = inp["topk_idx"].reshape(-1)
    valid = int(np.count_nonzero((idx >= 0) & (idx < w.E)))
    S = w.T * w.k
    return valid, S, S + (w.T if w.shared else 0)


def _rows_written(gu, inp):
    valid, S, R = _sorted_rows(inp)
    return torch.cat([gu[:valid], gu[S:R]]) if R > S else gu[:valid]


def _run_all(inp):
    """forward, forward_save_gu, the recomputing backward (its workspace kept)
    and the cached backward on the same seeded inputs."""
    import grouped_gemm_permute_amd as gg
    w = inp["workload"]
    d = device_inputs(inp)
    dy = dev(inp, "dy", w.dtype)
    args = (d["x"], d["topk_idx"], d["topk_w"], d["W1"], d["W3"], d["W2"], d["shared"])
    y = gg.forward(*args)
    y_save, gu = gg.forward_save_gu(*args)
    lay = gg.backward_workspace_layout(w.T, w.D, w.F, w.E, w.k, w.shared, d["x"].dtype)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device="cuda")
    g_re = gg.backward(*args, dy, workspace=ws)
    g_ca = gg.backward(*args, dy, gu=gu)
    torch.cuda.synchronize()
    R = w.T * w.k + (w.T if w.shared else 0)
    gu_re = ws[lay["gu"]:lay["gu"] + R * 2 * w.F * 2].view(torch.bfloat16).view(R, 2 * w.F)
    return y, y_save, gu, gu_re, g_re, g_ca


def _assert_same_grads(g_re, g_ca, label):
    for n in GRADS:
        if g_re[n] is None:
            assert g_ca[n] is None, n
            continue
        assert torch.equal(g_re[n], g_ca[n]), f"{label}: {n} differs from the recomputing backward"


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T{}_D{}_F{}_E{}_k{}_{}_{}".format(*c))
def test_saved_gate_up_and_cached_backward(case):
    T, D, F, E, k, sh, routing = case
    inp = moe_inputs.add_output_grad(make_case(T, D, F, E, k, sh, "bf16", routing, seed=41))
    say(f"cached backward T{T} D{D} F{F} E{E} k{k} sh{sh} {routing}")
    y, y_save, gu, gu_re, g_re, g_ca = _run_all(inp)
    assert torch.equal(y, y_save), "forward_save_gu's y differs from moe_ffn_forward's"
    assert torch.equal(_rows_written(gu, inp), _rows_written(gu_re, inp)), \
        "saved [g | u] differs from the backward's own recompute"
    _assert_same_grads(g_re, g_ca, f"T{T}")
    ref = oracle.forward_permuted(inp["x"], inp["topk_idx"], inp["topk_w"], inp["W1"], inp["W3"],
                                  inp["W2"], host_shared(inp), nthreads=oracle_threads(), with_gu=True)
    valid, S, R = _sorted_rows(inp)
    got = gu.float().cpu().numpy().astype(np.float64)
    rows = np.r_[0:valid, S:R]
    check_close(got[rows, :F], ref["gu"][rows, :F], "bf16", "gate products g")
    check_close(got[rows, F:], ref["gu"][rows, F:], "bf16", "up products u")


def test_cached_backward_invalid_ids():
    inp = moe_inputs.add_output_grad(make_case(400, 64, 128, 6, 2, True, "bf16", seed=9))
    inp["topk_idx"][10, 1] = 6
    inp["topk_idx"][11, 0] = -1
    say("cached backward invalid ids")
    y, y_save, gu, gu_re, g_re, g_ca = _run_all(inp)
    assert torch.equal(y, y_save)
    assert torch.equal(_rows_written(gu, inp), _rows_written(gu_re, inp))
    _assert_same_grads(g_re, g_ca, "invalid ids")
    assert float(g_ca["dtopk_w"][10, 1]) == 0.0 and float(g_ca["dtopk_w"][11, 0]) == 0.0
    # T = 0: nothing kept, weight gradients come back as zeros
    import grouped_gemm_permute_amd as gg
    inp0 = moe_inputs.add_output_grad(make_case(0, 64, 128, 3, 2, True, "bf16", seed=9))
    d0 = device_inputs(inp0)
    args0 = (d0["x"], d0["topk_idx"], d0["topk_w"], d0["W1"], d0["W3"], d0["W2"], d0["shared"])
    say("cached backward T0")
    y0, gu0 = gg.forward_save_gu(*args0)
    assert y0.shape == (0, 64) and gu0.shape == (0, 256)
    g0 = gg.backward(*args0, dev(inp0, "dy", "bf16"), gu=gu0)
    torch.cuda.synchronize()
    for n in ("dW1", "dW3", "dW2", "dWs1", "dWs3", "dWs2"):
        assert torch.count_nonzero(g0[n]).item() == 0, n


def test_cached_backward_step_workload():
    """The full step workload (32768 tokens, D 768, F 1536, 8 experts, top-2 +
    shared, Zipf): the up GEMM on whole 256-row tiles with its [g | u] pass.
    Bitwise checks only (the recomputing path's parity with the oracle is
    covered by the backward tests)."""
    inp = moe_inputs.add_output_grad(moe_inputs.make_inputs(2))
    say("cached backward step workload")
    y, y_save, gu, gu_re, g_re, g_ca = _run_all(inp)
    assert torch.equal(y, y_save)
    assert torch.equal(_rows_written(gu, inp), _rows_written(gu_re, inp))
    _assert_same_grads(g_re, g_ca, "step workload")


def test_cached_unsupported_dtype_and_variant():
    import grouped_gemm_permute_amd as gg
    from grouped_gemm_permute_amd import _lib
    inp = moe_inputs.add_output_grad(make_case(64, 64, 128, 4, 2, False, "f32", seed=3))
    d = device_inputs(inp)
    dy = dev(inp, "dy", "f32")
    args = (d["x"], d["topk_idx"], d["topk_w"], d["W1"], d["W3"], d["W2"], d["shared"])
    say("cached fp32 refused")
    with pytest.raises(gg.MoeError) as e:
        gg.forward_save_gu(*args)
    assert e.value.status == _lib.MOE_ERR_UNSUPPORTED
    gu = torch.zeros((64 * 2, 256), dtype=torch.float32, device="cuda")
    with pytest.raises(gg.MoeError) as e:
        gg.backward(*args, dy, gu=gu)
    assert e.value.status == _lib.MOE_ERR_UNSUPPORTED
    # the fused variant keeps no up product: refused before any launch
    b = make_case(128, 128, 256, 4, 2, False, "bf16", seed=3)
    db = device_inputs(b)
    y = torch.empty((128, 128), dtype=torch.bfloat16, device="cuda")
    gub = torch.empty((256, 512), dtype=torch.bfloat16, device="cuda")
    n = gg.workspace_size(128, 128, 256, 4, 2, False, torch.bfloat16, "fused")
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    st = gg.lib().moe_ffn_forward_save_gu(P(db["x"]), P(db["topk_idx"]), P(db["topk_w"]), P(db["W1"]),
                                          P(db["W3"]), P(db["W2"]), None, None, None, P(y), P(gub),
                                          128, 128, 256, 4, 2, _lib.MOE_BF16, _lib.MOE_VARIANT_FUSED,
                                          P(ws), ws.numel(), None)
    assert st == _lib.MOE_ERR_UNSUPPORTED
    torch.cuda.synchronize()
