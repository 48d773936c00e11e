"""moe_ffn_backward on the GPU against the fp64 oracle's backward.

Every output -- dx, dW1, dW3, dW2, the shared expert's weight gradients and
dtopk_w -- is compared element by element with oracle.backward on the same
seeded inputs, with the output tolerance of the call's dtype (bf16:
max|err| <= 1e-2 max|ref| + 1e-3; fp32: <= 1e-5 max|ref|), at sizes that
span several 256-row tiles, ragged tails, the multi-block permute, Zipf skew
and empty experts.  Also: bitwise run-to-run determinism, out-of-range ids
(flagged, contributing nothing), T = 0 (zero weight gradients).
"""
import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from gpu_util import check_close, dev, device_inputs, host_shared, make_case, oracle_threads, say, to_f64

pytestmark = pytest.mark.gpu




def gpu_backward(inp, workspace=None):
    import grouped_gemm_permute_amd as gg
    d = device_inputs(inp)
    dy = dev(inp, "dy", inp["workload"].dtype)
    g = gg.backward(d["x"], d["topk_idx"], d["topk_w"], d["W1"], d["W3"], d["W2"], d["shared"], dy,
                    workspace=workspace)
    torch.cuda.synchronize()
    return g


def oracle_grads(inp):
    return oracle.backward(inp["x"], inp["topk_idx"], inp["topk_w"], inp["W1"], inp["W3"],
                           inp["W2"], host_shared(inp), inp["dy"], nthreads=oracle_threads())


def compare_all(g, ref, dtype, label):
    for name in ("dx", "dW1", "dW3", "dW2", "dWs1", "dWs3", "dWs2"):
        if ref[name] is None:
            assert g[name] is None
            continue
        check_close(to_f64(g[name]), ref[name], dtype, f"{label} {name}")
    # routing-weight gradient: fp32 output for both dtypes, bf16 tolerance
    # for bf16 calls (its inputs h and dh' come from bf16 operands)
    check_close(to_f64(g["dtopk_w"]), ref["dw"], dtype, f"{label} dtopk_w")


CASES = [
    # T, D, F, E, k, shared, dtype, routing
    (64, 64, 128, 4, 2, False, "f32", "uniform"),
    (97, 64, 192, 3, 2, True, "f32", "uniform"),
    (300, 128, 256, 8, 2, True, "bf16", "uniform"),
    (700, 256, 512, 8, 2, True, "bf16", "zipf"),
    (1111, 64, 128, 16, 4, False, "bf16", "zipf"),      # empty / tiny experts
    (2500, 64, 192, 8, 2, True, "bf16", "uniform"),     # multi-block permute
    (200, 192, 320, 5, 1, False, "bf16", "uniform"),    # k = 1, column tails
    (9000, 64, 128, 4, 2, True, "bf16", "zipf"),        # groups over one 4096-row gradient chunk
    (3000, 64, 128, 70, 2, True, "bf16", "uniform"),    # 71 groups: lookups over two 64-group blocks
    (2000, 64, 128, 1024, 8, False, "bf16", "uniform"), # the expert limit
    (600, 64, 128, 8, 6, True, "bf16", "zipf"),         # top-k above 4 with a shared expert
    (400, 1024, 1600, 2, 1, True, "bf16", "uniform"),   # wide D and F (F = 25 * 64)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T{}_D{}_F{}_E{}_k{}_{}_{}_{}".format(*c))
def test_backward_full_parity(case):
    T, D, F, E, k, sh, dt, routing = case
    inp = moe_inputs.add_output_grad(make_case(T, D, F, E, k, sh, dt, routing, seed=41))
    say(f"backward full parity {case}")
    g = gpu_backward(inp)
    compare_all(g, oracle_grads(inp), dt, str(case))


def test_backward_tiny_workload():
    inp = moe_inputs.add_output_grad(moe_inputs.make_inputs(0))
    say("backward workload " + inp["workload"].name)
    compare_all(gpu_backward(inp), oracle_grads(inp), "f32", inp["workload"].name)


def test_backward_is_bitwise_deterministic():
    import grouped_gemm_permute_amd as gg
    inp = moe_inputs.add_output_grad(make_case(1500, 128, 256, 8, 2, True, "bf16", "zipf", seed=5))
    lay = gg.backward_workspace_layout(1500, 128, 256, 8, 2, True, torch.bfloat16)
    say("backward determinism T1500 D128 F256 E8 k2 shared")
    outs = []
    for fill in (0, 255):
        ws = torch.full((lay["total"],), fill, dtype=torch.uint8, device="cuda")
        g = gpu_backward(inp, workspace=ws)
        outs.append({n: v.view(torch.int16 if v.dtype == torch.bfloat16 else torch.int32).cpu()
                     for n, v in g.items() if v is not None})
    for n in outs[0]:
        assert torch.equal(outs[0][n], outs[1][n]), n


def test_backward_invalid_ids_and_empty_batch():
    import grouped_gemm_permute_amd as gg
    inp = moe_inputs.add_output_grad(make_case(400, 64, 128, 6, 2, True, "bf16", seed=9))
    inp["topk_idx"][10, 1] = 6
    inp["topk_idx"][11, 0] = -1
    lay = gg.backward_workspace_layout(400, 64, 128, 6, 2, True, torch.bfloat16)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device="cuda")
    say("backward invalid ids")
    g = gpu_backward(inp, workspace=ws)
    assert gg.device_error(ws) == 2
    ref = oracle_grads(inp)
    compare_all(g, ref, "bf16", "invalid ids")
    assert float(g["dtopk_w"][10, 1]) == 0.0 and float(g["dtopk_w"][11, 0]) == 0.0
    # T = 0: weight gradients come back as zeros
    inp0 = moe_inputs.add_output_grad(make_case(0, 64, 128, 3, 2, True, "bf16", seed=9))
    say("backward T0")
    g0 = gpu_backward(inp0)
    for n in ("dW1", "dW3", "dW2", "dWs1", "dWs3", "dWs2"):
        assert torch.count_nonzero(g0[n]).item() == 0, n
    assert g0["dx"].shape == (0, 64) and g0["dtopk_w"].shape == (0, 2)


@pytest.mark.parametrize("cfg", [1, 2])
def test_backward_workload_sampled(cfg):
    """Full-size workloads in the configuration the benchmark times: dx and
    dtopk_w on sampled tokens (both depend only on their own token, so the
    oracle runs on those tokens alone) and the weight gradients of the
    smallest expert (the oracle sums all of its rows)."""
    w = moe_inputs.WORKLOADS[cfg]
    inp = moe_inputs.add_output_grad(moe_inputs.make_inputs(cfg))
    say(f"backward workload {w.name}")
    g = gpu_backward(inp)
    rng = np.random.default_rng(200 + cfg)
    tokens = np.unique(np.concatenate([np.arange(4), np.arange(w.T - 4, w.T),
                                       rng.choice(w.T, 16, replace=False)]))
    sub = {n: inp[n][tokens] for n in ("x", "topk_idx", "topk_w", "dy")}
    ref = oracle.backward(sub["x"], sub["topk_idx"], sub["topk_w"], inp["W1"], inp["W3"], inp["W2"],
                          host_shared(inp), sub["dy"], nthreads=oracle_threads())
    check_close(to_f64(g["dx"])[tokens], ref["dx"], w.dtype, f"{w.name} dx")
    check_close(to_f64(g["dtopk_w"])[tokens], ref["dw"], w.dtype, f"{w.name} dtopk_w")
    counts = np.bincount(inp["topk_idx"].reshape(-1), minlength=w.E)
    e = int(np.argmin(counts))
    wg = oracle.backward_weight_grads(inp["x"], inp["topk_idx"], inp["topk_w"], inp["W1"], inp["W3"],
                                      inp["W2"], host_shared(inp), inp["dy"], [e], nthreads=oracle_threads())[e]
    for name, ref_e in zip(("dW1", "dW3", "dW2"), wg):
        check_close(to_f64(g[name][e]), ref_e, w.dtype, f"{w.name} {name}[{e}] ({counts[e]} rows)")
