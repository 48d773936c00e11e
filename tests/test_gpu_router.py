"""The router (moe_router_topk) and the routed forward (moe_ffn_forward_routed)
on the GPU against the oracle.

The router's top-k is an integer decision taken from fp32 logits; the
oracle takes it from fp64 logits.  A token's selection must match the
oracle's exactly unless two logits are closer than the fp32 summation error
bound, and then the GPU's choice must still be a valid top-k of the exact
logits within that bound; at least 99.9% of tokens must match exactly.
The routing weights are compared with the fp64 softmax of the exact logits
of the experts the GPU chose (1e-5 relative).  The routed forward must equal
moe_ffn_forward run on the router's own output bit for bit, its permute
must equal the oracle's counting sort of that output, and y must match the
oracle's layer on that routing within the dtype's tolerance.
"""
import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from oracle import brute
from gpu_util import check_close, dev, device_inputs, host_shared, make_case, say, to_f64

pytestmark = pytest.mark.gpu


def check_router(inp, idx_gpu, w_gpu, label):
    x = inp["x"].astype(np.float64)
    g = inp["gate_w"].astype(np.float64)
    k = idx_gpu.shape[1]
    _, _, logits = brute.router(x, g, k)
    ref_idx, _, _ = brute.router(x, g, k)
    bound = 1e-5 * (np.abs(x) @ np.abs(g)) + 1e-30          # fp32 summation error bound per logit
    T = x.shape[0]
    exact = np.all(idx_gpu == ref_idx, axis=1)
    for t in np.nonzero(~exact)[0]:
        chosen = idx_gpu[t]
        assert len(set(chosen.tolist())) == k, f"{label}: token {t} repeats an expert"
        others = np.setdiff1d(np.arange(g.shape[1]), chosen)
        lo = logits[t, chosen] + bound[t, chosen]
        if others.size:
            assert np.all(lo.min() >= logits[t, others] - bound[t, others]), f"{label}: token {t} misses a larger logit"
        assert np.all(np.diff(logits[t, chosen]) <= bound[t, chosen][1:] + bound[t, chosen][:-1]), \
            f"{label}: token {t} not in descending order"
    assert exact.mean() >= 0.999, f"{label}: only {exact.mean():.4f} of tokens match exactly"
    sel = np.take_along_axis(logits, idx_gpu.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    ref_w = z / z.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(w_gpu, ref_w, rtol=1e-5, atol=1e-7, err_msg=label)


ROUTER_CASES = [
    # T, D, E, k, dtype
    (1, 64, 4, 1, "bf16"),
    (700, 768, 8, 2, "bf16"),
    (5000, 256, 16, 4, "bf16"),
    (3000, 128, 64, 8, "bf16"),
    (300, 64, 4, 2, "f32"),
    (2049, 1024, 16, 2, "bf16"),
]


@pytest.mark.parametrize("case", ROUTER_CASES, ids=lambda c: "T{}_D{}_E{}_k{}_{}".format(*c))
def test_router_topk(case):
    import grouped_gemm_permute_amd as gg
    T, D, E, k, dt = case
    inp = moe_inputs.add_router(make_case(T, D, 64, E, k, False, dt, seed=61))
    say(f"router {case}")
    idx, w = gg.router_topk(dev(inp, "x", dt), dev(inp, "gate_w", dt), k)
    torch.cuda.synchronize()
    check_router(inp, idx.cpu().numpy(), w.cpu().numpy(), str(case))


def test_router_ties_take_the_lower_expert():
    import grouped_gemm_permute_amd as gg
    x = torch.ones((5, 64), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((64, 6), dtype=torch.bfloat16, device="cuda")
    g[0, 1] = g[0, 4] = 1.0         # logits [0, 1, 0, 0, 1, 0]
    say("router ties")
    idx, w = gg.router_topk(x, g, 3)
    torch.cuda.synchronize()
    assert idx.cpu().tolist() == [[1, 4, 0]] * 5


ROUTED_CASES = [
    # T, D, F, E, k, shared, dtype — S <= 4096 (one-block permute) and S > 4096 (router-fed histogram)
    (1500, 128, 256, 8, 2, True, "bf16"),
    (6000, 256, 512, 8, 2, True, "bf16"),
    (5000, 64, 128, 16, 4, False, "bf16"),
    (200, 64, 128, 4, 2, False, "f32"),
    (5000, 128, 128, 64, 4, False, "bf16"),   # histogram too fine for the fused scan: router, then permute
]


@pytest.mark.parametrize("case", ROUTED_CASES, ids=lambda c: "T{}_D{}_F{}_E{}_k{}_{}_{}".format(*c))
def test_forward_routed(case):
    import grouped_gemm_permute_amd as gg
    T, D, F, E, k, sh, dt = case
    inp = moe_inputs.add_router(make_case(T, D, F, E, k, sh, dt, seed=67))
    d = device_inputs(inp)
    gw = dev(inp, "gate_w", dt)
    lay = gg.workspace_layout(T, D, F, E, k, sh, d["x"].dtype)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device="cuda")
    say(f"forward routed {case}")
    y, idx, w = gg.forward_routed(d["x"], gw, d["W1"], d["W3"], d["W2"], d["shared"], k=k, workspace=ws)
    torch.cuda.synchronize()
    idx_h, w_h = idx.cpu().numpy(), w.cpu().numpy()
    check_router(inp, idx_h, w_h, "routed " + str(case))
    # the permute the routed forward left in its workspace
    ref = oracle.permute(idx_h, E, tile_rows=lay["tile_rows"], shared_rows=T if sh else 0)
    for name, n in (("counts", E), ("offsets", E + 1), ("perm", T * k), ("inv", T * k)):
        got = ws[lay[name]:lay[name] + 4 * n].view(torch.int32).cpu().numpy()
        np.testing.assert_array_equal(got, ref[name], err_msg=f"{case} {name}")
    # bit-identical to the plain forward on the router's output
    y2 = gg.forward(d["x"], idx, w, d["W1"], d["W3"], d["W2"], d["shared"])
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16 if dt == "bf16" else torch.int32),
                       y2.view(torch.int16 if dt == "bf16" else torch.int32))
    ref_y = oracle.forward_dense(inp["x"], idx_h, w_h, inp["W1"], inp["W3"], inp["W2"], host_shared(inp),
                                 nthreads=16)
    check_close(to_f64(y), ref_y, dt, "routed y " + str(case))
