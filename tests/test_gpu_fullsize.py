"""moe_ffn_forward at the workloads' full sizes, every output element checked.

The five workload shapes (the 4096-token GPT-OSS-Lite layer, the
32768-token Zipf step, the 512-token small-chunk case and the F > D case)
run in the launch configuration the benchmark times (a caller-owned
workspace, one call on the current stream), and every token of y is
compared with the fp64 oracle's dense path, with the tolerance of
``gpu_util.check_close``.  The fused variant is checked the same way on the
step, small-chunk (its tiles' F chunks split over workgroups) and F > D
workloads.

The permute the forward runs inside its own workspace (counts, offsets,
tile_off for the call's tile height, tile_off64 for 64-row tiles, perm, inv
and the invalid-slot count) is compared bit for bit with the oracle's
counting sort, since the grouped GEMMs read nothing else about the routing.
"""
import functools

import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from gpu_util import check_close, device_inputs, host_shared, oracle_threads, say, to_f64

pytestmark = pytest.mark.gpu

# (workload, variant), ordered so that each workload's oracle result is
# computed once and reused by both variants
CASES = [(0, "unfused"), (1, "unfused"), (2, "unfused"), (2, "fused"), (3, "unfused"),
         (3, "fused"), (4, "unfused"), (4, "fused")]


def case_id(v):
    return moe_inputs.WORKLOADS[v].name if isinstance(v, int) else v


@functools.lru_cache(maxsize=1)
def workload_inputs(cfg):
    return moe_inputs.make_inputs(cfg)


@functools.lru_cache(maxsize=1)
def oracle_y(cfg):
    inp = workload_inputs(cfg)
    return oracle.forward_dense(inp["x"], inp["topk_idx"], inp["topk_w"], inp["W1"], inp["W3"],
                                inp["W2"], host_shared(inp), nthreads=oracle_threads())


def run_forward(cfg, variant):
    """One forward as bench.py launches it; returns y and the workspace."""
    import grouped_gemm_permute_amd as gg
    w = moe_inputs.WORKLOADS[cfg]
    inp = workload_inputs(cfg)
    d = device_inputs(inp)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    # garbage in the workspace and y: the forward must overwrite what it reads
    ws = torch.full((gg.workspace_layout(w.T, w.D, w.F, w.E, w.k, w.shared, dt, variant)["total"],),
                    0x5A, dtype=torch.uint8, device="cuda")
    y = torch.full((w.T, w.D), float("nan"), dtype=dt, device="cuda")
    gg.forward(d["x"], d["topk_idx"], d["topk_w"], d["W1"], d["W3"], d["W2"], d["shared"], y=y,
               variant=variant, workspace=ws)
    torch.cuda.synchronize()
    return y, ws


@pytest.mark.parametrize("cfg,variant", CASES, ids=case_id)
def test_forward_full_size_every_token(cfg, variant):
    w = moe_inputs.WORKLOADS[cfg]
    say(f"full-size forward, every token: {w.name} {variant}")
    y, _ = run_forward(cfg, variant)
    got = to_f64(y)
    say(f"oracle on all {w.T} tokens, {oracle_threads()} threads")
    check_close(got, oracle_y(cfg), w.dtype, f"{variant} {w.name}")


def read_i32(ws, off, n):
    return ws[off:off + 4 * n].view(torch.int32).cpu().numpy()


@pytest.mark.parametrize("cfg,variant", CASES, ids=case_id)
def test_forward_workspace_permute_bit_exact(cfg, variant):
    import grouped_gemm_permute_amd as gg
    w = moe_inputs.WORKLOADS[cfg]
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    lay = gg.workspace_layout(w.T, w.D, w.F, w.E, w.k, w.shared, dt, variant)
    say(f"workspace permute of the forward: {w.name} {variant} (tile_rows {lay['tile_rows']}, "
        f"small_tiles {lay['small_tiles']})")
    _, ws = run_forward(cfg, variant)
    idx = workload_inputs(cfg)["topk_idx"]
    S, E = w.T * w.k, w.E
    sh_rows = w.T if w.shared else 0
    ref = oracle.permute(idx, E, lay["tile_rows"], sh_rows)
    ref64 = oracle.permute(idx, E, 64, sh_rows)
    got = {
        "err": read_i32(ws, lay["err"], 1),
        "counts": read_i32(ws, lay["counts"], E),
        "offsets": read_i32(ws, lay["offsets"], E + 1),
        "tile_off": read_i32(ws, lay["tile_off"], E + 2),
        "perm": read_i32(ws, lay["perm"], S),
        "inv": read_i32(ws, lay["inv"], S),
    }
    assert got["err"][0] == ref["bad"] == 0
    for name in ("counts", "offsets", "tile_off", "perm", "inv"):
        assert np.array_equal(got[name], ref[name]), f"{name} differs from the oracle"
    # written by every forward; the small-chunk down GEMM walks these 64-row tiles
    assert np.array_equal(read_i32(ws, lay["tile_off64"], E + 2), ref64["tile_off"])
    # the invariants the pins of the oracle rest on, on the GPU's own arrays
    assert got["counts"].sum() == S
    assert np.array_equal(np.sort(got["perm"]), np.arange(S))
    assert np.array_equal(got["inv"][got["perm"]], np.arange(S))
