"""expert_permute on the GPU against the oracle's counting sort: counts,
offsets, tile offsets, perm, inv and the invalid-slot count must be
bit-identical (the stable order is unique)."""
import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from gpu_util import say

pytestmark = pytest.mark.gpu


def run_and_compare(idx_np, E, tile_rows, shared_rows, label):
    import grouped_gemm_permute_amd as gg
    say(f"permute {label} S={idx_np.size} E={E} BM={tile_rows} shared_rows={shared_rows}")
    ref = oracle.permute(idx_np, E, tile_rows=tile_rows, shared_rows=shared_rows)
    out = gg.expert_permute(torch.from_numpy(idx_np).cuda(), E, tile_rows, shared_rows)
    torch.cuda.synchronize()
    for name in ("counts", "offsets", "tile_off", "perm", "inv"):
        got = out[name].cpu().numpy()
        np.testing.assert_array_equal(got, ref[name], err_msg=f"{label}: {name}")
    assert int(out["err"].item()) == ref["bad"], label


@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (64, 2, 4), (100, 3, 5), (2048, 2, 8),
                                   (2049, 2, 8), (5000, 2, 8), (40000, 2, 64), (3000, 4, 1024),
                                   # histogram tables past the fused-scan limit: separate scan launch
                                   (5000, 4, 1024), (200000, 2, 64)])
def test_permute_uniform(T, k, E):
    rng = np.random.default_rng(T + E)
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    run_and_compare(idx, E, 256, T, f"uniform T{T}k{k}E{E}")


@pytest.mark.parametrize("T", [333, 4096, 32768])
def test_permute_all_to_one_expert(T):
    idx = np.full((T, 2), 5, np.int32)
    idx[:, 1] = 6
    run_and_compare(idx, 8, 256, 0, f"two-experts T{T}")


def test_permute_invalid_ids():
    rng = np.random.default_rng(3)
    for T in (50, 9000):
        idx = rng.integers(-2, 10, (T, 2)).astype(np.int32)
        run_and_compare(idx, 8, 64, T, f"invalid T{T}")


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_permute_workloads(cfg):
    w = moe_inputs.WORKLOADS[cfg]
    inp = moe_inputs.make_inputs(cfg)
    import grouped_gemm_permute_amd as gg
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    run_and_compare(inp["topk_idx"], w.E, gg.tile_rows(dt), w.T if w.shared else 0, w.name)
