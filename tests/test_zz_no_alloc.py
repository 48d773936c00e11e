"""moe_ffn_forward_noalloc through the C ABI against moe_ffn_forward.

The no-allocation entry point runs the same kernels on the library's own
per-device workspace array, so its y must equal moe_ffn_forward's bit for
bit (and hence meet the same oracle tolerance).  Two calls in a row, the
second smaller than the first, check that the array's leftover contents from
a larger call do not leak into a smaller one; a third call takes the fused
variant.  A call that would need more than the array holds is refused on the
host with MOE_ERR_WORKSPACE before anything is launched.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_close, device_inputs, host_shared, make_case, oracle_threads, say, to_f64

pytestmark = pytest.mark.gpu


def both(inp, variant="unfused"):
    import grouped_gemm_permute_amd as gg
    d = device_inputs(inp)
    args = (d["x"], d["topk_idx"], d["topk_w"], d["W1"], d["W3"], d["W2"], d["shared"])
    ref = gg.forward(*args, variant=variant)
    got = gg.forward_noalloc(*args, variant=variant)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_forward_two_calls_shrinking():
    big = make_case(4096, 768, 1536, 8, 2, True, "bf16", "uniform", seed=91)
    say("noalloc call 1: T4096 D768 F1536 E8 k2 shared (the 4096-token layer)")
    ref, got = both(big)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    small = make_case(700, 256, 512, 8, 2, True, "bf16", "zipf", seed=92)
    say("noalloc call 2: T700 D256 F512 E8 k2 shared, smaller than call 1")
    ref, got = both(small)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    y_ref = oracle.forward_dense(small["x"], small["topk_idx"], small["topk_w"], small["W1"],
                                 small["W3"], small["W2"], host_shared(small), nthreads=oracle_threads())
    check_close(to_f64(got), y_ref, "bf16", "noalloc T700")


def test_noalloc_fused_and_fp32():
    inp = make_case(300, 256, 512, 4, 2, False, "bf16", "uniform", seed=93)
    say("noalloc fused T300 D256 F512 E4 k2")
    ref, got = both(inp, "fused")
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    inp = make_case(97, 64, 192, 3, 2, True, "f32", "uniform", seed=94)
    say("noalloc fp32 T97 D64 F192 E3 k2 shared")
    ref, got = both(inp)
    assert torch.equal(got, ref)


def test_noalloc_refuses_a_call_larger_than_its_array():
    import grouped_gemm_permute_amd as gg
    T, D, F, E, k = 32768, 768, 1536, 8, 2
    assert gg.workspace_size(T, D, F, E, k, True, torch.bfloat16) > gg.NOALLOC_SCRATCH_BYTES
    z = dict(dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((T, D), **z)
    W1 = torch.zeros((E, D, F), **z)
    W2 = torch.zeros((E, F, D), **z)
    sh = (torch.zeros((D, F), **z), torch.zeros((D, F), **z), torch.zeros((F, D), **z))
    idx = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    y = torch.full((T, D), 7.0, **z)
    say("noalloc T32768: refused (workspace beyond the array)")
    with pytest.raises(gg.MoeError) as e:
        gg.forward_noalloc(x, idx, w, W1, W1, W2, sh, y=y)
    assert e.value.status == 3          # MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())       # nothing was launched
