"""moe_ffn_forward on the GPU against the fp64 oracle.

* full element-by-element parity at sizes the oracle finishes in seconds,
  spanning several 256-row tiles, ragged tails, column tails, the
  multi-block permute, Zipf skew and empty experts;
* (the five workload shapes at full size, every token, are in
  test_gpu_fullsize.py)
* 2^20 tokens on sampled tokens the oracle computes one by one;
* the sorted-row intermediates h and Y on sampled rows;
* run-to-run bitwise determinism with garbage-filled workspaces;
* edge cases: T = 1, all tokens on one expert, zero routing weights,
  out-of-range expert ids (flagged and skipped), T = 0.
"""
import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from oracle import brute
from gpu_util import check_close, device_inputs, host_shared, make_case, oracle_threads, say, to_f64

pytestmark = pytest.mark.gpu


def gpu_forward(inp, variant="unfused", workspace=None):
    import grouped_gemm_permute_amd as gg
    d = device_inputs(inp)
    y = gg.forward(d["x"], d["topk_idx"], d["topk_w"], d["W1"], d["W3"], d["W2"], d["shared"],
                   variant=variant, workspace=workspace)
    torch.cuda.synchronize()
    return y, d


def oracle_y(inp, tokens=None):
    return oracle.forward_dense(inp["x"], inp["topk_idx"], inp["topk_w"], inp["W1"], inp["W3"],
                                inp["W2"], host_shared(inp), tokens=tokens, nthreads=oracle_threads())


FULL_CASES = [
    # T, D, F, E, k, shared, dtype, routing
    (64, 64, 128, 4, 2, False, "f32", "uniform"),
    (97, 64, 192, 3, 2, True, "f32", "uniform"),
    (700, 256, 512, 8, 2, True, "bf16", "uniform"),
    (2500, 128, 192, 8, 2, True, "bf16", "uniform"),     # multi-block permute, column tails
    (300, 64, 64, 1, 1, False, "bf16", "uniform"),
    (1500, 192, 320, 6, 3, True, "bf16", "zipf"),
    (1111, 320, 128, 16, 4, False, "bf16", "zipf"),      # empty / tiny experts
    # groups averaging < 256 rows run on the small-tile kernels
    (200, 512, 1024, 16, 2, False, "bf16", "zipf"),      # ~25 rows per expert, many empty
    (64, 768, 1536, 8, 2, True, "bf16", "uniform"),      # layer shape, tiny batch + shared
    (300, 128, 320, 4, 2, False, "bf16", "uniform"),     # up tiles of 192 rows, one per expert
    (1000, 64, 128, 32, 3, False, "bf16", "zipf"),       # 128-row up tiles, skewed: multi-tile groups
    (512, 768, 1536, 8, 2, True, "bf16", "uniform"),     # 256-row up tiles (half-stage operand reads)
    (640, 128, 256, 8, 2, True, "bf16", "zipf"),         # 224-row up tiles, multi-tile groups
    # more than 64 groups: the tile -> group lookup spans several 64-group blocks
    (3000, 128, 192, 100, 4, True, "bf16", "zipf"),      # small-chunk kernels, many empty experts
    (20000, 64, 128, 70, 2, True, "bf16", "uniform"),    # 256-row engine
    # top-k above 4: the combine's plain per-slot loop (up to 4 slots it
    # loads every slot's row up front)
    (400, 128, 256, 12, 6, True, "bf16", "uniform"),     # small-chunk kernels + shared
    (1500, 64, 128, 8, 8, False, "bf16", "uniform"),     # k = E: every token to every expert
    (64, 64, 128, 6, 5, True, "f32", "uniform"),
    # over twelve rounds of up tiles: whole 256-row tiles, two column groups
    # (12 x 448 x 256 weights per XCD outgrow its L2 share), D tail of 192
    (24000, 448, 1536, 8, 2, True, "bf16", "zipf"),
    (2000, 64, 128, 1024, 8, True, "bf16", "uniform"),   # the expert limit (1025 groups)
    # wide D and F with a 64-column tail (F = 10 * 256 + 64)
    (96, 2048, 2624, 3, 2, True, "bf16", "uniform"),     # small-chunk kernels
    (600, 2048, 2624, 2, 1, False, "bf16", "uniform"),   # 256-row engine, 64 K steps
]


@pytest.mark.parametrize("case", FULL_CASES, ids=lambda c: "T{}_D{}_F{}_E{}_k{}_{}_{}_{}".format(*c))
def test_forward_full_parity(case):
    T, D, F, E, k, sh, dt, routing = case
    inp = make_case(T, D, F, E, k, sh, dt, routing)
    say(f"forward full parity {case}")
    y, _ = gpu_forward(inp)
    check_close(to_f64(y), oracle_y(inp), dt, str(case))


FUSED_CASES = [
    # T, D, F, E, k, shared, routing
    (700, 256, 512, 8, 2, True, "uniform"),
    (1111, 128, 384, 5, 3, False, "zipf"),     # ragged 64-row tiles, empty experts possible
    (300, 1024, 256, 4, 2, True, "uniform"),   # widest accumulator (D = 1024)
    (513, 768, 640, 6, 2, False, "uniform"),
    (1, 384, 128, 2, 1, False, "uniform"),
    # tiles of the last round of 256 shared out over workgroups (F chunks
    # split, fp32 partial outputs summed after)
    (200, 512, 4096, 4, 2, True, "uniform"),   # ~11 tiles -> 16 splits of one chunk
    (64, 256, 2176, 3, 2, False, "zipf"),      # 2-3 tiles -> 16 splits of 9 chunks, the last a half chunk
    (9000, 128, 640, 8, 2, False, "zipf"),     # 256 whole tiles, then ~30 tiles in 2-3 splits
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "T{}_D{}_F{}_E{}_k{}_{}_{}".format(*c))
def test_fused_full_parity(case):
    T, D, F, E, k, sh, routing = case
    inp = make_case(T, D, F, E, k, sh, "bf16", routing, seed=31)
    say(f"fused full parity {case}")
    y, _ = gpu_forward(inp, variant="fused")
    check_close(to_f64(y), oracle_y(inp), "bf16", "fused " + str(case))


def test_forward_million_tokens_sampled():
    """2^20 tokens (2^21 routed slots plus the shared expert's 2^20 rows):
    the many-block permute and row offsets far past 2^16 tiles' worth of
    rows, checked on sampled tokens (each depends only on its own row)."""
    T = 1 << 20
    inp = make_case(T, 64, 128, 8, 2, True, "bf16", "zipf", seed=11)
    say(f"forward T={T} sampled")
    y, _ = gpu_forward(inp)
    rng = np.random.default_rng(5)
    tokens = np.unique(np.concatenate([np.arange(8), np.arange(T - 8, T), rng.choice(T, 48, replace=False)]))
    check_close(to_f64(y)[tokens], oracle_y(inp, tokens), "bf16", f"T={T}")


def test_forward_intermediates_sampled_rows():
    import grouped_gemm_permute_amd as gg
    inp = make_case(900, 192, 256, 5, 2, True, "bf16", "zipf", seed=21)
    T, D, F, E, k = 900, 192, 256, 5, 2
    lay = gg.workspace_layout(T, D, F, E, k, True, torch.bfloat16)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device="cuda")
    say("forward intermediates T900 D192 F256 E5 k2 shared")
    gpu_forward(inp, workspace=ws)
    R = T * k + T
    h = ws[lay["h"]:lay["h"] + R * F * 2].view(torch.bfloat16).view(R, F)
    Y = ws[lay["Y"]:lay["Y"] + R * D * 2].view(torch.bfloat16).view(R, D)
    ref = oracle.permute(inp["topk_idx"], E)
    rows = np.concatenate([np.arange(0, T * k, 37), np.arange(T * k - 5, T * k),
                           np.arange(T * k, R, 41), [R - 1]])
    flat = inp["topk_idx"].reshape(-1)
    hs = to_f64(h[torch.from_numpy(rows).cuda()])
    Ys = to_f64(Y[torch.from_numpy(rows).cuda()])
    for i, p in enumerate(rows):
        if p < T * k:
            s = ref["perm"][p]
            t, e = s // k, flat[s]
            w1, w3, w2 = inp["W1"][e], inp["W3"][e], inp["W2"][e]
        else:
            t = p - T * k
            w1, w3, w2 = inp["Ws1"], inp["Ws3"], inp["Ws2"]
        xv = inp["x"][t].astype(np.float64)
        g, u = xv @ w1, xv @ w3
        hh = brute.silu(g) * u
        check_close(hs[i], hh, "bf16", f"h row {p}")
        check_close(Ys[i], hh @ w2.astype(np.float64), "bf16", f"Y row {p}")


DETERMINISM_CASES = [
    # T, D, F, E, k, shared, routing, variant
    (3000, 256, 384, 8, 2, True, "zipf", "unfused"),      # 256-row engine
    (300, 256, 512, 8, 2, False, "uniform", "unfused"),   # small chunks, sort inside the up GEMM
    (300, 256, 1024, 8, 2, True, "uniform", "fused"),     # every tile split over F chunks
    (9000, 128, 640, 8, 2, False, "zipf", "fused"),       # whole rounds, then split tiles
]


@pytest.mark.parametrize("case", DETERMINISM_CASES, ids=lambda c: "T{}_D{}_F{}_E{}_k{}_{}_{}_{}".format(*c))
def test_forward_is_bitwise_deterministic(case):
    """Three calls with differently filled workspaces on fresh streams give
    the same bits: no atomics decide an order, and partial sums (split
    tiles, the combine) are added in a fixed order."""
    import grouped_gemm_permute_amd as gg
    T, D, F, E, k, sh, routing, variant = case
    inp = make_case(T, D, F, E, k, sh, "bf16", routing, seed=5)
    d = device_inputs(inp)
    lay = gg.workspace_layout(T, D, F, E, k, sh, torch.bfloat16, variant)
    say(f"determinism {case}")
    outs = []
    for fill in (0, 255, 77):
        ws = torch.full((lay["total"],), fill, dtype=torch.uint8, device="cuda")
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            y = gg.forward(d["x"], d["topk_idx"], d["topk_w"], d["W1"], d["W3"], d["W2"], d["shared"],
                           variant=variant, workspace=ws)
        s.synchronize()
        outs.append(y.view(torch.int16).cpu())
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_forward_edge_cases():
    import grouped_gemm_permute_amd as gg
    # one token
    inp = make_case(1, 128, 128, 4, 2, True, "bf16")
    say("edge T1")
    y, _ = gpu_forward(inp)
    check_close(to_f64(y), oracle_y(inp), "bf16", "T=1")
    # every token on the same two experts, the others empty
    inp = make_case(600, 128, 256, 8, 2, False, "bf16")
    inp["topk_idx"][:, 0] = 3
    inp["topk_idx"][:, 1] = 7
    say("edge all tokens on experts 3 and 7")
    y, _ = gpu_forward(inp)
    check_close(to_f64(y), oracle_y(inp), "bf16", "two experts")
    # zero routing weights leave the shared expert
    inp = make_case(200, 128, 128, 4, 2, True, "bf16")
    inp["topk_w"][:] = 0.0
    say("edge zero weights")
    y, _ = gpu_forward(inp)
    check_close(to_f64(y), oracle_y(inp), "bf16", "zero weights")
    # out-of-range ids: flagged, skipped
    inp = make_case(500, 128, 192, 6, 2, True, "bf16")
    inp["topk_idx"][10, 1] = 6
    inp["topk_idx"][11, 0] = -1
    inp["topk_idx"][499, 1] = 1000
    lay = gg.workspace_layout(500, 128, 192, 6, 2, True, torch.bfloat16)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device="cuda")
    say("edge invalid ids")
    y, _ = gpu_forward(inp, workspace=ws)
    assert gg.device_error(ws) == 3
    check_close(to_f64(y), oracle_y(inp), "bf16", "invalid ids")
    # T = 0: nothing launched, empty output
    inp = make_case(0, 64, 64, 2, 1, False, "bf16")
    y, _ = gpu_forward(inp)
    assert y.shape == (0, 64)


def test_stream_read_reads_every_word_once():
    """The measurement helper behind the small-chunk record's read peak: each
    16-byte chunk is read by exactly one thread, so the xor over all
    workgroups' sinks is the xor of every word of the buffer."""
    import grouped_gemm_permute_amd as gg
    n = (1 << 20) + 4 * 37                         # a tail past the unrolled passes
    host = np.random.default_rng(3).integers(-2**31, 2**31 - 1, size=n, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(host).cuda()
    for blocks in (1, 64, 1000):
        sink = torch.empty(blocks, dtype=torch.int32, device="cuda")
        say(f"stream_read blocks={blocks}")
        gg.stream_read(buf, sink)
        got = np.bitwise_xor.reduce(sink.cpu().numpy())
        assert got == np.bitwise_xor.reduce(host)
