"""Pins for the CPU oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  The oracle (oracle/moe_oracle.c) is
checked against things other than itself: numpy's bincount and stable
argsort (textbook routines), an independently written numpy brute force,
hand-derived closed forms (tests/golden/closed_form_cases.json), algebraic
special cases, and the page figures that fix the work accounting
(tests/golden/page_figures.json).
"""
import json
import math
import os

import numpy as np
import pytest

import moe_inputs
import oracle
from oracle import brute


def _rand_problem(rng, T, D, F, E, k, shared=False, distinct=True):
    x = rng.standard_normal((T, D))
    W1 = rng.standard_normal((E, D, F)) / math.sqrt(D)
    W3 = rng.standard_normal((E, D, F)) / math.sqrt(D)
    W2 = rng.standard_normal((E, F, D)) / math.sqrt(F)
    if distinct:
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    else:
        idx = rng.integers(0, E, (T, k)).astype(np.int32)
    w = rng.random((T, k))
    sh = None
    if shared:
        sh = (rng.standard_normal((D, F)) / math.sqrt(D), rng.standard_normal((D, F)) / math.sqrt(D),
              rng.standard_normal((F, D)) / math.sqrt(F))
    return x, idx, w, W1, W3, W2, sh


# ---------------------------------------------------------------- permutation

@pytest.mark.parametrize("T,k,E,skew", [(1, 1, 1, False), (7, 2, 4, False), (64, 2, 4, False),
                                        (1000, 2, 8, True), (513, 3, 16, False), (4096, 2, 8, True),
                                        (300, 4, 64, True)])
def test_permute_matches_numpy_counting_sort(T, k, E, skew):
    rng = np.random.default_rng(T * 31 + E)
    if skew:   # many empty experts
        idx = rng.integers(0, max(1, E // 3), (T, k)).astype(np.int32)
    else:
        idx = rng.integers(0, E, (T, k)).astype(np.int32)
    BM = 32
    r = oracle.permute(idx, E, tile_rows=BM, shared_rows=T)
    flat = idx.reshape(-1)
    ref_counts = np.bincount(flat, minlength=E)
    ref_perm = np.argsort(flat, kind="stable")
    assert r["bad"] == 0
    np.testing.assert_array_equal(r["counts"], ref_counts)
    np.testing.assert_array_equal(r["offsets"], np.concatenate([[0], np.cumsum(ref_counts)]))
    np.testing.assert_array_equal(r["perm"], ref_perm)
    ref_inv = np.empty_like(ref_perm)
    ref_inv[ref_perm] = np.arange(flat.size)
    np.testing.assert_array_equal(r["inv"], ref_inv)
    tiles = np.concatenate([-(-ref_counts // BM), [-(-T // BM)]])
    np.testing.assert_array_equal(r["tile_off"], np.concatenate([[0], np.cumsum(tiles)]))


def test_permute_invariants():
    rng = np.random.default_rng(5)
    inp = moe_inputs.make_inputs(2, T=2000)          # Zipf-skewed routing, E=8, k=2
    idx = inp["topk_idx"]
    S = idx.size
    r = oracle.permute(idx, 8)
    perm, inv, flat = r["perm"], r["inv"], idx.reshape(-1)
    assert sorted(perm.tolist()) == list(range(S))                # bijection
    assert r["counts"].sum() == S
    assert np.all(np.diff(r["offsets"]) >= 0) and r["offsets"][-1] == S
    assert np.all(np.diff(flat[perm]) >= 0)                       # sorted by expert
    for e in range(8):                                            # stable inside an expert
        seg = perm[r["offsets"][e]:r["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
    np.testing.assert_array_equal(inv[perm], np.arange(S))
    del rng


def test_permute_flags_out_of_range_ids():
    idx = np.array([[0, 5], [-1, 1], [1, 0]], np.int32)
    r = oracle.permute(idx, 2, tile_rows=2)
    assert r["bad"] == 2
    np.testing.assert_array_equal(r["counts"], [2, 2])
    np.testing.assert_array_equal(r["offsets"], [0, 2, 4])
    np.testing.assert_array_equal(r["perm"][:4], [0, 5, 3, 4])
    np.testing.assert_array_equal(r["perm"][4:], [-1, -1])
    np.testing.assert_array_equal(r["inv"], [0, -1, -1, 2, 3, 1])
    np.testing.assert_array_equal(r["tile_off"], [0, 1, 2, 2])


# ---------------------------------------------------------------- forward

@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("T,D,F,E,k", [(1, 3, 5, 1, 1), (9, 8, 12, 4, 2), (17, 16, 24, 5, 3)])
def test_dense_matches_numpy_brute_force(T, D, F, E, k, shared):
    rng = np.random.default_rng(T + D + F + E + k)
    x, idx, w, W1, W3, W2, sh = _rand_problem(rng, T, D, F, E, k, shared)
    y = oracle.forward_dense(x, idx, w, W1, W3, W2, sh)
    ref = brute.moe_forward(x, idx, w, W1, W3, W2, sh)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("shared", [False, True])
def test_permuted_path_equals_dense_path_bitwise(shared):
    rng = np.random.default_rng(11)
    x, idx, w, W1, W3, W2, sh = _rand_problem(rng, 40, 16, 32, 6, 2, shared)
    idx[3] = [5, 5]                                  # a duplicate id inside one token
    idx[:10, 0] = 1                                  # expert skew; expert 0 may go empty
    dense = oracle.forward_dense(x, idx, w, W1, W3, W2, sh, nthreads=3)
    perm = oracle.forward_permuted(x, idx, w, W1, W3, W2, sh, nthreads=2)
    assert np.array_equal(dense, perm["y"])


def test_one_expert_top1_is_dense_swiglu():
    rng = np.random.default_rng(3)
    T, D, F = 12, 16, 40
    x = rng.standard_normal((T, D))
    W1 = rng.standard_normal((1, D, F))
    W3 = rng.standard_normal((1, D, F))
    W2 = rng.standard_normal((1, F, D))
    idx = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1))
    g, u = x @ W1[0], x @ W3[0]
    ref = ((g / (1 + np.exp(-g))) * u) @ W2[0]
    for y in (oracle.forward_dense(x, idx, w, W1, W3, W2),
              oracle.forward_permuted(x, idx, w, W1, W3, W2)["y"]):
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_closed_form_fixtures(golden_dir):
    cases = json.load(open(os.path.join(golden_dir, "closed_form_cases.json")))["cases"]
    for c in cases:
        arr = {n: np.array(c[n], np.float64) for n in ("x", "W1", "W3", "W2", "topk_w")}
        idx = np.array(c["topk_idx"], np.int32)
        sh = tuple(np.array(a, np.float64) for a in c["shared"]) if "shared" in c else None
        for y in (oracle.forward_dense(arr["x"], idx, arr["topk_w"], arr["W1"], arr["W3"], arr["W2"], sh),
                  oracle.forward_permuted(arr["x"], idx, arr["topk_w"], arr["W1"], arr["W3"], arr["W2"], sh)["y"]):
            np.testing.assert_allclose(y, np.array(c["y"]), rtol=0, atol=1e-15, err_msg=c["name"])


def test_special_cases():
    rng = np.random.default_rng(7)
    T, D, F, E, k = 20, 12, 18, 4, 2
    x, idx, w, W1, W3, W2, sh = _rand_problem(rng, T, D, F, E, k, shared=True)
    base = oracle.forward_dense(x, idx, w, W1, W3, W2, sh)
    sh_only = oracle.forward_dense(x, idx, np.zeros_like(w), W1, W3, W2, sh)
    # zero routed weights leave the dense shared SwiGLU
    np.testing.assert_allclose(sh_only, brute.expert(x, *sh), rtol=1e-12, atol=1e-13)
    # scaling the routing weights scales the routed part
    scaled = oracle.forward_dense(x, idx, 3.0 * w, W1, W3, W2, sh)
    np.testing.assert_allclose(scaled - sh_only, 3.0 * (base - sh_only), rtol=1e-11, atol=1e-12)
    # one-hot weights pick out one expert
    onehot = np.zeros_like(w)
    onehot[:, 1] = 1.0
    y1 = oracle.forward_dense(x, idx, onehot, W1, W3, W2)
    for t in range(T):
        e = idx[t, 1]
        np.testing.assert_allclose(y1[t], brute.expert(x[t], W1[e], W3[e], W2[e]), rtol=1e-12,
                                   atol=1e-13)
    # x = 0 gives y = 0 (silu(0) = 0)
    assert np.all(oracle.forward_dense(np.zeros_like(x), idx, w, W1, W3, W2, sh) == 0.0)
    # W3 = 0 removes the routed experts
    np.testing.assert_array_equal(oracle.forward_dense(x, idx, w, W1, np.zeros_like(W3), W2, sh), sh_only)
    # swapping the k choices of every token leaves y unchanged up to rounding
    sw = oracle.forward_dense(x, idx[:, ::-1].copy(), w[:, ::-1].copy(), W1, W3, W2, sh)
    np.testing.assert_allclose(sw, base, rtol=1e-13, atol=1e-14)
    # a duplicated id acts as one expert with the summed weight
    idx2 = idx.copy()
    idx2[:, 1] = idx2[:, 0]
    yd = oracle.forward_dense(x, idx2, w, W1, W3, W2)
    yone = oracle.forward_dense(x, idx2[:, :1].copy(), w.sum(1, keepdims=True), W1, W3, W2)
    np.testing.assert_allclose(yd, yone, rtol=1e-12, atol=1e-13)


def test_permuted_intermediates_are_per_row_swiglu():
    rng = np.random.default_rng(9)
    T, D, F, E, k = 15, 8, 16, 3, 2
    x, idx, w, W1, W3, W2, sh = _rand_problem(rng, T, D, F, E, k, shared=True)
    r = oracle.forward_permuted(x, idx, w, W1, W3, W2, sh)
    S = T * k
    for p in range(S):
        s = r["perm"][p]
        t, e = s // k, idx.reshape(-1)[s]
        g, u = x[t] @ W1[e], x[t] @ W3[e]
        hh = (g / (1 + np.exp(-g))) * u
        np.testing.assert_allclose(r["h"][p], hh, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(r["Y"][p], hh @ W2[e], rtol=1e-12, atol=1e-13)
    for t in range(T):
        g, u = x[t] @ sh[0], x[t] @ sh[1]
        np.testing.assert_allclose(r["Y"][S + t], ((g / (1 + np.exp(-g))) * u) @ sh[2], rtol=1e-12,
                                   atol=1e-13)


def test_permuted_gate_up_products_per_row():
    """The sorted-row gate and up products a caching backward keeps
    ("Triton MoE Kernels & Memory Checkpointing", Part A section 8: g = v W1,
    u = v W3): against numpy's products of the row's token with its
    expert's matrices, h = silu(g) u to the last bit, zero rows for invalid
    slots."""
    rng = np.random.default_rng(21)
    T, D, F, E, k = 13, 8, 12, 4, 2
    x, idx, w, W1, W3, W2, sh = _rand_problem(rng, T, D, F, E, k, shared=True)
    idx[3, 1] = E + 2                                   # one invalid slot
    r = oracle.forward_permuted(x, idx, w, W1, W3, W2, sh, with_gu=True)
    S = T * k
    gu = r["gu"]
    assert gu.shape == (S + T, 2 * F)
    valid = r["offsets"][E]
    for p in range(S):
        if p >= valid:
            assert not gu[p].any()
            continue
        s = r["perm"][p]
        t, e = s // k, idx.reshape(-1)[s]
        np.testing.assert_allclose(gu[p, :F], x[t] @ W1[e], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(gu[p, F:], x[t] @ W3[e], rtol=1e-12, atol=1e-13)
    for t in range(T):
        np.testing.assert_allclose(gu[S + t, :F], x[t] @ sh[0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(gu[S + t, F:], x[t] @ sh[1], rtol=1e-12, atol=1e-13)
    g, u = gu[:, :F], gu[:, F:]
    # (numpy's exp and the C library's may differ in the last bit)
    np.testing.assert_allclose(r["h"], g / (1 + np.exp(-g)) * u, rtol=1e-15, atol=1e-300)
    # asking for them changes nothing else
    plain = oracle.forward_permuted(x, idx, w, W1, W3, W2, sh)
    for key in ("y", "h", "Y", "perm", "inv"):
        np.testing.assert_array_equal(plain[key], r[key])


def test_invalid_ids_contribute_nothing():
    rng = np.random.default_rng(13)
    x, idx, w, W1, W3, W2, _ = _rand_problem(rng, 10, 8, 8, 3, 2)
    bad = idx.copy()
    bad[2, 1] = 7
    bad[5, 0] = -3
    r = oracle.forward_permuted(x, bad, w, W1, W3, W2)
    assert r["bad"] == 2
    keep_w = w.copy()
    keep_w[2, 1] = 0.0
    keep_w[5, 0] = 0.0
    fixed = bad.copy()
    fixed[2, 1] = 0
    fixed[5, 0] = 0
    ref = brute.moe_forward(x, fixed, keep_w, W1, W3, W2)
    np.testing.assert_allclose(r["y"], ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(oracle.forward_dense(x, bad, w, W1, W3, W2), r["y"])


def test_page_figures_pin_flop_and_byte_accounting(golden_dir):
    fig = json.load(open(os.path.join(golden_dir, "page_figures.json")))
    f = fig["w1w3_gflop_per_layer_step"]
    wl = f["workload"]
    total = oracle.flops(wl["T"], wl["D"], wl["F"], wl["k"], wl["shared"])
    w1w3 = total * fig["w1w3_share_of_expert_flops"]["value"]
    assert abs(w1w3 / 1e9 - f["value"]) <= f["rel_tol"] * f["value"]
    b = fig["expert_weight_bytes_bf16"]
    assert round(b["shape"][0] * b["shape"][1] * b["bytes_per_element"] / 1e6, 2) == b["value_mb"]
    a = fig["activation_traffic_saved_mib_per_layer"]
    assert a["slots"] * a["d_ff"] * a["bytes_per_element"] * a["streams_saved"] / 2**20 == a["value"]
    # the workload table and the oracle agree on the FLOP formula
    for wk in moe_inputs.WORKLOADS:
        assert wk.flops() == oracle.flops(wk.T, wk.D, wk.F, wk.k, wk.shared)


# ---------------------------------------------------------------- inputs

def test_inputs_are_seeded_and_shaped():
    a = moe_inputs.make_inputs(0)
    b = moe_inputs.make_inputs(0)
    assert moe_inputs.input_digest(a) == moe_inputs.input_digest(b)
    w = moe_inputs.WORKLOADS[0]
    assert a["x"].shape == (w.T, w.D) and a["W1"].shape == (w.E, w.D, w.F)
    assert a["W2"].shape == (w.E, w.F, w.D) and a["topk_idx"].shape == (w.T, w.k)
    for row in a["topk_idx"]:
        assert len(set(row.tolist())) == w.k                     # distinct experts per token
    np.testing.assert_allclose(a["topk_w"].sum(1), 1.0, rtol=1e-6)
    c = moe_inputs.make_inputs(3)                                 # bf16 workload
    assert c["x_bits"].dtype == np.uint16
    np.testing.assert_array_equal(moe_inputs.bf16_bits_to_f32(c["x_bits"]), c["x"])


def test_bf16_rounding_is_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 1.0 + 2**-8 + 2**-20],
                    np.float32)
    got = moe_inputs.bf16_bits_to_f32(moe_inputs.f32_to_bf16_bits(vals))
    np.testing.assert_array_equal(got, np.array([1.0, 1.0, 1.0 + 4 * 2**-8, 1.0, -2.5, 1.0 + 2**-7],
                                                np.float32))


def test_zipf_routing_is_skewed_toward_low_ids():
    inp = moe_inputs.make_inputs(2, T=8192)
    counts = np.bincount(inp["topk_idx"].reshape(-1), minlength=8)
    assert np.all(np.diff(counts) < 0)           # p_e ~ (e+1)^-1.2 sampled without replacement
    assert counts.sum() == 2 * 8192


# ---------------------------------------------------------------- router

def test_router_matches_textbook_topk_and_softmax():
    rng = np.random.default_rng(17)
    x = rng.standard_normal((50, 12))
    gw = rng.standard_normal((12, 7))
    idx, w, logits = brute.router(x, gw, 3)
    # logits: plain matrix product, computed independently
    np.testing.assert_allclose(logits, np.einsum("td,de->te", x, gw), rtol=1e-13, atol=1e-13)
    # top-k: numpy's stable argsort of the negated logits
    ref = np.argsort(-logits, axis=1, kind="stable")[:, :3]
    np.testing.assert_array_equal(idx, ref)
    # weights: positive, sum to one, ordered like the logits, invariant to a shift of the logits
    assert np.all(w > 0) and np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)
    # a constant added to every logit (a ones column in x, a constant row in gate_w)
    xs = np.concatenate([x, np.ones((50, 1))], axis=1)
    gs = np.concatenate([gw, np.full((1, 7), 3.25)], axis=0)
    idx2, w_shift, _ = brute.router(xs, gs, 3)
    np.testing.assert_array_equal(idx2, idx)
    np.testing.assert_allclose(w_shift, w, rtol=1e-13)
    # closed form for k = 2: w0 = sigmoid(l0 - l1)
    i2, w2, lg = brute.router(x, gw, 2)
    l0 = np.take_along_axis(lg, i2[:, :1].astype(np.int64), 1)[:, 0]
    l1 = np.take_along_axis(lg, i2[:, 1:].astype(np.int64), 1)[:, 0]
    np.testing.assert_allclose(w2[:, 0], 1 / (1 + np.exp(-(l0 - l1))), rtol=1e-14)


def test_router_ties_take_the_lower_expert():
    x = np.ones((3, 2))
    gw = np.array([[1.0, 2.0, 2.0, 0.5], [0.0, 0.0, 0.0, 0.0]])   # logits [1, 2, 2, 0.5]
    idx, w, _ = brute.router(x, gw, 2)
    np.testing.assert_array_equal(idx, [[1, 2]] * 3)
    np.testing.assert_allclose(w, 0.5)
