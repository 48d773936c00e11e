"""Pins for the oracle's backward (oracle.backward) on the CPU.

The backward is checked against things that do not share its derivation:

* central finite differences of the forward oracle's scalar loss
  L = sum(dy * y), on sampled coordinates of every input (x, all weights,
  the routing weights);
* torch's float64 autograd on a plain torch forward expression of the layer
  (the derivative rules come from the library, not from the oracle's
  formulas);
* identities that tie it to the forward: the routing weights' gradient is
  dy[t] . (unweighted expert output), the gradient is linear in dy, a zero
  routing weight leaves that slot's weight gradients at zero, and a token's
  dx does not depend on any other token.

The mutant tests plant plausible mistakes in copies of the backward and
check that these pins catch each one.
"""
import math
import os
import subprocess

import numpy as np
import pytest

import oracle

SRC = open(os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")).read()


def _problem(rng, T, D, F, E, k, shared=True, distinct=True):
    x = rng.standard_normal((T, D))
    W1 = rng.standard_normal((E, D, F)) / math.sqrt(D)
    W3 = rng.standard_normal((E, D, F)) / math.sqrt(D)
    W2 = rng.standard_normal((E, F, D)) / math.sqrt(F)
    if distinct:
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    else:
        idx = rng.integers(0, E, (T, k)).astype(np.int32)
    w = rng.random((T, k)) + 0.1
    sh = None
    if shared:
        sh = (rng.standard_normal((D, F)) / math.sqrt(D), rng.standard_normal((D, F)) / math.sqrt(D),
              rng.standard_normal((F, D)) / math.sqrt(F))
    dy = rng.standard_normal((T, D))
    return dict(x=x, idx=idx, w=w, W1=W1, W3=W3, W2=W2, sh=sh, dy=dy)


def _loss(p):
    y = oracle.forward_dense(p["x"], p["idx"], p["w"], p["W1"], p["W3"], p["W2"], p["sh"])
    return float(np.sum(p["dy"] * y))


def _grads(p):
    return oracle.backward(p["x"], p["idx"], p["w"], p["W1"], p["W3"], p["W2"], p["sh"], p["dy"])


def _fd_check(p, g, rng, n=6, h=1e-5, rtol=1e-6):
    """Central differences on n random coordinates of every differentiable
    input; returns the worst relative disagreement."""
    worst = 0.0
    targets = [("x", "dx"), ("W1", "dW1"), ("W3", "dW3"), ("W2", "dW2"), ("w", "dw")]
    if p["sh"] is not None:
        targets += [(("sh", 0), "dWs1"), (("sh", 1), "dWs3"), (("sh", 2), "dWs2")]
    for src, gname in targets:
        arr = p[src[0]][src[1]] if isinstance(src, tuple) else p[src]
        for _ in range(n):
            i = tuple(int(rng.integers(0, s)) for s in arr.shape)
            old = arr[i]
            arr[i] = old + h
            lp = _loss(p)
            arr[i] = old - h
            lm = _loss(p)
            arr[i] = old
            fd = (lp - lm) / (2 * h)
            an = g[gname][i]
            worst = max(worst, abs(fd - an) / (1.0 + abs(an)))
    return worst


@pytest.mark.parametrize("shared,distinct", [(True, True), (False, True), (True, False)])
def test_backward_matches_finite_differences(shared, distinct):
    rng = np.random.default_rng(7 + shared + 2 * distinct)
    p = _problem(rng, 7, 5, 6, 3, 2, shared=shared, distinct=distinct)
    g = _grads(p)
    assert _fd_check(p, g, rng) < 1e-6


def _torch_grads(p):
    torch = pytest.importorskip("torch")
    t = {n: torch.tensor(p[n], dtype=torch.float64, requires_grad=True)
         for n in ("x", "w", "W1", "W3", "W2")}
    sh = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in p["sh"]] if p["sh"] else None
    idx = torch.tensor(p["idx"], dtype=torch.int64)

    def expert(v, a1, a3, a2):
        return (torch.nn.functional.silu(v @ a1) * (v @ a3)) @ a2

    T, k = p["idx"].shape
    y = expert(t["x"], *sh) if sh else torch.zeros_like(t["x"])
    for j in range(k):
        e = idx[:, j]
        a1, a3, a2 = t["W1"][e], t["W3"][e], t["W2"][e]        # per token: [T, D, F], [T, F, D]
        xv = t["x"][:, None, :]
        hh = torch.nn.functional.silu(torch.bmm(xv, a1)) * torch.bmm(xv, a3)
        y = y + t["w"][:, j:j + 1] * torch.bmm(hh, a2)[:, 0, :]
    loss = (torch.tensor(p["dy"]) * y).sum()
    inputs = [t["x"], t["w"], t["W1"], t["W3"], t["W2"]] + (sh or [])
    gr = torch.autograd.grad(loss, inputs)
    names = ["dx", "dw", "dW1", "dW3", "dW2"] + (["dWs1", "dWs3", "dWs2"] if sh else [])
    return {n: v.numpy() for n, v in zip(names, gr)}


@pytest.mark.parametrize("shared", [True, False])
def test_backward_matches_torch_autograd(shared):
    rng = np.random.default_rng(11 + shared)
    p = _problem(rng, 40, 16, 24, 5, 2, shared=shared)
    g = _grads(p)
    ref = _torch_grads(p)
    for n, r in ref.items():
        np.testing.assert_allclose(g[n], r, rtol=1e-10, atol=1e-12 * max(1.0, np.abs(r).max()),
                                   err_msg=n)


def test_routing_weight_gradient_is_dy_dot_expert_output():
    rng = np.random.default_rng(3)
    p = _problem(rng, 20, 8, 12, 4, 2)
    g = _grads(p)
    fp = oracle.forward_permuted(p["x"], p["idx"], p["w"], p["W1"], p["W3"], p["W2"], p["sh"])
    inv = fp["inv"].reshape(20, 2)
    for t in range(20):
        for j in range(2):
            o = fp["Y"][inv[t, j]]             # unweighted expert output of slot (t, j)
            assert abs(g["dw"][t, j] - float(p["dy"][t] @ o)) < 1e-12 * (1 + abs(g["dw"][t, j]))


def test_backward_is_linear_in_dy_and_local_in_tokens():
    rng = np.random.default_rng(4)
    p = _problem(rng, 12, 6, 10, 4, 2)
    g = _grads(p)
    q = dict(p, dy=2.5 * p["dy"])
    g2 = _grads(q)
    for n in ("dx", "dW1", "dW3", "dW2", "dw", "dWs1", "dWs3", "dWs2"):
        np.testing.assert_allclose(g2[n], 2.5 * g[n], rtol=1e-12, atol=1e-14, err_msg=n)
    # dy zero on all but token 5: only token 5's dx row and dw row can be non-zero
    dy = np.zeros_like(p["dy"])
    dy[5] = p["dy"][5]
    g3 = _grads(dict(p, dy=dy))
    others = np.arange(12) != 5
    assert np.all(g3["dx"][others] == 0.0) and np.all(g3["dw"][others] == 0.0)
    np.testing.assert_allclose(g3["dx"][5], g["dx"][5], rtol=0, atol=0)


def test_zero_routing_weight_contributes_no_weight_gradient():
    rng = np.random.default_rng(5)
    p = _problem(rng, 10, 6, 8, 4, 1, shared=False)
    p["idx"][:] = 2
    p["w"][:] = 0.0
    g = _grads(p)
    assert np.all(g["dW1"] == 0) and np.all(g["dW3"] == 0) and np.all(g["dW2"] == 0)
    assert np.all(g["dx"] == 0)
    # ... but the routing weights still get dy . o
    assert np.any(g["dw"] != 0)


def test_invalid_ids_contribute_nothing():
    rng = np.random.default_rng(6)
    p = _problem(rng, 9, 5, 7, 3, 2)
    q = {n: (v.copy() if isinstance(v, np.ndarray) else v) for n, v in p.items()}
    q["idx"][2, 1] = 3          # out of range
    q["idx"][4, 0] = -1
    g = _grads(q)
    assert g["dw"][2, 1] == 0.0 and g["dw"][4, 0] == 0.0
    # same as a zero routing weight on those slots with any valid id
    r = {n: (v.copy() if isinstance(v, np.ndarray) else v) for n, v in p.items()}
    r["w"][2, 1] = 0.0
    r["w"][4, 0] = 0.0
    gr = _grads(r)
    for n in ("dx", "dW1", "dW3", "dW2", "dWs1", "dWs3", "dWs2"):
        np.testing.assert_allclose(g[n], gr[n], rtol=1e-13, atol=1e-15, err_msg=n)


# ------------------------------------------------------------------ mutants

MUTANTS = {
    "dsilu_drops_term": ("return s * (1.0 + z * (1.0 - s));", "return s;"),
    "dh_drops_weight": ("acc += w2[d] * (wt * dyr[d]);", "acc += w2[d] * dyr[d];"),
    "dh_w2_transposed": ("const double *w2 = W2 + f * D;\n        double acc = 0.0;",
                         "const double *w2 = W2 + f;\n        double acc = 0.0;"),
    "swap_dg_du": ("dg[f] = dh[f] * u[f] * dsilu(g[f]);\n        du[f] = dh[f] * silu(g[f]);",
                   "du[f] = dh[f] * u[f] * dsilu(g[f]);\n        dg[f] = dh[f] * silu(g[f]);"),
    "dx_drops_w3": ("dx_acc[d] = dx_acc[d] + a1 + a3;", "dx_acc[d] = dx_acc[d] + a1;"),
    "dw2_uses_g": ("dW2[f * D + d] += h[f] * (wt * dyr[d]);", "dW2[f * D + d] += g[f] * (wt * dyr[d]);"),
    "dx_misses_shared": ("if (J->Ws1)\n            swiglu_row_backward(xr, dyr, 1.0,",
                         "if (0)\n            swiglu_row_backward(xr, dyr, 1.0,"),
    "dw1_wrong_token": ("swiglu_row_backward(J->x + t * D, J->dy + t * D,",
                        "swiglu_row_backward(J->x + ((t + 1) % J->T) * D, J->dy + t * D,"),
}


def _backward_pins_pass():
    rng = np.random.default_rng(21)
    try:
        p = _problem(rng, 6, 4, 5, 3, 2, shared=True)
        if _fd_check(p, _grads(p), rng, n=4) >= 1e-6:
            return False
        p = _problem(rng, 6, 4, 5, 3, 2, shared=False, distinct=False)
        if _fd_check(p, _grads(p), rng, n=4) >= 1e-6:
            return False
    except Exception:
        return False
    return True


def test_unmutated_backward_passes_the_compact_pins():
    assert _backward_pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_backward_mistake_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation anchor for {name} not unique in moe_oracle.c"
    src = tmp_path / "mutant.c"
    src.write_text(SRC.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-pthread",
                           "-std=c11", str(src), "-o", str(lib), "-lm"])
    saved = oracle._lib
    oracle._lib = None
    monkeypatch.setattr(oracle, "_LIB_PATH", str(lib))
    try:
        caught = not _backward_pins_pass()
    finally:
        oracle._lib = saved
    assert caught, f"no pin failed for planted mistake {name}"


def test_group_subset_matches_full_backward():
    rng = np.random.default_rng(8)
    p = _problem(rng, 30, 6, 8, 5, 2, shared=True)
    g = _grads(p)
    sub = oracle.backward_weight_grads(p["x"], p["idx"], p["w"], p["W1"], p["W3"], p["W2"], p["sh"],
                                       p["dy"], [3, 5, 0])
    for e in (0, 3):
        for got, ref in zip(sub[e], (g["dW1"][e], g["dW3"][e], g["dW2"][e])):
            np.testing.assert_array_equal(got, ref)
    for got, ref in zip(sub[5], (g["dWs1"], g["dWs3"], g["dWs2"])):
        np.testing.assert_array_equal(got, ref)
