"""The oracle's pins must catch plausible mistakes.

Each case below plants one mistake in a copy of oracle/moe_oracle.c (on the
CPU, in a temporary directory), builds it, and checks that at least one of
the pins from test_oracle.py's families fails against the mutant: numpy's
stable counting sort, the numpy brute force, the closed-form fixtures and
the dense/permuted agreement.
"""
import json
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import brute

SRC = open(os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")).read()

MUTANTS = {
    "swap_w1_w3": ("g[f] += xd * w1[f];\n            u[f] += xd * w3[f];",
                   "g[f] += xd * w3[f];\n            u[f] += xd * w1[f];"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "drop_up_product": ("h[f] = silu(g[f]) * u[f];", "h[f] = silu(g[f]);"),
    "w2_transposed": ("out[d] += hf * w2[d];", "out[d] += hf * W2[d * F + f];"),
    "token_index_mod": ("t = J->perm[p] / J->k;", "t = J->perm[p] % J->k;"),
    "combine_drops_weight": ("yr[d] = yr[d] + wt * Y_out[(int64_t)p * D + d];",
                             "yr[d] = yr[d] + Y_out[(int64_t)p * D + d];"),
    "unstable_sort": ("for (int64_t s = 0; s < S; ++s)\n            if (idx[s] == e) {",
                      "for (int64_t s = S - 1; s >= 0; --s)\n            if (idx[s] == e) {"),
    "dense_drops_shared": ("for (int64_t d = 0; d < D; ++d) yr[d] = o[d];",
                           "for (int64_t d = 0; d < D; ++d) yr[d] = 0.0;"),
    "tile_round_down": ("(counts[e] + BM - 1) / BM", "(counts[e]) / BM"),
    "offsets_off_by_one": ("offsets[e + 1] = offsets[e] + counts[e];",
                           "offsets[e + 1] = offsets[e] + counts[e] + (e == 0);"),
    "gu_columns_swapped": ("r[f] = g[f]; r[F + f] = u[f];", "r[f] = u[f]; r[F + f] = g[f];"),
    "gu_row_stride": ("double *r = J->gu_out + p * 2 * F;", "double *r = J->gu_out + p * F;"),
}


def _pins_pass(golden_dir) -> bool:
    """Run a compact set of pins against whatever library oracle._lib holds."""
    rng = np.random.default_rng(1)
    try:
        # counting sort against numpy
        idx = rng.integers(0, 5, (50, 2)).astype(np.int32)
        r = oracle.permute(idx, 6, tile_rows=4, shared_rows=50)
        flat = idx.reshape(-1)
        cnt = np.bincount(flat, minlength=6)
        if not (np.array_equal(r["counts"], cnt)
                and np.array_equal(r["offsets"], np.concatenate([[0], np.cumsum(cnt)]))
                and np.array_equal(r["perm"], np.argsort(flat, kind="stable"))
                and np.array_equal(r["tile_off"],
                                   np.concatenate([[0], np.cumsum(np.append(-(-cnt // 4), 13))]))):
            return False
        # brute force, with and without a shared expert, both oracle paths
        T, D, F, E, k = 9, 6, 10, 4, 2
        x = rng.standard_normal((T, D))
        W1, W3 = rng.standard_normal((E, D, F)), rng.standard_normal((E, D, F))
        W2 = rng.standard_normal((E, F, D))
        sh = (rng.standard_normal((D, F)), rng.standard_normal((D, F)), rng.standard_normal((F, D)))
        tidx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
        w = rng.random((T, k))
        for s in (None, sh):
            ref = brute.moe_forward(x, tidx, w, W1, W3, W2, s)
            for y in (oracle.forward_dense(x, tidx, w, W1, W3, W2, s),
                      oracle.forward_permuted(x, tidx, w, W1, W3, W2, s)["y"]):
                if not np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max()):
                    return False
        # the sorted rows' gate and up products against numpy's
        r = oracle.forward_permuted(x, tidx, w, W1, W3, W2, sh, with_gu=True)
        for p in range(T * k + T):
            if p < T * k:
                sl = r["perm"][p]
                v, A1, A3 = x[sl // k], W1[tidx.reshape(-1)[sl]], W3[tidx.reshape(-1)[sl]]
            else:
                v, A1, A3 = x[p - T * k], sh[0], sh[1]
            if not (np.allclose(r["gu"][p, :F], v @ A1, rtol=1e-12, atol=1e-12)
                    and np.allclose(r["gu"][p, F:], v @ A3, rtol=1e-12, atol=1e-12)):
                return False
        # closed forms
        cases = json.load(open(os.path.join(golden_dir, "closed_form_cases.json")))["cases"]
        for c in cases:
            a = {n: np.array(c[n], np.float64) for n in ("x", "W1", "W3", "W2", "topk_w")}
            s = tuple(np.array(v, np.float64) for v in c["shared"]) if "shared" in c else None
            y = oracle.forward_dense(a["x"], np.array(c["topk_idx"], np.int32), a["topk_w"],
                                     a["W1"], a["W3"], a["W2"], s)
            if not np.allclose(y, np.array(c["y"]), rtol=0, atol=1e-15):
                return False
    except Exception:
        return False
    return True


def test_unmutated_oracle_passes_the_compact_pins(golden_dir):
    assert _pins_pass(golden_dir)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path, golden_dir, monkeypatch):
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
        caught = not _pins_pass(golden_dir)
    finally:
        oracle._lib = saved
    assert caught, f"no pin failed for planted mistake {name}"
