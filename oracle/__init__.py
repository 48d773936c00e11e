"""CPU oracle for the top-k routed MoE SwiGLU FFN, forward and backward (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP path
(``grouped_gemm_permute_amd``) and never imports it; both are fed by
``moe_inputs``.

Two independent evaluations are offered:

* ``moe_oracle.c`` (through ctypes): fp64 loops.  ``forward_dense`` is the
  brute force over every (token, choice); ``forward_permuted`` takes the
  pages' order (counting sort, per-expert loop over sorted rows, unpermute,
  combine in j order) and also returns the sorted-row intermediates h and Y.
  ``permute`` is the stable counting sort with per-expert counts, offsets and
  row-tile offsets.  ``backward`` is the vector-Jacobian product of the
  layer (dx, the weight gradients and the routing weights' gradient) by the
  chain rule on the recomputed forward (Part A section 8 of the first page).
* ``brute.py``: a separate numpy fp64 brute force for tiny inputs.

Definitions followed are cited in ``moe_oracle.c`` ("Triton MoE Kernels &
Memory Checkpointing", Part A sections 2, 10.2, 10.3; "Chinchilla scaling,
MoE, and fused Triton kernels", section "PyTorch MoE implementation").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-pthread",
                               "-std=c11", "-Wall", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        ci = ctypes.c_int
        lib.moe_oracle_permute.restype = i64
        lib.moe_oracle_permute.argtypes = [P, i64, ci, ci, i64, P, P, P, P, P]
        lib.moe_oracle_forward_dense.restype = ci
        lib.moe_oracle_forward_dense.argtypes = [P, P, P, P, P, P, P, P, P, i64, i64, i64, ci, ci,
                                                 P, i64, P, ci]
        lib.moe_oracle_backward.restype = ci
        lib.moe_oracle_backward.argtypes = [P] * 10 + [i64, i64, i64, ci, ci] + [P] * 8 + [ci]
        lib.moe_oracle_backward_groups.restype = ci
        lib.moe_oracle_backward_groups.argtypes = [P] * 10 + [i64, i64, i64, ci, ci, P, ci] + [P] * 6 + [ci]
        lib.moe_oracle_forward_permuted.restype = i64
        lib.moe_oracle_forward_permuted.argtypes = [P, P, P, P, P, P, P, P, P, i64, i64, i64, ci,
                                                    ci, P, P, P, P, P, P, P, P, ci]
        _lib = lib
    return _lib


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data


def permute(topk_idx: np.ndarray, E: int, tile_rows: int = 1, shared_rows: int = 0) -> dict:
    """Stable counting sort of slots s = t*k + j by expert id.

    Returns counts [E], offsets [E+1], tile_off [E+2], perm [S], inv [S]
    (int32) and ``bad``, the number of slots whose id is outside [0, E)."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32).reshape(-1)
    S = idx.size
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    tile_off = np.empty(E + 2, np.int32)
    perm = np.empty(max(S, 1), np.int32)
    inv = np.empty(max(S, 1), np.int32)
    bad = _load().moe_oracle_permute(_ptr(idx), S, E, tile_rows, shared_rows, _ptr(counts),
                                     _ptr(offsets), _ptr(tile_off), _ptr(perm), _ptr(inv))
    return dict(counts=counts, offsets=offsets, tile_off=tile_off, perm=perm[:S], inv=inv[:S],
                bad=int(bad))


def _shared(shared):
    if shared is None:
        return None, None, None
    return tuple(_f64(a) for a in shared)


def forward_dense(x, topk_idx, topk_w, W1, W3, W2, shared=None, tokens=None, nthreads=1):
    """Path (i): y rows for ``tokens`` (all tokens when None), fp64."""
    x = _f64(x)
    T, D = x.shape
    E, _, F = W1.shape
    k = topk_idx.shape[1]
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    w = _f64(topk_w)
    W1, W3, W2 = _f64(W1), _f64(W3), _f64(W2)
    Ws1, Ws3, Ws2 = _shared(shared)
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
    n = T if tok is None else tok.size
    y = np.empty((n, D), np.float64)
    rc = _load().moe_oracle_forward_dense(_ptr(x), _ptr(idx), _ptr(w), _ptr(W1), _ptr(W3),
                                          _ptr(W2), _ptr(Ws1), _ptr(Ws3), _ptr(Ws2), T, D, F, E,
                                          k, _ptr(tok), n, _ptr(y), nthreads)
    if rc != 0:
        raise MemoryError("oracle allocation failed")
    return y


def forward_permuted(x, topk_idx, topk_w, W1, W3, W2, shared=None, nthreads=1,
                     with_gu=False) -> dict:
    """Path (ii): returns y [T,D], the sorted-row intermediates h [R,F] and
    Y [R,D] (R = T*k plus T shared rows), and counts/offsets/perm/inv; with
    with_gu also gu [R, 2F], each row's gate product g = v W1 (columns
    0..F-1) and up product u = v W3 (columns F..2F-1)."""
    x = _f64(x)
    T, D = x.shape
    E, _, F = W1.shape
    k = topk_idx.shape[1]
    S = T * k
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    w = _f64(topk_w)
    W1, W3, W2 = _f64(W1), _f64(W3), _f64(W2)
    Ws1, Ws3, Ws2 = _shared(shared)
    R = S + (T if Ws1 is not None else 0)
    y = np.empty((T, D), np.float64)
    h = np.empty((max(R, 1), F), np.float64)
    Y = np.empty((max(R, 1), D), np.float64)
    gu = np.empty((max(R, 1), 2 * F), np.float64) if with_gu else None
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(max(S, 1), np.int32)
    inv = np.empty(max(S, 1), np.int32)
    bad = _load().moe_oracle_forward_permuted(
        _ptr(x), _ptr(idx), _ptr(w), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(Ws1), _ptr(Ws3),
        _ptr(Ws2), T, D, F, E, k, _ptr(y), _ptr(h), _ptr(Y), _ptr(gu), _ptr(counts),
        _ptr(offsets), _ptr(perm), _ptr(inv), nthreads)
    if bad < 0:
        raise MemoryError("oracle allocation failed")
    out = dict(y=y, h=h[:R], Y=Y[:R], counts=counts, offsets=offsets, perm=perm[:S],
               inv=inv[:S], bad=int(bad))
    if with_gu:
        out["gu"] = gu[:R]
    return out


def backward(x, topk_idx, topk_w, W1, W3, W2, shared, dy, nthreads=1) -> dict:
    """Vector-Jacobian product of the layer for the incoming gradient dy
    [T,D], fp64: dx [T,D], dW1/dW3 [E,D,F], dW2 [E,F,D], dw [T,k] (the
    routing weights' gradient, 0 for invalid slots) and, with a shared
    expert, dWs1/dWs3 [D,F] and dWs2 [F,D] (else None)."""
    x = _f64(x)
    T, D = x.shape
    E, _, F = W1.shape
    k = topk_idx.shape[1]
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    w = _f64(topk_w)
    W1, W3, W2 = _f64(W1), _f64(W3), _f64(W2)
    Ws1, Ws3, Ws2 = _shared(shared)
    dy = _f64(dy)
    out = dict(dx=np.empty((T, D)), dW1=np.empty((E, D, F)), dW3=np.empty((E, D, F)),
               dW2=np.empty((E, F, D)), dw=np.empty((T, k)))
    sh = Ws1 is not None
    out.update(dWs1=np.empty((D, F)) if sh else None, dWs3=np.empty((D, F)) if sh else None,
               dWs2=np.empty((F, D)) if sh else None)
    rc = _load().moe_oracle_backward(
        _ptr(x), _ptr(idx), _ptr(w), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(Ws1), _ptr(Ws3),
        _ptr(Ws2), _ptr(dy), T, D, F, E, k, _ptr(out["dx"]), _ptr(out["dW1"]), _ptr(out["dW3"]),
        _ptr(out["dW2"]), _ptr(out["dWs1"]), _ptr(out["dWs3"]), _ptr(out["dWs2"]),
        _ptr(out["dw"]), nthreads)
    if rc != 0:
        raise MemoryError("oracle allocation failed")
    return out


def backward_weight_grads(x, topk_idx, topk_w, W1, W3, W2, shared, dy, groups, nthreads=1) -> dict:
    """The weight gradients of the listed groups only (0..E-1 routed, E the
    shared expert), fp64, computed as ``backward`` does: {group: (dW1, dW3,
    dW2)}."""
    x = _f64(x)
    T, D = x.shape
    E, _, F = W1.shape
    k = topk_idx.shape[1]
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    w = _f64(topk_w)
    W1, W3, W2 = _f64(W1), _f64(W3), _f64(W2)
    Ws1, Ws3, Ws2 = _shared(shared)
    dy = _f64(dy)
    g = np.ascontiguousarray(groups, dtype=np.int32)
    dW1, dW3, dW2 = np.zeros((E, D, F)), np.zeros((E, D, F)), np.zeros((E, F, D))
    sh = Ws1 is not None
    dWs = (np.zeros((D, F)), np.zeros((D, F)), np.zeros((F, D))) if sh else (None, None, None)
    rc = _load().moe_oracle_backward_groups(
        _ptr(x), _ptr(idx), _ptr(w), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(Ws1), _ptr(Ws3), _ptr(Ws2),
        _ptr(dy), T, D, F, E, k, _ptr(g), g.size, _ptr(dW1), _ptr(dW3), _ptr(dW2), _ptr(dWs[0]),
        _ptr(dWs[1]), _ptr(dWs[2]), nthreads)
    if rc != 0:
        raise MemoryError("oracle allocation failed")
    return {int(e): ((dW1[e], dW3[e], dW2[e]) if e < E else dWs) for e in g}


def backward_flops(T: int, D: int, F: int, k: int, shared: bool) -> int:
    """Algorithmic FLOPs of one backward with the gate and up products
    recomputed: per row, the two recomputed up products (4 D F), the
    gradient of h through W2 (2 D F), the W2 gradient (2 D F), the two W1/W3
    gradients (4 D F) and dx through W1 and W3 (4 D F): 16 D F."""
    return 16 * D * F * (T * k + (T if shared else 0))


def flops(T: int, D: int, F: int, k: int, shared: bool) -> int:
    """Algorithmic FLOPs of one forward: 2 per multiply-add of the three
    GEMMs (W1, W3: D x F each; W2: F x D) for every routed slot and, with a
    shared expert, every token once more."""
    return 6 * D * F * (T * k + (T if shared else 0))
