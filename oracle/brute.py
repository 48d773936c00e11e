"""Independent numpy fp64 brute force for tiny inputs (test infrastructure).

Written separately from ``moe_oracle.c``: a Python loop over tokens and
their k choices, each expert evaluated with numpy matrix products, no
permutation at all.  Follows the SwiGLU expert W2(silu(W1 x) * W3 x) of
"Triton MoE Kernels & Memory Checkpointing" (Part A, section 2) and the
weighted sum over a token's k experts of "Chinchilla scaling, MoE, and fused
Triton kernels" (section "PyTorch MoE implementation").
"""
from __future__ import annotations

import numpy as np


def silu(z):
    return z / (1.0 + np.exp(-z))


def expert(v, W1, W3, W2):
    """SwiGLU expert on row vector(s) v; weights [D,F], [D,F], [F,D]."""
    return (silu(v @ W1) * (v @ W3)) @ W2


def moe_forward(x, topk_idx, topk_w, W1, W3, W2, shared=None):
    x = np.asarray(x, np.float64)
    T, D = x.shape
    k = topk_idx.shape[1]
    W1, W3, W2 = (np.asarray(a, np.float64) for a in (W1, W3, W2))
    y = np.zeros((T, D))
    for t in range(T):
        acc = np.zeros(D)
        if shared is not None:
            acc = acc + expert(x[t], *(np.asarray(a, np.float64) for a in shared))
        for j in range(k):
            e = int(topk_idx[t, j])
            acc = acc + float(topk_w[t, j]) * expert(x[t], W1[e], W3[e], W2[e])
        y[t] = acc
    return y


def router(x, gate_w, k):
    """Top-k routing of "Chinchilla scaling, MoE, and fused Triton kernels"
    (section "PyTorch MoE implementation"): logits = x @ gate_w, the k largest
    logits of each token in descending order, routing weights = softmax over
    those k logits.  fp64 throughout.  Equal logits are taken in ascending
    expert order (the page leaves ties to torch.topk; this is the reading).
    Returns (topk_idx int32 [T,k], topk_w float64 [T,k], logits [T,E])."""
    x = np.asarray(x, np.float64)
    logits = x @ np.asarray(gate_w, np.float64)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))
        idx[t] = order[:k]
    sel = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return idx, z / z.sum(axis=1, keepdims=True), logits
