"""Helpers for the GPU parity tests: move seeded inputs to the device and
apply the output tolerances.

Tolerances (float outputs): bf16 max|y - y_ref| <= 1e-2 * max|y_ref| + 1e-3,
fp32 max|y - y_ref| <= 1e-5 * max|y_ref|; y_ref is the fp64 oracle.
"""
import os
import sys

import numpy as np
import torch

import moe_inputs

BF16_RTOL, BF16_ATOL = 1e-2, 1e-3
F32_RTOL = 1e-5


def oracle_threads():
    """Threads for the CPU oracle: the host cores this process may use,
    capped at 16 (a one-GPU machine's share of its host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def say(msg):
    """Name the case before touching the GPU, flushed."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(inp, name, dtype):
    if dtype == "bf16":
        return torch.from_numpy(inp[name + "_bits"].view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(inp[name], np.float32)).cuda()


def device_inputs(inp):
    w = inp["workload"]
    d = {n: dev(inp, n, w.dtype) for n in ("x", "W1", "W3", "W2")}
    d["shared"] = tuple(dev(inp, n, w.dtype) for n in ("Ws1", "Ws3", "Ws2")) if w.shared else None
    d["topk_idx"] = torch.from_numpy(inp["topk_idx"]).cuda()
    d["topk_w"] = torch.from_numpy(inp["topk_w"]).cuda()
    return d


def host_shared(inp):
    return (inp["Ws1"], inp["Ws3"], inp["Ws2"]) if "Ws1" in inp else None


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_close(got, ref, dtype, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref).max() if ref.size else 0.0
    scale = np.abs(ref).max() if ref.size else 0.0
    bound = BF16_RTOL * scale + BF16_ATOL if dtype == "bf16" else F32_RTOL * scale
    assert err <= bound, f"{what}: max|err| {err:.3e} > bound {bound:.3e} (max|ref| {scale:.3e})"
    return err, bound


def make_case(T, D, F, E, k, shared, dtype="bf16", routing="uniform", seed=7):
    w = moe_inputs.Workload(f"case_T{T}_D{D}_F{F}_E{E}_k{k}", T, D, F, E, k, shared, dtype, routing)
    return moe_inputs.make_inputs(w, seed=seed)
