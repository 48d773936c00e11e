#!/usr/bin/env python
"""Benchmark of the MoE SwiGLU FFN forward on one MI355X.

One step = one moe_ffn_forward call (permute, up+SwiGLU grouped GEMM, down
grouped GEMM, combine) over one batch of seeded synthetic input already
resident in HBM.  The default workload is the full-step layer: T = 32768
tokens (8 x 4096), d_model 768, d_ff 1536, 8 routed experts top-2 with
Zipf(1.2)-skewed routing, plus a shared expert, bf16 storage with fp32
accumulation.  Inputs and weights are rotated over enough copies that the
working set exceeds the on-die caches (MALL + L2), so each step streams from
HBM.

Prints one JSON line:
  value       whole-forward TFLOP/s (algorithmic FLOPs 6*D*F*(T*k + T) / time)
  roofline    the dominant kernel's achieved rate vs the MI355X peak, from
              HIP events recorded between the kernels on their stream during
              the timed loop (traffic: HBM bytes from rocprofv3 counters,
              when a counter summary for the current kernel source exists)
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE FFN fwd TFLOP/s + % bf16 MFMA peak, 32k tok D768 F1536 E8 top-2"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
STAGES = ("permute", "up_swiglu", "down", "combine")
BWD_METRIC = "MoE FFN bwd TFLOP/s (gate/up recomputed), 32k tok D768 F1536 E8 top-2"
BWD_STAGES = ("permute", "transpose", "gate_up", "dh", "dx_rows", "dw13", "dw2", "reduce_dtopk_combine")
KERNEL_SOURCES = {             # the source each stage's kernel is built from
    "permute": "grouped_gemm_permute_amd/csrc/permute.hip",
    "up_swiglu": "grouped_gemm_permute_amd/csrc/gemm_bf16.hip",
    "down": "grouped_gemm_permute_amd/csrc/gemm_bf16.hip",
    "combine": "grouped_gemm_permute_amd/csrc/combine.hip",
}
SMALL_SOURCES = {              # groups averaging under 256 rows (small_tiles)
    "up_swiglu": "grouped_gemm_permute_amd/csrc/gemm_bf16_slab.hip",
    "down": "grouped_gemm_permute_amd/csrc/gemm_bf16_small.hip",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(stage: str, variant: str = "unfused", small: bool = False) -> str:
    """Hash of the sources a kernel is built from (stale counters are not used)."""
    h = hashlib.sha256()
    src = SMALL_SOURCES.get(stage, KERNEL_SOURCES[stage]) if small else KERNEL_SOURCES[stage]
    if variant == "fused" and stage == "up_swiglu":
        src = "grouped_gemm_permute_amd/csrc/fused_bf16.hip"
    extra = {"grouped_gemm_permute_amd/csrc/gemm_bf16_slab.hip":     # its sort workgroup
             ("grouped_gemm_permute_amd/csrc/permute_device.h",)}
    for rel in (src, *extra.get(src, ()), "grouped_gemm_permute_amd/csrc/mfma_common.h",
                "grouped_gemm_permute_amd/csrc/moe_internal.h"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch has loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = ev.value
        return arr

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, arr):
        for ev in arr:
            self.hip.hipEventDestroy(ev)


def stage_work(w, counts):
    """Algorithmic FLOPs and compulsory bytes (each operand read once, each
    result written once) of one launch of every stage.  b = 2 (bf16)."""
    b = 2 if w.dtype == "bf16" else 4
    rows = w.T * w.k + (w.T if w.shared else 0)
    groups = int(sum(1 for c in counts if c > 0)) + (1 if w.shared else 0)
    wbytes = w.D * w.F * b
    S = w.T * w.k
    return {
        # topk_idx in; counts, offsets, tile prefixes, perm and inv out
        "permute": {"flop": 0, "bytes": S * 4 * 3 + 4 * (4 * w.E + 6)},
        # x once, [W1|W3] of every active group, h out
        "up_swiglu": {"flop": 4 * w.D * w.F * rows,
                      "bytes": w.T * w.D * b + 2 * wbytes * groups + rows * w.F * b},
        # h, W2 of every active group, Y out (storage dtype)
        "down": {"flop": 2 * w.D * w.F * rows,
                 "bytes": rows * w.F * b + wbytes * groups + rows * w.D * b},
        # Y, inv and routing weights in, y out
        "combine": {"flop": 2 * w.k * w.D * w.T,
                    "bytes": rows * w.D * b + S * 8 + w.T * w.D * b},
    }


def path_bytes(w, counts):
    """Bytes the whole forward must move: x, y, routing, and the three weight
    matrices of every active expert (intermediates excluded)."""
    b = 2 if w.dtype == "bf16" else 4
    groups = int(sum(1 for c in counts if c > 0)) + (1 if w.shared else 0)
    return 2 * w.T * w.D * b + w.T * w.k * 8 + 3 * w.D * w.F * b * groups


def load_traffic(workload_name, key, small=False):
    """Counter-derived HBM bytes per launch ("variant:stage" key), if
    profiles/traffic.json holds a figure taken from the current kernel
    source; otherwise None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(workload_name, {}).get(key)
    except (OSError, ValueError):
        return None
    stage = key.split(":")[-1]
    if not rec or rec.get("source_sha") != source_hash(stage, key.split(":")[0], small):
        return None
    return rec.get("bytes_per_launch")


def host_cpu():
    """The host's core counts and CPU model, and the oracle's thread count:
    the cores this process may run on, capped at 16 (one GPU's share of the
    GPU machine's host)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0))
    return {"threads": max(1, min(16, affinity)), "nproc": os.cpu_count(), "affinity": affinity,
            "cpu_model": model}


def cpu_baseline(inp, w, target_s):
    import numpy as np
    import oracle
    host = host_cpu()
    threads = host["threads"]
    shared = (inp["Ws1"], inp["Ws3"], inp["Ws2"]) if w.shared else None
    W = [np.ascontiguousarray(inp[n], np.float64) for n in ("W1", "W3", "W2")]
    sh = tuple(np.ascontiguousarray(a, np.float64) for a in shared) if shared else None

    def run(n):
        t0 = time.perf_counter()
        oracle.forward_permuted(inp["x"][:n], inp["topk_idx"][:n], inp["topk_w"][:n], *W, sh,
                                nthreads=threads)
        return time.perf_counter() - t0

    n0 = min(w.T, 8 * threads)
    t0 = run(n0)
    n = int(min(w.T, max(n0, target_s / max(t0, 1e-6) * n0)))
    t = run(n)
    flop = 6 * w.D * w.F * (n * w.k + (n if w.shared else 0))
    return {"value": round(flop / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": round(t, 3), "host_nproc": host["nproc"], "host_affinity_cores": host["affinity"],
            "cpu_model": host["cpu_model"],
            "sample": f"first {n} of {w.T} tokens of the same workload (same weights and routing), "
                      f"fp64 permuted oracle path, {threads} threads"}


def bwd_stage_work(w, counts):
    """Algorithmic FLOPs and compulsory bytes of the backward's kernels
    (16 D F FLOP per row in total: the recomputed gate and up products 4, dh
    2, the per-row dx 4, dW1/dW3 4, dW2 2)."""
    b = 2 if w.dtype == "bf16" else 4
    rows = w.T * w.k + (w.T if w.shared else 0)
    groups = int(sum(1 for c in counts if c > 0)) + (1 if w.shared else 0)
    D, F, T = w.D, w.F, w.T
    wb = D * F * b
    return {
        "gate_up": {"flop": 4 * D * F * rows, "bytes": T * D * b + 2 * wb * groups + rows * 2 * F * b},
        "dh": {"flop": 2 * D * F * rows,
               "bytes": T * D * b + wb * groups + rows * 2 * F * b * 2 + rows * F * b},
        "dx_rows": {"flop": 4 * D * F * rows, "bytes": rows * 2 * F * b + 2 * wb * groups + rows * D * b},
        "dw13": {"flop": 4 * D * F * rows, "bytes": T * D * b + rows * 2 * F * b + 2 * D * F * 4 * groups},
        "dw2": {"flop": 2 * D * F * rows, "bytes": rows * F * b + T * D * b + D * F * 4 * groups},
    }


def bwd_cpu_baseline(inp, w, target_s):
    import numpy as np
    import oracle
    host = host_cpu()
    threads = host["threads"]
    sh = (inp["Ws1"], inp["Ws3"], inp["Ws2"]) if w.shared else None

    def run(n):
        t0 = time.perf_counter()
        oracle.backward(inp["x"][:n], inp["topk_idx"][:n], inp["topk_w"][:n], inp["W1"], inp["W3"],
                        inp["W2"], sh, inp["dy"][:n], nthreads=threads)
        return time.perf_counter() - t0

    n0 = min(w.T, 8 * threads)
    t0 = run(n0)
    n = int(min(w.T, max(n0, target_s / max(t0, 1e-6) * n0)))
    t = run(n)
    flop = 16 * w.D * w.F * (n * w.k + (n if w.shared else 0))
    return {"value": round(flop / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": round(t, 3), "host_nproc": host["nproc"], "host_affinity_cores": host["affinity"],
            "cpu_model": host["cpu_model"],
            "sample": f"first {n} of {w.T} tokens of the same workload (same weights, routing and dy), "
                      f"fp64 oracle backward, {threads} threads"}


def run_backward(args):
    """One step = one moe_ffn_backward call over the workload's inputs and a
    seeded dy, inputs resident in HBM (rotated like the forward's)."""
    import numpy as np
    import torch

    import grouped_gemm_permute_amd as gg
    import moe_inputs

    w = moe_inputs.WORKLOADS[args.workload]
    log(f"backward workload {w.name}: drawing inputs")
    inp = moe_inputs.add_output_grad(moe_inputs.make_inputs(args.workload))
    counts = np.bincount(inp["topk_idx"].reshape(-1), minlength=w.E)
    torch.cuda.set_device(0)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def dev(name):
        if w.dtype == "bf16":
            return torch.from_numpy(inp[name + "_bits"].view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(inp[name]).cuda()

    base = {n: dev(n) for n in ("x", "W1", "W3", "W2", "dy")}
    if w.shared:
        base.update({n: dev(n) for n in ("Ws1", "Ws3", "Ws2")})
    base["idx"] = torch.from_numpy(inp["topk_idx"]).cuda()
    base["w"] = torch.from_numpy(inp["topk_w"]).cuda()
    set_bytes = sum(t.numel() * t.element_size() for t in base.values())
    R = max(2, math.ceil(args.rotate_bytes / set_bytes))
    sets = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(R - 1)]
    lay = gg.backward_workspace_layout(w.T, w.D, w.F, w.E, w.k, w.shared, dt)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device="cuda")
    out = None
    log(f"{R} rotated input sets of {set_bytes / 1e6:.1f} MB; workspace {ws.numel() / 1e6:.1f} MB")

    def step(i, events=None):
        nonlocal out
        s = sets[i % R]
        sh = (s["Ws1"], s["Ws3"], s["Ws2"]) if w.shared else None
        out = gg.backward(s["x"], s["idx"], s["w"], s["W1"], s["W3"], s["W2"], sh, s["dy"], out=out,
                          workspace=ws, events=events)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    hip = HipEvents()
    evs = [hip.create(9) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    stage_ms = {st: float(np.mean([hip.elapsed_ms(e[j], e[j + 1]) for e in evs]))
                for j, st in enumerate(BWD_STAGES)}
    for e in evs:
        hip.destroy(e)
    log(f"timed {args.steps} backward steps: {ms_per_step:.4f} ms/step; stages {stage_ms}")
    rows = w.T * w.k + (w.T if w.shared else 0)
    flop = 16 * w.D * w.F * rows
    value = flop / (ms_per_step * 1e-3) / 1e12
    work = bwd_stage_work(w, counts)
    dom = max(work, key=lambda st: stage_ms[st])
    sec = stage_ms[dom] * 1e-3
    mfma_bound = work[dom]["flop"] / work[dom]["bytes"] > PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3
    if mfma_bound:
        ach = work[dom]["flop"] / sec / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
    else:
        ach = work[dom]["bytes"] / sec / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4)}
    roof.update({"traffic": None, "kernel": dom, "launch_ms": round(stage_ms[dom], 5),
                 "algorithmic": work[dom]["flop"] if mfma_bound else work[dom]["bytes"]})
    cpu = None
    if args.cpu_seconds > 0:
        log("timing the CPU oracle backward baseline")
        cpu = bwd_cpu_baseline(inp, w, args.cpu_seconds)
    res = {
        "metric": BWD_METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "D": w.D, "F": w.F, "E": w.E, "k": w.k,
                   "shared_expert": w.shared, "routing": w.routing, "pass": "backward",
                   "rotated_sets": R},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "expert_rows": counts.tolist(),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def train_step_record(workload, steps, warmup, rotate_bytes):
    """The recompute-versus-keep trade-off of the gate and up products
    ("Triton MoE Kernels & Memory Checkpointing", Part A section 8), timed on
    one workload: a training step's forward and backward either as
    moe_ffn_forward + moe_ffn_backward (g and u recomputed by the backward)
    or as moe_ffn_forward_save_gu + moe_ffn_backward_cached (g and u kept
    from the forward, R x 2F values of the storage dtype).  Each of the four
    calls is timed alone over the rotated input sets (host clock between two
    synchronisations), and the whole step both ways; one JSON line."""
    import numpy as np
    import torch

    import grouped_gemm_permute_amd as gg
    import moe_inputs

    w = moe_inputs.WORKLOADS[workload]
    if w.dtype != "bf16":
        raise SystemExit("--train-step: the kept gate/up products exist on the bf16 path only")
    log(f"train-step workload {w.name}: drawing inputs")
    inp = moe_inputs.add_output_grad(moe_inputs.make_inputs(workload))
    torch.cuda.set_device(0)

    def dev(name):
        return torch.from_numpy(inp[name + "_bits"].view(np.int16)).view(torch.bfloat16).cuda()

    base = {n: dev(n) for n in ("x", "W1", "W3", "W2", "dy")}
    if w.shared:
        base.update({n: dev(n) for n in ("Ws1", "Ws3", "Ws2")})
    base["idx"] = torch.from_numpy(inp["topk_idx"]).cuda()
    base["w"] = torch.from_numpy(inp["topk_w"]).cuda()
    set_bytes = sum(t.numel() * t.element_size() for t in base.values())
    R = max(2, math.ceil(rotate_bytes / set_bytes))
    sets = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(R - 1)]
    rows = w.T * w.k + (w.T if w.shared else 0)
    gus = [torch.empty((rows, 2 * w.F), dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    fws = gg.alloc_workspace(w.T, w.D, w.F, w.E, w.k, w.shared, torch.bfloat16)
    lay = gg.backward_workspace_layout(w.T, w.D, w.F, w.E, w.k, w.shared, torch.bfloat16)
    bws = torch.empty(lay["total"], dtype=torch.uint8, device="cuda")
    y = torch.empty((w.T, w.D), dtype=torch.bfloat16, device="cuda")
    out = None
    log(f"{R} rotated input sets of {set_bytes / 1e6:.1f} MB, kept g/u {rows * 2 * w.F * 2 / 1e6:.1f} MB each")

    def args_of(s):
        sh = (s["Ws1"], s["Ws3"], s["Ws2"]) if w.shared else None
        return (s["x"], s["idx"], s["w"], s["W1"], s["W3"], s["W2"], sh)

    def fwd(i):
        gg.forward(*args_of(sets[i % R]), y=y, workspace=fws)

    def fwd_keep(i):
        gg.forward_save_gu(*args_of(sets[i % R]), y=y, gu=gus[i % R], workspace=fws)

    def bwd(i, gu=False):
        nonlocal out
        s = sets[i % R]
        out = gg.backward(*args_of(s), s["dy"], out=out, workspace=bws, gu=gus[i % R] if gu else None)

    calls = {
        "forward": fwd,
        "forward_save_gu": fwd_keep,
        "backward_recompute": lambda i: bwd(i),
        "backward_cached": lambda i: bwd(i, gu=True),
        "step_recompute": lambda i: (fwd(i), bwd(i)),
        "step_keep": lambda i: (fwd_keep(i), bwd(i, gu=True)),
    }
    for i in range(R):                   # every set's g/u, for the cached calls
        fwd_keep(i)
    ms = {}
    for name, f in calls.items():
        for i in range(warmup):
            f(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            f(i)
        torch.cuda.synchronize()
        ms[name] = (time.perf_counter() - t0) * 1e3 / steps
        log(f"{name}: {ms[name]:.4f} ms per call")
    flop = 22 * w.D * w.F * rows          # 6 D F forward + 16 D F backward per row
    flop_keep = 18 * w.D * w.F * rows     # the backward's 4 D F gate/up recompute left out
    res = {
        "metric": "MoE FFN training step ms, gate/up recomputed vs kept", "unit": "ms",
        "value": round(ms["step_keep"], 5), "higher_is_better": False, "n_gpus": 1,
        "steps": steps, "warmup": warmup, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "D": w.D, "F": w.F, "E": w.E, "k": w.k,
                   "shared_expert": w.shared, "routing": w.routing, "rotated_sets": R},
        "ms_per_call": {k: round(v, 5) for k, v in ms.items()},
        "step_tflops": {"recompute": round(flop / (ms["step_recompute"] * 1e-3) / 1e12, 2),
                        "keep": round(flop_keep / (ms["step_keep"] * 1e-3) / 1e12, 2),
                        "note": "FLOP executed per row: 22 D F recomputing, 18 D F keeping"},
        "kept_bytes": rows * 2 * w.F * 2,
        "saving_ms": round(ms["step_recompute"] - ms["step_keep"], 5),
    }
    del sets, gus, fws, bws, out
    torch.cuda.empty_cache()
    return res


def run_train_step(args):
    print(json.dumps(train_step_record(args.workload, args.steps, args.warmup, args.rotate_bytes)),
          flush=True)


def time_forward(w, variant, steps, warmup, rotate_bytes=512e6):
    """Wall time per forward call of workload w (inputs rotated as in the
    main bench), in ms."""
    import numpy as np
    import torch

    import grouped_gemm_permute_amd as gg
    import moe_inputs

    inp = moe_inputs.make_inputs(w, seed=4242)
    dt = torch.bfloat16

    def dev(name):
        return torch.from_numpy(inp[name + "_bits"].view(np.int16)).view(dt).cuda()

    base = {n: dev(n) for n in ("x", "W1", "W3", "W2")}
    base["idx"] = torch.from_numpy(inp["topk_idx"]).cuda()
    base["w"] = torch.from_numpy(inp["topk_w"]).cuda()
    set_bytes = sum(t.numel() * t.element_size() for t in base.values())
    R = max(2, math.ceil(rotate_bytes / set_bytes))
    sets = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(R - 1)]
    ws = gg.alloc_workspace(w.T, w.D, w.F, w.E, w.k, False, dt, variant)
    y = torch.empty((w.T, w.D), dtype=dt, device="cuda")

    def step(i):
        s = sets[i % R]
        gg.forward(s["x"], s["idx"], s["w"], s["W1"], s["W3"], s["W2"], None, y=y, variant=variant,
                   workspace=ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del sets, ws, y
    return ms


def run_sweep(args):
    """The fused-vs-unfused measurement variants of "Chinchilla scaling,
    MoE, and fused Triton kernels" (verification section): sweep the
    expansion ratio F/D at a fixed per-expert token count t, and sweep t at a
    fixed F/D, timing the unfused (h through HBM) and fused (h on chip)
    forwards.  Each point prints one JSON line with both times, the measured
    speedup, the traffic model's speedup and the arithmetic intensity.

    Traffic model for the SwiGLU expert in bf16 (two up matrices and one
    down matrix, each read once per expert): unfused 4tD + 4tF + 6DF bytes,
    fused 4tD + 6DF, so speedup ~ 1 + 4tF / (4tD + 6DF); intensity of the
    unfused layer 6tDF / (4tD + 4tF + 6DF) FLOP/B (the page's single-matrix
    forms are 4tD + 4tF + 4DF, 1 + tF/(tD + DF) and tFD/(tD + FD))."""
    import moe_inputs

    E, k = 16, 2
    if args.sweep == "fd":
        D, t = 1024, 512
        points = [(D, F, t) for F in (512, 1024, 2048, 4096, 8192)]
    else:
        D, F = 1024, 4096
        points = [(D, F, t) for t in (64, 128, 256, 512, 1024, 2048)]
    if args.sweep_point is not None:
        # one point, one variant (for counter collection under rocprofv3)
        D, F, t = points[args.sweep_point]
        T = t * E // k
        w = moe_inputs.Workload(f"sweep_{args.sweep}_T{T}_D{D}_F{F}_E{E}_top{k}", T, D, F, E, k, False,
                                "bf16", "uniform")
        ms = time_forward(w, args.variant, args.steps, args.warmup, args.rotate_bytes)
        print(json.dumps({"sweep": args.sweep, "point": args.sweep_point, "workload": w.name,
                          "T": T, "D": D, "F": F, "E": E, "k": k, "t_per_expert": t,
                          "variant": args.variant, "ms": round(ms, 5),
                          "tflops": round(6 * D * F * T * k / ms / 1e9, 1)}), flush=True)
        return
    for D, F, t in points:
        T = t * E // k
        w = moe_inputs.Workload(f"sweep_{args.sweep}_T{T}_D{D}_F{F}_E{E}_top{k}", T, D, F, E, k, False,
                                "bf16", "uniform")
        un = time_forward(w, "unfused", args.steps, args.warmup, args.rotate_bytes)
        fu = time_forward(w, "fused", args.steps, args.warmup, args.rotate_bytes)
        flop = 6 * D * F * T * k
        b_un = E * (4 * t * D + 4 * t * F + 6 * D * F)
        b_fu = E * (4 * t * D + 6 * D * F)
        print(json.dumps({
            "sweep": args.sweep, "T": T, "D": D, "F": F, "E": E, "k": k, "t_per_expert": t,
            "F_over_D": F / D, "unfused_ms": round(un, 5), "fused_ms": round(fu, 5),
            "speedup_measured": round(un / fu, 3), "speedup_model": round(b_un / b_fu, 3),
            "unfused_tflops": round(flop / un / 1e9, 1), "fused_tflops": round(flop / fu / 1e9, 1),
            "intensity_unfused_flop_per_byte": round(6 * t * D * F / (4 * t * D + 4 * t * F + 6 * D * F), 1),
            "intensity_fused_flop_per_byte": round(6 * t * D * F / (4 * t * D + 6 * D * F), 1),
            "ridge_flop_per_byte": round(PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3, 1),
        }), flush=True)


def copy_calibration(nbytes, steps):
    """A plain copy of known size: reads and writes nbytes per launch."""
    import torch
    n = nbytes // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_bytes": n * 4, "launches": steps + 1, "ms_per_copy": round(dt * 1e3, 4),
                      "gbs_read_plus_write": round(2 * n * 4 / dt / 1e9, 1)}), flush=True)


def percentiles(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 5), "p10": round(float(np.percentile(a, 10)), 5),
            "p90": round(float(np.percentile(a, 90)), 5), "mean": round(float(a.mean()), 5)}


def measure_forward(wid, variant="unfused", steps=50, warmup=10, rotate_bytes=512e6, routed=False,
                    sustained_ms=0.0):
    """Time moe_ffn_forward (or the routed forward) on workload wid with its
    inputs resident in HBM and rotated over enough copies to exceed the
    on-die caches.

    Region 1: `steps` plain calls between two synchronisations (host clock:
    ms_per_step), with one event between consecutive calls on the stream the
    kernels run on (per-call distribution) and an engine-clock sample on
    each side.  Region 2: the same calls with HIP events recorded between the
    kernels (moe_ffn_forward_timed) for per-kernel durations; each record
    costs a few microseconds of GPU time, so whole-call figures come from
    region 1 only.

    With sustained_ms > 0, a third region follows: the same calls, untimed,
    until the GPU has been kept busy for sustained_ms, then `steps` calls
    timed with no event inside (host clock and engine clock around them).
    The engine clock takes tens of milliseconds of sustained load to settle,
    so regions 1 and 2 right after a short warmup run partly on a rising
    clock; region 3 gives the settled rate beside them."""
    import numpy as np
    import torch

    import grouped_gemm_permute_amd as gg
    import moe_inputs

    w = moe_inputs.WORKLOADS[wid]
    log(f"workload {w.name}: drawing inputs")
    inp = moe_inputs.make_inputs(wid)
    if routed:
        moe_inputs.add_router(inp)
    counts = np.bincount(inp["topk_idx"].reshape(-1), minlength=w.E)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def dev(name):
        if w.dtype == "bf16":
            return torch.from_numpy(inp[name + "_bits"].view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(inp[name]).cuda()

    base = {n: dev(n) for n in ("x", "W1", "W3", "W2")}
    if w.shared:
        base.update({n: dev(n) for n in ("Ws1", "Ws3", "Ws2")})
    base["idx"] = torch.from_numpy(inp["topk_idx"]).cuda()
    base["w"] = torch.from_numpy(inp["topk_w"]).cuda()
    if routed:
        base["gate_w"] = dev("gate_w")
    set_bytes = sum(t.numel() * t.element_size() for t in base.values())
    R = max(2, math.ceil(rotate_bytes / set_bytes))
    sets = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(R - 1)]
    ws = gg.alloc_workspace(w.T, w.D, w.F, w.E, w.k, w.shared, dt, variant)
    y = torch.empty((w.T, w.D), dtype=dt, device="cuda")
    log(f"{R} rotated input sets of {set_bytes / 1e6:.1f} MB; workspace {ws.numel() / 1e6:.1f} MB")

    def step(i, events=None):
        s = sets[i % R]
        sh = (s["Ws1"], s["Ws3"], s["Ws2"]) if w.shared else None
        if routed:
            gg.forward_routed(s["x"], s["gate_w"], s["W1"], s["W3"], s["W2"], sh, k=w.k, y=y,
                              variant=variant, workspace=ws, events=events)
            return
        gg.forward(s["x"], s["idx"], s["w"], s["W1"], s["W3"], s["W2"], sh, y=y, variant=variant,
                   workspace=ws, events=events)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup {warmup} steps done")

    # Region 1
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    clk0 = gg.device_clock_sample()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        marks[i].record()
        step(i)
    marks[steps].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    clk1 = gg.device_clock_sample()
    torch.cuda.synchronize()
    ms_per_step = (t1 - t0) * 1e3 / steps
    per_call = [marks[i].elapsed_time(marks[i + 1]) for i in range(steps)]
    clocks = gg.engine_clock_ghz(clk0.cpu(), clk1.cpu())

    # Region 2
    hip = HipEvents()
    evs = [hip.create(5) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    stage_samples = {st: [hip.elapsed_ms(e[j], e[j + 1]) for e in evs] for j, st in enumerate(STAGES)}
    for e in evs:
        hip.destroy(e)

    # Region 3 (optional): settled clock
    sustained = None
    if sustained_ms > 0:
        t_end = time.perf_counter() + sustained_ms * 1e-3
        i = 0
        while time.perf_counter() < t_end:
            for _ in range(8):
                step(i)
                i += 1
            torch.cuda.synchronize()
        s_clk0 = gg.device_clock_sample()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for j in range(steps):
            step(i + j)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        s_clk1 = gg.device_clock_sample()
        torch.cuda.synchronize()
        sustained = {"ms_per_step": (t1 - t0) * 1e3 / steps, "calls_before": i,
                     "clocks": gg.engine_clock_ghz(s_clk0.cpu(), s_clk1.cpu())}
    if routed:
        sidx, _ = gg.router_topk(sets[0]["x"], sets[0]["gate_w"], w.k)
        counts = np.bincount(sidx.cpu().numpy().reshape(-1), minlength=w.E)
    small = bool(gg.workspace_layout(w.T, w.D, w.F, w.E, w.k, w.shared, dt, variant)["small_tiles"])
    log(f"timed {steps} steps of {w.name}: {ms_per_step:.4f} ms/step (host clock), per-call "
        f"median {np.median(per_call):.4f} ms; stage means "
        f"{ {k: round(float(np.mean(v)), 4) for k, v in stage_samples.items()} }")
    del sets, ws, y
    torch.cuda.empty_cache()
    return {"w": w, "inp": inp, "counts": counts, "R": R, "ms_per_step": ms_per_step,
            "per_call": per_call, "stage_samples": stage_samples, "clocks": clocks, "small": small,
            "sustained": sustained}


def dominant_roofline(m, variant):
    """The dominant kernel's algorithmic work over its mean event-timed launch
    duration, against the MFMA or HBM peak by its arithmetic intensity."""
    import numpy as np
    w, counts = m["w"], m["counts"]
    stage_ms = {st: float(np.mean(v)) for st, v in m["stage_samples"].items()}
    work = stage_work(w, counts)
    if variant == "fused":             # one kernel does up, SwiGLU and down
        b = 2 if w.dtype == "bf16" else 4
        groups = int(sum(1 for c in counts if c > 0)) + (1 if w.shared else 0)
        work["up_swiglu"]["flop"] += work["down"]["flop"]
        work["up_swiglu"]["bytes"] = (w.T * w.D * b + 3 * w.D * w.F * b * groups
                                      + (w.T * w.k + (w.T if w.shared else 0)) * w.D * b)
        kernels = ("up_swiglu",)
    else:
        kernels = ("up_swiglu", "down")
    dom = max(kernels, key=lambda s: stage_ms[s])
    sec = stage_ms[dom] * 1e-3
    mfma_bound = work[dom]["flop"] / work[dom]["bytes"] > PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3
    if mfma_bound:
        ach = work[dom]["flop"] / sec / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
    else:
        ach = work[dom]["bytes"] / sec / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4)}
    roof["traffic"] = load_traffic(w.name, f"{variant}:{dom}", m["small"])
    roof["kernel"] = "fused_up_act_down" if variant == "fused" else dom
    roof["launch_ms"] = round(stage_ms[dom], 5)
    roof["launch_ms_median"] = round(float(np.median(m["stage_samples"][dom])), 5)
    roof["algorithmic"] = work[dom]["flop"] if mfma_bound else work[dom]["bytes"]
    return roof, stage_ms


def clock_record(m, value_tflops):
    """Mean engine clock over the timed region (per XCD) and the bf16 MFMA
    peak at that clock: compute units x clock x 4096 dense bf16 FLOPs per CU
    per cycle (2.5 PFLOP/s at 256 CUs and 2.4 GHz)."""
    import numpy as np
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    c = m["clocks"]
    if not c:
        return {"compute_units": cus, "sclk_ghz_median": None}
    v = np.array(list(c.values()))
    med = float(np.median(v))
    per_xcd = {}
    for (x, _), g in c.items():
        per_xcd.setdefault(x, []).append(g)
    peak = cus * med * 1e9 * 4096 / 1e12
    return {"compute_units": cus, "units_sampled": len(c), "sclk_ghz_median": round(med, 4),
            "sclk_ghz_p10_p90": [round(float(np.percentile(v, 10)), 4),
                                 round(float(np.percentile(v, 90)), 4)],
            "sclk_ghz_median_per_xcd": {str(x): round(float(np.median(g)), 4)
                                        for x, g in sorted(per_xcd.items())},
            "peak_bf16_tflops_at_measured_clock": round(peak, 1),
            "frac_of_peak_at_measured_clock": round(value_tflops / peak, 4),
            "peak_bf16_tflops_at_2p4ghz": round(cus * 2.4e9 * 4096 / 1e12, 1)}


def sustained_record(m, w):
    """Region 3 of measure_forward: the same steps timed after the GPU has
    been kept busy (value is region 1, right after the warmup steps)."""
    import numpy as np
    s = m.get("sustained")
    if not s:
        return None
    c = s["clocks"]
    tf = w.flops() / (s["ms_per_step"] * 1e-3) / 1e12
    return {"ms_per_step": round(s["ms_per_step"], 5), "tflops": round(tf, 3),
            "pct_of_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
            "calls_before": s["calls_before"],
            "sclk_ghz_median": round(float(np.median(list(c.values()))), 4) if c else None,
            "note": "the same steps timed again (host clock, no events inside) after the "
                    "timed regions and calls_before further untimed calls; not the headline value"}


def measured_read_gbs(nbytes=2 << 30, blocks=(128, 192, 256), launches=10):
    """HBM read rate of a plain streaming kernel (moe_stream_read) over a
    buffer of nbytes (larger than the on-die caches): the best over the
    launch shapes `blocks` of the median over launches."""
    import numpy as np
    import torch

    import grouped_gemm_permute_amd as gg
    if isinstance(blocks, int):
        blocks = (blocks,)
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(1)
    best = 0.0
    for nb in blocks:
        sink = torch.empty(nb, dtype=torch.int32, device="cuda")
        gg.stream_read(buf, sink)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(launches + 1)]
        torch.cuda.synchronize()
        for i in range(launches):
            ev[i].record()
            gg.stream_read(buf, sink)
        ev[launches].record()
        torch.cuda.synchronize()
        ms = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(launches)]))
        best = max(best, nbytes / (ms * 1e-3) / 1e9)
    del buf
    torch.cuda.empty_cache()
    return round(best, 1)


def small_chunk_record(args):
    """The small-chunk workload (512 tokens, 8 experts of ~128 rows) in the
    same run: it is bound by streaming the experts' weights, so it is priced
    in HBM bytes (x, y, routing and the weights of every active expert) per
    forward, against 8 TB/s and against the read rate a plain streaming
    kernel measures on the same GPU."""
    import numpy as np
    m = measure_forward(3, "unfused", steps=max(args.steps, 200), warmup=max(args.warmup, 20),
                        rotate_bytes=args.rotate_bytes, sustained_ms=args.sustained_ms)
    w, counts = m["w"], m["counts"]
    nbytes = path_bytes(w, counts)
    pc = percentiles(m["per_call"])
    roof, stage_ms = dominant_roofline(m, "unfused")
    gbs = nbytes / (pc["median"] * 1e-3) / 1e9
    read_gbs = measured_read_gbs()
    return {"workload": w.name, "T": w.T, "D": w.D, "F": w.F, "E": w.E, "k": w.k,
            "steps": max(args.steps, 200), "rotated_sets": m["R"],
            "ms_per_call": pc, "ms_per_step_host_clock": round(m["ms_per_step"], 5),
            "bytes_alg": nbytes, "gbs": round(gbs, 1), "frac_of_8tbs": round(gbs / PEAK_HBM_GBS, 4),
            "stream_read_gbs_measured": read_gbs, "frac_of_measured_read": round(gbs / read_gbs, 4),
            "back_to_back": back_to_back_record(m, nbytes),
            "stage_ms_mean_with_events": {k: round(v, 5) for k, v in stage_ms.items()},
            "dominant": roof}


def back_to_back_record(m, nbytes):
    """Region 3 of measure_forward priced in bytes: the same calls issued
    back to back with no event between them, after the GPU has been kept
    busy.  At µs-scale calls each event record between calls costs GPU time
    of its own, so ms_per_call (one event between consecutive calls) sits
    above this figure."""
    s = m.get("sustained")
    if not s:
        return None
    gbs = nbytes / (s["ms_per_step"] * 1e-3) / 1e9
    return {"ms_per_call": round(s["ms_per_step"], 5), "gbs": round(gbs, 1),
            "frac_of_8tbs": round(gbs / PEAK_HBM_GBS, 4), "calls_before": s["calls_before"],
            "note": "host clock over the calls issued back to back (no event between them), "
                    "after calls_before untimed calls"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, help="index into moe_inputs.WORKLOADS")
    ap.add_argument("--variant", default="unfused", choices=("unfused", "fused"))
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target length of the CPU-oracle baseline sample; 0 skips it")
    ap.add_argument("--rotate-bytes", type=float, default=512e6,
                    help="rotate input copies until their total exceeds this many bytes")
    ap.add_argument("--no-small-chunk", action="store_true",
                    help="skip the same-run small-chunk (512-token) record")
    ap.add_argument("--backward", action="store_true",
                    help="time moe_ffn_backward (dx, weight gradients, dtopk_w) instead of the forward")
    ap.add_argument("--no-train-step", action="store_true",
                    help="skip the same-run training-step record (forward + backward, gate/up "
                         "recomputed vs kept)")
    ap.add_argument("--train-step", action="store_true",
                    help="time a training step's forward and backward with the gate/up products "
                         "recomputed by the backward or kept from the forward (bf16 workloads)")
    ap.add_argument("--routed", action="store_true",
                    help="time moe_ffn_forward_routed: the top-k router (x @ gate_w, top-k, softmax) "
                         "feeding the permute, then the same forward")
    ap.add_argument("--sweep", choices=("fd", "t"), default=None,
                    help="fused vs unfused forward over F/D at fixed tokens per expert (fd) or over "
                         "tokens per expert at fixed F/D (t); one JSON line per point")
    ap.add_argument("--sweep-point", type=int, default=None,
                    help="with --sweep: run only this point (index) and variant --variant, for "
                         "counter collection under rocprofv3")
    ap.add_argument("--sustained-ms", type=float, default=150.0,
                    help="after the timed regions, keep the GPU busy this long, then time the same "
                         "steps again (reported as 'sustained', beside value; 0 skips it)")
    ap.add_argument("--copy-bytes", type=float, default=0,
                    help="only run a plain device-to-device copy of this many bytes --steps times "
                         "(the reference kernel for scaling HBM byte counters); prints its timing")
    args = ap.parse_args()
    if args.copy_bytes > 0:
        copy_calibration(int(args.copy_bytes), args.steps)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this path has no multi-GPU implementation); "
              f"got --gpus {args.gpus}", file=sys.stderr)
        sys.exit(2)
    if args.backward:
        run_backward(args)
        return
    if args.train_step:
        run_train_step(args)
        return
    if args.sweep:
        run_sweep(args)
        return

    import torch

    import moe_inputs
    torch.cuda.set_device(0)
    m = measure_forward(args.workload, args.variant, args.steps, args.warmup, args.rotate_bytes,
                        args.routed, sustained_ms=args.sustained_ms)
    w, inp, counts = m["w"], m["inp"], m["counts"]
    value = w.flops() / (m["ms_per_step"] * 1e-3) / 1e12
    roof, stage_ms = dominant_roofline(m, args.variant)
    if args.variant == "fused":
        stage_ms.pop("down")           # an empty interval between two back-to-back events
    pc = percentiles(m["per_call"])

    small = None
    if args.workload == 2 and args.variant == "unfused" and not args.routed and not args.no_small_chunk:
        log("same-run small-chunk record")
        small = small_chunk_record(args)

    train = None
    if args.workload == 2 and args.variant == "unfused" and not args.routed and not args.no_train_step:
        log("same-run training-step record (gate/up recomputed vs kept)")
        train = train_step_record(args.workload, args.steps, args.warmup, args.rotate_bytes)
        train = {k: train[k] for k in ("ms_per_call", "step_tflops", "kept_bytes", "saving_ms",
                                       "steps", "warmup")}

    cpu = None
    if args.cpu_seconds > 0 and not args.routed:
        log("timing the CPU oracle baseline")
        cpu = cpu_baseline(inp, w, args.cpu_seconds)
    if args.routed:
        stage_ms["router_permute"] = stage_ms.pop("permute")

    out = {
        "metric": METRIC + (" (routed: router feeding the permute)" if args.routed else ""),
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(m["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "D": w.D, "F": w.F, "E": w.E, "k": w.k,
                   "shared_expert": w.shared, "routing": "router" if args.routed else w.routing,
                   "variant": args.variant, "rotated_sets": m["R"]},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "ms_per_call": pc,
        "tflops_at_median_call": round(w.flops() / (pc["median"] * 1e-3) / 1e12, 3),
        "clock": clock_record(m, value),
        "sustained": sustained_record(m, w),
        "hbm_gbs_path": round(path_bytes(w, counts) / (m["ms_per_step"] * 1e-3) / 1e9, 1),
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "stage_ms_median": {k: round(float(percentiles(v)["median"]), 5)
                            for k, v in m["stage_samples"].items() if k in stage_ms},
        "expert_rows": counts.tolist(),
        "input_sha256": moe_inputs.input_digest(inp),
        "roofline": roof,
        "small_chunk": small,
        "train_step": train,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
