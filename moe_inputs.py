"""Seeded synthetic inputs for the top-k routed MoE SwiGLU FFN forward.

This module only draws random numbers and rounds them to the storage type.
It holds none of the layer's arithmetic, and it is the one module that both
the CPU oracle (``oracle/``) and the HIP path (``grouped_gemm_permute_amd``)
are fed from.

Workload shapes follow the GPT-OSS-Lite layer described on "Triton MoE
Kernels & Memory Checkpointing" (Part A, section 2: d_model=768, d_ff=1536,
8 routed experts, top-2, one shared expert, 32,768 tokens per step).  The
value distributions are x ~ N(0,1), W1/W3 ~ N(0,1/D), W2 ~ N(0,1/F); routing
is either uniform over experts or Zipf(1.2)-skewed without replacement
(Gumbel top-k); routing weights are a softmax over k N(0,1) logits.

Draw order (one numpy PCG64 stream per workload, seed = 1000 + index):
x, W1, W3, W2, [Ws1, Ws3, Ws2], routing keys, weight logits.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    D: int
    F: int
    E: int
    k: int
    shared: bool
    dtype: str          # "f32" or "bf16"
    routing: str        # "uniform" or "zipf"
    zipf_s: float = 1.2
    note: str = field(default="", compare=False)

    @property
    def S(self) -> int:
        return self.T * self.k

    def flops(self) -> int:
        """Algorithmic FLOPs: 2 per multiply-add over the three GEMMs of every
        routed slot, plus the shared expert's T rows."""
        rows = self.T * self.k + (self.T if self.shared else 0)
        return 6 * self.D * self.F * rows


WORKLOADS = [
    Workload("tiny_fp32_T64_D64_F128_E4_top2", 64, 64, 128, 4, 2, False, "f32", "uniform",
             note="tiny fp32 case the oracle finishes instantly"),
    Workload("gptoss_lite_T4096_D768_F1536_E8_top2_shared", 4096, 768, 1536, 8, 2, True, "bf16",
             "uniform", note="one GPT-OSS-Lite MoE layer at one 4096-token sequence"),
    Workload("step_T32768_D768_F1536_E8_top2_shared_zipf", 32768, 768, 1536, 8, 2, True, "bf16",
             "zipf", note="full 8x4096-token step, Zipf(1.2) skewed routing"),
    Workload("smallchunk_T512_D768_F1536_E8_top2", 512, 768, 1536, 8, 2, False, "bf16", "uniform",
             note="small-chunk regime, weight-streaming bound"),
    Workload("fused_T16384_D1024_F4096_E16_top2", 16384, 1024, 4096, 16, 2, False, "bf16",
             "uniform", note="F > D case for the fused up-act-down variant"),
]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return the
    16-bit patterns as uint16.  Inputs are finite by construction."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(a: np.ndarray, dtype: str):
    """Return (values as float32, storage bits or None)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(a)
        return bf16_bits_to_f32(bits), bits
    return a, None


def draw_routing(rng: np.random.Generator, T: int, E: int, k: int, kind: str, zipf_s: float):
    if kind == "uniform":
        keys = rng.random((T, E))
        idx = np.argsort(keys, axis=1, kind="stable")[:, :k]
    elif kind == "zipf":
        # Gumbel-top-k: the k largest of log p_e + Gumbel(0,1) are k draws
        # without replacement from p, in draw order.
        logp = -zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
        keys = logp[None, :] + rng.gumbel(size=(T, E))
        idx = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    else:
        raise ValueError(f"unknown routing kind {kind!r}")
    return np.ascontiguousarray(idx, dtype=np.int32)


def draw_weights(rng: np.random.Generator, T: int, k: int):
    logits = rng.standard_normal((T, k))
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    return np.ascontiguousarray(z / z.sum(axis=1, keepdims=True), dtype=np.float32)


def make_inputs(w: Workload | int, seed: int | None = None, T: int | None = None) -> dict:
    """Draw one workload's inputs.  ``T`` overrides the token count (the
    weights are drawn first, so they do not depend on it; x and routing do).

    Returns float32 arrays holding exactly the stored values (for bf16, the
    rounded values), plus ``*_bits`` uint16 arrays for bf16 storage.
    """
    if isinstance(w, int):
        if seed is None:
            seed = 1000 + w
        w = WORKLOADS[w]
    if seed is None:
        seed = 1000 + WORKLOADS.index(w)
    T = w.T if T is None else T
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {"workload": w, "T": T, "seed": seed}

    def put(name, arr):
        vals, bits = _store(arr, w.dtype)
        out[name] = vals
        if bits is not None:
            out[name + "_bits"] = bits

    put("x", rng.standard_normal((T, w.D), dtype=np.float32))
    put("W1", rng.standard_normal((w.E, w.D, w.F), dtype=np.float32) / np.float32(np.sqrt(w.D)))
    put("W3", rng.standard_normal((w.E, w.D, w.F), dtype=np.float32) / np.float32(np.sqrt(w.D)))
    put("W2", rng.standard_normal((w.E, w.F, w.D), dtype=np.float32) / np.float32(np.sqrt(w.F)))
    if w.shared:
        put("Ws1", rng.standard_normal((w.D, w.F), dtype=np.float32) / np.float32(np.sqrt(w.D)))
        put("Ws3", rng.standard_normal((w.D, w.F), dtype=np.float32) / np.float32(np.sqrt(w.D)))
        put("Ws2", rng.standard_normal((w.F, w.D), dtype=np.float32) / np.float32(np.sqrt(w.F)))
    out["topk_idx"] = draw_routing(rng, T, w.E, w.k, w.routing, w.zipf_s)
    out["topk_w"] = draw_weights(rng, T, w.k)
    return out


def add_output_grad(inp: dict, seed: int | None = None) -> dict:
    """Draw the incoming gradient dy [T, D] ~ N(0, 1) for a backward pass,
    from its own stream (seed + 7919, so the forward inputs are unchanged),
    stored like x.  Adds ``dy`` (and ``dy_bits`` for bf16) to ``inp``."""
    w = inp["workload"]
    seed = inp["seed"] + 7919 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    vals, bits = _store(rng.standard_normal((inp["T"], w.D), dtype=np.float32), w.dtype)
    inp["dy"] = vals
    if bits is not None:
        inp["dy_bits"] = bits
    return inp


def add_router(inp: dict, seed: int | None = None) -> dict:
    """Draw a router matrix gate_w [D, E] ~ N(0, 1/D) from its own stream
    (seed + 104729), stored like the weights.  Adds ``gate_w`` (and
    ``gate_w_bits`` for bf16) to ``inp``."""
    w = inp["workload"]
    seed = inp["seed"] + 104729 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    g = rng.standard_normal((w.D, w.E), dtype=np.float32) / np.float32(np.sqrt(w.D))
    vals, bits = _store(g, w.dtype)
    inp["gate_w"] = vals
    if bits is not None:
        inp["gate_w_bits"] = bits
    return inp


def input_digest(inp: dict) -> str:
    """sha256 over the stored bytes of every input tensor, in a fixed order."""
    h = hashlib.sha256()
    for name in ("x", "W1", "W3", "W2", "Ws1", "Ws3", "Ws2", "topk_idx", "topk_w"):
        if name not in inp:
            continue
        arr = inp.get(name + "_bits", inp[name])
        h.update(name.encode())
        h.update(np.ascontiguousarray(arr).tobytes())
    return h.hexdigest()
