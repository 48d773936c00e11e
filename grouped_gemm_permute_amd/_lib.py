"""ctypes binding of libmoe_ffn.so (the C ABI in include/moe_ffn.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the layer runs in the library's kernels.
``torch`` is imported before the library is loaded so that the library
binds to the HIP runtime torch already holds (one runtime per process).
There is no fallback: if the library is missing, loading raises ImportError.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_ffn.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_VARIANT_UNFUSED, MOE_VARIANT_FUSED = 0, 1

# Every symbol include/moe_ffn.h declares.
EXPORTS = (
    "moe_status_string", "moe_ffn_tile_rows", "moe_ffn_workspace_layout", "moe_ffn_workspace_size",
    "moe_ffn_forward", "moe_ffn_forward_timed", "moe_expert_permute", "moe_expert_permute_scratch_size",
    "moe_ffn_get_device_error", "moe_ffn_backward_workspace_layout", "moe_ffn_backward_workspace_size",
    "moe_ffn_backward", "moe_ffn_backward_timed", "moe_router_topk", "moe_ffn_forward_routed",
    "moe_ffn_forward_routed_timed",
)


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("total", "err", "counts", "offsets", "tile_off", "tile_off64", "perm", "inv", "hist",
                 "h", "Y")] + \
               [("tile_rows", ctypes.c_int32), ("hist_blocks", ctypes.c_int32),
                ("small_tiles", ctypes.c_int32)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class BwdWsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("total", "err", "counts", "offsets", "tile_off", "chunk_off", "perm", "inv", "hist",
                 "gu", "dgu", "hw", "dxr", "dwpart", "w2t", "w13t", "partial", "zeros")] + \
               [("tile_rows", ctypes.c_int32), ("hist_blocks", ctypes.c_int32),
                ("chunk_rows", ctypes.c_int32)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m grouped_gemm_permute_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i64, ci, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ci]
        L.moe_ffn_tile_rows.restype = ci
        L.moe_ffn_tile_rows.argtypes = [ci, ci]
        L.moe_ffn_workspace_layout.restype = ci
        L.moe_ffn_workspace_layout.argtypes = [i64, ci, ci, ci, ci, ci, ci, ci, ctypes.POINTER(WsLayout)]
        L.moe_ffn_workspace_size.restype = sz
        L.moe_ffn_workspace_size.argtypes = [i64, ci, ci, ci, ci, ci, ci, ci]
        L.moe_ffn_forward.restype = ci
        L.moe_ffn_forward.argtypes = [P, P, P, P, P, P, P, P, P, P, i64, ci, ci, ci, ci, ci, ci, P, sz, P]
        L.moe_ffn_forward_timed.restype = ci
        L.moe_ffn_forward_timed.argtypes = [P, P, P, P, P, P, P, P, P, P, i64, ci, ci, ci, ci, ci, ci,
                                            P, sz, P, P]
        L.moe_expert_permute.restype = ci
        L.moe_expert_permute.argtypes = [P, i64, ci, ci, ci, i64, P, P, P, P, P, P, P, sz, P]
        L.moe_expert_permute_scratch_size.restype = sz
        L.moe_expert_permute_scratch_size.argtypes = [i64, ci, ci]
        L.moe_ffn_backward_workspace_layout.restype = ci
        L.moe_ffn_backward_workspace_layout.argtypes = [i64, ci, ci, ci, ci, ci, ci,
                                                        ctypes.POINTER(BwdWsLayout)]
        L.moe_ffn_backward_workspace_size.restype = sz
        L.moe_ffn_backward_workspace_size.argtypes = [i64, ci, ci, ci, ci, ci, ci]
        bwd_args = [P] * 18 + [i64, ci, ci, ci, ci, ci, P, sz, P]
        L.moe_ffn_backward.restype = ci
        L.moe_ffn_backward.argtypes = bwd_args
        L.moe_ffn_backward_timed.restype = ci
        L.moe_ffn_backward_timed.argtypes = bwd_args + [P]
        L.moe_router_topk.restype = ci
        L.moe_router_topk.argtypes = [P, P, i64, ci, ci, ci, ci, P, P, P]
        routed = [P] * 11 + [i64, ci, ci, ci, ci, ci, ci, P, sz, P]
        L.moe_ffn_forward_routed.restype = ci
        L.moe_ffn_forward_routed.argtypes = routed
        L.moe_ffn_forward_routed_timed.restype = ci
        L.moe_ffn_forward_routed_timed.argtypes = routed + [P]
        L.moe_ffn_get_device_error.restype = ci
        L.moe_ffn_get_device_error.argtypes = [P, P, ctypes.POINTER(ctypes.c_int32)]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, what)


def _dtype_enum(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return MOE_BF16
    if t == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {t}; use torch.bfloat16 or torch.float32")


def _variant_enum(v: str) -> int:
    return {"unfused": MOE_VARIANT_UNFUSED, "fused": MOE_VARIANT_FUSED}[v]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def tile_rows(dtype: torch.dtype, variant: str = "unfused") -> int:
    return lib().moe_ffn_tile_rows(_dtype_enum(dtype), _variant_enum(variant))


def workspace_layout(T, D, F, E, k, has_shared, dtype, variant="unfused") -> dict:
    L = WsLayout()
    _check(lib().moe_ffn_workspace_layout(T, D, F, E, k, int(has_shared), _dtype_enum(dtype),
                                          _variant_enum(variant), ctypes.byref(L)),
           "moe_ffn_workspace_layout")
    return L.as_dict()


def workspace_size(T, D, F, E, k, has_shared, dtype, variant="unfused") -> int:
    return lib().moe_ffn_workspace_size(T, D, F, E, k, int(has_shared), _dtype_enum(dtype),
                                        _variant_enum(variant))


def alloc_workspace(T, D, F, E, k, has_shared, dtype, variant="unfused", device="cuda"):
    n = workspace_layout(T, D, F, E, k, has_shared, dtype, variant)["total"]
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def forward(x, topk_idx, topk_w, W1, W3, W2, shared=None, y=None, variant="unfused",
            workspace=None, stream=None, events=None):
    """y = moe_ffn_forward(...).  x [T,D], topk_idx [T,k] int32, topk_w [T,k]
    fp32, W1/W3 [E,D,F], W2 [E,F,D], shared = (Ws1, Ws3, Ws2) or None.
    Tensors must be contiguous and on the current device.  ``events``: a
    ctypes array of five hipEvent_t handles to route the call through
    moe_ffn_forward_timed."""
    if topk_idx.dtype != torch.int32:
        raise TypeError("topk_idx must be int32")
    if topk_w.dtype != torch.float32:
        raise TypeError("topk_w must be float32")
    for t in (x, topk_idx, topk_w, W1, W3, W2, *(shared or ())):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    T, D = x.shape
    E, _, F = W1.shape
    k = topk_idx.shape[1]
    if W1.shape != (E, D, F) or W3.shape != (E, D, F) or W2.shape != (E, F, D):
        raise ValueError("weight shapes must be W1/W3 [E,D,F], W2 [E,F,D]")
    if topk_idx.shape != (T, k) or topk_w.shape != (T, k):
        raise ValueError("topk_idx / topk_w must be [T,k]")
    Ws1, Ws3, Ws2 = shared if shared is not None else (None, None, None)
    if shared is not None and (Ws1.shape != (D, F) or Ws3.shape != (D, F) or Ws2.shape != (F, D)):
        raise ValueError("shared weights must be [D,F], [D,F], [F,D]")
    dt = _dtype_enum(x.dtype)
    if y is None:
        y = torch.empty((T, D), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(T, D, F, E, k, shared is not None, x.dtype, variant, x.device)
    args = (_ptr(x), _ptr(topk_idx), _ptr(topk_w), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(Ws1),
            _ptr(Ws3), _ptr(Ws2), _ptr(y), T, D, F, E, k, dt, _variant_enum(variant),
            _ptr(workspace), workspace.numel(), _stream(stream))
    if events is None:
        _check(lib().moe_ffn_forward(*args), "moe_ffn_forward")
    else:
        _check(lib().moe_ffn_forward_timed(*args, events), "moe_ffn_forward_timed")
    return y


def expert_permute(topk_idx, E, tile_rows_=1, shared_rows=0, stream=None) -> dict:
    """Stable counting sort of the slots on the device; returns device int32
    tensors counts [E], offsets [E+1], tile_off [E+2], perm, inv [T*k], err [1]."""
    if topk_idx.dtype != torch.int32 or not topk_idx.is_contiguous():
        raise TypeError("topk_idx must be contiguous int32")
    T, k = topk_idx.shape
    dev = topk_idx.device
    out = {n: torch.empty(sz, dtype=torch.int32, device=dev) for n, sz in
           (("counts", E), ("offsets", E + 1), ("tile_off", E + 2), ("perm", max(T * k, 1)),
            ("inv", max(T * k, 1)), ("err", 1))}
    nscr = lib().moe_expert_permute_scratch_size(T, k, E)
    scratch = torch.empty(max(nscr // 4, 1), dtype=torch.int32, device=dev)
    st = lib().moe_expert_permute(_ptr(topk_idx), T, k, E, tile_rows_, shared_rows,
                                  _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["tile_off"]),
                                  _ptr(out["perm"]), _ptr(out["inv"]), _ptr(out["err"]),
                                  _ptr(scratch), nscr, _stream(stream))
    _check(st, "moe_expert_permute")
    out["perm"] = out["perm"][:T * k]
    out["inv"] = out["inv"][:T * k]
    return out


def device_error(workspace, stream=None) -> int:
    v = ctypes.c_int32(-1)
    _check(lib().moe_ffn_get_device_error(_ptr(workspace), _stream(stream), ctypes.byref(v)),
           "moe_ffn_get_device_error")
    return int(v.value)


def backward_workspace_layout(T, D, F, E, k, has_shared, dtype) -> dict:
    L = BwdWsLayout()
    _check(lib().moe_ffn_backward_workspace_layout(T, D, F, E, k, int(has_shared), _dtype_enum(dtype),
                                                   ctypes.byref(L)),
           "moe_ffn_backward_workspace_layout")
    return L.as_dict()


def backward(x, topk_idx, topk_w, W1, W3, W2, shared, dy, out=None, workspace=None, stream=None,
             events=None) -> dict:
    """moe_ffn_backward(...): gradients of the layer for the incoming dy [T,D].
    Returns dx [T,D] (x's dtype), dW1/dW3 [E,D,F], dW2 [E,F,D], dWs1/dWs3
    [D,F], dWs2 [F,D] (None without a shared expert) and dtopk_w [T,k], all
    fp32 except dx.  ``out`` may supply any of these tensors.  ``events``: a
    ctypes array of nine hipEvent_t handles (moe_ffn_backward_timed)."""
    if topk_idx.dtype != torch.int32 or topk_w.dtype != torch.float32:
        raise TypeError("topk_idx must be int32 and topk_w float32")
    for t in (x, topk_idx, topk_w, W1, W3, W2, dy, *(shared or ())):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    T, D = x.shape
    E, _, F = W1.shape
    k = topk_idx.shape[1]
    if dy.shape != (T, D) or dy.dtype != x.dtype:
        raise ValueError("dy must be [T,D] with x's dtype")
    if W1.shape != (E, D, F) or W3.shape != (E, D, F) or W2.shape != (E, F, D):
        raise ValueError("weight shapes must be W1/W3 [E,D,F], W2 [E,F,D]")
    dev = x.device
    f32 = dict(dtype=torch.float32, device=dev)
    o = dict(out or {})
    o.setdefault("dx", torch.empty((T, D), dtype=x.dtype, device=dev))
    o.setdefault("dW1", torch.empty((E, D, F), **f32))
    o.setdefault("dW3", torch.empty((E, D, F), **f32))
    o.setdefault("dW2", torch.empty((E, F, D), **f32))
    o.setdefault("dtopk_w", torch.empty((T, k), **f32))
    if shared is not None:
        o.setdefault("dWs1", torch.empty((D, F), **f32))
        o.setdefault("dWs3", torch.empty((D, F), **f32))
        o.setdefault("dWs2", torch.empty((F, D), **f32))
    else:
        o["dWs1"] = o["dWs3"] = o["dWs2"] = None
    Ws1, Ws3, Ws2 = shared if shared is not None else (None, None, None)
    if workspace is None:
        n = backward_workspace_layout(T, D, F, E, k, shared is not None, x.dtype)["total"]
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    args = (_ptr(x), _ptr(topk_idx), _ptr(topk_w), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(Ws1),
            _ptr(Ws3), _ptr(Ws2), _ptr(dy), _ptr(o["dx"]), _ptr(o["dW1"]), _ptr(o["dW3"]),
            _ptr(o["dW2"]), _ptr(o["dWs1"]), _ptr(o["dWs3"]), _ptr(o["dWs2"]), _ptr(o["dtopk_w"]),
            T, D, F, E, k, _dtype_enum(x.dtype), _ptr(workspace), workspace.numel(), _stream(stream))
    if events is None:
        _check(lib().moe_ffn_backward(*args), "moe_ffn_backward")
    else:
        _check(lib().moe_ffn_backward_timed(*args, events), "moe_ffn_backward_timed")
    return o


def router_topk(x, gate_w, k, stream=None):
    """moe_router_topk: (topk_idx int32 [T,k], topk_w fp32 [T,k]) for x [T,D]
    and gate_w [D,E] of x's dtype."""
    if not (x.is_contiguous() and gate_w.is_contiguous()) or gate_w.dtype != x.dtype:
        raise ValueError("x and gate_w must be contiguous and of one dtype")
    T, D = x.shape
    E = gate_w.shape[1]
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    _check(lib().moe_router_topk(_ptr(x), _ptr(gate_w), T, D, E, k, _dtype_enum(x.dtype), _ptr(idx),
                                 _ptr(w), _stream(stream)), "moe_router_topk")
    return idx, w


def forward_routed(x, gate_w, W1, W3, W2, shared=None, k=2, y=None, variant="unfused",
                   workspace=None, stream=None, events=None):
    """moe_ffn_forward_routed: returns (y, topk_idx, topk_w)."""
    for t in (x, gate_w, W1, W3, W2, *(shared or ())):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    T, D = x.shape
    E, _, F = W1.shape
    Ws1, Ws3, Ws2 = shared if shared is not None else (None, None, None)
    if y is None:
        y = torch.empty((T, D), dtype=x.dtype, device=x.device)
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(T, D, F, E, k, shared is not None, x.dtype, variant, x.device)
    args = (_ptr(x), _ptr(gate_w), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(Ws1), _ptr(Ws3), _ptr(Ws2),
            _ptr(y), _ptr(idx), _ptr(w), T, D, F, E, k, _dtype_enum(x.dtype), _variant_enum(variant),
            _ptr(workspace), workspace.numel(), _stream(stream))
    if events is None:
        _check(lib().moe_ffn_forward_routed(*args), "moe_ffn_forward_routed")
    else:
        _check(lib().moe_ffn_forward_routed_timed(*args, events), "moe_ffn_forward_routed_timed")
    return y, idx, w
