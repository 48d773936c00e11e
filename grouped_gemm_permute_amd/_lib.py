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
    "moe_ffn_forward_routed_timed", "moe_device_clock_sample", "moe_ffn_forward_noalloc",
    "moe_stream_read", "moe_ffn_forward_save_gu", "moe_ffn_backward_cached",
    "moe_ffn_backward_cached_timed",
)

# Bytes of the per-device workspace array behind moe_ffn_forward_noalloc.
NOALLOC_SCRATCH_BYTES = 64 << 20


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
        L.moe_ffn_forward_save_gu.restype = ci
        L.moe_ffn_forward_save_gu.argtypes = [P] * 11 + [i64, ci, ci, ci, ci, ci, ci, P, sz, P]
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
        cached_args = [P] * 19 + [i64, ci, ci, ci, ci, ci, P, sz, P]
        L.moe_ffn_backward_cached.restype = ci
        L.moe_ffn_backward_cached.argtypes = cached_args
        L.moe_ffn_backward_cached_timed.restype = ci
        L.moe_ffn_backward_cached_timed.argtypes = cached_args + [P]
        L.moe_router_topk.restype = ci
        L.moe_router_topk.argtypes = [P, P, i64, ci, ci, ci, ci, P, P, P]
        routed = [P] * 11 + [i64, ci, ci, ci, ci, ci, ci, P, sz, P]
        L.moe_ffn_forward_routed.restype = ci
        L.moe_ffn_forward_routed.argtypes = routed
        L.moe_ffn_forward_routed_timed.restype = ci
        L.moe_ffn_forward_routed_timed.argtypes = routed + [P]
        L.moe_ffn_forward_noalloc.restype = ci
        L.moe_ffn_forward_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, P, i64, ci, ci, ci, ci, ci, ci, P]
        L.moe_device_clock_sample.restype = ci
        L.moe_device_clock_sample.argtypes = [P, ci, P]
        L.moe_stream_read.restype = ci
        L.moe_stream_read.argtypes = [P, ctypes.c_size_t, P, ci, P]
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


def _same_device(ref, named):
    """Every tensor must live on ref's device, which must be a GPU: the C ABI
    takes raw device pointers and cannot tell a host pointer from one."""
    if ref.device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU device, got {ref.device}")
    for name, t in named.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _expect(name, t, shape, dtype):
    if t.shape != shape:
        raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_layer(x, W1, W3, W2, shared, y):
    """Shapes, dtypes, contiguity and device of the layer's tensors; returns
    (T, D, F, E).  Weights and y take x's dtype, so the library's element
    size matches every buffer it touches."""
    _dtype_enum(x.dtype)
    if x.dim() != 2 or W1.dim() != 3:
        raise ValueError("x must be [T,D] and W1 [E,D,F]")
    T, D = x.shape
    E, _, F = W1.shape
    _expect("x", x, (T, D), x.dtype)
    _expect("W1", W1, (E, D, F), x.dtype)
    _expect("W3", W3, (E, D, F), x.dtype)
    _expect("W2", W2, (E, F, D), x.dtype)
    if shared is not None:
        if len(shared) != 3:
            raise ValueError("shared must be (Ws1, Ws3, Ws2)")
        _expect("Ws1", shared[0], (D, F), x.dtype)
        _expect("Ws3", shared[1], (D, F), x.dtype)
        _expect("Ws2", shared[2], (F, D), x.dtype)
    if y is not None:
        _expect("y", y, (T, D), x.dtype)
    return T, D, F, E


def _layer_tensors(W1, W3, W2, shared, y):
    sh = dict(zip(("Ws1", "Ws3", "Ws2"), shared)) if shared is not None else {}
    return dict(W1=W1, W3=W3, W2=W2, y=y, **sh)


def _check_routing(x, topk_idx, topk_w, T):
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [T,k]")
    k = topk_idx.shape[1]
    _expect("topk_idx", topk_idx, (T, k), torch.int32)
    _expect("topk_w", topk_w, (T, k), torch.float32)
    return k


def _check_workspace(x, workspace, need):
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous uint8 tensor")
    _same_device(x, dict(workspace=workspace))
    if workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, the call needs {need}")


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
    T, D, F, E = _check_layer(x, W1, W3, W2, shared, y)
    k = _check_routing(x, topk_idx, topk_w, T)
    _same_device(x, dict(topk_idx=topk_idx, topk_w=topk_w, **_layer_tensors(W1, W3, W2, shared, y)))
    Ws1, Ws3, Ws2 = shared if shared is not None else (None, None, None)
    dt = _dtype_enum(x.dtype)
    if y is None:
        y = torch.empty((T, D), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(T, D, F, E, k, shared is not None, x.dtype, variant, x.device)
    _check_workspace(x, workspace, workspace_size(T, D, F, E, k, shared is not None, x.dtype, variant))
    args = (_ptr(x), _ptr(topk_idx), _ptr(topk_w), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(Ws1),
            _ptr(Ws3), _ptr(Ws2), _ptr(y), T, D, F, E, k, dt, _variant_enum(variant),
            _ptr(workspace), workspace.numel(), _stream(stream))
    if events is None:
        _check(lib().moe_ffn_forward(*args), "moe_ffn_forward")
    else:
        _check(lib().moe_ffn_forward_timed(*args, events), "moe_ffn_forward_timed")
    return y


def forward_save_gu(x, topk_idx, topk_w, W1, W3, W2, shared=None, y=None, gu=None, workspace=None,
                    stream=None):
    """(y, gu) = moe_ffn_forward_save_gu(...): the unfused bf16 forward that
    also returns each sorted row's gate and up products, gu [R, 2F] bf16
    (R = T*k + T with a shared expert), for backward(..., gu=gu)."""
    T, D, F, E = _check_layer(x, W1, W3, W2, shared, y)
    k = _check_routing(x, topk_idx, topk_w, T)
    R = T * k + (T if shared is not None else 0)
    if gu is None:
        gu = torch.empty((R, 2 * F), dtype=x.dtype, device=x.device)
    _expect("gu", gu, (R, 2 * F), x.dtype)
    _same_device(x, dict(topk_idx=topk_idx, topk_w=topk_w, gu=gu,
                         **_layer_tensors(W1, W3, W2, shared, y)))
    Ws1, Ws3, Ws2 = shared if shared is not None else (None, None, None)
    if y is None:
        y = torch.empty((T, D), dtype=x.dtype, device=x.device)
    n = workspace_size(T, D, F, E, k, shared is not None, x.dtype, "unfused")
    if workspace is None:
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=x.device)
    _check_workspace(x, workspace, n)
    _check(lib().moe_ffn_forward_save_gu(_ptr(x), _ptr(topk_idx), _ptr(topk_w), _ptr(W1), _ptr(W3),
                                         _ptr(W2), _ptr(Ws1), _ptr(Ws3), _ptr(Ws2), _ptr(y), _ptr(gu),
                                         T, D, F, E, k, _dtype_enum(x.dtype), MOE_VARIANT_UNFUSED,
                                         _ptr(workspace), workspace.numel(), _stream(stream)),
           "moe_ffn_forward_save_gu")
    return y, gu


def forward_noalloc(x, topk_idx, topk_w, W1, W3, W2, shared=None, y=None, variant="unfused",
                    stream=None):
    """y = moe_ffn_forward_noalloc(...): the forward on the library's own
    per-device workspace array (no allocation by the library; ``y`` is
    allocated here only when not given).  Calls overlapping on one GPU race
    on that array."""
    T, D, F, E = _check_layer(x, W1, W3, W2, shared, y)
    k = _check_routing(x, topk_idx, topk_w, T)
    _same_device(x, dict(topk_idx=topk_idx, topk_w=topk_w, **_layer_tensors(W1, W3, W2, shared, y)))
    Ws1, Ws3, Ws2 = shared if shared is not None else (None, None, None)
    if y is None:
        y = torch.empty((T, D), dtype=x.dtype, device=x.device)
    _check(lib().moe_ffn_forward_noalloc(_ptr(x), _ptr(topk_idx), _ptr(topk_w), _ptr(W1), _ptr(W3),
                                         _ptr(W2), _ptr(Ws1), _ptr(Ws3), _ptr(Ws2), _ptr(y), T, D, F,
                                         E, k, _dtype_enum(x.dtype), _variant_enum(variant),
                                         _stream(stream)),
           "moe_ffn_forward_noalloc")
    return y


def expert_permute(topk_idx, E, tile_rows_=1, shared_rows=0, stream=None) -> dict:
    """Stable counting sort of the slots on the device; returns device int32
    tensors counts [E], offsets [E+1], tile_off [E+2], perm, inv [T*k], err [1]."""
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [T,k]")
    T, k = topk_idx.shape
    _expect("topk_idx", topk_idx, (T, k), torch.int32)
    _same_device(topk_idx, {})
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


def device_clock_sample(blocks=1024, stream=None):
    """Issue a clock sample on the stream; returns the device int64 [blocks, 3]
    tensor (compute unit, shader-clock cycles, 100 MHz counter) it will hold."""
    out = torch.empty((blocks, 3), dtype=torch.int64, device="cuda")
    _check(lib().moe_device_clock_sample(_ptr(out), blocks, _stream(stream)), "moe_device_clock_sample")
    return out


def stream_read(buf, sink, stream=None):
    """Read every byte of the device tensor buf once (moe_stream_read) with
    sink.numel() workgroups; sink is a device int32 tensor."""
    if not (buf.is_cuda and sink.is_cuda and sink.dtype == torch.int32 and buf.is_contiguous()):
        raise TypeError("stream_read: buf and sink must be contiguous GPU tensors, sink int32")
    _check(lib().moe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), sink.numel(),
                                 _stream(stream)), "moe_stream_read")


def engine_clock_ghz(before, after):
    """Mean engine clock (GHz) between two device_clock_sample results (host
    copies) of every compute unit sampled in both, keyed by (XCD, unit)."""
    first = {}
    for loc, cyc, rt in before.tolist():
        first.setdefault(loc, (cyc, rt))
    out = {}
    for loc, cyc, rt in after.tolist():
        if loc in first and loc not in out and rt > first[loc][1]:
            out[(loc >> 16, loc & 0xffff)] = (cyc - first[loc][0]) / (rt - first[loc][1]) * 0.1
    return out


def backward_workspace_layout(T, D, F, E, k, has_shared, dtype) -> dict:
    L = BwdWsLayout()
    _check(lib().moe_ffn_backward_workspace_layout(T, D, F, E, k, int(has_shared), _dtype_enum(dtype),
                                                   ctypes.byref(L)),
           "moe_ffn_backward_workspace_layout")
    return L.as_dict()


def backward(x, topk_idx, topk_w, W1, W3, W2, shared, dy, out=None, workspace=None, stream=None,
             events=None, gu=None) -> dict:
    """moe_ffn_backward(...): gradients of the layer for the incoming dy [T,D].
    Returns dx [T,D] (x's dtype), dW1/dW3 [E,D,F], dW2 [E,F,D], dWs1/dWs3
    [D,F], dWs2 [F,D] (None without a shared expert) and dtopk_w [T,k], all
    fp32 except dx.  ``out`` may supply any of these tensors.  ``events``: a
    ctypes array of nine hipEvent_t handles (moe_ffn_backward_timed).
    ``gu``: the gate and up products forward_save_gu returned for the same
    inputs; the call then goes to moe_ffn_backward_cached(_timed), which
    skips their recompute."""
    T, D, F, E = _check_layer(x, W1, W3, W2, shared, None)
    k = _check_routing(x, topk_idx, topk_w, T)
    _expect("dy", dy, (T, D), x.dtype)
    if gu is not None:
        _expect("gu", gu, (T * k + (T if shared is not None else 0), 2 * F), x.dtype)
        _same_device(x, dict(gu=gu))
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
    shapes = dict(dx=((T, D), x.dtype), dW1=((E, D, F), torch.float32), dW3=((E, D, F), torch.float32),
                  dW2=((E, F, D), torch.float32), dtopk_w=((T, k), torch.float32),
                  dWs1=((D, F), torch.float32), dWs3=((D, F), torch.float32),
                  dWs2=((F, D), torch.float32))
    for name, (shape, dtype) in shapes.items():
        if o.get(name) is not None:
            _expect(name, o[name], shape, dtype)
    _same_device(x, dict(topk_idx=topk_idx, topk_w=topk_w, dy=dy,
                         **_layer_tensors(W1, W3, W2, shared, None),
                         **{n: t for n, t in o.items() if n in shapes}))
    Ws1, Ws3, Ws2 = shared if shared is not None else (None, None, None)
    n = backward_workspace_layout(T, D, F, E, k, shared is not None, x.dtype)["total"]
    if workspace is None:
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    _check_workspace(x, workspace, n)
    args = (_ptr(x), _ptr(topk_idx), _ptr(topk_w), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(Ws1),
            _ptr(Ws3), _ptr(Ws2), _ptr(dy), _ptr(o["dx"]), _ptr(o["dW1"]), _ptr(o["dW3"]),
            _ptr(o["dW2"]), _ptr(o["dWs1"]), _ptr(o["dWs3"]), _ptr(o["dWs2"]), _ptr(o["dtopk_w"]),
            T, D, F, E, k, _dtype_enum(x.dtype), _ptr(workspace), workspace.numel(), _stream(stream))
    if gu is not None:
        cargs = args[:9] + (_ptr(gu),) + args[9:]
        if events is None:
            _check(lib().moe_ffn_backward_cached(*cargs), "moe_ffn_backward_cached")
        else:
            _check(lib().moe_ffn_backward_cached_timed(*cargs, events), "moe_ffn_backward_cached_timed")
    elif events is None:
        _check(lib().moe_ffn_backward(*args), "moe_ffn_backward")
    else:
        _check(lib().moe_ffn_backward_timed(*args, events), "moe_ffn_backward_timed")
    return o


def router_topk(x, gate_w, k, stream=None):
    """moe_router_topk: (topk_idx int32 [T,k], topk_w fp32 [T,k]) for x [T,D]
    and gate_w [D,E] of x's dtype."""
    _dtype_enum(x.dtype)
    if x.dim() != 2 or gate_w.dim() != 2:
        raise ValueError("x must be [T,D] and gate_w [D,E]")
    T, D = x.shape
    E = gate_w.shape[1]
    _expect("x", x, (T, D), x.dtype)
    _expect("gate_w", gate_w, (D, E), x.dtype)
    _same_device(x, dict(gate_w=gate_w))
    if not 1 <= k <= E:
        raise ValueError(f"k must be in [1, E={E}], got {k}")
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    _check(lib().moe_router_topk(_ptr(x), _ptr(gate_w), T, D, E, k, _dtype_enum(x.dtype), _ptr(idx),
                                 _ptr(w), _stream(stream)), "moe_router_topk")
    return idx, w


def forward_routed(x, gate_w, W1, W3, W2, shared=None, k=2, y=None, variant="unfused",
                   workspace=None, stream=None, events=None):
    """moe_ffn_forward_routed: returns (y, topk_idx, topk_w)."""
    T, D, F, E = _check_layer(x, W1, W3, W2, shared, y)
    _expect("gate_w", gate_w, (D, E), x.dtype)
    if not 1 <= k <= E:
        raise ValueError(f"k must be in [1, E={E}], got {k}")
    _same_device(x, dict(gate_w=gate_w, **_layer_tensors(W1, W3, W2, shared, y)))
    Ws1, Ws3, Ws2 = shared if shared is not None else (None, None, None)
    if y is None:
        y = torch.empty((T, D), dtype=x.dtype, device=x.device)
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(T, D, F, E, k, shared is not None, x.dtype, variant, x.device)
    _check_workspace(x, workspace, workspace_size(T, D, F, E, k, shared is not None, x.dtype, variant))
    args = (_ptr(x), _ptr(gate_w), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(Ws1), _ptr(Ws3), _ptr(Ws2),
            _ptr(y), _ptr(idx), _ptr(w), T, D, F, E, k, _dtype_enum(x.dtype), _variant_enum(variant),
            _ptr(workspace), workspace.numel(), _stream(stream))
    if events is None:
        _check(lib().moe_ffn_forward_routed(*args), "moe_ffn_forward_routed")
    else:
        _check(lib().moe_ffn_forward_routed_timed(*args, events), "moe_ffn_forward_routed_timed")
    return y, idx, w
