"""C-ABI checks that need no GPU: the library loads, exports every function
include/moe_ffn.h declares, sizes its workspace, and rejects bad arguments on
the host before enqueueing anything (no pointer here is ever dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ffn.h")

gg = pytest.importorskip("grouped_gemm_permute_amd")
from grouped_gemm_permute_amd import _lib as L  # noqa: E402

FAKE = 0x7F0000000000          # 256-byte aligned, never dereferenced by host validation


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    names = declared_functions()
    assert names, "no declarations found"
    assert sorted(L.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def test_status_strings_and_tile_rows():
    for s in range(5):
        assert L.status_string(s).startswith("MOE_")
    assert L.lib().moe_ffn_tile_rows(L.MOE_BF16, 0) == 256
    assert L.lib().moe_ffn_tile_rows(L.MOE_F32, 0) > 0


def test_workspace_layout_is_aligned_and_sized():
    import torch
    lay = L.workspace_layout(32768, 768, 1536, 8, 2, True, torch.bfloat16)
    R = 32768 * 3
    for key in ("err", "counts", "offsets", "tile_off", "perm", "inv", "hist", "h", "Y"):
        assert lay[key] % 256 == 0
    assert lay["err"] == 0
    assert lay["Y"] + R * 768 * 2 <= lay["total"]   # bf16 expert outputs
    assert lay["h"] + R * 1536 * 2 <= lay["Y"]
    assert lay["hist_blocks"] == 65536 // 1024          # 1024-slot permute blocks
    assert L.workspace_size(32768, 768, 1536, 8, 2, True, torch.bfloat16) == lay["total"]
    small = L.workspace_layout(512, 768, 1536, 8, 2, False, torch.bfloat16)
    assert small["hist_blocks"] == 0
    # 128 rows per expert on average: up tiles of 160 rows hold a whole group
    assert small["small_tiles"] == 1 and small["tile_rows"] == 160
    assert lay["small_tiles"] == 0 and lay["tile_rows"] == 256
    # with the shared expert's 512 rows, 160-row tiles would need 12 x 24 up
    # workgroups (two rounds of 256): the tile grows to 256 rows (10 x 24)
    assert L.workspace_layout(512, 768, 1536, 8, 2, True, torch.bfloat16)["tile_rows"] == 256
    # 160 rows per expert on average: 1.25x that is 200 -> 224-row tiles
    assert L.workspace_layout(640, 128, 256, 8, 2, True, torch.bfloat16)["tile_rows"] == 224


def _fwd(**over):
    a = dict(x=FAKE, idx=FAKE, w=FAKE, W1=FAKE, W3=FAKE, W2=FAKE, Ws1=None, Ws3=None, Ws2=None,
             y=FAKE, T=16, D=64, F=128, E=4, k=2, dt=L.MOE_BF16, v=0, ws=FAKE, nbytes=1 << 40)
    a.update(over)
    return L.lib().moe_ffn_forward(a["x"], a["idx"], a["w"], a["W1"], a["W3"], a["W2"], a["Ws1"],
                                   a["Ws3"], a["Ws2"], a["y"], a["T"], a["D"], a["F"], a["E"],
                                   a["k"], a["dt"], a["v"], a["ws"], a["nbytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(k=5), L.MOE_ERR_INVALID_ARG),                 # k > E
    (dict(k=0), L.MOE_ERR_INVALID_ARG),
    (dict(E=0, k=1), L.MOE_ERR_INVALID_ARG),
    (dict(E=1025, k=2), L.MOE_ERR_INVALID_ARG),
    (dict(T=-1), L.MOE_ERR_INVALID_ARG),
    (dict(D=0), L.MOE_ERR_INVALID_ARG),
    (dict(dt=7), L.MOE_ERR_INVALID_ARG),
    (dict(v=9), L.MOE_ERR_INVALID_ARG),
    (dict(x=None), L.MOE_ERR_INVALID_ARG),
    (dict(W2=None), L.MOE_ERR_INVALID_ARG),
    (dict(ws=None), L.MOE_ERR_INVALID_ARG),
    (dict(x=FAKE + 8), L.MOE_ERR_INVALID_ARG),          # misaligned activations
    (dict(idx=FAKE + 2), L.MOE_ERR_INVALID_ARG),
    (dict(ws=FAKE + 64), L.MOE_ERR_INVALID_ARG),         # workspace must be 256-byte aligned
    (dict(Ws1=FAKE), L.MOE_ERR_INVALID_ARG),             # only part of the shared expert
    (dict(D=96), L.MOE_ERR_UNSUPPORTED),                 # bf16 needs D % 64 == 0
    (dict(F=200), L.MOE_ERR_UNSUPPORTED),
    (dict(v=1, D=192), L.MOE_ERR_UNSUPPORTED),           # fused needs D % 128 == 0
    (dict(v=1, D=1152), L.MOE_ERR_UNSUPPORTED),          # fused needs D <= 1024
    (dict(v=1, F=192), L.MOE_ERR_UNSUPPORTED),           # fused needs F % 128 == 0
    (dict(v=1, dt=L.MOE_F32), L.MOE_ERR_UNSUPPORTED),    # fused is bf16 only
    (dict(nbytes=1024), L.MOE_ERR_WORKSPACE),
    (dict(T=1 << 30, k=2), L.MOE_ERR_INVALID_ARG),       # T*k + T >= 2^31
    (dict(T=0, x=None, idx=None, w=None, y=None), L.MOE_OK),   # nothing to do, nothing launched
])
def test_forward_rejects_bad_arguments_on_host(over, status):
    assert _fwd(**over) == status


def test_fused_layout_64_row_tiles_and_partial_outputs():
    """The fused variant keeps h on chip; its h slot holds the fp32 partial
    outputs of the tiles it shares out over several workgroups: at most 256
    workgroups of 64 x D floats, fewer when the tiles times the 256-column
    chunks are fewer."""
    import torch
    D, F, E, k = 1024, 4096, 16, 2
    lay = L.workspace_layout(16384, D, F, E, k, False, torch.bfloat16, "fused")
    assert lay["tile_rows"] == 64 and lay["Y"] - lay["h"] == 256 * 64 * D * 4
    assert L.lib().moe_ffn_tile_rows(L.MOE_BF16, L.MOE_VARIANT_FUSED) == 64
    # 32 rows in 2 groups: at most 3 tiles x 1 chunk of 256 columns
    lay = L.workspace_layout(32, 256, 256, 2, 1, False, torch.bfloat16, "fused")
    assert lay["Y"] - lay["h"] == 3 * 64 * 256 * 4
    # 1024 rows in 16 groups, F = 384: at most 32 tiles x 2 chunks
    lay = L.workspace_layout(512, D, 384, E, k, False, torch.bfloat16, "fused")
    assert lay["Y"] - lay["h"] == 64 * 64 * D * 4


def test_stream_read_rejects_bad_arguments_on_host():
    lib = L.lib()
    assert lib.moe_stream_read(None, 1024, FAKE, 8, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_stream_read(FAKE, 1000, FAKE, 8, None) == L.MOE_ERR_INVALID_ARG   # not 16-byte sized
    assert lib.moe_stream_read(FAKE, 0, FAKE, 8, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_stream_read(FAKE, 1024, FAKE, 0, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_stream_read(FAKE + 8, 1024, FAKE, 8, None) == L.MOE_ERR_INVALID_ARG  # misaligned


def test_permute_rejects_bad_arguments_on_host():
    lib = L.lib()
    args = [FAKE, 10, 2, 4, 256, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None]
    bad = list(args); bad[3] = 0
    assert lib.moe_expert_permute(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(args); bad[4] = 0
    assert lib.moe_expert_permute(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(args); bad[6] = None
    assert lib.moe_expert_permute(*bad) == L.MOE_ERR_INVALID_ARG
    big = list(args); big[1] = 10000                     # needs scratch for the multi-block path
    assert lib.moe_ffn_forward is not None
    assert lib.moe_expert_permute(*big) == L.MOE_ERR_WORKSPACE
    assert lib.moe_expert_permute_scratch_size(10000, 2, 4) == 5 * ((20000 + 1023) // 1024) * 4
    assert lib.moe_expert_permute_scratch_size(100, 2, 4) == 0


def test_device_error_rejects_null():
    v = ctypes.c_int32()
    assert L.lib().moe_ffn_get_device_error(None, None, ctypes.byref(v)) == L.MOE_ERR_INVALID_ARG


def test_backward_layout_is_aligned_and_sized():
    import torch
    lay = L.backward_workspace_layout(32768, 768, 1536, 8, 2, True, torch.bfloat16)
    R = 32768 * 3
    for key in ("err", "counts", "offsets", "tile_off", "perm", "inv", "hist", "gu", "dgu", "hw",
                "dxr", "dwpart"):
        assert lay[key] % 256 == 0
    assert lay["gu"] + R * 2 * 1536 * 2 <= lay["dgu"]
    assert lay["dgu"] + R * 2 * 1536 * 2 <= lay["hw"]
    assert lay["hw"] + R * 1536 * 2 <= lay["dxr"]
    assert lay["dxr"] + R * 768 * 2 <= lay["dwpart"]
    assert lay["dwpart"] + R * (1536 // 64) * 4 <= lay["total"]
    assert L.lib().moe_ffn_backward_workspace_size(32768, 768, 1536, 8, 2, 1, L.MOE_BF16) == lay["total"]


def _bwd(**over):
    a = dict(x=FAKE, idx=FAKE, w=FAKE, W1=FAKE, W3=FAKE, W2=FAKE, Ws1=None, Ws3=None, Ws2=None,
             dy=FAKE, dx=FAKE, dW1=FAKE, dW3=FAKE, dW2=FAKE, dWs1=None, dWs3=None, dWs2=None,
             dtw=FAKE, T=16, D=64, F=128, E=4, k=2, dt=L.MOE_BF16, ws=FAKE, nbytes=1 << 40)
    a.update(over)
    return L.lib().moe_ffn_backward(
        a["x"], a["idx"], a["w"], a["W1"], a["W3"], a["W2"], a["Ws1"], a["Ws3"], a["Ws2"], a["dy"],
        a["dx"], a["dW1"], a["dW3"], a["dW2"], a["dWs1"], a["dWs3"], a["dWs2"], a["dtw"], a["T"],
        a["D"], a["F"], a["E"], a["k"], a["dt"], a["ws"], a["nbytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(k=5), L.MOE_ERR_INVALID_ARG),
    (dict(T=-1), L.MOE_ERR_INVALID_ARG),
    (dict(dt=3), L.MOE_ERR_INVALID_ARG),
    (dict(dy=None), L.MOE_ERR_INVALID_ARG),
    (dict(dx=None), L.MOE_ERR_INVALID_ARG),
    (dict(dW2=None), L.MOE_ERR_INVALID_ARG),
    (dict(dtw=None), L.MOE_ERR_INVALID_ARG),
    (dict(dx=FAKE + 8), L.MOE_ERR_INVALID_ARG),
    (dict(dW1=FAKE + 4), L.MOE_ERR_INVALID_ARG),
    (dict(Ws1=FAKE, Ws3=FAKE, Ws2=FAKE), L.MOE_ERR_INVALID_ARG),     # shared weights without their gradients
    (dict(dWs1=FAKE, dWs3=FAKE, dWs2=FAKE), L.MOE_ERR_INVALID_ARG),  # gradients without shared weights
    (dict(D=96), L.MOE_ERR_UNSUPPORTED),
    (dict(nbytes=1024), L.MOE_ERR_WORKSPACE),
    (dict(ws=FAKE + 64), L.MOE_ERR_INVALID_ARG),
])
def test_backward_rejects_bad_arguments_on_host(over, status):
    assert _bwd(**over) == status


@pytest.mark.parametrize("args,status", [
    (dict(E=65, k=2), L.MOE_ERR_UNSUPPORTED),            # more experts than one wavefront routes
    (dict(D=100), L.MOE_ERR_UNSUPPORTED),                # D % 8 != 0
    (dict(D=1024, E=32), L.MOE_ERR_UNSUPPORTED),         # gate matrix over 16384 entries
    (dict(k=9), L.MOE_ERR_INVALID_ARG),                  # k > E
    (dict(x=None), L.MOE_ERR_INVALID_ARG),
    (dict(idx=FAKE + 2), L.MOE_ERR_INVALID_ARG),
    (dict(dt=5), L.MOE_ERR_INVALID_ARG),
    (dict(T=0, x=None, idx=None, w=None), L.MOE_OK),
])
def test_router_rejects_bad_arguments_on_host(args, status):
    a = dict(x=FAKE, g=FAKE, T=16, D=64, E=8, k=2, dt=L.MOE_BF16, idx=FAKE, w=FAKE)
    a.update(args)
    assert L.lib().moe_router_topk(a["x"], a["g"], a["T"], a["D"], a["E"], a["k"], a["dt"], a["idx"],
                                   a["w"], None) == status
