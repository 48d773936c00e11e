"""MI355X (gfx950) top-k routed MoE SwiGLU FFN: forward and backward.

Hand-written HIP kernels behind a C ABI (include/moe_ffn.h, built into
libmoe_ffn.so): stable counting-sort expert permute, bf16-MFMA grouped
GEMMs over [W1|W3] with a fused silu(g)*u epilogue and over W2, and a
deterministic unpermute/combine, and the layer's backward.  This package is the Python binding:
torch supplies device memory and streams, nothing else.
"""
from ._lib import (MoeError, alloc_workspace, backward, backward_workspace_layout,  # noqa: F401
                   device_clock_sample, device_error, engine_clock_ghz, expert_permute, forward,
                   forward_noalloc, forward_routed, forward_save_gu, lib, router_topk, status_string, stream_read, tile_rows,
                   workspace_layout, workspace_size, EXPORTS, LIB_PATH, NOALLOC_SCRATCH_BYTES)
