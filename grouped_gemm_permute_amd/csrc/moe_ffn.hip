// moe_ffn.hip -- host side of the C ABI declared in include/moe_ffn.h:
// argument validation, workspace carving and the launch order
//   permute -> up+SwiGLU grouped GEMM -> down grouped GEMM -> combine
// on the caller's stream, with no host synchronisation.
//
// The error conventions follow the no-silent-fallback rule of "Triton MoE
// Kernels & Memory Checkpointing" (Part A, section 9): a shape the kernels do
// not implement is an error (MOE_ERR_UNSUPPORTED), never a silent switch to
// another path or precision.
#include "moe_ffn.h"
#include "moe_internal.h"
#include "moe_router_internal.h"

#include <stdint.h>

#include <mutex>

namespace {

using namespace moe;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status make_layout(int64_t T, int D, int F, int E, int k, int has_shared, moe_dtype dt,
                       moe_variant v, moe_ws_layout* L) {
    if (!L) return MOE_ERR_INVALID_ARG;
    if (T < 0 || D <= 0 || F <= 0 || E <= 0 || k < 1 || k > E || E > kMaxExperts)
        return MOE_ERR_INVALID_ARG;
    if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
    if (v != MOE_VARIANT_UNFUSED && v != MOE_VARIANT_FUSED) return MOE_ERR_INVALID_ARG;
    const int64_t S = T * (int64_t)k;
    const int64_t R = S + (has_shared ? T : 0);
    if (R >= ((int64_t)1 << 31)) return MOE_ERR_INVALID_ARG;
    if (dt == MOE_BF16 && (D % 64 != 0 || F % 64 != 0)) return MOE_ERR_UNSUPPORTED;
    if (v == MOE_VARIANT_FUSED && (dt != MOE_BF16 || D % 128 != 0 || D > 1024 || F % 128 != 0))
        return MOE_ERR_UNSUPPORTED;
    const bool fused = v == MOE_VARIANT_FUSED;

    const size_t esize = dt == MOE_BF16 ? 2 : 4;
    const int nb = permute_hist_blocks(S);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    L->err = take(sizeof(int32_t));
    L->counts = take(sizeof(int32_t) * (size_t)E);
    L->offsets = take(sizeof(int32_t) * (size_t)(E + 1));
    L->tile_off = take(sizeof(int32_t) * (size_t)(E + 2));
    L->tile_off64 = take(sizeof(int32_t) * (size_t)(E + 2));
    L->perm = take(sizeof(int32_t) * (size_t)S);
    L->inv = take(sizeof(int32_t) * (size_t)S);
    // multi-block permute histogram; kRouterSub columns per block when the
    // router writes it
    L->hist = take(sizeof(int32_t) * (size_t)(E + 1) * (size_t)nb * kRouterSub);
    // The fused variant keeps h on chip; this slot then holds the fp32
    // partial outputs of the tiles it shares out over several workgroups.
    const int G = E + (has_shared ? 1 : 0);
    L->h = take(fused ? fused_partial_bytes(R, G, D, F) : esize * (size_t)R * (size_t)F);
    L->Y = take(esize * (size_t)R * (size_t)D);
    L->total = off;
    // bf16 unfused: groups averaging under one 256-row tile are bound by
    // streaming their weights; they run on the small-tile kernels.
    // Their up GEMM tiles hold a whole typical group (tile_off); the down
    // GEMM runs on 64-row tiles (tile_off64).
    L->small_tiles = (!fused && dt == MOE_BF16 && R < (int64_t)kBf16TileRows * G) ? 1 : 0;
    L->tile_rows = fused ? kFusedTileRows
                         : (dt == MOE_BF16 ? (L->small_tiles ? 32 * slab_row_blocks(S, has_shared ? T : 0, E, F)
                                                             : kBf16TileRows)
                                           : kF32TileRows);
    L->hist_blocks = nb;
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape or variant not implemented";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
        case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime error";
    }
    return "MOE_ERR_UNKNOWN";
}

int moe_ffn_tile_rows(moe_dtype dtype, moe_variant variant) {
    if (variant == MOE_VARIANT_FUSED) return kFusedTileRows;
    return dtype == MOE_BF16 ? kBf16TileRows : kF32TileRows;
}

moe_status moe_ffn_workspace_layout(int64_t T, int D, int F, int E, int k, int has_shared,
                                    moe_dtype dtype, moe_variant variant, moe_ws_layout* layout) {
    return make_layout(T, D, F, E, k, has_shared, dtype, variant, layout);
}

size_t moe_ffn_workspace_size(int64_t T, int D, int F, int E, int k, int has_shared,
                              moe_dtype dtype, moe_variant variant) {
    moe_ws_layout L;
    return make_layout(T, D, F, E, k, has_shared, dtype, variant, &L) == MOE_OK ? L.total : 0;
}

size_t moe_expert_permute_scratch_size(int64_t T, int k, int E) {
    if (T < 0 || k < 1 || E < 1 || E > kMaxExperts) return 0;
    return sizeof(int32_t) * (size_t)(E + 1) * (size_t)permute_hist_blocks(T * (int64_t)k);
}

moe_status moe_expert_permute(const int32_t* topk_idx, int64_t T, int k, int E, int tile_rows,
                              int64_t shared_rows, int32_t* counts, int32_t* offsets,
                              int32_t* tile_off, int32_t* perm, int32_t* inv, int32_t* err,
                              void* scratch, size_t scratch_bytes, hipStream_t stream) {
    if (T < 0 || k < 1 || E < 1 || E > kMaxExperts || tile_rows < 1 || shared_rows < 0)
        return MOE_ERR_INVALID_ARG;
    const int64_t S = T * (int64_t)k;
    if (S >= ((int64_t)1 << 31)) return MOE_ERR_INVALID_ARG;
    if (!counts || !offsets || !tile_off || !err) return MOE_ERR_INVALID_ARG;
    if (S > 0 && (!topk_idx || !perm || !inv)) return MOE_ERR_INVALID_ARG;
    const int nb = permute_hist_blocks(S);
    const size_t need = sizeof(int32_t) * (size_t)(E + 1) * (size_t)nb;
    if (scratch_bytes < need || (need > 0 && !scratch)) return MOE_ERR_WORKSPACE;
    if (need > 0 && !aligned(scratch, 4)) return MOE_ERR_INVALID_ARG;
    (void)hipGetLastError();
    if (launch_permute(topk_idx, S, E, tile_rows, shared_rows, counts, offsets, tile_off, perm, inv,
                       err, (int32_t*)scratch, nb, stream) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

}  // extern "C"

namespace {

// The forward; with gate_w the router writes topk_idx / topk_w first (and,
// when the permute can take it, the permute's histogram).
moe_status forward_impl(const void* x, const void* gate_w, const int32_t* topk_idx,
                        const float* topk_w, const void* W1, const void* W3, const void* W2,
                        const void* Ws1, const void* Ws3, const void* Ws2, void* y, int64_t T, int D,
                        int F, int E, int k, moe_dtype dtype, moe_variant variant, void* workspace,
                        size_t ws_bytes, hipStream_t stream, hipEvent_t* events, void* gu = nullptr) {
    const int nsh = (Ws1 != nullptr) + (Ws3 != nullptr) + (Ws2 != nullptr);
    if (nsh != 0 && nsh != 3) return MOE_ERR_INVALID_ARG;
    const bool has_shared = nsh == 3;
    moe_ws_layout L;
    const moe_status st = make_layout(T, D, F, E, k, has_shared, dtype, variant, &L);
    if (st != MOE_OK) return st;
    if (!W1 || !W3 || !W2 || !workspace) return MOE_ERR_INVALID_ARG;
    if (T > 0 && (!x || !topk_idx || !topk_w || !y)) return MOE_ERR_INVALID_ARG;
    const void* vec_ptrs[] = {x, W1, W3, W2, Ws1, Ws3, Ws2, y};
    for (const void* p : vec_ptrs)
        if (p && !aligned(p, 16)) return MOE_ERR_INVALID_ARG;
    if (!aligned(topk_idx, 4) || !aligned(topk_w, 4) || !aligned(workspace, kAlign))
        return MOE_ERR_INVALID_ARG;
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    if (T == 0) return MOE_OK;
    if (gu && !aligned(gu, 16)) return MOE_ERR_INVALID_ARG;

    char* ws = (char*)workspace;
    int32_t* err = (int32_t*)(ws + L.err);
    int32_t* counts = (int32_t*)(ws + L.counts);
    int32_t* offsets = (int32_t*)(ws + L.offsets);
    int32_t* tile_off = (int32_t*)(ws + L.tile_off);
    int32_t* tile_off64 = (int32_t*)(ws + L.tile_off64);
    int32_t* perm = (int32_t*)(ws + L.perm);
    int32_t* inv = (int32_t*)(ws + L.inv);
    int32_t* hist = (int32_t*)(ws + L.hist);
    void* h = ws + L.h;
    void* Y = ws + L.Y;
    const int64_t S = T * (int64_t)k;

    (void)hipGetLastError();
    auto mark = [&](int i) {
        return events ? hipEventRecord(events[i], stream) : hipSuccess;
    };
    if (mark(0) != hipSuccess) return MOE_ERR_HIP;
    // Small chunks with at most kPermuteSingleMax slots: the up GEMM does the
    // counting sort itself (no permute launch); it writes the same outputs.
    const bool sort_in_up = dtype == MOE_BF16 && variant == MOE_VARIANT_UNFUSED && L.small_tiles &&
                            S <= kPermuteSingleMax && E <= kRouteMaxExperts;
    if (gate_w) {
        const bool fine = !sort_in_up && permute_fine_ok(S, E, kRouterSub);
        if (launch_router(x, gate_w, T, D, E, k, dtype == MOE_BF16, (int32_t*)topk_idx,
                          (float*)topk_w, fine ? hist : nullptr, stream) != hipSuccess)
            return MOE_ERR_HIP;
        if (sort_in_up) {
        } else if (fine) {
            if (launch_permute_from_hist(topk_idx, S, E, L.tile_rows, has_shared ? T : 0, counts,
                                         offsets, tile_off, perm, inv, err, hist, kRouterSub, stream,
                                         64, tile_off64) != hipSuccess)
                return MOE_ERR_HIP;
        } else if (launch_permute(topk_idx, S, E, L.tile_rows, has_shared ? T : 0, counts, offsets,
                                  tile_off, perm, inv, err, hist, L.hist_blocks, stream, 64,
                                  tile_off64) != hipSuccess) {
            return MOE_ERR_HIP;
        }
    } else if (!sort_in_up &&
               launch_permute(topk_idx, S, E, L.tile_rows, has_shared ? T : 0, counts, offsets,
                              tile_off, perm, inv, err, hist, L.hist_blocks, stream, 64,
                              tile_off64) != hipSuccess) {
        return MOE_ERR_HIP;
    }
    if (mark(1) != hipSuccess) return MOE_ERR_HIP;

    GroupArgs g{offsets, tile_off, perm, S, T, E, k, E + (has_shared ? 1 : 0)};
    hipError_t e;
    if (variant == MOE_VARIANT_FUSED) {
        // one launch does up, SwiGLU and down (mark 2); the sum of the split
        // tiles' partial outputs follows (mark 3)
        e = launch_fused_bf16(g, x, W1, W3, W2, Ws1, Ws3, Ws2, Y, (float*)h, D, F, stream);
        if (e == hipSuccess) e = mark(2);
        if (e == hipSuccess) e = launch_fused_reduce(g, (const float*)h, Y, D, F, stream);
    } else if (sort_in_up) {
        e = launch_up_swiglu_bf16_slab_routed(g, L.tile_rows / 32, topk_idx, counts, offsets, tile_off,
                                              tile_off64, perm, inv, err, x, W1, W3, Ws1, Ws3, W2, Ws2, h, D,
                                              F, stream, gu);
        if (e == hipSuccess) e = mark(2);
    } else if (dtype == MOE_BF16 && L.small_tiles) {
        e = launch_up_swiglu_bf16_slab(g, L.tile_rows / 32, x, W1, W3, Ws1, Ws3, h, D, F, stream, gu);
        if (e == hipSuccess) e = mark(2);
    } else if (dtype == MOE_BF16) {
        e = gu ? launch_up_swiglu_gu_bf16(g, x, W1, W3, Ws1, Ws3, h, gu, D, F, stream)
               : launch_up_swiglu_bf16(g, x, W1, W3, Ws1, Ws3, h, D, F, stream);
        if (e == hipSuccess) e = mark(2);
    } else {
        e = launch_up_swiglu_f32(g, (const float*)x, (const float*)W1, (const float*)W3,
                                 (const float*)Ws1, (const float*)Ws3, (float*)h, D, F, stream);
        if (e == hipSuccess) e = mark(2);
    }
    if (e == hipSuccess && variant != MOE_VARIANT_FUSED) {
        if (dtype == MOE_BF16 && L.small_tiles) {
            GroupArgs g64 = g;
            g64.tile_off = tile_off64;
            e = launch_down_bf16_small(g64, h, W2, Ws2, Y, D, F, stream);
        }
        else if (dtype == MOE_BF16)
            e = launch_down_bf16(g, h, W2, Ws2, Y, D, F, stream);
        else
            e = launch_down_f32(g, (const float*)h, (const float*)W2, (const float*)Ws2, (float*)Y,
                                D, F, stream);
    }
    if (e == hipSuccess) e = mark(3);
    if (e == hipSuccess)
        e = launch_combine(Y, inv, topk_w, y, T, D, k, has_shared, dtype == MOE_BF16, stream);
    if (e == hipSuccess) e = mark(4);
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

bool router_shape_ok(int D, int E) {
    return E <= kRouterMaxExperts && D % 8 == 0 && (int64_t)D * E <= kRouterMaxGateElems;
}

}  // namespace

extern "C" {

moe_status moe_ffn_forward_timed(const void* x, const int32_t* topk_idx, const float* topk_w,
                                 const void* W1, const void* W3, const void* W2, const void* Ws1,
                                 const void* Ws3, const void* Ws2, void* y, int64_t T, int D,
                                 int F, int E, int k, moe_dtype dtype, moe_variant variant,
                                 void* workspace, size_t ws_bytes, hipStream_t stream,
                                 hipEvent_t* events) {
    return forward_impl(x, nullptr, topk_idx, topk_w, W1, W3, W2, Ws1, Ws3, Ws2, y, T, D, F, E, k,
                        dtype, variant, workspace, ws_bytes, stream, events);
}

moe_status moe_router_topk(const void* x, const void* gate_w, int64_t T, int D, int E, int k,
                           moe_dtype dtype, int32_t* topk_idx, float* topk_w, hipStream_t stream) {
    if (T < 0 || D <= 0 || E < 1 || k < 1 || k > E || (dtype != MOE_F32 && dtype != MOE_BF16))
        return MOE_ERR_INVALID_ARG;
    if (!router_shape_ok(D, E)) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !gate_w || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(gate_w, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4))
        return MOE_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return launch_router(x, gate_w, T, D, E, k, dtype == MOE_BF16, topk_idx, topk_w, nullptr,
                         stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_ffn_forward_routed_timed(const void* x, const void* gate_w, const void* W1,
                                        const void* W3, const void* W2, const void* Ws1,
                                        const void* Ws3, const void* Ws2, void* y,
                                        int32_t* topk_idx, float* topk_w, int64_t T, int D, int F,
                                        int E, int k, moe_dtype dtype, moe_variant variant,
                                        void* workspace, size_t ws_bytes, hipStream_t stream,
                                        hipEvent_t* events) {
    if (T < 0 || D <= 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
    if (!router_shape_ok(D, E)) return MOE_ERR_UNSUPPORTED;
    if (T > 0 && !gate_w) return MOE_ERR_INVALID_ARG;
    if (gate_w && !aligned(gate_w, 4)) return MOE_ERR_INVALID_ARG;
    return forward_impl(x, T > 0 ? gate_w : nullptr, topk_idx, topk_w, W1, W3, W2, Ws1, Ws3, Ws2, y,
                        T, D, F, E, k, dtype, variant, workspace, ws_bytes, stream, events);
}

moe_status moe_ffn_forward_routed(const void* x, const void* gate_w, const void* W1, const void* W3,
                                  const void* W2, const void* Ws1, const void* Ws3, const void* Ws2,
                                  void* y, int32_t* topk_idx, float* topk_w, int64_t T, int D,
                                  int F, int E, int k, moe_dtype dtype, moe_variant variant,
                                  void* workspace, size_t ws_bytes, hipStream_t stream) {
    return moe_ffn_forward_routed_timed(x, gate_w, W1, W3, W2, Ws1, Ws3, Ws2, y, topk_idx, topk_w, T,
                                        D, F, E, k, dtype, variant, workspace, ws_bytes, stream,
                                        nullptr);
}

moe_status moe_ffn_forward_save_gu(const void* x, const int32_t* topk_idx, const float* topk_w,
                                   const void* W1, const void* W3, const void* W2, const void* Ws1,
                                   const void* Ws3, const void* Ws2, void* y, void* gu, int64_t T,
                                   int D, int F, int E, int k, moe_dtype dtype, moe_variant variant,
                                   void* workspace, size_t ws_bytes, hipStream_t stream) {
    // the gate and up products exist as bf16 tiles only on the unfused bf16 path
    if (dtype != MOE_BF16 || variant != MOE_VARIANT_UNFUSED) {
        moe_ws_layout L;
        const int nsh = (Ws1 != nullptr) + (Ws3 != nullptr) + (Ws2 != nullptr);
        const moe_status st = make_layout(T, D, F, E, k, nsh == 3, dtype, variant, &L);
        return st != MOE_OK ? st : MOE_ERR_UNSUPPORTED;
    }
    if (T > 0 && !gu) return MOE_ERR_INVALID_ARG;
    return forward_impl(x, nullptr, topk_idx, topk_w, W1, W3, W2, Ws1, Ws3, Ws2, y, T, D, F, E, k,
                        dtype, variant, workspace, ws_bytes, stream, nullptr, gu);
}

moe_status moe_ffn_forward(const void* x, const int32_t* topk_idx, const float* topk_w,
                           const void* W1, const void* W3, const void* W2, const void* Ws1,
                           const void* Ws3, const void* Ws2, void* y, int64_t T, int D, int F,
                           int E, int k, moe_dtype dtype, moe_variant variant, void* workspace,
                           size_t ws_bytes, hipStream_t stream) {
    return moe_ffn_forward_timed(x, topk_idx, topk_w, W1, W3, W2, Ws1, Ws3, Ws2, y, T, D, F, E, k,
                                 dtype, variant, workspace, ws_bytes, stream, nullptr);
}

}  // extern "C"

namespace {

// Workspace of moe_ffn_forward_noalloc: one array per device, resolved to a
// device address once per device with hipGetSymbolAddress (the array's name
// in host code is only a host-side stand-in and must never reach a kernel).
__device__ __attribute__((aligned(256))) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, or null.
void* scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

moe_status moe_ffn_forward_noalloc(const void* x, const int32_t* topk_idx, const float* topk_w,
                                   const void* W1, const void* W3, const void* W2, const void* Ws1,
                                   const void* Ws3, const void* Ws2, void* y, int64_t T, int D,
                                   int F, int E, int k, moe_dtype dtype, moe_variant variant,
                                   hipStream_t stream) {
    const int nsh = (Ws1 != nullptr) + (Ws3 != nullptr) + (Ws2 != nullptr);
    if (nsh != 0 && nsh != 3) return MOE_ERR_INVALID_ARG;
    moe_ws_layout L;
    const moe_status st = make_layout(T, D, F, E, k, nsh == 3, dtype, variant, &L);
    if (st != MOE_OK) return st;
    if (L.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    void* ws = scratch_ptr();
    if (!ws) return MOE_ERR_HIP;
    return forward_impl(x, nullptr, topk_idx, topk_w, W1, W3, W2, Ws1, Ws3, Ws2, y, T, D, F, E, k,
                        dtype, variant, ws, MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

moe_status moe_ffn_get_device_error(const void* workspace, hipStream_t stream, int32_t* out) {
    if (!workspace || !out) return MOE_ERR_INVALID_ARG;
    if (hipMemcpyAsync(out, workspace, sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess)
        return MOE_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

}  // extern "C"
