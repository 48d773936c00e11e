// moe_bwd.hip -- host side of the backward entry points declared in
// include/moe_ffn.h: argument validation, workspace carving and the launch
// order
//   permute -> (bf16: weight transposes) -> gate/up recompute -> dh stage
//   -> per-row dx -> dW1/dW3 -> dW2 -> dtopk_w and the dx combine
// on the caller's stream, with no host synchronisation.  A shape the kernels
// do not implement is an error, never a switch to another path ("Triton MoE
// Kernels & Memory Checkpointing", Part A section 9).
#include "moe_ffn.h"
#include "moe_bwd_internal.h"

#include <stdint.h>

namespace {

using namespace moe;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status make_bwd_layout(int64_t T, int D, int F, int E, int k, int has_shared, moe_dtype dt,
                           moe_bwd_ws_layout* L) {
    if (!L) return MOE_ERR_INVALID_ARG;
    if (T < 0 || D <= 0 || F <= 0 || E <= 0 || k < 1 || k > E || E > kMaxExperts)
        return MOE_ERR_INVALID_ARG;
    if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
    const int64_t S = T * (int64_t)k;
    const int64_t R = S + (has_shared ? T : 0);
    if (R >= ((int64_t)1 << 31)) return MOE_ERR_INVALID_ARG;
    if (dt == MOE_BF16 && (D % 64 != 0 || F % 64 != 0)) return MOE_ERR_UNSUPPORTED;
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
    L->chunk_off = take(sizeof(int32_t) * (size_t)(E + 2));
    L->perm = take(sizeof(int32_t) * (size_t)S);
    L->inv = take(sizeof(int32_t) * (size_t)S);
    L->hist = take(sizeof(int32_t) * (size_t)(E + 1) * (size_t)nb);
    L->gu = take(esize * (size_t)R * 2 * (size_t)F);
    L->dgu = take(esize * (size_t)R * 2 * (size_t)F);
    L->hw = take(esize * (size_t)R * (size_t)F);
    L->dxr = take(esize * (size_t)R * (size_t)D);
    L->dwpart = take(sizeof(float) * (size_t)R * (size_t)bwd_dw_blocks(F));
    // bf16: transposed weights for the engine's [K, N] weight tiles
    const size_t G = (size_t)E + (has_shared ? 1 : 0);
    const bool tr = dt == MOE_BF16;
    L->w2t = take(tr ? 2 * G * (size_t)D * (size_t)F : 0);
    L->w13t = take(tr ? 2 * G * 2 * (size_t)F * (size_t)D : 0);
    // dW1/dW3 partials [chunks, D, 2F], then dW2's [chunks, F, D]: both
    // GEMMs run before either reduction
    const size_t MN = 3 * (size_t)D * (size_t)F;
    const int kc = wgrad_chunk_rows(R, D, F);
    L->partial = take(tr ? sizeof(float) * (size_t)wgrad_chunks_upper(R, (int)G, kc) * MN : 0);
    L->zeros = take(tr ? 256 : 0);
    L->total = off;
    L->chunk_rows = tr ? kc : 0;
    L->tile_rows = dt == MOE_BF16 ? kBf16TileRows : kF32TileRows;
    L->hist_blocks = nb;
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_ffn_backward_workspace_layout(int64_t T, int D, int F, int E, int k, int has_shared,
                                             moe_dtype dtype, moe_bwd_ws_layout* layout) {
    return make_bwd_layout(T, D, F, E, k, has_shared, dtype, layout);
}

size_t moe_ffn_backward_workspace_size(int64_t T, int D, int F, int E, int k, int has_shared,
                                       moe_dtype dtype) {
    moe_bwd_ws_layout L;
    return make_bwd_layout(T, D, F, E, k, has_shared, dtype, &L) == MOE_OK ? L.total : 0;
}

}  // extern "C"

namespace {

// The backward; with gu_in (bf16 only) the gate and up products come from
// the caller (the forward that saved them) instead of the recompute launch.
moe_status backward_impl(const void* x, const int32_t* topk_idx, const float* topk_w,
                         const void* W1, const void* W3, const void* W2, const void* Ws1,
                         const void* Ws3, const void* Ws2, const void* dy, void* dx, float* dW1,
                         float* dW3, float* dW2, float* dWs1, float* dWs3, float* dWs2,
                         float* dtopk_w, int64_t T, int D, int F, int E, int k, moe_dtype dtype,
                         void* workspace, size_t ws_bytes, hipStream_t stream, hipEvent_t* events,
                         const void* gu_in) {
    const int nsh = (Ws1 != nullptr) + (Ws3 != nullptr) + (Ws2 != nullptr);
    const int ndsh = (dWs1 != nullptr) + (dWs3 != nullptr) + (dWs2 != nullptr);
    if ((nsh != 0 && nsh != 3) || ndsh != nsh) return MOE_ERR_INVALID_ARG;
    const bool has_shared = nsh == 3;
    moe_bwd_ws_layout L;
    const moe_status st = make_bwd_layout(T, D, F, E, k, has_shared, dtype, &L);
    if (st != MOE_OK) return st;
    if (!W1 || !W3 || !W2 || !dW1 || !dW3 || !dW2 || !workspace) return MOE_ERR_INVALID_ARG;
    if (T > 0 && (!x || !topk_idx || !topk_w || !dy || !dx || !dtopk_w)) return MOE_ERR_INVALID_ARG;
    const void* vec_ptrs[] = {x, W1, W3, W2, Ws1, Ws3, Ws2, dy, dx, dW1, dW3, dW2, dWs1, dWs3, dWs2};
    for (const void* p : vec_ptrs)
        if (p && !aligned(p, 16)) return MOE_ERR_INVALID_ARG;
    if (!aligned(topk_idx, 4) || !aligned(topk_w, 4) || !aligned(dtopk_w, 4) ||
        !aligned(workspace, kAlign))
        return MOE_ERR_INVALID_ARG;
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    if (gu_in && !aligned(gu_in, 16)) return MOE_ERR_INVALID_ARG;

    char* ws = (char*)workspace;
    int32_t* err = (int32_t*)(ws + L.err);
    int32_t* counts = (int32_t*)(ws + L.counts);
    int32_t* offsets = (int32_t*)(ws + L.offsets);
    int32_t* tile_off = (int32_t*)(ws + L.tile_off);
    int32_t* chunk_off = (int32_t*)(ws + L.chunk_off);
    int32_t* perm = (int32_t*)(ws + L.perm);
    int32_t* inv = (int32_t*)(ws + L.inv);
    int32_t* hist = (int32_t*)(ws + L.hist);
    const void* gu = gu_in ? gu_in : ws + L.gu;
    void* dgu = ws + L.dgu;
    void* hw = ws + L.hw;
    void* dxr = ws + L.dxr;
    float* dwpart = (float*)(ws + L.dwpart);
    const int64_t S = T * (int64_t)k;
    const bool bf16 = dtype == MOE_BF16;

    (void)hipGetLastError();
    auto mark = [&](int i) { return events ? hipEventRecord(events[i], stream) : hipSuccess; };
    hipError_t e = mark(0);
    if (e == hipSuccess)
        e = launch_permute(topk_idx, S, E, L.tile_rows, has_shared ? T : 0, counts, offsets,
                           tile_off, perm, inv, err, hist, L.hist_blocks, stream,
                           bf16 ? L.chunk_rows : 0, bf16 ? chunk_off : nullptr);
    if (e == hipSuccess) e = mark(1);
    const BwdArgs a{GroupArgs{offsets, tile_off, perm, S, T, E, k, E + (has_shared ? 1 : 0)},
                    topk_w, D, F, bf16};
    if (T > 0 && bf16) {
        // W2 -> W2t [E(+1), D, F]; W1, W3 -> W13t [E(+1), 2F, D] (W1^T rows first)
        uint16_t* w2t = (uint16_t*)(ws + L.w2t);
        uint16_t* w13t = (uint16_t*)(ws + L.w13t);
        const int64_t df = (int64_t)D * F;
        // the shared expert's matrix, when there is one, as batch E of the same launch
        if (e == hipSuccess)
            e = launch_transpose_bf16(W2, E, F, D, w2t, df, F, 0, stream, has_shared ? Ws2 : nullptr);
        if (e == hipSuccess)
            e = launch_transpose_bf16(W1, E, D, F, w13t, 2 * df, D, 0, stream, has_shared ? Ws1 : nullptr);
        if (e == hipSuccess)
            e = launch_transpose_bf16(W3, E, D, F, w13t, 2 * df, D, F, stream, has_shared ? Ws3 : nullptr);
        if (e == hipSuccess) e = launch_zero_fill(ws + L.zeros, 256, stream);
        if (e == hipSuccess) e = mark(2);
        if (e == hipSuccess && !gu_in)
            e = launch_bwd_gate_up_bf16(a.g, x, W1, W3, Ws1, Ws3, ws + L.gu, D, F, stream);
        if (e == hipSuccess) e = mark(3);
        if (e == hipSuccess)
            e = launch_bwd_dh_bf16(a.g, topk_w, dy, w2t, has_shared ? w2t + E * df : nullptr, gu, dgu,
                                   hw, dwpart, D, F, stream);
        if (e == hipSuccess) e = mark(4);
        if (e == hipSuccess)
            e = launch_down_bf16(a.g, dgu, w13t, has_shared ? w13t + 2 * E * df : nullptr, dxr, D,
                                 2 * F, stream);
        if (e == hipSuccess) e = mark(5);
    } else if (T > 0) {
        if (e == hipSuccess) e = mark(2);
        if (e == hipSuccess) e = launch_bwd_gate_up(a, x, W1, W3, Ws1, Ws3, ws + L.gu, stream);
        if (e == hipSuccess) e = mark(3);
        if (e == hipSuccess) e = launch_bwd_dh(a, dy, W2, Ws2, gu, dgu, hw, dwpart, stream);
        if (e == hipSuccess) e = mark(4);
        if (e == hipSuccess) e = launch_bwd_dx_rows(a, dgu, W1, W3, Ws1, Ws3, dxr, stream);
        if (e == hipSuccess) e = mark(5);
    } else {
        for (int i = 2; i <= 5 && e == hipSuccess; ++i) e = mark(i);
    }
    // weight gradients: every element written, zero for a group without rows
    const GroupArgs chunks{offsets, chunk_off, perm, S, T, E, k, E + (has_shared ? 1 : 0)};
    float* partial13 = (float*)(ws + L.partial);
    float* partial2 = partial13 + (bf16 ? wgrad_chunks_upper(S + (has_shared ? T : 0), chunks.G,
                                                             L.chunk_rows) * 2 * (int64_t)D * F
                                        : 0);
    if (bf16) {
        const void* zeros = ws + L.zeros;
        const int64_t R = S + (has_shared ? T : 0);
        if (e == hipSuccess)
            e = launch_wgrad_bf16(chunks, L.chunk_rows, x, true, dgu, false, D, 2 * F, partial13,
                                  zeros, F, dW1, dW3, dWs1, dWs3, R, stream);
        if (e == hipSuccess) e = mark(6);
        if (e == hipSuccess)
            e = launch_wgrad_bf16(chunks, L.chunk_rows, hw, false, dy, true, F, D, partial2, zeros, D,
                                  dW2, nullptr, dWs2, nullptr, R, stream);
        if (e == hipSuccess) e = mark(7);
        if (e == hipSuccess)
            e = launch_wgrad_reduce(partial13, chunks, D, 2 * F, F, dW1, dW3, dWs1, dWs3, stream);
        if (e == hipSuccess)
            e = launch_wgrad_reduce(partial2, chunks, F, D, D, dW2, nullptr, dWs2, nullptr, stream);
    } else {
        if (e == hipSuccess) e = launch_bwd_dw13(a, x, dgu, dW1, dW3, dWs1, dWs3, stream);
        if (e == hipSuccess) e = mark(6);
        if (e == hipSuccess) e = launch_bwd_dw2(a, hw, dy, dW2, dWs2, stream);
        if (e == hipSuccess) e = mark(7);
    }
    if (T > 0) {
        if (e == hipSuccess) e = launch_bwd_dtopk(a, inv, dwpart, dtopk_w, stream);
        if (e == hipSuccess)
            e = launch_combine(dxr, inv, nullptr, dx, T, D, k, has_shared, bf16, stream);
    }
    if (e == hipSuccess) e = mark(8);
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace

extern "C" {

moe_status moe_ffn_backward_timed(const void* x, const int32_t* topk_idx, const float* topk_w,
                                  const void* W1, const void* W3, const void* W2, const void* Ws1,
                                  const void* Ws3, const void* Ws2, const void* dy, void* dx,
                                  float* dW1, float* dW3, float* dW2, float* dWs1, float* dWs3,
                                  float* dWs2, float* dtopk_w, int64_t T, int D, int F, int E,
                                  int k, moe_dtype dtype, void* workspace, size_t ws_bytes,
                                  hipStream_t stream, hipEvent_t* events) {
    return backward_impl(x, topk_idx, topk_w, W1, W3, W2, Ws1, Ws3, Ws2, dy, dx, dW1, dW3, dW2, dWs1,
                         dWs3, dWs2, dtopk_w, T, D, F, E, k, dtype, workspace, ws_bytes, stream,
                         events, nullptr);
}

moe_status moe_ffn_backward_cached_timed(const void* x, const int32_t* topk_idx,
                                         const float* topk_w, const void* W1, const void* W3,
                                         const void* W2, const void* Ws1, const void* Ws3,
                                         const void* Ws2, const void* gu, const void* dy, void* dx,
                                         float* dW1, float* dW3, float* dW2, float* dWs1,
                                         float* dWs3, float* dWs2, float* dtopk_w, int64_t T, int D,
                                         int F, int E, int k, moe_dtype dtype, void* workspace,
                                         size_t ws_bytes, hipStream_t stream, hipEvent_t* events) {
    if (dtype != MOE_BF16) {
        const int nsh = (Ws1 != nullptr) + (Ws3 != nullptr) + (Ws2 != nullptr);
        moe_bwd_ws_layout L;
        const moe_status st = make_bwd_layout(T, D, F, E, k, nsh == 3, dtype, &L);
        return st != MOE_OK ? st : MOE_ERR_UNSUPPORTED;
    }
    if (T > 0 && !gu) return MOE_ERR_INVALID_ARG;
    return backward_impl(x, topk_idx, topk_w, W1, W3, W2, Ws1, Ws3, Ws2, dy, dx, dW1, dW3, dW2, dWs1,
                         dWs3, dWs2, dtopk_w, T, D, F, E, k, dtype, workspace, ws_bytes, stream,
                         events, T > 0 ? gu : nullptr);
}

moe_status moe_ffn_backward_cached(const void* x, const int32_t* topk_idx, const float* topk_w,
                                   const void* W1, const void* W3, const void* W2, const void* Ws1,
                                   const void* Ws3, const void* Ws2, const void* gu, const void* dy,
                                   void* dx, float* dW1, float* dW3, float* dW2, float* dWs1,
                                   float* dWs3, float* dWs2, float* dtopk_w, int64_t T, int D, int F,
                                   int E, int k, moe_dtype dtype, void* workspace, size_t ws_bytes,
                                   hipStream_t stream) {
    return moe_ffn_backward_cached_timed(x, topk_idx, topk_w, W1, W3, W2, Ws1, Ws3, Ws2, gu, dy, dx,
                                         dW1, dW3, dW2, dWs1, dWs3, dWs2, dtopk_w, T, D, F, E, k,
                                         dtype, workspace, ws_bytes, stream, nullptr);
}

moe_status moe_ffn_backward(const void* x, const int32_t* topk_idx, const float* topk_w,
                            const void* W1, const void* W3, const void* W2, const void* Ws1,
                            const void* Ws3, const void* Ws2, const void* dy, void* dx, float* dW1,
                            float* dW3, float* dW2, float* dWs1, float* dWs3, float* dWs2,
                            float* dtopk_w, int64_t T, int D, int F, int E, int k,
                            moe_dtype dtype, void* workspace, size_t ws_bytes,
                            hipStream_t stream) {
    return moe_ffn_backward_timed(x, topk_idx, topk_w, W1, W3, W2, Ws1, Ws3, Ws2, dy, dx, dW1, dW3,
                                  dW2, dWs1, dWs3, dWs2, dtopk_w, T, D, F, E, k, dtype, workspace,
                                  ws_bytes, stream, nullptr);
}

}  // extern "C"
