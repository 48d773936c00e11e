// moe_bwd_internal.h -- launchers of the backward pass shared between the
// translation units of libmoe_ffn.so.  Not part of the public ABI.
#pragma once

#include "moe_internal.h"

namespace moe {

// Width of the column blocks whose partial sums of dy . o the dh kernel
// writes (one fp32 per row and block).
constexpr int kBwdDwBlock = 64;
inline int bwd_dw_blocks(int F) { return (F + kBwdDwBlock - 1) / kBwdDwBlock; }

// Everything the backward kernels read about the problem besides the
// tensors of one stage.
struct BwdArgs {
    GroupArgs g;
    const float* topk_w;   // [S] routing weight of each slot
    int D, F;
    bool bf16;             // element type of x, dy, weights and the row buffers
};

// gu[p] = [x W1 | x W3] of row p (gate in columns 0..F-1, up in F..2F-1),
// fp32 accumulation, stored in the row element type.
hipError_t launch_bwd_gate_up(const BwdArgs& a, const void* x, const void* W1, const void* W3,
                              const void* Ws1, const void* Ws3, void* gu, hipStream_t s);

// From dh' = dy[tok(p)] W2[grp]^T (fp32 accumulation) and the row's g, u:
//   dwpart[p][b] = sum over columns f of block b of dh'[f] * h[f], h = silu(g) * u
//   dgu[p] = [dg | du] with dh = w dh', dg = dh * u * silu'(g), du = dh * silu(g)
//   hw[p]  = w * h
// (w = the routing weight of the row's slot, 1 on shared rows).
hipError_t launch_bwd_dh(const BwdArgs& a, const void* dy, const void* W2, const void* Ws2,
                         const void* gu, void* dgu, void* hw, float* dwpart, hipStream_t s);

// dxr[p] = dg W1[grp]^T + du W3[grp]^T (fp32 accumulation, row element type).
hipError_t launch_bwd_dx_rows(const BwdArgs& a, const void* dgu, const void* W1, const void* W3,
                              const void* Ws1, const void* Ws3, void* dxr, hipStream_t s);

// Weight gradients, fp32, every element written (zero for an empty group):
//   [dW1 | dW3][grp] = sum over the group's rows p of x[tok(p)]^T dgu[p]
//   dW2[grp]         = sum over the group's rows p of hw[p]^T dy[tok(p)]
hipError_t launch_bwd_dw13(const BwdArgs& a, const void* x, const void* dgu, float* dW1,
                           float* dW3, float* dWs1, float* dWs3, hipStream_t s);
hipError_t launch_bwd_dw2(const BwdArgs& a, const void* hw, const void* dy, float* dW2,
                          float* dWs2, hipStream_t s);

// dtopk_w[s] = sum_b dwpart[inv[s]][b] in b order (0 for an invalid slot).
hipError_t launch_bwd_dtopk(const BwdArgs& a, const int32_t* inv, const float* dwpart,
                            float* dtopk_w, hipStream_t s);

// bf16 MFMA versions (gemm_bf16.hip), same results up to summation order.
// gate_up: as launch_bwd_gate_up.  dh: as launch_bwd_dh with the transposed
// down weights W2t [E, D, F] (Ws2t [D, F]).  The dx rows run as
// launch_down_bf16 with F := 2F over the stacked transposes [W1^T ; W3^T]
// ([E, 2F, D]) and A = dgu.  Needs D, F multiples of 64.
hipError_t launch_bwd_gate_up_bf16(const GroupArgs& g, const void* x, const void* W1, const void* W3,
                                   const void* Ws1, const void* Ws3, void* gu, int D, int F,
                                   hipStream_t s);
hipError_t launch_bwd_dh_bf16(const GroupArgs& g, const float* topk_w, const void* dy,
                              const void* W2t, const void* Ws2t, const void* gu, void* dgu, void* hw,
                              float* dwpart, int D, int F, hipStream_t s);

// Weight gradients on bf16 MFMA (gemm_bf16_wgrad.hip).  Each group's rows
// are cut into chunks of KC rows (chunks.tile_off: the chunk prefix of the
// permute, KC rows per tile); every chunk's partial sum
//   sum over its rows p of A[p]^T B[p]   (A [., M] row p or its token's row,
//                                         B [., N] likewise)
// goes to partial [chunks, M, N] in fp32 (launch_wgrad_bf16; a one-chunk
// group writes its result directly), and launch_wgrad_reduce adds the
// groups' chunk partials in chunk order: columns n < split into out0
// [G', M, split], the rest into out1 [G', M, N - split] (the shared group
// into out0_sh / out1_sh), zero for a group without rows.  zeros: at least
// 16 zero bytes.  Needs M, N multiples of 64, KC a multiple of 32 no larger
// than kWgradChunkRows.
constexpr int kWgradChunkRows = 4096;
int64_t wgrad_chunks_upper(int64_t R, int G, int KC);
// Chunk height for R rows (512 .. kWgradChunkRows, a multiple of 256).
int wgrad_chunk_rows(int64_t R, int D, int F);
hipError_t launch_wgrad_bf16(const GroupArgs& chunks, int KC, const void* am, bool gather_m,
                             const void* bn, bool gather_n, int M, int N, float* partial,
                             const void* zeros, int split, float* out0, float* out1,
                             float* out0_sh, float* out1_sh, int64_t R, hipStream_t s);
hipError_t launch_wgrad_reduce(const float* partial, const GroupArgs& chunks, int M, int N, int split,
                               float* out0, float* out1, float* out0_sh, float* out1_sh,
                               hipStream_t s);
hipError_t launch_zero_fill(void* p, int64_t bytes, hipStream_t s);

// dst[b][dst_row0 + c][r] = src[b][r][c] for b < batches, r < rows, c < cols
// (bf16, rows and cols multiples of 64); dst rows hold dst_ld elements and
// dst batches are dst_batch_stride elements apart.  With src_extra, batch
// `batches` (one more) is read from that matrix instead.
hipError_t launch_transpose_bf16(const void* src, int64_t batches, int rows, int cols, void* dst,
                                 int64_t dst_batch_stride, int dst_ld, int dst_row0, hipStream_t s,
                                 const void* src_extra = nullptr);

}  // namespace moe
