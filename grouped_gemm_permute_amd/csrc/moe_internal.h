// moe_internal.h -- launchers shared between the translation units of
// libmoe_ffn.so.  Not part of the public ABI (include/moe_ffn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Slot blocks of the multi-block permute; a single workgroup handles
// T*k <= kPermuteSingleMax.
constexpr int kPermuteBlockSlots = 1024;
constexpr int64_t kPermuteSingleMax = 4096;
constexpr int kMaxExperts = 1024;

inline int permute_hist_blocks(int64_t S) {
    return S <= kPermuteSingleMax ? 0 : (int)((S + kPermuteBlockSlots - 1) / kPermuteBlockSlots);
}

// Stable counting sort of slots by expert (see moe_expert_permute).
// hist: int32 [(E+1) * nblocks] when nblocks > 0.  tile_off2 (optional,
// [E+2]) receives the row-tile prefix for tiles of tile_rows2 rows.
hipError_t launch_permute(const int32_t* idx, int64_t S, int E, int tile_rows, int64_t shared_rows,
                          int32_t* counts, int32_t* offsets, int32_t* tile_off, int32_t* perm,
                          int32_t* inv, int32_t* err, int32_t* hist, int nblocks, hipStream_t s,
                          int tile_rows2 = 0, int32_t* tile_off2 = nullptr);

// Grid for a kernel whose `upper` tiles (an upper bound) are spread over the
// 8 XCDs by xcd_remap_work: a multiple of 8 no smaller than upper.
inline unsigned grid_for_work(int64_t upper) { return (unsigned)((upper + 7) / 8 * 8); }

// Everything the grouped GEMMs read about the routed groups.
struct GroupArgs {
    const int32_t* offsets;   // [E+1] routed row starts
    const int32_t* tile_off;  // [G+1] row-tile prefix, G = E + has_shared
    const int32_t* perm;      // [S] sorted row -> slot
    int64_t S;                // T*k: first shared row
    int64_t T;
    int E;
    int k;
    int G;                    // E + has_shared
};

// bf16 MFMA grouped GEMMs.
constexpr int kBf16TileRows = 256;
hipError_t launch_up_swiglu_bf16(const GroupArgs& g, const void* x, const void* W1, const void* W3,
                                 const void* Ws1, const void* Ws3, void* h, int D, int F,
                                 hipStream_t s);
// The same, also storing each row's gate and up products gu[p] = [g | u]
// rounded to bf16 ([R, 2F], the layout of the backward's gate/up recompute).
hipError_t launch_up_swiglu_gu_bf16(const GroupArgs& g, const void* x, const void* W1,
                                    const void* W3, const void* Ws1, const void* Ws3, void* h,
                                    void* gu, int D, int F, hipStream_t s);
// Down GEMM output: Y[p] = h[p] . W2[grp] rounded to bf16 (the routing
// weight is applied by the combine).
hipError_t launch_down_bf16(const GroupArgs& g, const void* h, const void* W2, const void* Ws2,
                            void* Y, int D, int F, hipStream_t s);

// Small-chunk grouped GEMMs (bf16), for groups too small to fill the GPU
// with 256-row tiles.  The up GEMM runs on row tiles of 32 * rb rows that hold
// a whole typical group (rb from slab_row_blocks), each weight slab streamed
// once; the down GEMM on 64-row x 64-column tiles with a 4-deep load ring.
constexpr int kSmallTileRows = 64;
constexpr int kSlabMaxRowBlocks = 8;
// Workgroups of one round of the slab kernel (one per compute unit).
constexpr int kSlabRoundTiles = 256;
// Largest expert count whose counting sort the small-chunk up GEMM runs itself.
constexpr int kRouteMaxExperts = 512;
// rb for S routed rows over E experts, shared_rows shared-expert rows (0:
// none) and F output columns.
int slab_row_blocks(int64_t S, int64_t shared_rows, int E, int F);
// gu (optional, may be null): each row's [g | u] rounded to bf16, [R, 2F].
hipError_t launch_up_swiglu_bf16_slab(const GroupArgs& g, int rb, const void* x, const void* W1,
                                      const void* W3, const void* Ws1, const void* Ws3, void* h,
                                      int D, int F, hipStream_t s, void* gu = nullptr);
// The same with the counting sort of the permute done inside the kernel
// (S = T*k <= kPermuteSingleMax, E <= kRouteMaxExperts): reads the expert id of
// every slot and writes counts, offsets, tile_off (tile rows 32 rb),
// tile_off64, perm, inv and err exactly as launch_permute would; g's
// offsets, tile_off and perm are not read.  W2 [E, F, D] and Ws2 (or null)
// are only read, by idle CUs, to leave them in the last-level cache for the
// down GEMM.
hipError_t launch_up_swiglu_bf16_slab_routed(const GroupArgs& g, int rb, const int32_t* idx,
                                             int32_t* counts, int32_t* offsets, int32_t* tile_off,
                                             int32_t* tile_off64, int32_t* perm, int32_t* inv,
                                             int32_t* err, const void* x, const void* W1,
                                             const void* W3, const void* Ws1, const void* Ws3,
                                             const void* W2, const void* Ws2,
                                             void* h, int D, int F, hipStream_t s,
                                             void* gu = nullptr);
hipError_t launch_down_bf16_small(const GroupArgs& g, const void* h, const void* W2, const void* Ws2,
                                  void* Y, int D, int F, hipStream_t s);

// Fused up-act-down (bf16): token tiles of kFusedTileRows rows, h kept on
// chip; writes the same Y as the down GEMM.  Needs D % 128 == 0,
// D <= 1024, F % 128 == 0.
constexpr int kFusedTileRows = 64;
// Work plan of one fused launch, from the actual number of 64-row tiles W
// (tile_off[G], known on the device only).  Tiles run whole in full rounds
// of kFusedUnits workgroups (one per compute unit); each of the
// r = W mod kFusedUnits tiles of the last, partial round is shared out over
// s workgroups, s the largest power of two with r s <= kFusedUnits and
// s <= the number of 256-column F chunks, so the last round fills the GPU
// as far as the chunk count allows.  Split tiles write fp32 partial outputs
// that launch_fused_reduce sums in split order.
constexpr int kFusedUnits = 256;
struct FusedPlan {
    int whole;   // tiles 0 .. whole-1 run whole (a multiple of kFusedUnits)
    int r;       // tiles whole .. W-1 form the last round
    int s;       // workgroups per tile of the last round
};
__host__ __device__ inline FusedPlan fused_plan(int W, int chunks) {
    FusedPlan p;
    p.r = W % kFusedUnits;
    p.whole = W - p.r;
    p.s = 1;
    if (p.r > 0)
        while (2 * p.s <= chunks && p.r * 2 * p.s <= kFusedUnits) p.s *= 2;
    return p;
}
// Bytes of the fp32 partial outputs of a call with R rows and G groups: at
// most kFusedUnits split workgroups, 64 x D floats each.
size_t fused_partial_bytes(int64_t R, int G, int D, int F);
// Y [R, D] bf16 for whole tiles; split tiles write P and need
// launch_fused_reduce afterwards, on the same stream (always launched: the
// split tiles are known on the device only; with none, its workgroups exit
// at once).
hipError_t launch_fused_bf16(const GroupArgs& g, const void* x, const void* W1, const void* W3,
                             const void* W2, const void* Ws1, const void* Ws3, const void* Ws2,
                             void* Y, float* P, int D, int F, hipStream_t s);
hipError_t launch_fused_reduce(const GroupArgs& g, const float* P, void* Y, int D, int F, hipStream_t s);

// fp32 grouped GEMMs (plain fp32 FMA; correctness-first path).
constexpr int kF32TileRows = 64;
hipError_t launch_up_swiglu_f32(const GroupArgs& g, const float* x, const float* W1,
                                const float* W3, const float* Ws1, const float* Ws3, float* h,
                                int D, int F, hipStream_t s);
hipError_t launch_down_f32(const GroupArgs& g, const float* h, const float* W2, const float* Ws2,
                           float* Y, int D, int F, hipStream_t s);

// y[t] = Y[S+t] (shared, if any) + sum_j topk_w[t,j] * Y[inv[t*k+j]], in fp32
// in j order, rounded once.  Y is bf16 when bf16 is set, else fp32; y has
// the same type.
hipError_t launch_combine(const void* Y, const int32_t* inv, const float* topk_w, void* y,
                          int64_t T, int D, int k, bool has_shared, bool bf16, hipStream_t s);

}  // namespace moe
