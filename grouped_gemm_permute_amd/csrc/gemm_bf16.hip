// gemm_bf16.hip -- grouped GEMMs of the expert FFN on gfx950 bf16 MFMA.
//
// Two kernels share one tile engine:
//
//  up_swiglu:  for every row p of every group (routed experts in sorted
//              order, then the shared expert on all tokens),
//                g = x[tok(p)] . W1[grp],  u = x[tok(p)] . W3[grp]   (fp32 accumulate)
//                h[p] = bf16(silu(g) * u)
//              x rows are gathered straight from the token matrix while the
//              token tile is loaded, and W1 and W3 columns of the same output
//              column sit in one workgroup tile, so g and u never leave the
//              registers.  This is the fused gate/up/SiLU-multiply grouped
//              GEMM of "Triton MoE Kernels & Memory Checkpointing" (Part A,
//              sections 6 and 10.1) with fp32 SiLU and a single cast of the
//              product to the storage type.
//  down:       Y[p] = bf16(h[p] . W2[grp])   (fp32 accumulate), the per-expert
//              W2 product of the same page's section 10.3; the combine applies
//              the routing weight (its step 4).
//
// and, for the backward (the same page's Part A section 8: recompute the
// gate and up products, then the chain rule through silu(g) * u):
//
//  gate_up:    gu[p] = [g | u] rounded to bf16 (g in columns 0..F-1, u in
//              F..2F-1): the up GEMM with the activation left out.
//  up_gu:      up_swiglu that also stores gate_up's [g | u] (the forward
//              that keeps the gate and up products for the backward instead
//              of their recompute; the same K loop, two epilogue passes).
//  dh:         dh' = dy[tok(p)] . W2t[grp] with W2t[grp] = W2[grp]^T ([D, F]),
//              then per element, with g, u read back from gu and w the row's
//              routing weight (1 on shared rows):
//                h = silu(g) u,  dg = w dh' u silu'(g),  du = w dh' silu(g)
//                dgu[p] = [dg | du],  hw[p] = w h   (bf16)
//                dwpart[p][b] = sum over the 64 columns of block b of dh' h (fp32)
//  The backward's dx rows are the down mode run with K = 2F over the
//  transposed, stacked [W1^T ; W3^T] and A = dgu.
//
// Tile engine:
//  * the MFMA computes the transposed tile C^T = W^T . X^T: its A operand is
//    a 32-feature block of the weights, its B operand a 32-token block of
//    rows, so each lane ends with 4 consecutive output features of one token
//    and stores 8 bytes at a time;
//  * row tiles of 256 tokens x 256 MFMA features (up: 128 W1 + 128 W3
//    columns of the same 128 outputs), in one of two workgroup shapes
//    (waves_of below), each chosen by interleaved A/Bs with bitwise-equal
//    results:
//      - whole tiles, 8 wavefronts (up and gate_up on long grids, down): two
//        wavefronts per SIMD, wavefront w owning features 64 (w % 4) .. +63
//        of rows 128 (w / 4) .. +127 (2 x 4 v_mfma_f32_32x32x16_bf16
//        accumulators), one workgroup per CU and a ring of four 32 KiB
//        stages; one wavefront's MFMAs run while its partner is held issuing
//        a load into a busy memory pipe;
//      - half tiles, 4 wavefronts (up and gate_up when the whole-tile grid
//        is under twelve rounds of the CUs, dh always): a workgroup takes one
//        128-token half of a row tile, wavefront w owning features
//        64 w .. +63 of its 128 rows (2 x 4 accumulators, a ring of three
//        24 KiB stages, 72 KiB; dh adds 8 KiB for its epilogue), so two
//        workgroups share a CU and one's prologue and epilogue (the SiLU,
//        or dh's store-heavy one) run under the other's MFMAs;
//    spreading the wavefronts over the features rather than 2 x 2 halves the
//    slow transposed weight reads per MFMA;
//  * K step 32; both tiles go global -> LDS with global_load_lds (16 bytes
//    per lane, no registers) into the ring of stages;
//  * token rows are K-contiguous in memory and in LDS (read with
//    ds_read_b128); the weights stay [K][N] (N contiguous) in LDS and the
//    MFMA's K-consecutive operand is produced by ds_read_b64_tr_b16, which
//    hands each lane 4 consecutive K values of its own column;
//  * LDS rows are XOR-swizzled in 16-byte chunks (64-byte token rows by
//    (row / 4) & 3, 512-byte weight rows by 4 (k & 3)); since global_load_lds
//    writes each wavefront's 1 KiB contiguously, the swizzle is applied by
//    choosing which global chunk each lane fetches.
//
// Row tiles never cross a group: group g owns tiles tile_off[g] ..
// tile_off[g+1]-1 (computed by the permute on the device), the grid is sized
// by the host from an upper bound, and workgroups past tile_off[G] exit, so
// no host synchronisation is needed.  Rows past a group's end are clamped
// to their group's last row on load and never stored.
#include "mfma_common.h"

#include <type_traits>

namespace moe {
namespace {

using namespace mfma;

constexpr int TT = kBf16TileRows;   // 256 tokens (rows) per tile
constexpr int TF = 256;             // MFMA features per tile (up: 128 g + 128 u)
constexpr int BK = 32;
constexpr int X_ROW = BK * 2;                        // 64 B per token row
constexpr int W_ROW = TF * 2;                        // 512 B per k row
constexpr int W_BYTES = BK * W_ROW;                  // 16 KiB weight tile

static_assert(TT == 256 && TF == 256 && BK == 32, "index math below assumes these");

// 64-byte token rows (4 chunks): 16 consecutive rows read at one logical
// chunk hit 16 distinct bank groups.
__device__ __forceinline__ int swz_x(int row) { return (row >> 2) & 3; }

// Kernel modes.
enum : int {
    M_UP = 0,      // x gathered . [W1 | W3] -> h = silu(g) u
    M_DOWN = 1,    // rows . W2 -> Y (also the backward's dx rows)
    M_GU = 2,      // x gathered . [W1 | W3] -> [g | u]
    M_DH = 3,      // dy gathered . W2t -> dgu, hw, dwpart
    M_UPGU = 4,    // x gathered . [W1 | W3] -> [g | u] and h = silu(g) u
};

// Workgroup shapes, each chosen by measurement (interleaved A/Bs):
//  * whole tiles (HALF = false): 8 wavefronts, two per SIMD, on a 256-row
//    tile, one workgroup per CU (a 4-stage ring of 32 KiB), so one
//    wavefront's MFMAs cover the other's stalls issuing loads;
//  * half tiles (HALF = true; up, gate/up and dh): 4 wavefronts on one 128-row half
//    of a tile (a 3-stage ring of 24 KiB), two workgroups per CU, so the
//    epilogue and the prologue of one overlap the other's MFMAs and the
//    last round is finer.  It stages 1.5x the bytes per MFMA: the up GEMM
//    takes it when its whole-tile grid is short (up_half_tiles), where it
//    measured 3-9% faster; on long grids it is even to 1% slower.  gate/up
//    follows the same rule (4% faster at 4096 tokens, 4% slower at 32768);
//    the down GEMM is slower on it at every size.  dh, whose epilogue moves 640 KiB per
//    256-row tile, always takes it: 522 -> 487 us at 32768 tokens and
//    110 -> 83 us at 4096 (D = 768, F = 1536, E = 8; before, 4 wavefronts
//    on a whole tile, one workgroup per CU).
template <int MODE, bool HALF>
constexpr int waves_of() {
    return HALF ? 4 : 8;
}

struct GemmArgs {
    GroupArgs g;
    const uint16_t* a;        // up, gu: x [T, D]; down: h [R, F]; dh: dy [T, D]
    const uint16_t* b0;       // up, gu: W1 [E, D, F]; down: W2 [E, F, D]; dh: W2t [E, D, F]
    const uint16_t* b1;       // up, gu: W3; otherwise unused
    const uint16_t* bs0;      // shared expert: Ws1 / Ws2 / Ws2t
    const uint16_t* bs1;      // up, gu: Ws3
    void* out;                // up: h [R, F]; down: Y [R, D]; gu: gu [R, 2F]; dh: dgu [R, 2F]
    int D, F;
    int n_tiles;              // column tiles
    int col_groups;           // column-tile groups (divides n_tiles and 8)
    // dh only
    const float* topk_w;      // [S] routing weight of each slot
    const uint16_t* gu;       // [R, 2F] recomputed g and u
    uint16_t* hw;             // [R, F] w * h
    float* dwpart;            // [R, F / 64] partial sums of dh' * h
    // up with the gate and up products kept (M_UPGU) only
    void* gu_out;             // [R, 2F] g and u, as the gate/up mode stores them
};

// Target of the dh epilogue's stores for rows and columns outside the tile.
__device__ __attribute__((aligned(16))) u32x4_t dh_trash[1];

template <int MODE, bool HALF>
__global__ __launch_bounds__((64 * waves_of<MODE, HALF>()), (HALF ? 2 : 1)) void grouped_gemm_bf16_kernel(
    const GemmArgs a) {
    constexpr bool UP = MODE != M_DOWN;         // A gathered by token, K = D, N = F
    constexpr bool PAIR = MODE == M_UP || MODE == M_GU || MODE == M_UPGU;   // g / u column pairs from W1, W3
    static_assert(!HALF || MODE != M_DOWN, "half tiles are built for the up, gate/up and dh GEMMs");
    constexpr int NW = waves_of<MODE, HALF>();
    constexpr int NT = 64 * NW;
    constexpr int ROWS = HALF ? TT / 2 : TT;   // rows of the workgroup's tile
    constexpr int NJ = ROWS * 4 / (32 * NW);   // 32-row blocks per wavefront
    constexpr int XJ = ROWS / (16 * NW);       // token-tile DMA instructions per wavefront
    constexpr int WJ = 16 / NW;                // weight-tile DMA instructions per wavefront
    constexpr int XBYTES = ROWS * X_ROW;       // token tile
    constexpr int SBYTES = XBYTES + W_BYTES;   // one stage
    constexpr int NS = HALF ? 3 : 4;           // ring stages
    // The stage buffers as separate LDS objects: every access names its
    // buffer statically, so the compiler knows reads of one buffer do not
    // alias the asynchronous global_load_lds writes into the others.
    __shared__ __attribute__((aligned(1024))) char st0[SBYTES];
    __shared__ __attribute__((aligned(1024))) char st1[SBYTES];
    __shared__ __attribute__((aligned(1024))) char st2[SBYTES];
    // (dh: an 8 KiB fourth buffer for its epilogue's g/u scratch)
    __shared__ __attribute__((aligned(1024))) char st3[NS == 4 ? SBYTES : MODE == M_DH ? 8192 : 16];

    const int K = UP ? a.D : a.F;      // reduction length
    const int N = UP ? a.F : a.D;      // output columns
    const int ldw = N;                 // weight row stride (elements)

    // ---- this workgroup's tile.  The column tiles are split into col_groups
    // groups of ncol; the 8 / col_groups XCDs of group c (XCD x = workgroups
    // b with b % 8 == x, dispatched round-robin) split its row tiles x ncol
    // tiles (row-major; with half tiles each row tile counts as its two
    // halves) into contiguous, equal ranges.  An XCD thus keeps one weight
    // slab of ncol column tiles in its L2 while row tiles stream through;
    // with one group this is xcd_remap_work over all tiles.
    int mt, hf, nt;
    {
        const int m_tiles = a.g.tile_off[a.g.G];
        const int xpg = 8 / a.col_groups, ncol = a.n_tiles / a.col_groups;
        const int xcd = blockIdx.x & 7;
        const int c = xcd / xpg, share = xcd - c * xpg;
        const int items = (HALF ? 2 : 1) * m_tiles * ncol;
        const int per = items / xpg, rem = items - per * xpg;
        const int i = blockIdx.x >> 3;
        if (i >= per + (share < rem ? 1 : 0)) return;
        const int j = share * per + min(share, rem) + i;
        const int mh = j / ncol;
        mt = HALF ? mh >> 1 : mh;
        hf = HALF ? mh & 1 : 0;
        nt = c * ncol + (j - mh * ncol);
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int fw = wave & 3;           // MFMA features 64 fw .. 64 fw + 63
    const int rw = wave >> 2;          // rows 32 NJ rw .. +32 NJ - 1 (eight wavefronts)

    // ---- the group owning row tile mt, and the tile's rows.
    if (mt >= a.g.tile_off[a.g.G]) return;
    const TileGroup tg = find_tile_group(a.g, mt, TT, lane);
    const int grp = tg.grp;
    const bool shared = grp >= a.g.E;
    const int64_t tile_r0 = tg.tile_r0 + ROWS * hf;
    const int valid_rows = min(tg.valid_rows - ROWS * hf, ROWS);
    if (valid_rows <= 0) return;       // an empty second half, or tile_off disagreeing with offsets

    // ---- token tile sources: DMA instruction j (0..XJ-1) of wavefront w fills
    // rows 16 XJ w + 16 j .. +15; lane -> row 16 XJ w + 16 j + lane/4, physical
    // chunk lane%4 holding logical chunk (lane%4) ^ swz_x(row).  Routed rows of
    // the up GEMM gather token perm[p] / k (all index loads in flight at
    // once); shared rows read token p - S; the down GEMM reads row p of h.
    const char* x_src[XJ];
    {
        int64_t src_row[XJ];
#pragma unroll
        for (int j = 0; j < XJ; ++j)
            src_row[j] = tile_r0 + min(16 * XJ * wave + 16 * j + (lane >> 2), valid_rows - 1);
        if (UP && !shared) {
            int32_t slot[XJ];
#pragma unroll
            for (int j = 0; j < XJ; ++j) slot[j] = a.g.perm[src_row[j]];
#pragma unroll
            for (int j = 0; j < XJ; ++j) src_row[j] = slot[j] / a.g.k;
        } else if (UP) {
#pragma unroll
            for (int j = 0; j < XJ; ++j) src_row[j] -= a.g.S;
        }
#pragma unroll
        for (int j = 0; j < XJ; ++j) {
            const int row = 16 * XJ * wave + 16 * j + (lane >> 2);
            x_src[j] = (const char*)(a.a + src_row[j] * (int64_t)K + 8 * ((lane & 3) ^ swz_x(row)));
        }
    }
    // ---- weight tile sources: DMA instruction j (0..WJ-1) of wavefront w fills
    // k rows 2 WJ w + 2 j, +1; lane -> k row 2 WJ w + 2 j + lane/32, physical chunk
    // lane%32 holding logical chunk cl = phys ^ swz_tr(k) = MFMA features
    // 8 cl .. 8 cl + 7.  Up: wavefront block wb = cl / 8, g when (cl / 4) is
    // even, u when odd, output column 32 wb + 8 (cl % 4) of the tile's 128.
    const int64_t gstride = (int64_t)a.D * a.F;
    const char* w_src[WJ];
#pragma unroll
    for (int j = 0; j < WJ; ++j) {
        const int kr = 2 * WJ * wave + 2 * j + (lane >> 5);
        const int cl = (lane & 31) ^ swz_tr(kr);
        int col;
        const uint16_t* base;
        if (PAIR) {
            const int kind = (cl >> 2) & 1;
            col = nt * (TF / 2) + 32 * (cl >> 3) + 8 * (cl & 3);
            base = shared ? (kind ? a.bs1 : a.bs0) : (kind ? a.b1 : a.b0) + grp * gstride;
        } else {
            col = nt * TF + 8 * cl;
            base = shared ? a.bs0 : a.b0 + grp * gstride;
        }
        if (col >= N) col = 0;                 // past the last column: a valid chunk, never stored
        w_src[j] = (const char*)(base + (int64_t)kr * ldw + col);
    }
    const int64_t w_step = (int64_t)BK * ldw * 2;      // bytes per K step in the weights

    auto issue = [&](int kt, char* st) {
#pragma unroll
        for (int j = 0; j < XJ; ++j)
            load_lds16(x_src[j] + (int64_t)kt * X_ROW, st + (16 * XJ * wave + 16 * j) * X_ROW);
#pragma unroll
        for (int j = 0; j < WJ; ++j)
            load_lds16(w_src[j] + kt * w_step, st + XBYTES + (2 * WJ * wave + 2 * j) * W_ROW);
    };

    // ---- MFMA operand read offsets (bytes within a stage).
    // Weight operand (A), transposed read: lane = 16 G + s of k16 slice ks
    // reads k = 16 ks + 8 (G / 2) + 4 r + s / 4 (r = 0, 1 for the two halves),
    // feature 64 w + 32 mi + 16 (G % 2) + 4 (s % 4).
    const int G = lane >> 4, sl = lane & 15;
    int w_off[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int k = 8 * (G >> 1) + 4 * r + (sl >> 2);
            const int R = 64 * fw + 32 * mi + 16 * (G & 1) + 4 * (sl & 3);
            w_off[mi][r] = XBYTES + k * W_ROW + (((R >> 3) ^ swz_tr(k)) << 4) + 8 * ((R >> 2) & 1);
        }
    // Token operand (B): lane reads row 32 nj + lane%32, logical chunk
    // 2 ks + lane/32; rows 32 nj + l and l share swz_x, so one offset serves
    // all eight blocks.
    const int xr = lane & 31;
    const int x_base = (32 * NJ * rw + xr) * X_ROW;
    const int x_sw = swz_x(xr);

    f32x16_t acc[2][NJ];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) acc[mi][nj] = f32x16_t{};

    struct Frags {
        bf16x8_t w[2][2], x[2][NJ];     // [k16 slice][block]
    };
    auto read_frags = [&](const char* st, Frags& f) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                f.w[ks][mi] = cat_bf16(read_tr(st + w_off[mi][0] + ks * 16 * W_ROW),
                                       read_tr(st + w_off[mi][1] + ks * 16 * W_ROW));
            const int c = ((2 * ks + (lane >> 5)) ^ x_sw) << 4;
#pragma unroll
            for (int nj = 0; nj < NJ; ++nj)
                f.x[ks][nj] = __builtin_bit_cast(
                    bf16x8_t, *(const u32x4_t*)(st + x_base + nj * 32 * X_ROW + c));
        }
    };
    auto mfmas = [&](const Frags& f) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
                    acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.w[ks][mi], f.x[ks][nj],
                                                                          acc[mi][nj], 0, 0, 0);
    };
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

    // ---- 4-stage ring, software-pipelined one stage deep in registers.
    // Step s (its operands fc already in registers):
    //   wait until stage s+1 has landed (one later stage of this wavefront's
    //   loads may still be outstanding) and fc's LDS reads have returned;
    //   barrier;
    //   issue the loads of stage s+3 into the buffer of stage s-1;
    //   read stage s+1's operands into fn;
    //   the MFMAs on fc -- the reads of fn land under them.
    // The buffer of stage s-1 is free at step s: its operands were read in
    // step s-2 and consumed by the MFMAs of step s-1, which every wavefront
    // finished before arriving at this barrier.  Loads past the last stage
    // re-read the last stage (into buffers never computed on), so the number
    // of loads per stage stays fixed.
    const int KT = K / BK;
    constexpr int PER_STAGE = XJ + WJ; // global_load_lds per wavefront per stage
    auto wait_stage = [] {
        // four stages: one later stage may still be in flight; three: none
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(NS == 4 ? PER_STAGE : 0, 0));
        __builtin_amdgcn_s_barrier();
    };
    auto step = [&](Frags& fc, Frags& fn, const char* nxt, char* dma, int kl) {
        wait_stage();
        fence();
        issue(kl, dma);
        read_frags(nxt, fn);
        mfmas(fc);
        // A wavefront issues in order and stalls on a load or LDS read while
        // that pipe is backed up, so bursts of either would idle its MFMAs.
        // Half tiles (16 MFMAs, 6 loads, 16 reads per step): the loads one per
        // MFMA over the first half of the step, so the only stage in flight
        // lands before the next step's wait.  Eight wavefronts (16 MFMAs, 4
        // loads, 16 reads): one load per 4 MFMAs over the whole step (the
        // front-loaded and the compiler's own orders measured 1-4% slower).
        if constexpr (NW == 8) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // vector memory
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        } else {
            static_assert(HALF, "four wavefronts run half tiles");
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // vector memory
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
        fence();
    };
    Frags fa, fb;
    issue(0, st0);
    issue(min(1, KT - 1), st1);
    if constexpr (NS == 4) issue(min(2, KT - 1), st2);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm((NS - 2) * PER_STAGE, 15));   // stage 0 landed
    __builtin_amdgcn_s_barrier();
    fence();
    read_frags(st0, fa);
    fence();
    int kt = 0;
    if constexpr (NS == 4) {
        // stage s in buffer s % 4; step s issues stage s + 3
        for (; kt + 4 <= KT; kt += 4) {
            step(fa, fb, st1, st3, min(kt + 3, KT - 1));
            step(fb, fa, st2, st0, min(kt + 4, KT - 1));
            step(fa, fb, st3, st1, min(kt + 5, KT - 1));
            step(fb, fa, st0, st2, min(kt + 6, KT - 1));
        }
        if (kt < KT) {
            step(fa, fb, st1, st3, KT - 1);
            if (kt + 1 < KT) {
                step(fb, fa, st2, st0, KT - 1);
                if (kt + 2 < KT) step(fa, fb, st3, st1, KT - 1);
            }
        }
    } else {
        // stage s in buffer s % 3; step s issues stage s + 2.  The operand
        // registers alternate with period 2 and the buffers with period 3, so
        // after three steps the next stage's operands are in fb: swap.
        for (; kt + 3 <= KT; kt += 3) {
            step(fa, fb, st1, st2, min(kt + 2, KT - 1));
            step(fb, fa, st2, st0, min(kt + 3, KT - 1));
            step(fa, fb, st0, st1, min(kt + 4, KT - 1));
            Frags t = fa;
            fa = fb;
            fb = t;
        }
        // at most two steps left (stage kt in st0); every stage they need is
        // already in flight, their own loads re-read the last stage
        if (kt < KT) {
            step(fa, fb, st1, st2, KT - 1);
            if (kt + 1 < KT) step(fb, fa, st2, st0, KT - 1);
        }
    }
    wait_vmem();

    // ---- epilogue, staged through LDS so that every store instruction
    // writes whole row segments (16 bytes per lane, 256 or 512 contiguous
    // bytes per row) instead of 8-byte pieces of 32 rows.  acc[mi][nj]
    // element v of lane l: token 32 NJ rw + 32 nj + l%32, MFMA feature
    // 64 fw + 32 mi + 8 (v/4) + 4 (l/32) + v%4.  Up: h column 32 fw + the
    // feature's offset in its 32-block (g in mi = 0, u in mi = 1); down:
    // output column = MFMA feature.  The tile's rows are staged RPS to a
    // stage buffer, 16-byte chunks XOR-swizzled by the row's low 4 bits.
    if constexpr (MODE == M_DH) {
        static_assert(HALF && NW == 4 && NJ == 4 && NS == 3,
                      "the dh epilogue lays out one wavefront per 64 columns of a 128-row half tile");
        // Element v of acc[mi][nj] on lane l: token 32 nj + l%32, column
        // nt*256 + 64 w + 32 mi + 8 (v/4) + 4 (l/32) + v%4; each lane handles
        // four consecutive columns at a time.  The wavefront's 64 columns are
        // one dwpart block; the two lane halves holding a token's columns are
        // added with one cross-lane exchange.  g and u of the next 32-row
        // block are loaded while this block is stored; dg, du and w h go
        // through LDS (one block at a time: dg in the lower 16 KiB of st0,
        // du of st1, w h of st2, 512-byte rows, 16-byte chunks XOR-swizzled
        // by the row) so that the stores write whole 512-byte row segments.
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
        __syncthreads();                         // every wavefront is done with the stage buffers
        const int F = a.F;
        const int nbk = F / 64;
        const int blk = nt * 4 + wave;
        const bool cols_ok = nt * TF + 64 * wave < F;   // F % 64 == 0: all or none of a wavefront's
        int64_t prow[NJ];
        float wrow[NJ];
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) prow[nj] = tile_r0 + min(32 * nj + (lane & 31), valid_rows - 1);
        if (shared) {
#pragma unroll
            for (int nj = 0; nj < NJ; ++nj) wrow[nj] = 1.f;
        } else {
            int32_t slot[NJ];
#pragma unroll
            for (int nj = 0; nj < NJ; ++nj) slot[nj] = a.g.perm[prow[nj]];
#pragma unroll
            for (int nj = 0; nj < NJ; ++nj) wrow[nj] = a.topk_w[slot[nj]];
        }
        // g, u of the lane's 4 columns nt*256 + 64 w + 32 mi + 8 vg + 4 (l/32) + 0..3
        struct GU {
            uint2 g[2][4], u[2][4];   // [mi][vg]
        };
        // g and u of a 32-row block are loaded as whole 128-byte row segments
        // (instruction j: rows 8 (j%4) .. +7 of the block, g for j < 4 else u;
        // lane: row + lane/8, 16-byte chunk lane%8 of the wavefront's 64
        // columns), then rearranged into the accumulator layout through an
        // 8 KiB LDS scratch of the wavefront's own (the upper 8 KiB of stage
        // buffer w, or st3 for w = 3), 16-byte chunks XOR-swizzled by row / 2.
        struct Raw {
            u32x4_t v[8];
        };
        char* const gus = wave == 0 ? st0 + 16384 : wave == 1 ? st1 + 16384
                        : wave == 2 ? st2 + 16384 : st3;
        const int fc0 = cols_ok ? nt * TF + 64 * wave : 0;   // the wavefront's first column (readable)
        auto swz_gu = [](int r) { return (r >> 1) & 7; };
        auto load_raw = [&](int nj, Raw& R) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int row = 8 * (j & 3) + (lane >> 3);
                const int64_t p = tile_r0 + min(32 * nj + row, valid_rows - 1);
                R.v[j] = *(const u32x4_t*)(a.gu + p * 2 * F + (j >> 2) * F + fc0 + 8 * (lane & 7));
            }
        };
        auto unpack = [&](const Raw& R, GU& b) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int row = 8 * (j & 3) + (lane >> 3);
                *(u32x4_t*)(gus + (j >> 2) * 4096 + row * 128 + (((lane & 7) ^ swz_gu(row)) << 4)) = R.v[j];
            }
            const int r = lane & 31, h = lane >> 5;
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int vg = 0; vg < 4; ++vg) {
                    const int off = r * 128 + (((4 * mi + vg) ^ swz_gu(r)) << 4) + 8 * h;
                    b.g[mi][vg] = *(const uint2*)(gus + off);
                    b.u[mi][vg] = *(const uint2*)(gus + 4096 + off);
                }
        };
        const int r_l = lane & 31;
        auto finish_block = [&](int nj, const GU& b) {
            char* sdg = st0 + r_l * 512;
            char* sdu = st1 + r_l * 512;
            char* shw = st2 + r_l * 512;
            const float w = wrow[nj];
            float part = 0.f;
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
                const f32x16_t& c = acc[mi][nj];
#pragma unroll
                for (int vg = 0; vg < 4; ++vg) {
                    const uint2 gq = b.g[mi][vg], uq = b.u[mi][vg];
                    const float gv[4] = {__uint_as_float(gq.x << 16), __uint_as_float(gq.x & 0xffff0000u),
                                         __uint_as_float(gq.y << 16), __uint_as_float(gq.y & 0xffff0000u)};
                    const float uv[4] = {__uint_as_float(uq.x << 16), __uint_as_float(uq.x & 0xffff0000u),
                                         __uint_as_float(uq.y << 16), __uint_as_float(uq.y & 0xffff0000u)};
                    float dg[4], du[4], hv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float dhp = c[4 * vg + i];
                        const float sg = __builtin_amdgcn_rcpf(
                            1.0f + __builtin_amdgcn_exp2f(-gv[i] * 1.4426950408889634f));
                        const float act = gv[i] * sg;
                        const float h = act * uv[i];
                        part = fmaf(dhp, h, part);
                        const float dh = w * dhp;
                        dg[i] = dh * uv[i] * (sg * (1.0f + gv[i] * (1.0f - sg)));
                        du[i] = dh * act;
                        hv[i] = w * h;
                    }
                    const int ch = 8 * wave + 4 * mi + vg;          // 16-byte chunk of the tile row
                    const int off = 8 * (lane >> 5);
                    *(uint2*)(sdg + ((ch ^ r_l) << 4) + off) =
                        make_uint2(pack_bf16(dg[0], dg[1]), pack_bf16(dg[2], dg[3]));
                    *(uint2*)(sdu + ((ch ^ r_l) << 4) + off) =
                        make_uint2(pack_bf16(du[0], du[1]), pack_bf16(du[2], du[3]));
                    *(uint2*)(shw + ((ch ^ r_l) << 4) + off) =
                        make_uint2(pack_bf16(hv[0], hv[1]), pack_bf16(hv[2], hv[3]));
                }
            }
            part += __shfl_xor(part, 32);
            // both lane halves hold the row's sum and store it (the same value)
            const bool ok = cols_ok && 32 * nj + r_l < valid_rows;
            *(ok ? a.dwpart + prow[nj] * nbk + blk : (float*)dh_trash) = part;
        };
        // rows 32 nj .. 32 nj + 31 of the staged block go out as whole 16-byte
        // chunks: dg and du 32 chunks per row each (chunk c < 32 of dg, else
        // of du), w h 32 chunks per row.  Every thread issues the same 12
        // stores per block whatever the tile's valid rows and columns (the
        // others go to a 16-byte trash slot), so that the compiler can count
        // the stores issued after a block's g/u loads and wait for those
        // loads alone.
        auto store_block = [&](int nj) {
            const int c = tid & 63;
            const int col = nt * TF + 8 * (c & 31);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = (tid >> 6) + 4 * i;
                const bool ok = col < F && 32 * nj + r < valid_rows;
                const int64_t p = tile_r0 + 32 * nj + r;
                const u32x4_t v = *(const u32x4_t*)((c < 32 ? st0 : st1) + r * 512 + (((c & 31) ^ r) << 4));
                *(ok ? (u32x4_t*)((uint16_t*)a.out + p * 2 * F + (c < 32 ? 0 : F) + col) : dh_trash) = v;
            }
            const int c2 = tid & 31;
            const int col2 = nt * TF + 8 * c2;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = (tid >> 5) + 8 * i;
                const bool ok = col2 < F && 32 * nj + r < valid_rows;
                const int64_t p = tile_r0 + 32 * nj + r;
                const u32x4_t v = *(const u32x4_t*)(st2 + r * 512 + ((c2 ^ r) << 4));
                *(ok ? (u32x4_t*)(a.hw + p * F + col2) : dh_trash) = v;
            }
        };
        Raw raw;
        load_raw(0, raw);
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) {
            GU cur;
            unpack(raw, cur);
            finish_block(nj, cur);
            // the next block's g and u go out now, into the registers cur
            // held (at two workgroups per CU registers are short)
            if (nj + 1 < NJ) load_raw(nj + 1, raw);
            // the staged block is complete in LDS; a barrier that waits on
            // LDS only, so block nj + 1's loads stay in flight
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
            __builtin_amdgcn_s_barrier();
            store_block(nj);
            // one staging buffer: every wavefront has read it out before the
            // next block overwrites it
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
            __builtin_amdgcn_s_barrier();
        }
        return;
    }
    if constexpr (MODE == M_UPGU) {
        // Two passes through the stage buffers: [g | u] as the gate/up mode
        // stages and stores it (staged columns 0..127 g, 128..255 u, to
        // gu_out [R, 2F]), then h as the up mode does (to out [R, F]).
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
        __syncthreads();
        auto pass = [&](auto GUc) {
            constexpr bool GU = decltype(GUc)::value;
            constexpr int OCOLS = GU ? TF : TF / 2;
            constexpr int OROW = OCOLS * 2;
            constexpr int OCH = OROW / 16;
            constexpr int RPS = SBYTES / OROW;
            static_assert(RPS % 16 == 0 && NS * RPS >= ROWS, "the stage buffers hold the staged tile");
            auto orow = [&](int r) -> char* {
                const int q = r / RPS;
                char* b = q == 0 ? st0 : q == 1 ? st1 : q == 2 ? st2 : st3;
                return b + (r - q * RPS) * OROW;
            };
#pragma unroll
            for (int nj = 0; nj < NJ; ++nj) {
                const int t = 32 * NJ * rw + 32 * nj + (lane & 31);
                char* rowp = orow(t);
                const int sw = t & 15;
                if constexpr (GU) {
#pragma unroll
                    for (int mi = 0; mi < 2; ++mi) {
                        const f32x16_t& c = acc[mi][nj];
#pragma unroll
                        for (int vg = 0; vg < 4; ++vg) {
                            const int v = 4 * vg;
                            const int ch = 16 * mi + 4 * fw + vg;
                            *(uint2*)(rowp + ((ch ^ sw) << 4) + 8 * (lane >> 5)) =
                                make_uint2(pack_bf16(c[v], c[v + 1]), pack_bf16(c[v + 2], c[v + 3]));
                        }
                    }
                } else {
                    const f32x16_t& g = acc[0][nj];
                    const f32x16_t& u = acc[1][nj];
#pragma unroll
                    for (int vg = 0; vg < 4; ++vg) {
                        const int v = 4 * vg;
                        const int c = 4 * fw + vg;
                        *(uint2*)(rowp + ((c ^ sw) << 4) + 8 * (lane >> 5)) =
                            make_uint2(pack_bf16(silu_mul(g[v], u[v]), silu_mul(g[v + 1], u[v + 1])),
                                       pack_bf16(silu_mul(g[v + 2], u[v + 2]), silu_mul(g[v + 3], u[v + 3])));
                    }
                }
            }
            __syncthreads();
            constexpr int ROWS_PER_PASS = NT / OCH;
            const int c = tid % OCH;
            const int col = GU ? (c < 16 ? nt * 128 + 8 * c : N + nt * 128 + 8 * (c - 16)) : nt * OCOLS + 8 * c;
            const int ldo = GU ? 2 * N : N;
            const bool col_ok = GU ? nt * 128 + 8 * (c & 15) < N : col < N;
            uint16_t* out = (uint16_t*)(GU ? a.gu_out : a.out);
#pragma unroll 4
            for (int r = tid / OCH; r < ROWS; r += ROWS_PER_PASS) {
                if (r >= valid_rows) break;
                const u32x4_t v = *(const u32x4_t*)(orow(r) + ((c ^ (r & 15)) << 4));
                if (col_ok) *(u32x4_t*)(out + (tile_r0 + r) * (int64_t)ldo + col) = v;
            }
        };
        pass(std::true_type{});
        __syncthreads();          // every wavefront has read the [g | u] pass out of LDS
        pass(std::false_type{});
        return;
    }
    constexpr int OCOLS = MODE == M_UP ? TF / 2 : TF;   // output columns of the tile
    constexpr int OROW = OCOLS * 2;             // bytes per staged row
    constexpr int OCH = OROW / 16;              // 16-byte chunks per row
    constexpr int RPS = SBYTES / OROW;         // staged rows per stage buffer
    static_assert(RPS % 16 == 0 && NS * RPS >= ROWS, "the stage buffers hold the staged tile");
    auto orow = [&](int r) -> char* {
        const int q = r / RPS;
        char* b = q == 0 ? st0 : q == 1 ? st1 : q == 2 ? st2 : st3;
        return b + (r - q * RPS) * OROW;
    };
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));   // this wavefront's loads and LDS reads done
    __syncthreads();                                // ... and every other wavefront's
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) {
        const int t = 32 * NJ * rw + 32 * nj + (lane & 31);
        char* rowp = orow(t);
        const int sw = t & 15;
        if (MODE == M_GU) {
            // g (mi = 0) to staged columns 32 fw + ..., u (mi = 1) to 128 + 32 fw + ...
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
                const f32x16_t& c = acc[mi][nj];
#pragma unroll
                for (int vg = 0; vg < 4; ++vg) {
                    const int v = 4 * vg;
                    const int ch = 16 * mi + 4 * fw + vg;
                    *(uint2*)(rowp + ((ch ^ sw) << 4) + 8 * (lane >> 5)) =
                        make_uint2(pack_bf16(c[v], c[v + 1]), pack_bf16(c[v + 2], c[v + 3]));
                }
            }
        } else if (MODE == M_UP) {
            const f32x16_t& g = acc[0][nj];
            const f32x16_t& u = acc[1][nj];
#pragma unroll
            for (int vg = 0; vg < 4; ++vg) {
                const int v = 4 * vg;
                const int c = 4 * fw + vg;
                *(uint2*)(rowp + ((c ^ sw) << 4) + 8 * (lane >> 5)) =
                    make_uint2(pack_bf16(silu_mul(g[v], u[v]), silu_mul(g[v + 1], u[v + 1])),
                               pack_bf16(silu_mul(g[v + 2], u[v + 2]), silu_mul(g[v + 3], u[v + 3])));
            }
        } else {
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
                const f32x16_t& c = acc[mi][nj];
#pragma unroll
                for (int vg = 0; vg < 4; ++vg) {
                    const int v = 4 * vg;
                    const int ch = 8 * fw + 4 * mi + vg;
                    *(uint2*)(rowp + ((ch ^ sw) << 4) + 8 * (lane >> 5)) =
                        make_uint2(pack_bf16(c[v], c[v + 1]), pack_bf16(c[v + 2], c[v + 3]));
                }
            }
        }
    }
    __syncthreads();
    constexpr int ROWS_PER_PASS = NT / OCH;
    const int c = tid % OCH;
    // gate_up: staged columns 0..127 are g, 128..255 u, of h columns nt*128 + ...
    const int col = MODE == M_GU ? (c < 16 ? nt * 128 + 8 * c : N + nt * 128 + 8 * (c - 16))
                                 : nt * OCOLS + 8 * c;
    const int ldo = MODE == M_GU ? 2 * N : N;
    const bool col_ok = MODE == M_GU ? nt * 128 + 8 * (c & 15) < N : col < N;
#pragma unroll 4
    for (int r = tid / OCH; r < ROWS; r += ROWS_PER_PASS) {
        if (r >= valid_rows) break;
        const u32x4_t v = *(const u32x4_t*)(orow(r) + ((c ^ (r & 15)) << 4));
        if (col_ok) *(u32x4_t*)((uint16_t*)a.out + (tile_r0 + r) * (int64_t)ldo + col) = v;
    }
}

// Column groups for a GEMM with n_tiles column tiles over a K-row weight
// slab: the smallest split (dividing n_tiles and 8) whose per-XCD slab
// (n_tiles / groups column tiles of K x 256 bf16) fits in 2.5 MiB of the
// XCD's 4 MiB L2; one group when none does.
int column_groups(int n_tiles, int K) {
    for (int cg = 1; cg <= 8; cg *= 2)
        if (n_tiles % cg == 0 && (int64_t)(n_tiles / cg) * K * TF * 2 <= (int64_t)5 << 19) return cg;
    return 1;
}

// Whether the up GEMM runs on half tiles: when its grid of whole tiles
// (an upper bound, known on the host) is under twelve rounds of 256 CUs.
// Measured (D = 768, F = 1536, E = 8): half tiles 3-9% faster at 4096 to
// 16384 tokens (2.4 to 9.4 rounds), even to 1% slower at 32768 (18 rounds).
bool up_half_tiles(int64_t tiles) { return tiles < 12 * 256; }

int m_tiles_upper(const GroupArgs& g) {
    const int64_t rows = g.S + (g.G > g.E ? g.T : 0);
    return (int)((rows + TT - 1) / TT) + g.G;
}

}  // namespace

hipError_t launch_up_swiglu_bf16(const GroupArgs& g, const void* x, const void* W1, const void* W3,
                                 const void* Ws1, const void* Ws3, void* h, int D, int F,
                                 hipStream_t s) {
    GemmArgs a{g, (const uint16_t*)x, (const uint16_t*)W1, (const uint16_t*)W3,
               (const uint16_t*)Ws1, (const uint16_t*)Ws3, h, D, F, (F + TF / 2 - 1) / (TF / 2)};
    a.col_groups = column_groups(a.n_tiles, D);
    const int64_t tiles = (int64_t)m_tiles_upper(g) * a.n_tiles;
    if (up_half_tiles(tiles))
        grouped_gemm_bf16_kernel<M_UP, true><<<grid_for_work(2 * tiles), 64 * waves_of<M_UP, true>(), 0, s>>>(a);
    else
        grouped_gemm_bf16_kernel<M_UP, false><<<grid_for_work(tiles), 64 * waves_of<M_UP, false>(), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_up_swiglu_gu_bf16(const GroupArgs& g, const void* x, const void* W1,
                                    const void* W3, const void* Ws1, const void* Ws3, void* h,
                                    void* gu, int D, int F, hipStream_t s) {
    GemmArgs a{g, (const uint16_t*)x, (const uint16_t*)W1, (const uint16_t*)W3,
               (const uint16_t*)Ws1, (const uint16_t*)Ws3, h, D, F, (F + TF / 2 - 1) / (TF / 2)};
    a.col_groups = column_groups(a.n_tiles, D);
    a.gu_out = gu;
    const int64_t tiles = (int64_t)m_tiles_upper(g) * a.n_tiles;
    if (up_half_tiles(tiles))
        grouped_gemm_bf16_kernel<M_UPGU, true><<<grid_for_work(2 * tiles), 64 * waves_of<M_UPGU, true>(), 0, s>>>(a);
    else
        grouped_gemm_bf16_kernel<M_UPGU, false><<<grid_for_work(tiles), 64 * waves_of<M_UPGU, false>(), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_down_bf16(const GroupArgs& g, const void* h, const void* W2, const void* Ws2,
                            void* Y, int D, int F, hipStream_t s) {
    GemmArgs a{g, (const uint16_t*)h, (const uint16_t*)W2, nullptr, (const uint16_t*)Ws2, nullptr,
               Y, D, F, (D + TF - 1) / TF};
    a.col_groups = column_groups(a.n_tiles, F);
    const int64_t blocks = (int64_t)m_tiles_upper(g) * a.n_tiles;
    grouped_gemm_bf16_kernel<M_DOWN, false><<<grid_for_work(blocks), 64 * waves_of<M_DOWN, false>(), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_bwd_gate_up_bf16(const GroupArgs& g, const void* x, const void* W1, const void* W3,
                                   const void* Ws1, const void* Ws3, void* gu, int D, int F,
                                   hipStream_t s) {
    GemmArgs a{g, (const uint16_t*)x, (const uint16_t*)W1, (const uint16_t*)W3,
               (const uint16_t*)Ws1, (const uint16_t*)Ws3, gu, D, F, (F + TF / 2 - 1) / (TF / 2)};
    a.col_groups = column_groups(a.n_tiles, D);
    const int64_t blocks = (int64_t)m_tiles_upper(g) * a.n_tiles;
    // half tiles on short grids, as the forward's up GEMM (gate/up measured
    // 4% faster on them at 4096 tokens, 4% slower at 32768)
    if (up_half_tiles(blocks))
        grouped_gemm_bf16_kernel<M_GU, true><<<grid_for_work(2 * blocks), 64 * waves_of<M_GU, true>(), 0, s>>>(a);
    else
        grouped_gemm_bf16_kernel<M_GU, false><<<grid_for_work(blocks), 64 * waves_of<M_GU, false>(), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_bwd_dh_bf16(const GroupArgs& g, const float* topk_w, const void* dy,
                              const void* W2t, const void* Ws2t, const void* gu, void* dgu, void* hw,
                              float* dwpart, int D, int F, hipStream_t s) {
    GemmArgs a{g, (const uint16_t*)dy, (const uint16_t*)W2t, nullptr, (const uint16_t*)Ws2t, nullptr,
               dgu, D, F, (F + TF - 1) / TF, 1, topk_w, (const uint16_t*)gu, (uint16_t*)hw, dwpart};
    a.col_groups = column_groups(a.n_tiles, D);
    const int64_t blocks = (int64_t)m_tiles_upper(g) * a.n_tiles;
    // half tiles: two 128-row workgroups per 256-row tile
    grouped_gemm_bf16_kernel<M_DH, true><<<grid_for_work(2 * blocks), 64 * waves_of<M_DH, true>(), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
