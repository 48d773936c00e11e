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
//  down:       Yw[p] = bf16(w(p) * (h[p] . W2[grp]))   (fp32 accumulate), the
//              per-expert W2 product followed by the scaling with the routing
//              weight of the same page's section 10.3 step 4; w(p) is the
//              weight of the slot in row p (1 on shared rows).
//
// Tile engine (256 threads = 4 wavefronts, one per SIMD):
//  * the MFMA computes the transposed tile C^T = W^T . X^T: its A operand is
//    a 32-feature block of the weights, its B operand a 32-token block of
//    rows, so each lane ends with 4 consecutive output features of one token
//    and stores 8 bytes (h, bf16) or 16 bytes (Y, fp32) at a time;
//  * workgroup tile 256 tokens x 256 MFMA features (up: 128 W1 + 128 W3
//    columns of the same 128 outputs), K step 64, wave tile 128 x 128 =
//    4 x 4 v_mfma_f32_32x32x16_bf16 accumulators;
//  * both tiles go global -> LDS with global_load_lds (16 bytes per lane, no
//    registers), double-buffered (2 x 64 KiB); the loads of step k+1 are in
//    flight while step k computes;
//  * token rows are K-contiguous in memory and in LDS (read with
//    ds_read_b128); the weights stay [K][N] (N contiguous) in LDS and the
//    MFMA's K-consecutive operand is produced by ds_read_b64_tr_b16, which
//    hands each lane 4 consecutive K values of its own column;
//  * LDS rows are XOR-swizzled in 16-byte chunks (token rows by
//    (row ^ row/8) & 7, weight rows by 4 (k & 3)); since global_load_lds
//    writes each wavefront's 1 KiB contiguously, the swizzle is applied by
//    choosing which global chunk each lane fetches.
//
// Row tiles never cross a group: group g owns tiles tile_off[g] ..
// tile_off[g+1]-1 (computed by the permute on the device), the grid is sized
// by the host from an upper bound, and workgroups past tile_off[G] exit, so
// no host synchronisation is needed.  Rows past a group's end are clamped
// to its last row on load and never stored.
#include "mfma_common.h"

namespace moe {
namespace {

using namespace mfma;

constexpr int TT = kBf16TileRows;   // 256 tokens (rows) per tile
constexpr int TF = 256;             // MFMA features per tile (up: 128 g + 128 u)
constexpr int BK = 64;
constexpr int NT = 256;
constexpr int X_BYTES = TT * BK * 2;                 // 32 KiB token tile
constexpr int W_BYTES = BK * TF * 2;                 // 32 KiB weight tile
constexpr int STAGE_BYTES = X_BYTES + W_BYTES;
constexpr int X_ROW = BK * 2;                        // 128 B per token row
constexpr int W_ROW = TF * 2;                        // 512 B per k row

static_assert(TT == 256 && TF == 256 && BK == 64 && NT == 256, "index math below assumes these");

__device__ __forceinline__ int swz_x(int row) { return swz8(row); }
__device__ __forceinline__ int swz_w(int k) { return swz_tr(k); }

struct GemmArgs {
    GroupArgs g;
    const uint16_t* a;        // up: x [T, D]; down: h [R, F]
    const uint16_t* b0;       // up: W1 [E, D, F]; down: W2 [E, F, D]
    const uint16_t* b1;       // up: W3; down: unused
    const uint16_t* bs0;      // shared expert: up Ws1, down Ws2
    const uint16_t* bs1;      // up Ws3
    void* out;                // up: h bf16 [R, F]; down: Yw bf16 [R, D]
    int D, F;
    int n_tiles;              // column tiles
};

template <bool UP>
__global__ __launch_bounds__(NT, 1) void grouped_gemm_bf16_kernel(const GemmArgs a) {
    // Two stage buffers as separate LDS objects: every access names its buffer
    // statically, so the compiler knows reads of one buffer do not alias the
    // asynchronous global_load_lds writes into the other and does not wait
    // for them.
    __shared__ __attribute__((aligned(1024))) char lds0[STAGE_BYTES];   // 64 KiB
    __shared__ __attribute__((aligned(1024))) char lds1[STAGE_BYTES];   // 64 KiB

    const int K = UP ? a.D : a.F;      // reduction length
    const int N = UP ? a.F : a.D;      // output columns
    const int ldw = N;                 // weight row stride (elements)

    const int bid = xcd_remap_work(blockIdx.x, a.g.tile_off[a.g.G] * a.n_tiles);
    if (bid < 0) return;
    const int mt = bid / a.n_tiles, nt = bid - mt * a.n_tiles;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wf = wave >> 1, wt = wave & 1;   // wave's feature half, token half

    // ---- the group owning row tile mt, and the tile's rows.
    const int32_t* tile_off = a.g.tile_off;
    if (mt >= tile_off[a.g.G]) return;
    const TileGroup tg = find_tile_group(a.g, mt, TT, lane);
    const int grp = tg.grp;
    const bool shared = grp >= a.g.E;
    const int64_t tile_r0 = tg.tile_r0;
    const int valid_rows = tg.valid_rows;
    if (valid_rows <= 0) return;       // only if tile_off disagrees with offsets

    // ---- token tile sources: wave instruction j fills LDS rows 64 wave + 8 j .. +7;
    // lane -> row 64 wave + 8 j + lane/8, physical chunk lane%8.  Routed rows of
    // the up GEMM gather token perm[p] / k (all eight index loads in flight at
    // once); shared rows read token p - S; the down GEMM reads row p of h.
    int64_t src_row[8];
    if (UP && !shared) {
        int32_t slot[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            slot[j] = a.g.perm[tile_r0 + min(64 * wave + 8 * j + (lane >> 3), valid_rows - 1)];
#pragma unroll
        for (int j = 0; j < 8; ++j) src_row[j] = slot[j] / a.g.k;
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            src_row[j] = tile_r0 + min(64 * wave + 8 * j + (lane >> 3), valid_rows - 1) -
                         (UP ? a.g.S : 0);
    }
    // Down GEMM: routing weight of each of this lane's 4 output rows (1 on shared rows).
    float row_w[4] = {1.f, 1.f, 1.f, 1.f};
    if (!UP && !shared) {
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) {
            const int t = min(128 * wt + 32 * nj + (lane & 31), valid_rows - 1);
            row_w[nj] = a.g.topk_w[a.g.perm[tile_r0 + t]];
        }
    }
    const char* x_src[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int row = 64 * wave + 8 * j + (lane >> 3);
        const int c = (lane & 7) ^ swz_x(row);
        x_src[j] = (const char*)(a.a + src_row[j] * (int64_t)K + 8 * c);
    }

    // ---- weight tile sources: wave instruction j fills k rows 16 wave + 2 j, +1;
    // lane -> row 16 wave + 2 j + lane/32, physical chunk lane%32.
    const int64_t gstride = (int64_t)a.D * a.F;
    const char* w_src[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int kr = 16 * wave + 2 * j + (lane >> 5);
        const int c = (lane & 31) ^ swz_w(kr);          // logical chunk: 8 feature columns
        int col;
        const uint16_t* base;
        if (UP) {
            const int half = c >> 4, kind = (c >> 3) & 1;   // kind 0: W1 (g), 1: W3 (u)
            col = nt * (TF / 2) + half * 64 + (c & 7) * 8;
            base = shared ? (kind ? a.bs1 : a.bs0) : (kind ? a.b1 : a.b0) + grp * gstride;
        } else {
            col = nt * TF + c * 8;
            base = shared ? a.bs0 : a.b0 + grp * gstride;
        }
        if (col >= N) col = 0;                 // past the last column: a valid chunk, never stored
        w_src[j] = (const char*)(base + (int64_t)kr * ldw + col);
    }
    const int64_t w_step = (int64_t)BK * ldw * 2;      // bytes per K step in the weights

    // One global_load_lds of the stage-kt tiles into buffer xs: instruction
    // q < 8 is token-tile instruction q, q >= 8 weight-tile instruction q - 8.
    auto dma = [&](int kt, char* xs, int q) {
        if (q < 8)
            load_lds16(x_src[q] + (int64_t)kt * X_ROW, xs + (64 * wave + 8 * q) * X_ROW);
        else
            load_lds16(w_src[q - 8] + kt * w_step, xs + X_BYTES + (16 * wave + 2 * (q - 8)) * W_ROW);
    };

    // ---- MFMA operand read offsets (bytes within a stage).
    // Weight operand (A): lane = 16 G + s reads k = 16 ks + 8 (G>>1) + 4 r + s/4,
    // feature R = 128 wf + 32 mi + 16 (G&1) + 4 (s&3).
    const int G = lane >> 4, s = lane & 15;
    int w_off[4][2];   // [mi][r] for ks = 0; later ks add 16 rows (swizzle repeats every 4 rows)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int k = 8 * (G >> 1) + 4 * r + (s >> 2);
            const int R = 128 * wf + 32 * mi + 16 * (G & 1) + 4 * (s & 3);
            w_off[mi][r] = X_BYTES + k * W_ROW + (((R >> 3) ^ swz_w(k)) << 4) + 8 * (s & 1);
        }
    // Token operand (B): lane reads row 128 wt + 32 nj + lane%32, logical chunk 2 ks + lane/32.
    int x_row_off[4], x_swz[4];
#pragma unroll
    for (int nj = 0; nj < 4; ++nj) {
        const int row = 128 * wt + 32 * nj + (lane & 31);
        x_row_off[nj] = row * X_ROW;
        x_swz[nj] = swz_x(row);
    }

    f32x16_t acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) acc[mi][nj] = f32x16_t{};

    struct Frags {
        bf16x8_t w[4], x[4];
    };
    auto read_frags = [&](const char* st, int ks, Frags& f) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            f.w[mi] = cat_bf16(read_tr(st + w_off[mi][0] + ks * 16 * W_ROW),
                               read_tr(st + w_off[mi][1] + ks * 16 * W_ROW));
        }
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) {
            const int c = (2 * ks + (lane >> 5)) ^ x_swz[nj];
            f.x[nj] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(st + x_row_off[nj] + (c << 4)));
        }
    };
    auto mfmas = [&](const Frags& f) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int nj = 0; nj < 4; ++nj)
                acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.w[mi], f.x[nj], acc[mi][nj],
                                                                      0, 0, 0);
    };
    // One K step on stage buffer st (its ks = 0 operands already in fa) while
    // stage kl streams into nx.  Each k16 slice first issues the next slice's
    // 12 LDS reads and 4 of the next stage's global_load_lds, then its own 16
    // independent MFMAs; the scheduling fences keep that order, so every LDS
    // read has 16 MFMAs (~512 cycles) to land before it is used.
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    auto step = [&](const char* st, char* nx, int kl, Frags& fa, Frags& fb) {
        read_frags(st, 1, fb);
#pragma unroll
        for (int q = 0; q < 4; ++q) dma(kl, nx, q);
        fence();
        mfmas(fa);
        fence();
        read_frags(st, 2, fa);
#pragma unroll
        for (int q = 4; q < 8; ++q) dma(kl, nx, q);
        fence();
        mfmas(fb);
        fence();
        read_frags(st, 3, fb);
#pragma unroll
        for (int q = 8; q < 12; ++q) dma(kl, nx, q);
        fence();
        mfmas(fa);
        fence();
#pragma unroll
        for (int q = 12; q < 16; ++q) dma(kl, nx, q);
        fence();
        mfmas(fb);
        fence();
    };

    // K loop, unrolled by two so the stage buffer of every access is static.
    // The step after the last one reloads the last stage into the idle buffer
    // (an L2 hit) instead of branching around the loads.
    const int KT = K / BK;
#pragma unroll
    for (int q = 0; q < 16; ++q) dma(0, lds0, q);
    wait_vmem();
    __syncthreads();
    Frags fa, fb;
    read_frags(lds0, 0, fa);
    int kt = 0;
    for (; kt + 2 <= KT; kt += 2) {
        step(lds0, lds1, kt + 1, fa, fb);
        wait_vmem();
        __syncthreads();
        read_frags(lds1, 0, fa);
        step(lds1, lds0, min(kt + 2, KT - 1), fa, fb);
        wait_vmem();
        __syncthreads();
        read_frags(lds0, 0, fa);
    }
    if (kt < KT) {                     // odd step count: the last step sits in lds0
        step(lds0, lds1, KT - 1, fa, fb);
        wait_vmem();
    }

    // ---- epilogue.  acc[mi][nj] element v of lane l: token 128 wt + 32 nj + l%32,
    // feature 128 wf + 32 mi + 8 (v/4) + 4 (l/32) + v%4.
#pragma unroll
    for (int nj = 0; nj < 4; ++nj) {
        const int t = 128 * wt + 32 * nj + (lane & 31);
        if (t >= valid_rows) continue;
        const int64_t row = tile_r0 + t;
        uint16_t* out = (uint16_t*)a.out + row * (int64_t)N;
        if (UP) {
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int vg = 0; vg < 4; ++vg) {
                    const int col = nt * (TF / 2) + 64 * wf + 32 * mi + 8 * vg + 4 * (lane >> 5);
                    if (col >= N) continue;
                    const f32x16_t& g = acc[mi][nj];
                    const f32x16_t& u = acc[mi + 2][nj];
                    const int v = 4 * vg;
                    *(uint2*)(out + col) =
                        make_uint2(pack_bf16(silu_mul(g[v], u[v]), silu_mul(g[v + 1], u[v + 1])),
                                   pack_bf16(silu_mul(g[v + 2], u[v + 2]), silu_mul(g[v + 3], u[v + 3])));
                }
        } else {
            const float wt_row = row_w[nj];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int vg = 0; vg < 4; ++vg) {
                    const int col = nt * TF + 128 * wf + 32 * mi + 8 * vg + 4 * (lane >> 5);
                    if (col >= N) continue;
                    const f32x16_t& c = acc[mi][nj];
                    const int v = 4 * vg;
                    *(uint2*)(out + col) = make_uint2(pack_bf16(wt_row * c[v], wt_row * c[v + 1]),
                                                      pack_bf16(wt_row * c[v + 2], wt_row * c[v + 3]));
                }
        }
    }
}

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
    const int64_t blocks = (int64_t)m_tiles_upper(g) * a.n_tiles;
    grouped_gemm_bf16_kernel<true><<<grid_for_work(blocks), NT, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_down_bf16(const GroupArgs& g, const void* h, const void* W2, const void* Ws2,
                            void* Y, int D, int F, hipStream_t s) {
    GemmArgs a{g, (const uint16_t*)h, (const uint16_t*)W2, nullptr, (const uint16_t*)Ws2, nullptr,
               Y, D, F, (D + TF - 1) / TF};
    const int64_t blocks = (int64_t)m_tiles_upper(g) * a.n_tiles;
    grouped_gemm_bf16_kernel<false><<<grid_for_work(blocks), NT, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
