// gemm_bf16_small.hip -- the down grouped GEMM for small per-expert chunks.
//
// The same product as gemm_bf16.hip's down mode, Y = bf16(h . W2), shaped
// for the regime where each expert sees only tens to a few hundred rows and
// the weights dominate the traffic (the "small chunks" that "Triton MoE
// Kernels & Memory Checkpointing", Part A sections 2 and 6.1, calls the
// pathological regime).  There the product is bound by streaming each
// expert's weights once, so the tile is small in both directions to spread
// the weights over many workgroups (the up product of this regime is
// gemm_bf16_slab.hip):
//
//  * tile 64 rows x 64 output columns, K step 64;
//  * 256 threads = 4 wavefronts (2 column x 2 row blocks), one 32 x 32
//    v_mfma_f32_32x32x16_bf16 block each; two workgroups per CU;
//  * a 4-deep ring of LDS stages (16 KiB each) filled with global_load_lds
//    (two stages in flight while one computes), and the next stage's
//    operands read from LDS while the current stage's MFMAs run;
//  * tiles run m-major (all column tiles of one row tile back to back), so
//    an XCD works through one group's whole weight matrix with neighbouring
//    workgroups reading neighbouring parts of each weight row, and the
//    group's next row tile finds the weights in that XCD's L2.
#include "mfma_common.h"

namespace moe {
namespace {

using namespace mfma;

constexpr int TT = kSmallTileRows;   // 64 rows per tile
constexpr int TF = 64;               // output columns per tile
constexpr int BK = 64;
constexpr int NT = 256;
constexpr int X_ROW = BK * 2;                  // 128 B
constexpr int X_BYTES = TT * X_ROW;            // 8 KiB
constexpr int W_ROW = TF * 2;                  // 128 B (64 columns of one k row)
constexpr int W_BYTES = BK * W_ROW;            // 8 KiB
constexpr int STAGE_BYTES = X_BYTES + W_BYTES; // 16 KiB

static_assert(TT == 64 && TF == 64 && BK == 64 && NT == 256, "index math below assumes these");

// [K][N] rows of 128 B read with ds_read_b64_tr_b16: rows k and k+2 (same
// bank half) land on disjoint chunk sets.
__device__ __forceinline__ int swz_tr128(int k) { return 4 * ((k >> 1) & 1); }

struct SmallArgs {
    GroupArgs g;
    const uint16_t* a;        // h [R, F]
    const uint16_t* b0;       // W2 [E, F, D]
    const uint16_t* bs0;      // shared expert's Ws2 [F, D]
    uint16_t* out;            // Y [R, D]
    int D, F;
    int n_tiles;
};

__global__ __launch_bounds__(NT, 2) void grouped_gemm_small_down_kernel(const SmallArgs a) {
    __shared__ __attribute__((aligned(1024))) char st0[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char st1[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char st2[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char st3[STAGE_BYTES];

    const int K = a.F;
    const int N = a.D;
    // the group lookup's loads go out with the tile count's (one round trip)
    const GroupBlock gblock = load_group_block(a.g, 0, threadIdx.x & 63);
    const int total = a.g.tile_off[a.g.G];
    const int id = xcd_remap_work(blockIdx.x, total * a.n_tiles);
    if (id < 0) return;
    const int mt = id / a.n_tiles, nt = id - mt * a.n_tiles;     // m-major
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wf = wave >> 1, wt = wave & 1;
    const TileGroup tg = find_tile_group(a.g, mt, TT, lane, gblock);
    const int grp = tg.grp;
    const bool shared = grp >= a.g.E;
    const int64_t tile_r0 = tg.tile_r0;
    const int valid_rows = tg.valid_rows;
    if (valid_rows <= 0) return;

    // ---- row tile: DMA instruction j (0, 1) of wavefront w fills rows 16 w +
    // 8 j .. +7 (rows past the group's end re-read its last row, never stored).
    const char* x_src[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = 16 * wave + 8 * j + (lane >> 3);
        const int64_t src_row = tile_r0 + min(row, valid_rows - 1);
        x_src[j] = (const char*)(a.a + src_row * (int64_t)K + 8 * ((lane & 7) ^ swz8(row)));
    }
    // ---- weight tile [64 k][64 columns]: DMA instruction j (0, 1) of
    // wavefront w fills k rows 16 w + 8 j .. +7; lane -> k row 16 w + 8 j +
    // lane/8, physical chunk lane%8 holding logical chunk lc = phys ^ swz(k),
    // output columns 8 lc .. 8 lc + 7 of the tile.
    const int64_t gstride = (int64_t)a.D * a.F;
    const char* w_src[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int kr = 16 * wave + 8 * j + (lane >> 3);
        const int lc = (lane & 7) ^ swz_tr128(kr);
        int col = nt * TF + 8 * lc;
        const uint16_t* base = shared ? a.bs0 : a.b0 + grp * gstride;
        if (col >= N) col = 0;                 // past the last column: a valid chunk, never stored
        w_src[j] = (const char*)(base + (int64_t)kr * N + col);
    }
    const int64_t w_step = (int64_t)BK * N * 2;

    auto issue = [&](int kt, char* st) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            load_lds16(x_src[j] + (int64_t)kt * X_ROW, st + (16 * wave + 8 * j) * X_ROW);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            load_lds16(w_src[j] + kt * w_step, st + X_BYTES + (16 * wave + 8 * j) * W_ROW);
    };

    // ---- operands: weights (A) through transposed reads: lane = 16 G + s
    // reads k = 16 ks + 8 (G>>1) + 4 r + s/4, feature 32 wf + 16 (G&1) + 4 (s&3);
    // rows (B): row 32 wt + lane%32, logical chunk 2 ks + lane/32.
    const int G = lane >> 4, sl = lane & 15;
    int w_off[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int k = 8 * (G >> 1) + 4 * r + (sl >> 2);
        const int R = 32 * wf + 16 * (G & 1) + 4 * (sl & 3);
        w_off[r] = X_BYTES + k * W_ROW + (((R >> 3) ^ swz_tr128(k)) << 4) + 8 * (sl & 1);
    }
    const int xrow = 32 * wt + (lane & 31);
    const int x_off = xrow * X_ROW, x_swz = swz8(xrow);

    f32x16_t acc = {};
    struct Frags {
        bf16x8_t w[BK / 16], x[BK / 16];
    };
    auto read_frags = [&](const char* st, Frags& f) {
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            f.w[ks] = cat_bf16(read_tr(st + w_off[0] + ks * 16 * W_ROW),
                               read_tr(st + w_off[1] + ks * 16 * W_ROW));
            const int c = (2 * ks + (lane >> 5)) ^ x_swz;
            f.x[ks] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(st + x_off + (c << 4)));
        }
    };
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

    // ---- 4-stage ring, software-pipelined one stage deep in registers.
    // Step s (its operands fc already in registers): wait until stage s+1
    // has landed (one later stage of this wavefront's loads may still be
    // outstanding) and fc's LDS reads have returned, then a bare s_barrier
    // (__syncthreads() would also wait for the stage in flight and drain the
    // ring); issue the loads of stage s+3 into the buffer of stage s-1; read
    // stage s+1's operands into fn; MFMAs on fc, the reads landing under
    // them.  The buffer of stage s-1 is free: its operands were read in step
    // s-2 and consumed by the MFMAs of step s-1, which every wavefront
    // finished before this barrier.  Loads past the last stage re-read the
    // last stage (never computed on), so each stage has the same load count.
    const int KT = K / BK;
    constexpr int PER_STAGE = 4;       // global_load_lds per wavefront per stage
    auto step = [&](Frags& fc, Frags& fn, const char* nxt, char* dma, int kl) {
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(PER_STAGE, 0));
        __builtin_amdgcn_s_barrier();
        fence();
        issue(kl, dma);
        read_frags(nxt, fn);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fc.w[ks], fc.x[ks], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < BK / 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // vector memory
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // LDS read
        }
        fence();
    };
    Frags fa, fb;
    issue(0, st0);
    issue(min(1, KT - 1), st1);
    issue(min(2, KT - 1), st2);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * PER_STAGE, 15));   // stage 0 landed
    __builtin_amdgcn_s_barrier();
    fence();
    read_frags(st0, fa);
    fence();
    int kt = 0;
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
    wait_vmem();

    // ---- epilogue.  acc element v of lane l: row 32 wt + l%32, MFMA feature
    // 32 wf + 8 (v/4) + 4 (l/32) + v%4.
    const int t = xrow;
    if (t >= valid_rows) return;
    uint16_t* out = a.out + (tile_r0 + t) * (int64_t)N;
#pragma unroll
    for (int vg = 0; vg < 4; ++vg) {
        const int col = nt * TF + 32 * wf + 8 * vg + 4 * (lane >> 5);
        if (col >= N) continue;
        const int v = 4 * vg;
        *(uint2*)(out + col) = make_uint2(pack_bf16(acc[v], acc[v + 1]),
                                          pack_bf16(acc[v + 2], acc[v + 3]));
    }
}

int m_tiles_upper_small(const GroupArgs& g) {
    const int64_t rows = g.S + (g.G > g.E ? g.T : 0);
    return (int)((rows + TT - 1) / TT) + g.G;
}

}  // namespace

hipError_t launch_down_bf16_small(const GroupArgs& g, const void* h, const void* W2, const void* Ws2,
                                  void* Y, int D, int F, hipStream_t s) {
    SmallArgs a{g, (const uint16_t*)h, (const uint16_t*)W2, (const uint16_t*)Ws2, (uint16_t*)Y, D, F,
                (D + TF - 1) / TF};
    const int64_t blocks = (int64_t)m_tiles_upper_small(g) * a.n_tiles;
    grouped_gemm_small_down_kernel<<<grid_for_work(blocks), NT, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
