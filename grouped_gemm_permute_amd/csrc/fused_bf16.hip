// fused_bf16.hip -- fused up-act-down variant of the expert FFN (bf16 MFMA).
//
// "Chinchilla scaling, MoE, and fused Triton kernels" (sections "Fused
// Triton kernel mechanism" and "Triton fused kernel implementation")
// describes one program per token tile that keeps the tile's output
// accumulator [tokens, D] on chip and streams the expanded dimension F in
// tiles: for each F tile, h = act(x . Wup[:, f]) and acc += h . Wdown[f, :],
// so h never makes the HBM round trip (saving the 4 t F bytes of that page's
// traffic model).  Here the activation is SwiGLU, as everywhere in this
// library:
//
//   for each chunk of CH = 256 h columns f (the last one may hold 128):
//     g, u = x_tile . W1[:, f], x_tile . W3[:, f]        (fp32 accumulate, K = D)
//     h    = bf16(silu(g) * u)                           (into LDS)
//     acc += h . W2[f, :]                                (fp32 accumulate, K = CH)
//   Y[row] = bf16(acc[row])                              (the combine applies the routing weight)
//
// Shapes and placement on gfx950 (512 threads = 8 wavefronts, two per SIMD,
// one workgroup per CU):
//  * token tile TT = 64 rows of one group; the fp32 accumulator acc is
//    64 x D (D <= 1024 -> at most 128 accumulator registers per lane, which
//    two wavefronts per SIMD can hold).  With D / 128 even, wavefront w owns
//    output columns w D / 8 .. +D/8 - 1 of all 64 rows; otherwise columns
//    (w % 4) D / 4 .. +D/4 - 1 of rows 32 (w / 4) .. +31;
//  * up phase: MFMA tile 512 features x 64 tokens per chunk; wavefront w
//    owns two 32-feature blocks, each 16 W1 columns followed by the same 16
//    W3 columns (h columns 32 w .. 32 w + 31), for both 32-row blocks, so
//    accumulator elements v (g) and v + 8 (u) of a lane belong to the same h
//    element and every operand fragment read from LDS feeds two MFMAs (the
//    LDS read rate, not the MFMA rate, bounds a tile this short);
//  * the up phase (K step 16: token rows [64][16], weights [16][512]) and
//    the down phase (16 rows of W2 [16][D] per step) share one stream of
//    stages through a ring of four 32 KiB LDS buffers, two stages in flight
//    while one is computed, all filled with global_load_lds; weights stay
//    [K][N] and reach the MFMA through ds_read_b64_tr_b16, token rows and h
//    are K-contiguous; h of the current chunk sits in its own 32 KiB buffer
//    (160 KiB of LDS in all);
//  * token rows are loaded with the non-temporal policy: each tile re-reads
//    its own 128 KiB of x once per chunk, and 32 tiles' worth would fill an
//    XCD's L2 and evict the weight chunks its workgroups share;
//  * tiles are numbered group-major and each XCD takes a contiguous range,
//    so the workgroups of one XCD work on the same expert at the same time
//    and share each weight chunk through that XCD's L2, each starting the
//    chunk's steps at a different point;
//  * the tiles of the last, partial round of 256 workgroups (all tiles when
//    there are fewer than 256) are shared out over s workgroups each
//    (fused_plan): workgroup (tile, sp) runs chunks sp NCH / s ..
//    (sp + 1) NCH / s - 1 and stores its fp32 accumulator as a partial
//    output; fused_reduce_kernel adds a tile's partials in split order and
//    rounds once to bf16 Y.  Ragged group ends make the tile count a little
//    over a multiple of 256 (16384 tokens on 16 experts: 528 tiles), and
//    the few tiles past it would otherwise cost a whole extra round.
//
// Measured on the 16384-token F > D workload (D 1024, F 4096, 16 experts):
// the kernel stages ~27 MB per 64-row tile (each tile re-streams its
// expert's weights), ~50 MB per CU per launch, and sustains ~40 GB/s of
// weight staging per CU; with no loads at all its loop alone takes half the
// launch.  The unfused pair stages 4x fewer bytes per FLOP and is faster.
#include <algorithm>

#include "mfma_common.h"

namespace moe {
namespace {

using namespace mfma;

constexpr int TT = kFusedTileRows;   // 64 tokens per tile
constexpr int CH = 256;              // h columns per F chunk
constexpr int NW = 8;                // wavefronts
constexpr int NT = 64 * NW;
constexpr int UP_BK = 16;                        // up K step
constexpr int X_ROW = UP_BK * 2;                 // 32 B token row (K-contiguous)
constexpr int X_BYTES = TT * X_ROW;              // 2 KiB
constexpr int WGU_ROW = 2 * CH * 2;              // 1 KiB: 512 features of one k row
constexpr int WGU_BYTES = UP_BK * WGU_ROW;       // 16 KiB
constexpr int UP_LOADS = (X_BYTES + WGU_BYTES) / 1024;   // 1 KiB DMA instructions per up stage
constexpr int DN_K = 16;                         // W2 rows per down stage
constexpr int DN_STEPS = CH / DN_K;              // 16 down stages per whole chunk
constexpr int STAGE_BYTES = 32 * 1024;           // >= max(18 KiB up, 16 * 2 D down)
constexpr int H_ROW = CH * 2;                    // 512 B
constexpr int H_BYTES = TT * H_ROW;              // 32 KiB

static_assert(TT == 64 && CH == 256 && NW == 8 && UP_BK == 16, "index math below assumes these");
static_assert(X_BYTES + WGU_BYTES <= STAGE_BYTES && 4 * STAGE_BYTES + H_BYTES <= 160 * 1024,
              "four stages and h fit in LDS");

// 32-byte token rows (2 chunks): the 16 rows one ds_read_b128 phase reads
// at one logical chunk fill distinct bank groups.
__device__ __forceinline__ int swz_x(int row) { return (row >> 3) & 1; }

// Only wavefronts 0 .. LW-1 (one per SIMD) issue the stage loads: DMA
// instructions j = w, w + LW, ... (< n) of a stage belong to wavefront w < LW.
// A wavefront stalls issuing a load while the memory pipe is full; with one
// loader per SIMD its partner keeps the SIMD's MFMAs going meanwhile (3-6%
// faster than all eight wavefronts issuing, measured).
constexpr int LW = 4;
__host__ __device__ constexpr int per_wave(int n, int w) { return w < LW && n > w ? (n - w + LW - 1) / LW : 0; }

// s_waitcnt vmcnt(n) for a wave-uniform n in 0..16 (the immediate must be a
// compile-time constant).
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
        case 0: __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0)); break;
        case 1: __builtin_amdgcn_s_waitcnt(waitcnt_imm(1, 0)); break;
        case 2: __builtin_amdgcn_s_waitcnt(waitcnt_imm(2, 0)); break;
        case 3: __builtin_amdgcn_s_waitcnt(waitcnt_imm(3, 0)); break;
        case 4: __builtin_amdgcn_s_waitcnt(waitcnt_imm(4, 0)); break;
        case 5: __builtin_amdgcn_s_waitcnt(waitcnt_imm(5, 0)); break;
        case 6: __builtin_amdgcn_s_waitcnt(waitcnt_imm(6, 0)); break;
        case 7: __builtin_amdgcn_s_waitcnt(waitcnt_imm(7, 0)); break;
        case 8: __builtin_amdgcn_s_waitcnt(waitcnt_imm(8, 0)); break;
        case 9: __builtin_amdgcn_s_waitcnt(waitcnt_imm(9, 0)); break;
        case 10: __builtin_amdgcn_s_waitcnt(waitcnt_imm(10, 0)); break;
        case 11: __builtin_amdgcn_s_waitcnt(waitcnt_imm(11, 0)); break;
        case 12: __builtin_amdgcn_s_waitcnt(waitcnt_imm(12, 0)); break;
        case 13: __builtin_amdgcn_s_waitcnt(waitcnt_imm(13, 0)); break;
        case 14: __builtin_amdgcn_s_waitcnt(waitcnt_imm(14, 0)); break;
        case 15: __builtin_amdgcn_s_waitcnt(waitcnt_imm(15, 0)); break;
        default: __builtin_amdgcn_s_waitcnt(waitcnt_imm(16, 0)); break;
    }
}

struct FusedArgs {
    GroupArgs g;
    const uint16_t* x;                     // [T, D]
    const uint16_t *W1, *W3, *W2;          // [E, D, F], [E, D, F], [E, F, D]
    const uint16_t *Ws1, *Ws3, *Ws2;       // shared expert or null
    uint16_t* Y;                           // [R, D] bf16 expert outputs (whole tiles)
    float* P;                              // [r s][64][D] fp32 partial outputs (split tiles)
    int D, F;
};

// Workgroup bid -> (tile mt, split sp) under plan p.  XCD x = bid % 8 runs,
// in its first whole / 8 slots, whole tiles x whole / 8 .. (x + 1) whole / 8 - 1
// (whole rounds, contiguous tiles sharing their weights in the XCD's L2),
// then the split units x rs / 8 .. (x + 1) rs / 8 - 1 of the last round
// (unit u: tile whole + u / s, split u % s).  False: nothing to do.
__device__ __forceinline__ bool fused_unit(int bid, const FusedPlan& p, int& mt, int& sp) {
    const int x = bid & 7, i = bid >> 3;
    const int nw = p.whole >> 3;
    if (i < nw) {
        mt = x * nw + i;
        sp = 0;
        return true;
    }
    const int units = p.r * p.s;
    const int u = x * units / 8 + (i - nw);
    if (u >= (x + 1) * units / 8) return false;
    mt = p.whole + u / p.s;
    sp = u - (u / p.s) * p.s;
    return true;
}

// D = 128 * NFB.
template <int NFB>
__global__ __launch_bounds__(NT, 1) void fused_up_act_down_kernel(const FusedArgs a) {
    // Separate LDS objects per stage buffer, each named statically by the
    // unrolled loops below: the compiler then knows reads of one never alias
    // the asynchronous global_load_lds writes into another.
    __shared__ __attribute__((aligned(1024))) char st0[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char st1[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char st2[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char st3[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char hbuf[H_BYTES];

    constexpr int D = 128 * NFB;
    constexpr int DN_ROW = 2 * D;              // bytes of one W2 row in LDS
    constexpr int DN_LOADS = DN_K * DN_ROW / 1024;   // 4 NFB DMA instructions per down stage
    constexpr int KU = D / UP_BK;              // up stages per chunk (8 NFB)
    constexpr int SPC = KU + DN_STEPS;         // stages per whole chunk (a multiple of 4)
    // output layout: NCG column groups of CBW 32-column blocks, RBW row blocks per wavefront
    constexpr int NCG = NFB % 2 == 0 ? 8 : 4;
    constexpr int CBW = 4 * NFB / NCG;
    constexpr int RBW = NCG == 8 ? 2 : 1;
    static_assert(DN_K * DN_ROW <= STAGE_BYTES && SPC % 4 == 0 && KU % 4 == 0, "stage shapes");
    const int F = a.F;
    const int NCH = (F + CH - 1) / CH;         // chunks; the last holds 128 columns when F % 256 != 0
    const bool half = F % CH != 0;

    // work item = (tile mt, split sp of ns): chunks c0 .. c1-1 of tile mt
    const FusedPlan plan = fused_plan(a.g.tile_off[a.g.G], NCH);
    int mt, sp;
    if (!fused_unit(blockIdx.x, plan, mt, sp)) return;
    const int ns = mt >= plan.whole ? plan.s : 1;
    const int c0 = sp * NCH / ns, c1 = (sp + 1) * NCH / ns;
    const int NSTEP = (c1 - c0) * SPC - (half && c1 == NCH ? DN_STEPS / 2 : 0);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const TileGroup tg = find_tile_group(a.g, mt, TT, lane);
    const int grp = tg.grp;
    const bool shared = grp >= a.g.E;
    const int64_t tile_r0 = tg.tile_r0;
    const int valid_rows = tg.valid_rows;
    if (valid_rows <= 0) return;

    const int64_t gstride = (int64_t)D * F;
    const uint16_t* W1g = shared ? a.Ws1 : a.W1 + grp * gstride;
    const uint16_t* W3g = shared ? a.Ws3 : a.W3 + grp * gstride;
    const uint16_t* W2g = shared ? a.Ws2 : a.W2 + grp * gstride;

    // DMA loads of this wavefront per stage (fixed per stage kind).
    const int up_n = per_wave(UP_LOADS, wave);
    const int dn_n = per_wave(DN_LOADS, wave);

    // ---- up stage: instruction j (0..17) fills LDS bytes 1024 j .. +1023.
    // j < 2: token rows 32 j .. 32 j + 31 (lane -> row 32 j + lane/2,
    // physical chunk lane%2 holding logical chunk (lane%2) ^ swz_x(row));
    // j >= 2: weight k row j - 2 (lane = physical chunk, holding logical chunk
    // cl = lane ^ swz_tr(k): MFMA features 8 cl .. 8 cl + 7 = wavefront block
    // cl / 8, its 32-feature block (cl / 4) % 2, W3 when (cl / 2) is odd, h
    // column 32 (cl / 8) + 16 ((cl / 4) % 2) + 8 (cl % 2)).  Loader w < 4
    // issues j = w, w + 4, ..., w + 16 (< 18): waves 0 and 1 own token block w,
    // and loader w owns weight rows (w + 2) % 4 + 4 i, i = 0..3.  A
    // wavefront's weight rows share k % 4, hence one per-lane source.
    const char* x_src = nullptr;
    if (wave < 2) {
        const int row = 32 * wave + (lane >> 1);
        const int64_t p = tile_r0 + min(row, valid_rows - 1);
        const int64_t tok = shared ? p - a.g.S : (int64_t)(a.g.perm[p] / a.g.k);
        x_src = (const char*)(a.x + tok * D + 8 * ((lane & 1) ^ swz_x(row)));
    }
    const int kw0 = (wave + 2) & 3;                   // first weight k row of loader wavefront w < LW: rows kw0 + 4 i
    int col_hi;                                       // 128 when this lane's column is in the chunk's upper half
    const uint16_t* w_src;
    {
        const int cl = lane ^ swz_tr(kw0);
        const int col = 32 * (cl >> 3) + 16 * ((cl >> 2) & 1) + 8 * (cl & 1);
        col_hi = col >= 128 ? 128 : 0;
        w_src = (((cl >> 1) & 1) ? W3g : W1g) + col;
    }
    auto issue_up = [&](int c, int ks, char* st) {
        if (wave < 2) load_lds16_nt(x_src + ks * X_ROW, st + 1024 * wave);
        // a last chunk of 128 columns re-reads the lower half for the upper
        // (valid addresses; those features are never used)
        const uint16_t* base = w_src + c * CH - (half && c == NCH - 1 ? col_hi : 0);
        const int64_t k0 = (int64_t)ks * UP_BK + kw0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            load_lds16(base + (k0 + 4 * i) * F, st + X_BYTES + 1024 * (kw0 + 4 * i));
    };
    // ---- down stage: W2 rows [16][D] = 256 NFB chunks; instruction j
    // covers linear chunks 64 j + lane: row L / (16 NFB), physical chunk
    // L % (16 NFB) holding logical chunk phys ^ swz_tr(row).
    auto issue_down = [&](int c, int q, char* st) {
        const uint16_t* base = W2g + (int64_t)(c * CH + DN_K * q) * D;
#pragma unroll
        for (int i = 0; i < (DN_LOADS + LW - 1) / LW; ++i) {
            const int j = wave + LW * i;
            if (j < DN_LOADS) {
                const int L = 64 * j + lane;
                const int row = L / (16 * NFB), pc = L - row * (16 * NFB);
                load_lds16(base + row * D + 8 * (pc ^ swz_tr(row)), st + 1024 * j);
            }
        }
    };
    // stage s of the stream: chunk c = c0 + s / SPC, up step (s % SPC) < KU,
    // else down step (s % SPC) - KU.  Stages past the last re-load the last one
    // (a down stage, into a buffer never computed on), so every stage issues
    // its kind's fixed number of loads.
    // Neighbouring tiles (which run at the same time on one XCD) walk a
    // chunk's up and down steps from 8 different starting points, so they
    // request different weight rows of the shared chunk at any moment
    // instead of all the same lines (3.5% faster than all starting at 0,
    // measured; the order is fixed per tile, so results stay reproducible).
    const int rot = mt % 8;
    auto issue = [&](int s, char* st) {
        if (wave >= LW) return;
        s = min(s, NSTEP - 1);
        const int r = s - (s / SPC) * SPC, c = c0 + s / SPC;
        if (r < KU) issue_up(c, (r + rot * (KU / 8)) % KU, st);
        else {
            const int dsn = half && c == NCH - 1 ? DN_STEPS / 2 : DN_STEPS;
            issue_down(c, (r - KU + rot * (dsn / 8)) % dsn, st);
        }
    };
    auto loads_of = [&](int s) {
        s = min(s, NSTEP - 1);
        return s - (s / SPC) * SPC < KU ? up_n : dn_n;
    };

    // ---- operand read offsets.  Transposed weight reads: lane = 16 G + s
    // reads k = 8 (G>>1) + 4 r + s/4, feature R = ... + 16 (G&1) + 4 (s&3);
    // the r = 1 read is the r = 0 one plus four rows.
    const int G = lane >> 4, sl = lane & 15;
    const int tk = 8 * (G >> 1) + (sl >> 2);
    int gu_off[2];
#pragma unroll
    for (int fb = 0; fb < 2; ++fb) {
        const int R = 64 * wave + 32 * fb + 16 * (G & 1) + 4 * (sl & 3);
        gu_off[fb] = X_BYTES + tk * WGU_ROW + (((R >> 3) ^ swz_tr(tk)) << 4) + 8 * ((R >> 2) & 1);
    }
    const int cb0 = NCG == 8 ? wave * CBW : (wave & 3) * CBW;   // first 32-column block
    const int rb0 = NCG == 8 ? 0 : (wave >> 2);                  // first 32-row block
    int dn_off[CBW];
#pragma unroll
    for (int i = 0; i < CBW; ++i) {
        const int R = 32 * (cb0 + i) + 16 * (G & 1) + 4 * (sl & 3);
        dn_off[i] = tk * DN_ROW + (((R >> 3) ^ swz_tr(tk)) << 4) + 8 * ((R >> 2) & 1);
    }
    const int xr = lane & 31;                      // token / h row within a 32-row block
    const int x_off = xr * X_ROW + (((lane >> 5) ^ swz_x(xr)) << 4);   // + 32 nj rows

    f32x16_t acc_y[CBW][RBW];
#pragma unroll
    for (int i = 0; i < CBW; ++i)
#pragma unroll
        for (int j = 0; j < RBW; ++j) acc_y[i][j] = f32x16_t{};
    f32x16_t acc_up[2][2];

    // One up K step (16) on stage st: 2 weight frags x 2 token frags = 4 MFMAs;
    // stage s + 3 is issued into dma between the operand reads and the MFMAs.
    auto compute_up = [&](const char* st, int s, char* dma) {
        bf16x8_t wf[2], xf[2];
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
            wf[fb] = cat_bf16(read_tr(st + gu_off[fb]), read_tr(st + gu_off[fb] + 4 * WGU_ROW));
#pragma unroll
        for (int nj = 0; nj < 2; ++nj)
            xf[nj] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(st + x_off + 32 * nj * X_ROW));
        __builtin_amdgcn_sched_barrier(0);
        issue(s + 3, dma);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
#pragma unroll
            for (int nj = 0; nj < 2; ++nj)
                acc_up[fb][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[fb], xf[nj], acc_up[fb][nj], 0, 0, 0);
    };
    // One down K step (16 rows of W2) on stage st, h slice q of the chunk;
    // stage s + 3 is issued once the h slice and the first weight fragment
    // are requested.
    auto compute_down = [&](const char* st, int q, int s, char* dma) {
        bf16x8_t hf[RBW];
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
            const int row = 32 * (rb0 + j) + xr;
            const int c = (2 * q + (lane >> 5)) ^ swz16(row);
            hf[j] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(hbuf + row * H_ROW + (c << 4)));
        }
        const bf16x8_t wf0 = cat_bf16(read_tr(st + dn_off[0]), read_tr(st + dn_off[0] + 4 * DN_ROW));
        __builtin_amdgcn_sched_barrier(0);
        issue(s + 3, dma);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < CBW; ++i) {
            const bf16x8_t wf = i == 0 ? wf0 : cat_bf16(read_tr(st + dn_off[i]), read_tr(st + dn_off[i] + 4 * DN_ROW));
#pragma unroll
            for (int j = 0; j < RBW; ++j)
                acc_y[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, hf[j], acc_y[i][j], 0, 0, 0);
        }
    };
    // h = silu(g) * u for the chunk, bf16, into hbuf (token rows, K-contiguous).
    // acc_up[fb][nj] element v of lane l: token 32 nj + l%32, h column
    // 32 w + 16 fb + 8 (v/4) + 4 (l/32) + v%4 for v < 8 (g), its u at v + 8.
    auto write_h = [&]() {
#pragma unroll
        for (int nj = 0; nj < 2; ++nj) {
            const int t = 32 * nj + xr;
#pragma unroll
            for (int fb = 0; fb < 2; ++fb) {
                const f32x16_t& c = acc_up[fb][nj];
#pragma unroll
                for (int vg = 0; vg < 2; ++vg) {
                    const int v = 4 * vg;
                    const int ch = (4 * wave + 2 * fb + vg) ^ swz16(t);
                    *(uint2*)(hbuf + t * H_ROW + (ch << 4) + 8 * (lane >> 5)) =
                        make_uint2(pack_bf16(silu_mul(c[v], c[v + 8]), silu_mul(c[v + 1], c[v + 9])),
                                   pack_bf16(silu_mul(c[v + 2], c[v + 10]), silu_mul(c[v + 3], c[v + 11])));
                }
            }
        }
    };
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

    // ---- step s (buffer s % 4): wait until stage s has landed (stages s+1
    // and s+2 of this wavefront may still be in flight) and every LDS access
    // of the previous step is done; barrier; read stage s's operands, then
    // issue stage s + 3 into the buffer of stage s - 1 (free: its last
    // readers finished before this barrier), then the MFMAs.  Issuing the
    // loads after the operand reads rather than before them lets the reads
    // go out while the memory pipe is still busy with earlier stages (a
    // wavefront stalls at a load while that pipe is backed up): 8-10% off the
    // kernel, measured.  Each chunk runs its KU up steps, writes h,
    // then its down steps (16, or 8 for a last chunk of 128 columns); every
    // count is a multiple of 4, so every phase starts in buffer 0 and the
    // buffers are named statically.  The barrier of the first down step
    // orders the h writes before the down steps' reads, and the barriers of
    // the next chunk's up phase order those reads before the next write.
    auto begin_step = [&](int s) {
        wait_vm(loads_of(s + 1) + loads_of(s + 2));
        __builtin_amdgcn_s_barrier();
        fence();
    };
    issue(0, st0);
    issue(1, st1);
    issue(2, st2);
    for (int c = c0; c < c1; ++c) {
        const int s0 = (c - c0) * SPC;
#pragma unroll
        for (int fb = 0; fb < 2; ++fb) acc_up[fb][0] = acc_up[fb][1] = f32x16_t{};
        for (int u = 0; u < KU; u += 4) {
            begin_step(s0 + u);
            compute_up(st0, s0 + u, st3);
            fence();
            begin_step(s0 + u + 1);
            compute_up(st1, s0 + u + 1, st0);
            fence();
            begin_step(s0 + u + 2);
            compute_up(st2, s0 + u + 2, st1);
            fence();
            begin_step(s0 + u + 3);
            compute_up(st3, s0 + u + 3, st2);
            fence();
        }
        write_h();
        const int ds = half && c == NCH - 1 ? DN_STEPS / 2 : DN_STEPS;
        const int qr = rot * (ds / 8);
        for (int q = 0; q < ds; q += 4) {
            begin_step(s0 + KU + q);
            compute_down(st0, (q + qr) % ds, s0 + KU + q, st3);
            fence();
            begin_step(s0 + KU + q + 1);
            compute_down(st1, (q + 1 + qr) % ds, s0 + KU + q + 1, st0);
            fence();
            begin_step(s0 + KU + q + 2);
            compute_down(st2, (q + 2 + qr) % ds, s0 + KU + q + 2, st1);
            fence();
            begin_step(s0 + KU + q + 3);
            compute_down(st3, (q + 3 + qr) % ds, s0 + KU + q + 3, st2);
            fence();
        }
    }
    wait_vm(0);

    // ---- epilogue: acc_y[i][j] element v of lane l: token 32 (rb0 + j) + l%32,
    // output column 32 (cb0 + i) + 8 (v/4) + 4 (l/32) + v%4.  The lane index
    // is read again here (not kept live through the loop, where the widest
    // accumulator leaves no register for it).
    const int el = __lane_id(), ex = el & 31, eh = el >> 5;
    if (ns > 1) {
        const int unit = (mt - plan.whole) * ns + sp;
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
            const int t = 32 * (rb0 + j) + ex;
            if (t >= valid_rows) continue;
            float* out = a.P + ((int64_t)unit * TT + t) * D;
#pragma unroll
            for (int i = 0; i < CBW; ++i)
#pragma unroll
                for (int vg = 0; vg < 4; ++vg) {
                    const int col = 32 * (cb0 + i) + 8 * vg + 4 * eh;
                    const f32x16_t& y = acc_y[i][j];
                    const int v = 4 * vg;
                    *(float4*)(out + col) = make_float4(y[v], y[v + 1], y[v + 2], y[v + 3]);
                }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < RBW; ++j) {
        const int t = 32 * (rb0 + j) + ex;
        if (t >= valid_rows) continue;
        uint16_t* out = a.Y + (tile_r0 + t) * (int64_t)D;
#pragma unroll
        for (int i = 0; i < CBW; ++i)
#pragma unroll
            for (int vg = 0; vg < 4; ++vg) {
                const int col = 32 * (cb0 + i) + 8 * vg + 4 * eh;
                const f32x16_t& y = acc_y[i][j];
                const int v = 4 * vg;
                *(uint2*)(out + col) = make_uint2(pack_bf16(y[v], y[v + 1]),
                                                  pack_bf16(y[v + 2], y[v + 3]));
            }
    }
}

// Split tile whole + j (j < r) of the plan: Y[row] = bf16(sum over sp of
// its partial outputs), fp32 adds in split order (reproducible).  Workgroup
// b takes rows RED_ROWS (b % (TT / RED_ROWS)) .. + RED_ROWS - 1 of split
// tile b / (TT / RED_ROWS); one thread per 8 columns of a row.
constexpr int RED_ROWS = 8;
__global__ __launch_bounds__(256) void fused_reduce_kernel(const GroupArgs g, const float* __restrict__ P,
                                                          uint16_t* __restrict__ Y, int D, int chunks) {
    const FusedPlan plan = fused_plan(g.tile_off[g.G], chunks);
    const int j = blockIdx.x / (TT / RED_ROWS), rb = blockIdx.x % (TT / RED_ROWS);
    if (plan.s == 1 || j >= plan.r) return;
    const TileGroup tg = find_tile_group(g, plan.whole + j, TT, threadIdx.x & 63);
    const int cg = D / 8;
    const int rows = min(RED_ROWS, tg.valid_rows - RED_ROWS * rb);
    for (int it = threadIdx.x; it < rows * cg; it += 256) {
        const int t = RED_ROWS * rb + it / cg, c = (it % cg) * 8;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int sp = 0; sp < plan.s; ++sp) {
            typedef __attribute__((ext_vector_type(4))) float f4;
            const f4* src = (const f4*)(P + ((int64_t)(j * plan.s + sp) * TT + t) * D + c);
            const f4 lo = __builtin_nontemporal_load(src), hi = __builtin_nontemporal_load(src + 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[i] += lo[i];
                acc[4 + i] += hi[i];
            }
        }
        *(uint4*)(Y + (tg.tile_r0 + t) * D + c) =
            make_uint4(pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]),
                       pack_bf16(acc[4], acc[5]), pack_bf16(acc[6], acc[7]));
    }
}

// Upper bound of the tile count of a call with R rows in G groups.
int64_t fused_tiles_upper(int64_t R, int G) { return (R + TT - 1) / TT + G; }

}  // namespace

size_t fused_partial_bytes(int64_t R, int G, int D, int F) {
    const int64_t chunks = (F + CH - 1) / CH;
    const int64_t units = std::min<int64_t>(kFusedUnits, fused_tiles_upper(R, G) * chunks);
    return sizeof(float) * (size_t)units * TT * (size_t)D;
}

hipError_t launch_fused_reduce(const GroupArgs& g, const float* P, void* Y, int D, int F, hipStream_t s) {
    const int64_t rows = g.S + (g.G > g.E ? g.T : 0);
    const int blocks = (int)std::min<int64_t>(kFusedUnits, fused_tiles_upper(rows, g.G)) * (TT / RED_ROWS);
    fused_reduce_kernel<<<blocks, 256, 0, s>>>(g, P, (uint16_t*)Y, D, (F + CH - 1) / CH);
    return hipGetLastError();
}

hipError_t launch_fused_bf16(const GroupArgs& g, const void* x, const void* W1, const void* W3,
                             const void* W2, const void* Ws1, const void* Ws3, const void* Ws2,
                             void* Y, float* P, int D, int F, hipStream_t s) {
    FusedArgs a{g, (const uint16_t*)x, (const uint16_t*)W1, (const uint16_t*)W3,
                (const uint16_t*)W2, (const uint16_t*)Ws1, (const uint16_t*)Ws3,
                (const uint16_t*)Ws2, (uint16_t*)Y, P, D, F};
    const int64_t rows = g.S + (g.G > g.E ? g.T : 0);
    // whole tiles (at most the upper bound, whole / 8 slots per XCD) plus at
    // most kFusedUnits / 8 split units per XCD
    const unsigned blocks = grid_for_work(fused_tiles_upper(rows, g.G)) + kFusedUnits + 8;
    switch (D / 128) {
        case 1: fused_up_act_down_kernel<1><<<grid_for_work(blocks), NT, 0, s>>>(a); break;
        case 2: fused_up_act_down_kernel<2><<<grid_for_work(blocks), NT, 0, s>>>(a); break;
        case 3: fused_up_act_down_kernel<3><<<grid_for_work(blocks), NT, 0, s>>>(a); break;
        case 4: fused_up_act_down_kernel<4><<<grid_for_work(blocks), NT, 0, s>>>(a); break;
        case 5: fused_up_act_down_kernel<5><<<grid_for_work(blocks), NT, 0, s>>>(a); break;
        case 6: fused_up_act_down_kernel<6><<<grid_for_work(blocks), NT, 0, s>>>(a); break;
        case 7: fused_up_act_down_kernel<7><<<grid_for_work(blocks), NT, 0, s>>>(a); break;
        case 8: fused_up_act_down_kernel<8><<<grid_for_work(blocks), NT, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace moe
