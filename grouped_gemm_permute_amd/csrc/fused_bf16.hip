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
//   for each chunk of CH = 128 h columns f:
//     g, u = x_tile . W1[:, f], x_tile . W3[:, f]        (fp32 accumulate, K = D)
//     h    = bf16(silu(g) * u)                           (into LDS)
//     acc += h . W2[f, :]                                (fp32 accumulate, K = CH)
//   Y[row] = bf16(acc[row])                              (the combine applies the routing weight)
//
// Shapes and placement on gfx950 (256 threads = 4 wavefronts, one per SIMD):
//  * token tile TT = 64 rows of one group; the fp32 accumulator acc is
//    64 x D, each wavefront owning D/4 output columns (D <= 1024 -> at most
//    256 accumulator registers per lane);
//  * up phase per chunk: MFMA tile 256 features (128 g + 128 u) x 64 tokens,
//    K step 64; wavefront w holds g and u of h columns 32 w .. 32 w + 31;
//  * down phase per chunk: 8 K steps of 16 rows of W2 [16, D];
//  * all operand tiles stream global -> LDS with global_load_lds (double
//    buffered, 40 KiB per stage); weights stay [K][N] and reach the MFMA
//    through ds_read_b64_tr_b16; token rows and h are K-contiguous;
//  * tiles are numbered group-major and each XCD takes a contiguous range,
//    so the workgroups of one XCD work on the same expert at the same time
//    and share each weight chunk through that XCD's L2 instead of streaming
//    it from HBM once per token tile.
#include "mfma_common.h"

namespace moe {
namespace {

using namespace mfma;

constexpr int TT = kFusedTileRows;   // 64 tokens per tile
constexpr int CH = 128;              // h columns per F chunk
constexpr int NT = 256;
constexpr int UP_BK = 64;
constexpr int X_ROW = UP_BK * 2;                 // 128 B token row (K-contiguous)
constexpr int X_BYTES = TT * X_ROW;              // 8 KiB
constexpr int WGU_ROW = 2 * CH * 2;              // 512 B: 256 features of one k row
constexpr int WGU_BYTES = UP_BK * WGU_ROW;       // 32 KiB
constexpr int STAGE_BYTES = X_BYTES + WGU_BYTES; // 40 KiB (a down stage [16][D] needs <= 32 KiB)
constexpr int H_ROW = CH * 2;                    // 256 B
constexpr int H_BYTES = TT * H_ROW;              // 16 KiB
constexpr int DN_STEPS = CH / 16;                // 8 down steps per chunk

static_assert(TT == 64 && CH == 128 && NT == 256, "index math below assumes these");

struct FusedArgs {
    GroupArgs g;
    const uint16_t* x;                     // [T, D]
    const uint16_t *W1, *W3, *W2;          // [E, D, F], [E, D, F], [E, F, D]
    const uint16_t *Ws1, *Ws3, *Ws2;       // shared expert or null
    uint16_t* Y;                           // [R, D] bf16 expert outputs
    int D, F;
};

// D = 128 * NFB.
template <int NFB>
__global__ __launch_bounds__(NT, 1) void fused_up_act_down_kernel(const FusedArgs a) {
    // Separate LDS objects per stage buffer: the compiler then knows reads of
    // one never alias the asynchronous global_load_lds writes into the other.
    __shared__ __attribute__((aligned(1024))) char lds0[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds1[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char hbuf[H_BYTES];

    constexpr int D = 128 * NFB;
    constexpr int DN_ROW = 2 * D;          // bytes of one W2 row in LDS
    constexpr int WCOLS = 32 * NFB;        // output columns per wavefront
    constexpr int KU = D / UP_BK;          // up K steps per chunk (even)
    const int F = a.F;
    const int NC = F / CH;

    const int mt = xcd_remap_work(blockIdx.x, a.g.tile_off[a.g.G]);
    if (mt < 0) return;
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

    // ---- token rows: DMA instruction j (0, 1) of wavefront w fills rows
    // 16 w + 8 j .. +7; lane -> row 16 w + 8 j + lane/8, physical chunk lane%8.
    const char* x_src[2];
    {
        int64_t src_row[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t p = tile_r0 + min(16 * wave + 8 * j + (lane >> 3), valid_rows - 1);
            src_row[j] = p;
        }
        if (!shared) {
            const int32_t s0 = a.g.perm[src_row[0]], s1 = a.g.perm[src_row[1]];
            src_row[0] = s0 / a.g.k;
            src_row[1] = s1 / a.g.k;
        } else {
            src_row[0] -= a.g.S;
            src_row[1] -= a.g.S;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = 16 * wave + 8 * j + (lane >> 3);
            const int c = (lane & 7) ^ swz8(row);
            x_src[j] = (const char*)(a.x + src_row[j] * (int64_t)D + 8 * c);
        }
    }

    // ---- up weights: DMA instruction j (0..7) of wavefront w fills k rows
    // 16 w + 2 j, +1; lane -> k row 16 w + 2 j + lane/32, physical chunk
    // lane%32 holding logical chunk cl = phys ^ swz_tr(k).  Logical chunk cl
    // (8 features): wavefront block wb = cl / 8, g when (cl / 4) is even, u
    // when odd, h column 32 wb + 8 (cl % 4) within the chunk.
    // (The per-lane source is rebuilt at every issue: a few integer ops are
    // cheaper than keeping eight 64-bit pointers live next to the accumulators.)
    auto wgu_src = [&](int j) {
        const int kr = 16 * wave + 2 * j + (lane >> 5);
        const int cl = (lane & 31) ^ swz_tr(kr);
        const int col = 32 * (cl >> 3) + 8 * (cl & 3);
        return (((cl >> 2) & 1) ? W3g : W1g) + (int64_t)kr * F + col;
    };
    // ---- down weights: a stage is W2 rows [16][D] = 256 NFB chunks; DMA
    // instruction j (0..NFB-1) of wavefront w covers linear chunks
    // 64 (w NFB + j) + lane: row L / (16 NFB), physical chunk L % (16 NFB).

    auto issue_up = [&](int c, int s, char* st) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            load_lds16(x_src[j] + (int64_t)s * X_ROW, st + (16 * wave + 8 * j) * X_ROW);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            load_lds16(wgu_src(j) + (int64_t)s * UP_BK * F + c * CH,
                       st + X_BYTES + (16 * wave + 2 * j) * WGU_ROW);
    };
    auto issue_down = [&](int c, int q, char* st) {
        const uint16_t* base = W2g + (int64_t)(c * CH + 16 * q) * D;
#pragma unroll
        for (int j = 0; j < NFB; ++j) {
            const int L = 64 * (wave * NFB + j) + lane;
            const int row = L / (16 * NFB), pc = L - row * (16 * NFB);
            load_lds16(base + row * D + 8 * (pc ^ swz_tr(row)), st + 1024 * (wave * NFB + j));
        }
    };

    // ---- operand read offsets.  Transposed reads: lane = 16 G + s reads
    // k = 8 (G>>1) + 4 r + s/4 (+16 ks), feature R = ... + 16 (G&1) + 4 (s&3).
    const int G = lane >> 4, sl = lane & 15;
    int gu_off[2][2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int k = 8 * (G >> 1) + 4 * r + (sl >> 2);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
            const int R = 64 * wave + 32 * mi + 16 * (G & 1) + 4 * (sl & 3);
            gu_off[mi][r] = X_BYTES + k * WGU_ROW + (((R >> 3) ^ swz_tr(k)) << 4) + 8 * (sl & 1);
        }
    }
    // Down weight operand: k = 8 (G>>1) + 4 r + s/4 within the 16-row stage,
    // column R = WCOLS w + 32 fb + 16 (G&1) + 4 (s&3); the chunk index is
    // recomputed per block (cheaper than keeping 2 NFB offsets live).
    const int dn_k0 = 8 * (G >> 1) + (sl >> 2);
    const int dn_c0 = (WCOLS * wave + 16 * (G & 1) + 4 * (sl & 3)) >> 3;
    const int dn_b = 8 * (sl & 1);
    auto dn_off = [&](int fb, int r) {
        const int k = dn_k0 + 4 * r;
        return k * DN_ROW + (((dn_c0 + 4 * fb) ^ swz_tr(k)) << 4) + dn_b;
    };
    int tok_off[2], tok_swz8[2], tok_swz16[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int t = 32 * tb + (lane & 31);
        tok_off[tb] = t;
        tok_swz8[tb] = swz8(t);
        tok_swz16[tb] = swz16(t);
    }

    f32x16_t acc_y[NFB][2];
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) acc_y[fb][0] = acc_y[fb][1] = f32x16_t{};
    f32x16_t acc_up[2][2];

    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    // One up K step (64) on stage st: 4 slices x (2 weight frags, 2 token frags, 4 MFMAs).
    auto compute_up = [&](const char* st) {
#pragma unroll
        for (int ks = 0; ks < UP_BK / 16; ++ks) {
            bf16x8_t wf[2], xf[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                wf[mi] = cat_bf16(read_tr(st + gu_off[mi][0] + ks * 16 * WGU_ROW),
                                  read_tr(st + gu_off[mi][1] + ks * 16 * WGU_ROW));
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const int c = (2 * ks + (lane >> 5)) ^ tok_swz8[tb];
                xf[tb] = __builtin_bit_cast(bf16x8_t,
                                            *(const u32x4_t*)(st + tok_off[tb] * X_ROW + (c << 4)));
            }
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
                    acc_up[mi][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[mi], xf[tb],
                                                                             acc_up[mi][tb], 0, 0, 0);
        }
    };
    // One down K step (16 rows of W2) on stage st, h slice q of the chunk.
    // Weight fragments are read in groups of up to 4 column blocks to bound
    // the live registers next to the 32 NFB accumulator registers.
    auto compute_down = [&](const char* st, int q) {
        bf16x8_t hf[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int c = (2 * q + (lane >> 5)) ^ tok_swz16[tb];
            hf[tb] = __builtin_bit_cast(bf16x8_t,
                                        *(const u32x4_t*)(hbuf + tok_off[tb] * H_ROW + (c << 4)));
        }
        constexpr int GRP = NFB < 4 ? NFB : 4;
#pragma unroll
        for (int f0 = 0; f0 < NFB; f0 += GRP) {
            bf16x8_t wf[GRP];
#pragma unroll
            for (int i = 0; i < GRP && f0 + i < NFB; ++i)
                wf[i] = cat_bf16(read_tr(st + dn_off(f0 + i, 0)), read_tr(st + dn_off(f0 + i, 1)));
#pragma unroll
            for (int i = 0; i < GRP && f0 + i < NFB; ++i)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
                    acc_y[f0 + i][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        wf[i], hf[tb], acc_y[f0 + i][tb], 0, 0, 0);
        }
    };
    // h = silu(g) * u for the chunk, bf16, into hbuf (token rows, K-contiguous).
    // acc_up[mi][tb] element v of lane l: token 32 tb + l%32, h column
    // 32 w + 8 (v/4) + 4 (l/32) + v%4 (g for mi = 0, u for mi = 1).
    auto write_h = [&]() {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int vg = 0; vg < 4; ++vg) {
                const f32x16_t& g = acc_up[0][tb];
                const f32x16_t& u = acc_up[1][tb];
                const int v = 4 * vg;
                const int c = (4 * wave + vg) ^ tok_swz16[tb];
                *(uint2*)(hbuf + tok_off[tb] * H_ROW + (c << 4) + 8 * (lane >> 5)) =
                    make_uint2(pack_bf16(silu_mul(g[v], u[v]), silu_mul(g[v + 1], u[v + 1])),
                               pack_bf16(silu_mul(g[v + 2], u[v + 2]), silu_mul(g[v + 3], u[v + 3])));
            }
    };

    // ---- stage stream: per chunk KU up steps then DN_STEPS down steps (an
    // even count, so chunk step i always uses buffer i % 2); the loads of
    // step i+1 are in flight while step i computes.  After the very last step
    // the last down stage is reloaded into the idle buffer instead of
    // branching around the loads.
    issue_up(0, 0, lds0);
    wait_vmem();
    __syncthreads();
    for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) acc_up[mi][0] = acc_up[mi][1] = f32x16_t{};
        for (int s = 0; s < KU; s += 2) {
            issue_up(c, s + 1, lds1);
            fence();
            compute_up(lds0);
            fence();
            wait_vmem();
            __syncthreads();
            if (s + 2 < KU) issue_up(c, s + 2, lds0);
            else issue_down(c, 0, lds0);
            fence();
            compute_up(lds1);
            fence();
            wait_vmem();
            __syncthreads();
        }
        write_h();
        __syncthreads();
        for (int q = 0; q < DN_STEPS; q += 2) {
            issue_down(c, q + 1, lds1);
            fence();
            compute_down(lds0, q);
            fence();
            wait_vmem();
            __syncthreads();
            if (q + 2 < DN_STEPS) issue_down(c, q + 2, lds0);
            else if (c + 1 < NC) issue_up(c + 1, 0, lds0);
            else issue_down(c, DN_STEPS - 1, lds0);
            fence();
            compute_down(lds1, q + 1);
            fence();
            wait_vmem();
            __syncthreads();
        }
    }

    // ---- epilogue: acc_y[fb][tb] element v of lane l: token 32 tb + l%32,
    // output column WCOLS w + 32 fb + 8 (v/4) + 4 (l/32) + v%4.
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int t = 32 * tb + (lane & 31);
        if (t >= valid_rows) continue;
        uint16_t* out = a.Y + (tile_r0 + t) * (int64_t)D;
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
            for (int vg = 0; vg < 4; ++vg) {
                const int col = WCOLS * wave + 32 * fb + 8 * vg + 4 * (lane >> 5);
                const f32x16_t& y = acc_y[fb][tb];
                const int v = 4 * vg;
                *(uint2*)(out + col) = make_uint2(pack_bf16(y[v], y[v + 1]),
                                                  pack_bf16(y[v + 2], y[v + 3]));
            }
    }
}

}  // namespace

hipError_t launch_fused_bf16(const GroupArgs& g, const void* x, const void* W1, const void* W3,
                             const void* W2, const void* Ws1, const void* Ws3, const void* Ws2,
                             void* Y, int D, int F, hipStream_t s) {
    FusedArgs a{g, (const uint16_t*)x, (const uint16_t*)W1, (const uint16_t*)W3,
                (const uint16_t*)W2, (const uint16_t*)Ws1, (const uint16_t*)Ws3,
                (const uint16_t*)Ws2, (uint16_t*)Y, D, F};
    const int64_t rows = g.S + (g.G > g.E ? g.T : 0);
    const unsigned blocks = (unsigned)((rows + TT - 1) / TT + g.G);
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
