// gemm_bf16_slab.hip -- up+SwiGLU grouped GEMM for small per-expert chunks.
//
// Same product as the up GEMM of gemm_bf16.hip (h = bf16(silu(x . W1) *
// (x . W3)) on the rows of each group), shaped for the regime where every
// expert sees at most a few hundred rows and streaming the weights is the
// cost (the "small chunks" that "Triton MoE Kernels & Memory Checkpointing",
// Part A sections 2 and 6.1, calls the pathological regime).  Given a gu
// array it also stores each row's [g | u] rounded to bf16 beside h, for the
// forward that keeps the gate and up products for the backward.
//
// Every byte a workgroup stages passes through its CU's memory pipe, which
// moves a few tens of bytes per clock; the kernel is bound by the total
// bytes staged, i.e. by how often each operand is re-read.  A row tile of
// 32 RB rows is chosen by the host to hold a whole typical group, so each
// group's weight slab is streamed exactly once, and the token rows (which
// are small) are the operand re-read once per column slab:
//
//  * tile = 32 RB rows x 128 MFMA features = 64 output columns (four MFMA
//    blocks, each 16 W1 columns followed by the same 16 W3 columns, so
//    accumulator elements v (g) and v + 8 (u) of a lane pair up);
//  * 256 threads = 4 wavefronts; wavefront w owns feature block w for all RB
//    row blocks (RB v_mfma_f32_32x32x16_bf16 accumulators), so the slow
//    transposed weight reads are not replicated across wavefronts;
//  * K step 64; a ring of 4 LDS stages (3 for the tallest tiles) filled with
//    global_load_lds, and the operands of the next stage are read from LDS
//    while the MFMAs of the current one run; rows past the group's end are clamped to
//    its last row, which costs the memory pipe next to nothing (all lanes of
//    an instruction then hit one line) and keeps every wavefront's load count
//    per stage fixed, so the waits are compile-time counts;
//  * tiles run m-major (all column slabs of one row tile back to back), so
//    the workgroups of one XCD stream whole weight rows of one group in step
//    and share that group's token rows through the XCD's L2.
//
// Routed form (ROUTE, up to kPermuteSingleMax slots): the counting sort of
// the permute runs inside this kernel, so the forward needs no permute
// launch.  Workgroup (g, nt) is fixed by its block index alone: it issues
// its weight slab's first stages at entry, before it knows anything about
// the routing, then reads the slots' expert ids, counts the slots of lower
// experts (its group's first sorted row) and ranks its own group's slots in
// slot order -- the same stable order as the permute -- into an LDS row
// table, from which the token rows are gathered.  A group with more rows
// than a tile walks its row tiles in turn.  One more workgroup, beside the
// GEMM workgroups, runs the permute's one-workgroup counting sort and writes
// counts, offsets, both row-tile prefixes, perm, inv and the invalid-slot
// count, which only the later launches read.  Up to 64 more workgroups, on
// the CUs the GEMM leaves idle (the grid stays within one workgroup per CU),
// read the down GEMM's weights W2 (and the shared expert's) once, so that
// the down launch finds them in the 256 MB last-level cache instead of HBM:
// 6% off the small-chunk forward (its down GEMM 15.0 -> 11.9 us), measured;
// loaded with the non-temporal policy they are not kept there and nothing
// is gained.
#include <algorithm>

#include "mfma_common.h"
#include "permute_device.h"

namespace moe {
namespace {

using namespace mfma;

constexpr int FB = 4;                  // MFMA feature blocks per tile (one per wavefront)
constexpr int TFM = 32 * FB;           // 128 MFMA features
constexpr int TCOL = TFM / 2;          // 64 output columns
constexpr int BK = 64;
constexpr int NT = 256;
constexpr int X_ROW = BK * 2;          // 128 B per token row
constexpr int W_ROW = TFM * 2;         // 256 B per k row
constexpr int W_BYTES = BK * W_ROW;    // 16 KiB

static_assert(NT == 256 && FB == 4 && BK == 64 && W_BYTES == 16384, "index math below assumes these");

struct SlabArgs {
    GroupArgs g;              // ROUTE: only S, T, E, k, G are read
    const uint16_t* x;        // [T, D]
    const uint16_t* w1;       // [E, D, F]
    const uint16_t* w3;
    const uint16_t* ws1;      // shared expert [D, F]
    const uint16_t* ws3;
    uint16_t* h;              // [R, F]
    int D, F;
    int n_tiles;
    // ROUTE only: the routing in, the permute's outputs out
    const int32_t* idx;       // [S] expert id of each slot
    int32_t *counts, *offsets, *tile_off, *tile_off64, *perm, *inv, *err;
    int tile_rows;            // row-tile height of tile_off (32 RB)
    int sh_tiles;             // row tiles of the shared group (one workgroup per column slab each)
    // ROUTE: workgroups past the sort's read the down GEMM's weights once
    // (into a scratch LDS area), leaving them in the last-level cache
    const uint16_t* w2;       // [E, F, D]
    const uint16_t* ws2;      // [F, D] or null
    int64_t w2_bytes, ws2_bytes;
    int pf_blocks;
    // optional: each row's gate and up products [R, 2F] (g in columns
    // 0..F-1, u in F..2F-1), rounded to bf16, for a backward that keeps them
    uint16_t* gu;
};

constexpr int kRouteSlotsPerThread = kPermuteSingleMax / 256;

template <int RB, bool ROUTE>
__global__ __launch_bounds__(NT, 1) void up_swiglu_slab_kernel(const SlabArgs a) {
    constexpr int TT = 32 * RB;
    constexpr int X_BYTES = TT * X_ROW;
    constexpr int STAGE_BYTES = X_BYTES + W_BYTES;
    constexpr int PER_STAGE = RB + W_BYTES / 1024 / 4;     // global_load_lds per wavefront per stage
    // LDS of the in-kernel routing: the row table and reduction slots
    constexpr int ROUTE_LDS = ROUTE ? 4 * (TT + 16) : 0;
    // Four stage buffers when they fit in LDS, else three; separate LDS
    // objects so the compiler sees that reads of one do not alias the
    // asynchronous loads into another.
    constexpr int NS = 4 * STAGE_BYTES + ROUTE_LDS <= 160 * 1024 ? 4 : 3;
    // operands read half a stage at a time: tall tiles, and three-stage rings
    // (the routed form at RB 6, whose LDS holds only three)
    constexpr bool HALF = RB >= 7 || NS == 3;
    __shared__ __attribute__((aligned(1024))) char st0[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char st1[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char st2[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char st3[NS == 4 ? STAGE_BYTES : 16];
    __shared__ int32_t rtab[ROUTE ? TT : 1];                 // slot of each row of the tile
    __shared__ int32_t rred[ROUTE ? 16 : 1];

    // ROUTE: the last workgroup of the grid does the counting sort's
    // bookkeeping for the later launches (counts, offsets, both row-tile
    // prefixes, perm, inv, the invalid-slot count), in parallel with the
    // GEMM workgroups, with the stage buffers as its scratch.
    const int gemm_blocks = (a.g.E + a.sh_tiles) * a.n_tiles;
    if (ROUTE && (int)blockIdx.x > gemm_blocks) {
        // prefetch workgroup p: bytes [p chunk, (p + 1) chunk) of W2 then Ws2,
        // 4 KiB per round (1 KiB per wavefront), into a scratch LDS area
        const int p = blockIdx.x - gemm_blocks - 1;
        const int64_t total = a.w2_bytes + a.ws2_bytes;
        const int64_t chunk = (total + a.pf_blocks * 4096 - 1) / (a.pf_blocks * 4096) * 4096;
        const int64_t lo = p * chunk, hi = min(total, lo + chunk);
        const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
        for (int64_t o = lo + 1024 * w + 16 * l; o + 16 <= hi; o += 4096) {
            const char* src = o < a.w2_bytes ? (const char*)a.w2 + o : (const char*)a.ws2 + (o - a.w2_bytes);
            load_lds16(src, st0 + 1024 * w);
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
        return;
    }
    if (ROUTE && (int)blockIdx.x == gemm_blocks) {
        static_assert(4 * (6 * kRouteMaxExperts + 1) <= STAGE_BYTES, "the sort's scratch fits a stage");
        int32_t* scratch = (int32_t*)st0;
        permute_dev::permute_one_workgroup<NT>(
            a.idx, a.g.S, a.g.E, permute_dev::TileSpec{a.tile_rows, a.tile_off},
            permute_dev::TileSpec{64, a.tile_off64}, a.g.G > a.g.E ? a.g.T : 0, a.counts, a.offsets,
            a.perm, a.inv, a.err, scratch, scratch + kMaxExperts + 1, scratch + 2 * kMaxExperts + 1);
        return;
    }
    const int K = a.D, N = a.F;
    const int KT = K / BK;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int grp, nt;
    bool shared;
    int64_t tile_r0 = 0;
    int valid_rows = 0;
    int sh_rt = 0;                    // ROUTE: row tile of a shared-group workgroup
    if constexpr (ROUTE) {
        // (group, column slab) from the block index alone, m-major
        const int id = xcd_remap(blockIdx.x, (a.g.E + a.sh_tiles) * a.n_tiles);
        const int m = id / a.n_tiles;
        nt = id - m * a.n_tiles;
        shared = m >= a.g.E;
        grp = shared ? a.g.E : m;
        sh_rt = m - a.g.E;
    } else {
        // the group lookup's loads go out with the tile count's (one round trip)
        const GroupBlock gblock = load_group_block(a.g, 0, lane);
        const int total = a.g.tile_off[a.g.G];
        const int id = xcd_remap_work(blockIdx.x, total * a.n_tiles);
        if (id < 0) return;
        const int mt = id / a.n_tiles;
        nt = id - mt * a.n_tiles;     // m-major
        const TileGroup tg = find_tile_group(a.g, mt, TT, lane, gblock);
        grp = tg.grp;
        shared = grp >= a.g.E;
        tile_r0 = tg.tile_r0;
        valid_rows = tg.valid_rows;
        if (valid_rows <= 0) return;
    }

    // ---- weight slab [64 k][128 features]: DMA instruction j (0..3) of
    // wavefront w fills k rows 4 q .. 4 q + 3 with q = w + 4 j; lane -> k row
    // 4 q + lane/16, physical chunk lane%16 holding logical chunk
    // cl = phys ^ swz_tr(k) = MFMA features 8 cl .. 8 cl + 7: block cl / 4,
    // W3 when (cl / 2) is odd, output column 16 (cl / 4) + 8 (cl % 2).
    const int64_t gstride = (int64_t)a.D * a.F;
    const char* w_src[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int kr = 4 * (wave + 4 * j) + (lane >> 4);
        const int cl = (lane & 15) ^ swz_tr(kr);
        const int kind = (cl >> 1) & 1;
        int col = nt * TCOL + 16 * (cl >> 2) + 8 * (cl & 1);
        if (col >= N) col = 0;                 // past the last column: a valid chunk, never stored
        const uint16_t* base = shared ? (kind ? a.ws3 : a.ws1) : (kind ? a.w3 : a.w1) + grp * gstride;
        w_src[j] = (const char*)(base + (int64_t)kr * N + col);
    }
    const int64_t w_step = (int64_t)BK * N * 2;
    auto issue_w = [&](int kt, char* st) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            load_lds16(w_src[j] + kt * w_step, st + X_BYTES + 4 * (wave + 4 * j) * W_ROW);
    };

    // ---- ROUTE: the weight slab's first stages go out now, before the routing.
    int n_rows = 0, row0 = 0, eq_base = 0, s0 = 0;
    uint32_t eq_mask = 0;
    // A barrier that waits for this wavefront's LDS accesses only (a plain
    // __syncthreads would also drain the weight stages in flight).
    auto lds_barrier = [] {
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
        __builtin_amdgcn_s_barrier();
    };
    if constexpr (ROUTE) {
        auto issue_w_first = [&] {
#pragma unroll
            for (int i = 0; i < NS - 1; ++i) issue_w(min(i, KT - 1), i == 0 ? st0 : i == 1 ? st1 : st2);
        };
        if (shared) issue_w_first();
        if (!shared) {
            // The slots' expert ids come into the last stage buffer (not used
            // before the first K step) by LDS DMA ahead of the weight stages:
            // DMA loads retire in order, so once at most the weight stages'
            // loads are outstanding the ids are in, and the routing below
            // runs while the weights are still in flight.  Instruction i
            // (i = w, w + 4, ...) covers slots 64 i .. 64 i + 63, 4 bytes a lane
            // (addresses clamped to the last slot).
            const int S = (int)a.g.S, E = a.g.E;
            char* ids_lds = NS == 4 ? st3 : st2;
            for (int i = wave; i < (S + 63) / 64; i += 4)
                __builtin_amdgcn_global_load_lds(a.idx + min(64 * i + lane, S - 1),
                                                 (lds_void_t*)(ids_lds + 256 * i), 4, 0, 0);
            issue_w_first();
            // (Pulling further weight stages into L2 here, while the routing
            // waits on memory, measured slower: every DMA instruction must be
            // issued into the busy memory pipe before the ids can be used.)
            __builtin_amdgcn_s_waitcnt(waitcnt_imm((NS - 1) * 4, 15));   // the ids are in
            __builtin_amdgcn_s_barrier();
            // Slots 16 tid .. 16 tid + 15 of this thread, in slot order across
            // the workgroup.  Keys: the expert id when valid, E when out of
            // range, E + 1 past the last slot.
            s0 = kRouteSlotsPerThread * tid;
            int key[kRouteSlotsPerThread];
#pragma unroll
            for (int q = 0; q < kRouteSlotsPerThread / 4; ++q) {
                const u32x4_t v = *(const u32x4_t*)(ids_lds + 4 * (s0 + 4 * q));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int e = (int)v[i];
                    key[4 * q + i] = s0 + 4 * q + i >= S ? E + 1 : (e >= 0 && e < E ? e : E);
                }
            }
            int lt = 0;
#pragma unroll
            for (int j = 0; j < kRouteSlotsPerThread; ++j) {
                lt += key[j] < grp ? 1 : 0;
                eq_mask |= (key[j] == grp ? 1u : 0u) << j;
            }
            // the group's first sorted row (slots of lower experts), its row
            // count (slots of this expert) and this thread's first rank
            const int eqc = __popc(eq_mask);
            int inc = eqc;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int t = __shfl_up(inc, d);
                if (lane >= d) inc += t;
            }
            int ltw = lt;
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) ltw += __shfl_xor(ltw, d);
            if (lane == 63) rred[wave] = inc;
            if (lane == 0) rred[4 + wave] = ltw;
            lds_barrier();
            int before = 0;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                before += w < wave ? rred[w] : 0;
                n_rows += rred[w];
                row0 += rred[4 + w];
            }
            eq_base = before + inc - eqc;
        }
    }
    const int ntile = !ROUTE ? 1 : shared ? 1 : (n_rows + TT - 1) / TT;
    if (ntile == 0) {
        wait_vmem();                  // no rows: drain the weight stages before leaving
        return;
    }
    for (int rt = 0; rt < ntile; ++rt) {
    if constexpr (ROUTE) {
        if (rt > 0) __syncthreads();  // every wavefront is done with the previous tile's LDS
        if (shared) {
            tile_r0 = a.g.S + (int64_t)sh_rt * TT;
            valid_rows = min(TT, (int)(a.g.T - (int64_t)sh_rt * TT));
        } else {
            tile_r0 = row0 + rt * TT;
            valid_rows = min(TT, n_rows - rt * TT);
            int r = eq_base;
#pragma unroll
            for (int j = 0; j < kRouteSlotsPerThread; ++j)
                if ((eq_mask >> j) & 1u) {
                    if (r >= rt * TT && r < rt * TT + TT) rtab[r - rt * TT] = s0 + j;
                    ++r;
                }
            lds_barrier();
        }
    }

    // ---- token rows: DMA instruction j (0 .. RB-1) of wavefront w fills rows
    // 8 q .. 8 q + 7 with q = w + 4 j; lane -> row 8 q + lane/8, physical
    // chunk lane%8 holding logical chunk (lane%8) ^ swz8(row).  Routed rows
    // gather token slot / k, the slot from perm (or, routed in this kernel,
    // from the row table); shared rows read token row - S.
    const char* x_src[RB];
    {
        int64_t src_row[RB];
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            const int row = min(8 * (wave + 4 * j) + (lane >> 3), valid_rows - 1);
            src_row[j] = ROUTE && !shared ? row : tile_r0 + row;
        }
        if (!shared) {
            int32_t slot[RB];
#pragma unroll
            for (int j = 0; j < RB; ++j) slot[j] = ROUTE ? rtab[src_row[j]] : a.g.perm[src_row[j]];
#pragma unroll
            for (int j = 0; j < RB; ++j) src_row[j] = slot[j] / a.g.k;
        } else {
#pragma unroll
            for (int j = 0; j < RB; ++j) src_row[j] -= a.g.S;
        }
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            const int row = 8 * (wave + 4 * j) + (lane >> 3);
            x_src[j] = (const char*)(a.x + src_row[j] * (int64_t)K + 8 * ((lane & 7) ^ swz8(row)));
        }
    }
    auto issue_x = [&](int kt, char* st) {
#pragma unroll
        for (int j = 0; j < RB; ++j)
            load_lds16(x_src[j] + (int64_t)kt * X_ROW, st + 8 * (wave + 4 * j) * X_ROW);
    };
    auto issue = [&](int kt, char* st) {
        issue_x(kt, st);
        issue_w(kt, st);
    };
    // The prologue's stages: only the token rows when the weights went out at
    // entry.  Then stage 0 has landed once at most the later stages' token
    // loads are outstanding (loads complete in order); that stricter count
    // is also right for the usual order.
    const bool w_early = ROUTE && rt == 0;
    auto issue_first = [&](int kt, char* st) {
        if (w_early) issue_x(kt, st);
        else issue(kt, st);
    };
    constexpr int FIRST_WAIT = ROUTE ? (NS - 2) * RB : (NS - 2) * PER_STAGE;

    // ---- operand reads.  Weights (A), transposed: lane = 16 G + s reads
    // k = 16 ks + 8 (G>>1) + 4 r + s/4, feature 32 w + 16 (G&1) + 4 (s&3).
    // Rows (B): row 32 j + lane%32, logical chunk 2 ks + lane/32.
    const int G = lane >> 4, sl = lane & 15;
    int w_off[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int k = 8 * (G >> 1) + 4 * r + (sl >> 2);
        const int R = 32 * wave + 16 * (G & 1) + 4 * (sl & 3);
        w_off[r] = X_BYTES + k * W_ROW + (((R >> 3) ^ swz_tr(k)) << 4) + 8 * ((R >> 2) & 1);
    }
    const int xl = lane & 31;

    f32x16_t acc[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) acc[j] = f32x16_t{};

    struct Frags {
        bf16x8_t w[BK / 16], x[BK / 16][RB];
    };
    auto read_frags = [&](const char* st, Frags& f) {
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            f.w[ks] = cat_bf16(read_tr(st + w_off[0] + ks * 16 * W_ROW),
                               read_tr(st + w_off[1] + ks * 16 * W_ROW));
#pragma unroll
            for (int j = 0; j < RB; ++j) {
                const int row = 32 * j + xl;
                const int c = (2 * ks + (lane >> 5)) ^ swz8(row);
                f.x[ks][j] =
                    __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(st + row * X_ROW + (c << 4)));
            }
        }
    };
    auto mfmas = [&](const Frags& f) {
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
            for (int j = 0; j < RB; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.w[ks], f.x[ks][j], acc[j], 0, 0, 0);
    };
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

    // ---- ring of NS stages, software-pipelined one stage deep in registers.
    // Step s (its operands fc already in registers):
    //   wait until stage s+1 has landed (at most NS-3 later stages of this
    //   wavefront's loads outstanding) and fc's reads have returned, barrier;
    //   issue the loads of stage s+NS-1 into the buffer of stage s-1;
    //   read stage s+1's operands into fn;
    //   MFMAs on fc -- the reads of fn land under them.
    // The buffer of stage s-1 is free at step s: its operands were read in
    // step s-2 and consumed by the MFMAs of step s-1, which every wavefront
    // finished before arriving at this barrier.  Loads past the last stage
    // re-read the last stage (into buffers never computed on), so the number
    // of loads per stage stays fixed; operands read past the last stage are
    // never used.
    constexpr int WAIT_N = (NS - 3) * PER_STAGE;
    auto wait_stage = [] {
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(WAIT_N, 0));
        __builtin_amdgcn_s_barrier();
    };
    if constexpr (!HALF) {
        auto step = [&](Frags& fc, Frags& fn, const char* nxt, char* dma, int kl) {
            wait_stage();
            fence();
            issue(kl, dma);
            read_frags(nxt, fn);
            mfmas(fc);
            // The in-order wavefront stalls on a load or LDS read while that pipe
            // is backed up; spread them between the MFMAs (4 RB MFMAs, RB + 4
            // loads, 4 RB + 8 reads per step): each MFMA is followed by one load
            // and two reads until those run out.
#pragma unroll
            for (int i = 0; i < 4 * RB; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // vector memory
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS read
            }
            fence();
        };
        Frags fa, fb;
#pragma unroll
        for (int i = 0; i < NS - 1; ++i)
            issue_first(min(i, KT - 1), i == 0 ? st0 : i == 1 ? st1 : st2);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(FIRST_WAIT, 15));   // stage 0 landed
        __builtin_amdgcn_s_barrier();
        fence();
        read_frags(st0, fa);
        fence();
        // weights issued first: stage 1 has landed once at most stage 2's
        // token loads are outstanding (the steps' own waits allow a whole stage)
        if (ROUTE && NS == 4) __builtin_amdgcn_s_waitcnt(waitcnt_imm(RB, 15));
        int kt = 0;
        if constexpr (NS == 4) {
            // buffers rotate with period 4, operand sets with period 2
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
            // buffers rotate with period 3, operand sets with period 2
            for (; kt + 6 <= KT; kt += 6) {
                step(fa, fb, st1, st2, min(kt + 2, KT - 1));
                step(fb, fa, st2, st0, min(kt + 3, KT - 1));
                step(fa, fb, st0, st1, min(kt + 4, KT - 1));
                step(fb, fa, st1, st2, min(kt + 5, KT - 1));
                step(fa, fb, st2, st0, min(kt + 6, KT - 1));
                step(fb, fa, st0, st1, min(kt + 7, KT - 1));
            }
            if (kt < KT) {
                step(fa, fb, st1, st2, KT - 1);
                if (kt + 1 < KT) {
                    step(fb, fa, st2, st0, KT - 1);
                    if (kt + 2 < KT) {
                        step(fa, fb, st0, st1, KT - 1);
                        if (kt + 3 < KT) {
                            step(fb, fa, st1, st2, KT - 1);
                            if (kt + 4 < KT) step(fa, fb, st2, st0, KT - 1);
                        }
                    }
                }
            }
        }
    } else {
        // Tall tiles (RB >= 7): the operands of a whole stage do not fit twice in
        // registers, so a stage is consumed in two halves of 32 k: the second
        // half of the current stage is read while the MFMAs of its first half
        // run, and the first half of the next stage while those of its second
        // half run.  Same stage ring, waits and barrier as above.
        struct Half {
            bf16x8_t w[2], x[2][RB];
        };
        auto read_half = [&](const char* st, int h, Half& f) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int ks = 2 * h + q;
                f.w[q] = cat_bf16(read_tr(st + w_off[0] + ks * 16 * W_ROW), read_tr(st + w_off[1] + ks * 16 * W_ROW));
#pragma unroll
                for (int j = 0; j < RB; ++j) {
                    const int row = 32 * j + xl;
                    const int c = (2 * ks + (lane >> 5)) ^ swz8(row);
                    f.x[q][j] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(st + row * X_ROW + (c << 4)));
                }
            }
        };
        auto mfmas_half = [&](const Half& f) {
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int j = 0; j < RB; ++j)
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.w[q], f.x[q][j], acc[j], 0, 0, 0);
        };
        auto step_half = [&](Half& f0, Half& f1, const char* cur, const char* nxt, char* dma, int kl) {
            wait_stage();
            fence();
            issue(kl, dma);
            read_half(cur, 1, f1);
            mfmas_half(f0);
            // 2 RB MFMAs, RB + 4 loads, 2 RB + 4 reads: each MFMA followed by a
            // load and a read until those run out
#pragma unroll
            for (int i = 0; i < 2 * RB + 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // vector memory
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
            }
            fence();
            read_half(nxt, 0, f0);
            mfmas_half(f1);
#pragma unroll
            for (int i = 0; i < 2 * RB + 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            fence();
        };
        static_assert(!HALF || NS == 3, "tall tiles use three stages");
        Half h0, h1;
#pragma unroll
        for (int i = 0; i < NS - 1; ++i) issue_first(min(i, KT - 1), i == 0 ? st0 : st1);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(FIRST_WAIT, 15));   // stage 0 landed
        __builtin_amdgcn_s_barrier();
        fence();
        read_half(st0, 0, h0);
        fence();
        int kt = 0;
        // stage s in buffer s % 3: step s reads stages s and s + 1 and loads
        // stage s + 2 into the buffer of stage s - 1
        for (; kt + 3 <= KT; kt += 3) {
            step_half(h0, h1, st0, st1, st2, min(kt + 2, KT - 1));
            step_half(h0, h1, st1, st2, st0, min(kt + 3, KT - 1));
            step_half(h0, h1, st2, st0, st1, min(kt + 4, KT - 1));
        }
        if (kt < KT) {
            step_half(h0, h1, st0, st1, st2, KT - 1);
            if (kt + 1 < KT) step_half(h0, h1, st1, st2, st0, KT - 1);
        }
    }
    wait_vmem();

    // ---- epilogue.  acc[j] element v of lane l: row 32 j + l%32, MFMA
    // feature 32 w + 8 (v/4) + 4 (l/32) + v%4; g at v < 8, its u at v + 8.
#pragma unroll
    for (int j = 0; j < RB; ++j) {
        const int t = 32 * j + xl;
        if (t >= valid_rows) continue;
        uint16_t* out = a.h + (tile_r0 + t) * (int64_t)N;
#pragma unroll
        for (int vg = 0; vg < 2; ++vg) {
            const int col = nt * TCOL + 16 * wave + 8 * vg + 4 * (lane >> 5);
            if (col >= N) continue;
            const int v = 4 * vg;
            const f32x16_t& c = acc[j];
            *(uint2*)(out + col) =
                make_uint2(pack_bf16(silu_mul(c[v], c[v + 8]), silu_mul(c[v + 1], c[v + 9])),
                           pack_bf16(silu_mul(c[v + 2], c[v + 10]), silu_mul(c[v + 3], c[v + 11])));
            if (a.gu) {
                uint16_t* gu = a.gu + (tile_r0 + t) * (int64_t)(2 * N);
                *(uint2*)(gu + col) = make_uint2(pack_bf16(c[v], c[v + 1]), pack_bf16(c[v + 2], c[v + 3]));
                *(uint2*)(gu + N + col) =
                    make_uint2(pack_bf16(c[v + 8], c[v + 9]), pack_bf16(c[v + 10], c[v + 11]));
            }
        }
    }
#pragma unroll
    for (int j = 0; j < RB; ++j) acc[j] = f32x16_t{};
    }   // row tiles
}

template <int RB>
hipError_t launch_rb(const SlabArgs& a, hipStream_t s) {
    const int64_t rows = a.g.S + (a.g.G > a.g.E ? a.g.T : 0);
    const int64_t m_upper = (rows + 32 * RB - 1) / (32 * RB) + a.g.G;
    const int64_t blocks = m_upper * a.n_tiles;
    if (a.idx) {
        // one more workgroup than tiles: the sort's bookkeeping
        up_swiglu_slab_kernel<RB, true><<<(unsigned)((a.g.E + a.sh_tiles) * a.n_tiles + 1 + a.pf_blocks), NT, 0, s>>>(a);
    } else {
        up_swiglu_slab_kernel<RB, false><<<grid_for_work(blocks), NT, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

int slab_row_blocks(int64_t S, int64_t shared_rows, int E, int F) {
    // A tile of 32 rb rows holds a routed group of 1.25x the average size;
    // taller while that still leaves more than one round of workgroups (the
    // shared expert's rows count as a group of their own): every workgroup
    // pays the same fixed start-up, so a second, nearly empty round would
    // cost as much as the first.
    const int64_t want = (E > 0 ? S / E : S) * 5 / 4;
    const int64_t base = (want + 31) / 32;
    const int rb0 = (int)(base < 1 ? 1 : (base > kSlabMaxRowBlocks ? kSlabMaxRowBlocks : base));
    const int64_t cols = (F + TCOL - 1) / TCOL;
    for (int rb = rb0; rb <= kSlabMaxRowBlocks; ++rb) {
        const int64_t tr = 32 * rb;
        const int64_t tiles = (int64_t)E * ((want + tr - 1) / tr) + (shared_rows + tr - 1) / tr;
        if (tiles * cols <= kSlabRoundTiles) return rb;
    }
    return rb0;
}

namespace {
hipError_t launch_slab(const SlabArgs& a, int rb, hipStream_t s);
}  // namespace

hipError_t launch_up_swiglu_bf16_slab(const GroupArgs& g, int rb, const void* x, const void* W1,
                                      const void* W3, const void* Ws1, const void* Ws3, void* h,
                                      int D, int F, hipStream_t s, void* gu) {
    SlabArgs a{g, (const uint16_t*)x, (const uint16_t*)W1, (const uint16_t*)W3,
               (const uint16_t*)Ws1, (const uint16_t*)Ws3, (uint16_t*)h, D, F,
               (F + TCOL - 1) / TCOL};
    a.gu = (uint16_t*)gu;
    return launch_slab(a, rb, s);
}

hipError_t launch_up_swiglu_bf16_slab_routed(const GroupArgs& g, int rb, const int32_t* idx,
                                             int32_t* counts, int32_t* offsets, int32_t* tile_off,
                                             int32_t* tile_off64, int32_t* perm, int32_t* inv,
                                             int32_t* err, const void* x, const void* W1,
                                             const void* W3, const void* Ws1, const void* Ws3,
                                             const void* W2, const void* Ws2,
                                             void* h, int D, int F, hipStream_t s, void* gu) {
    if (g.S > kPermuteSingleMax || g.S < 1 || g.E > kRouteMaxExperts) return hipErrorInvalidValue;
    SlabArgs a{g, (const uint16_t*)x, (const uint16_t*)W1, (const uint16_t*)W3,
               (const uint16_t*)Ws1, (const uint16_t*)Ws3, (uint16_t*)h, D, F,
               (F + TCOL - 1) / TCOL, idx, counts, offsets, tile_off, tile_off64, perm, inv, err,
               32 * rb, g.G > g.E ? (int)((g.T + 32 * rb - 1) / (32 * rb)) : 0};
    a.w2 = (const uint16_t*)W2;
    a.ws2 = (const uint16_t*)Ws2;
    a.w2_bytes = (int64_t)g.E * F * D * 2;
    a.ws2_bytes = Ws2 ? (int64_t)F * D * 2 : 0;
    const int gemm_blocks = (g.E + a.sh_tiles) * a.n_tiles;
    // prefetch workgroups only on CUs the GEMM and the sort leave idle (256
    // CUs, one workgroup each), so they never delay the GEMM's last round
    a.pf_blocks = std::max(0, std::min(64, 256 - gemm_blocks - 1));
    a.gu = (uint16_t*)gu;
    return launch_slab(a, rb, s);
}

namespace {
hipError_t launch_slab(const SlabArgs& a, int rb, hipStream_t s) {
    switch (rb) {
        case 1: return launch_rb<1>(a, s);
        case 2: return launch_rb<2>(a, s);
        case 3: return launch_rb<3>(a, s);
        case 4: return launch_rb<4>(a, s);
        case 5: return launch_rb<5>(a, s);
        case 6: return launch_rb<6>(a, s);
        case 7: return launch_rb<7>(a, s);
        case 8: return launch_rb<8>(a, s);
    }
    return hipErrorInvalidValue;
}
}  // namespace

}  // namespace moe
