// gemm_bf16_wgrad.hip -- the backward's weight gradients on bf16 MFMA.
//
// For every group (routed expert, then the shared expert) the gradient of
// a weight matrix is a sum over the group's rows of outer products,
//
//   [dW1 | dW3][grp] = sum_p x[tok(p)]^T [dg | du][p]      (M = D, N = 2F)
//   dW2[grp]         = sum_p (w h)[p]^T dy[tok(p)]         (M = F, N = D)
//
// the outer products of the gate/up gradients with the inputs that "Triton
// MoE Kernels & Memory Checkpointing" (Part A, section 8) names, and the
// same for W2.  The contraction runs over rows, so both operands arrive as
// [rows, features] and both are read from LDS with ds_read_b64_tr_b16.
//
// Work: each group's rows are cut into chunks of KC rows (the permute's
// second tile prefix, chunk_off); a workgroup computes one 256 x 256 tile
// of one chunk's partial sum in fp32 and stores it to a partial buffer
// [chunks, M, N] (a group of one chunk writes its gradient directly);
// wgrad_reduce then adds a group's chunk partials in chunk order (fixed
// summation order, no atomics) and writes the fp32 gradient, zero for a
// group without rows.
//
// Tile engine: 512 threads = 8 wavefronts, two per SIMD (one issues MFMAs
// while the other is held issuing a load); the MFMA's A operand is 32
// N-features, its B operand 32 M-features; wavefront w owns N features
// 64 (w % 4) .. +63 of M features 128 (w / 4) .. +127, so each lane ends
// with four consecutive N values of one M row.  K step 32 rows,
// a 4-stage ring of 32 KiB stages (M tile, then N tile, each 32 rows x 512
// bytes, XOR-swizzled in 16-byte chunks as the forward's weight tiles),
// filled with global_load_lds.  Gathered rows (x and dy read through the
// token index) take their token from an LDS table of the chunk.  Rows past
// the chunk's end read the M operand's last row and a zero row for the N
// operand, so they add nothing.
#include "mfma_common.h"
#include "moe_bwd_internal.h"

namespace moe {
namespace {

using namespace mfma;

constexpr int TM = 256, TN = 256, BK = 32, NT = 512;
constexpr int ROW = 512;                       // bytes per k row of a 256-feature tile
constexpr int TILE_BYTES = BK * ROW;           // 16 KiB
constexpr int STAGE_BYTES = 2 * TILE_BYTES;    // M tile, then N tile
constexpr int KC_MAX = kWgradChunkRows;

struct WgradArgs {
    GroupArgs g;              // tile_off: the chunk prefix (KC rows per chunk)
    const uint16_t* am;       // M operand rows [., M]
    const uint16_t* bn;       // N operand rows [., N]
    int M, N, KC;
    int m_tiles, n_tiles;
    float* partial;           // [chunks, M, N]
    const uint16_t* zeros;    // >= 16 bytes of zeros
    int split;                // output columns n < split -> out0, others -> out1
    float *out0, *out1, *out0_sh, *out1_sh;
};

// GM / GN: the M / N operand's row p is its token's row (x, dy) rather than
// row p itself.
template <bool GM, bool GN>
__global__ __launch_bounds__(NT, 1) void wgrad_bf16_kernel(const WgradArgs a) {
    __shared__ __attribute__((aligned(1024))) char st0[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char st1[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char st2[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char st3[STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) uint32_t tok[KC_MAX];

    const int per_chunk = a.m_tiles * a.n_tiles;
    const int bid = xcd_remap_work(blockIdx.x, a.g.tile_off[a.g.G] * per_chunk);
    if (bid < 0) return;
    const int ck = bid / per_chunk;
    const int rem = bid - ck * per_chunk;
    const int tm = rem / a.n_tiles, tn = rem - tm * a.n_tiles;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int fw = wave & 3;           // N features 64 fw .. 64 fw + 63
    const int rw = wave >> 2;          // M features 128 rw .. 128 rw + 127

    if (ck >= a.g.tile_off[a.g.G]) return;
    const TileGroup tg = find_tile_group(a.g, ck, a.KC, lane);
    const bool shared = tg.grp >= a.g.E;
    const uint32_t r0 = (uint32_t)tg.tile_r0;   // rows < 2^31
    const int valid = tg.valid_rows;
    if (valid <= 0) return;
    const int KT = (valid + BK - 1) / BK;

    // ---- the chunk's token table, padded to KT * BK rows with the last
    // row's token and stored in issue order: entry ((kt * 2 + h) * 8 + w) * 2
    // + j holds row kt * BK + 4 w + 2 j + h, so a lane's two DMA rows of a
    // K step are one 8-byte LDS read.
    // All of a thread's index loads are issued before the first is used (one
    // memory round trip rather than one per entry).
    if (GM || GN) {
        constexpr int PER = KC_MAX / NT;
        uint32_t v[PER];
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int i = tid + q * NT;
            const uint32_t p = r0 + (uint32_t)min(i, valid - 1);
            v[q] = shared ? p - (uint32_t)a.g.S : (i < KT * BK ? (uint32_t)a.g.perm[p] : 0u);
        }
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int i = tid + q * NT;
            if (i < KT * BK) {
                const int kt = i >> 5, kr = i & 31;
                const int e = ((kt * 2 + (kr & 1)) * 8 + (kr >> 2)) * 2 + ((kr >> 1) & 1);
                tok[e] = shared ? v[q] : v[q] / (uint32_t)a.g.k;
            }
        }
        __syncthreads();
    }

    // ---- loads: DMA instruction j (0, 1) of wavefront w fills k rows
    // 4 w + 2 j, +1 of each tile; lane -> k row 4 w + 2 j + lane/32,
    // physical chunk lane%32 holding logical chunk cl = phys ^ swz_tr(k),
    // i.e. features 8 cl .. 8 cl + 7.  Row addresses are the row index (32
    // bits) times the row pitch plus a per-lane column base: one
    // v_mad_u64_u32 per load, no divergent code on the way to the DMA.
    const int M = a.M, N = a.N;
    const uint32_t pitch_m = 2u * (uint32_t)M, pitch_n = 2u * (uint32_t)N;
    const char* m_base[2];
    const char* n_base[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int kr = 4 * wave + 2 * j + (lane >> 5);
        const int cl = (lane & 31) ^ swz_tr(kr);
        int m = tm * TM + 8 * cl, n = tn * TN + 8 * cl;
        if (m >= M) m = 0;                 // a valid address; its sums are never stored
        if (n >= N) n = 0;
        m_base[j] = (const char*)(a.am + m);
        n_base[j] = (const char*)(a.bn + n);
    }
    const uint32_t own0 = 4 * wave + (lane >> 5);   // + 2 j: the lane's rows in a K step
    uint2 tok_pf = {0u, 0u};           // tokens of the next stage's rows
    auto fetch_tok = [&](int kt) {
        if (GM || GN) tok_pf = *(const uint2*)&tok[((kt * 2 + (lane >> 5)) * 8 + wave) * 2];
    };
    auto issue = [&](int kt, char* st) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t i = (uint32_t)(kt * BK) + own0 + 2 * j;
            const uint32_t own = r0 + min(i, (uint32_t)valid - 1);
            const uint32_t tk = j ? tok_pf.y : tok_pf.x;
            const uint32_t rm = GM ? tk : own;
            const uint32_t rn = GN ? tk : own;
            const char* sm = m_base[j] + (uint64_t)rm * pitch_m;
            const char* row_n = n_base[j] + (uint64_t)rn * pitch_n;
            // opaque to the optimiser, so the multiply is not sunk into a
            // divergent branch (exec-mask writes end a scheduling region)
            asm volatile("" : "+v"(row_n));
            const char* sn = i < (uint32_t)valid ? row_n : (const char*)a.zeros;
            load_lds16(sm, st + (4 * wave + 2 * j) * ROW);
            load_lds16(sn, st + TILE_BYTES + (4 * wave + 2 * j) * ROW);
        }
    };

    // ---- MFMA operand read offsets: lane = 16 G + s of k16 slice ks reads
    // k = 16 ks + 8 (G / 2) + 4 r + s / 4 (r = 0, 1), feature base + 16 (G % 2)
    // + 4 (s % 4) of a 32-feature block.
    const int G = lane >> 4, sl = lane & 15;
    auto tr_off = [&](int tile, int R, int r) {
        const int k = 8 * (G >> 1) + 4 * r + (sl >> 2);
        return tile + k * ROW + (((R >> 3) ^ swz_tr(k)) << 4) + 8 * ((R >> 2) & 1);
    };
    int n_off[2][2], m_off[4][2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
            n_off[mi][r] = tr_off(TILE_BYTES, 64 * fw + 32 * mi + 16 * (G & 1) + 4 * (sl & 3), r);
#pragma unroll
        for (int nj = 0; nj < 4; ++nj)
            m_off[nj][r] = tr_off(0, 128 * rw + 32 * nj + 16 * (G & 1) + 4 * (sl & 3), r);
    }

    f32x16_t acc[2][4];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) acc[mi][nj] = f32x16_t{};

    struct Frags {
        bf16x8_t n[2][2], m[2][4];      // [k16 slice][block]
    };
    auto read_frags = [&](const char* st, Frags& f) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                f.n[ks][mi] = cat_bf16(read_tr(st + n_off[mi][0] + ks * 16 * ROW),
                                       read_tr(st + n_off[mi][1] + ks * 16 * ROW));
#pragma unroll
            for (int nj = 0; nj < 4; ++nj)
                f.m[ks][nj] = cat_bf16(read_tr(st + m_off[nj][0] + ks * 16 * ROW),
                                       read_tr(st + m_off[nj][1] + ks * 16 * ROW));
        }
    };
    auto mfmas = [&](const Frags& f) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int nj = 0; nj < 4; ++nj)
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
                    acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.n[ks][mi], f.m[ks][nj],
                                                                          acc[mi][nj], 0, 0, 0);
    };
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

    // ---- 4-stage ring, one stage of operands in registers ahead (as the
    // forward engine): step s waits for stage s+1, issues stage s+3 into the
    // buffer of stage s-1, reads stage s+1's operands and runs stage s's
    // MFMAs.  The tokens for the next issue are read from LDS during the
    // step and waited for at the next step's barrier.
    constexpr int PER_STAGE = 4;
    auto step = [&](Frags& fc, Frags& fn, const char* nxt, char* dma, int kl) {
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(PER_STAGE, 0));
        __builtin_amdgcn_s_barrier();
        fence();
        issue(kl, dma);
        fetch_tok(min(kl + 1, KT - 1));
        read_frags(nxt, fn);
        mfmas(fc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // vector memory
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS reads
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        fence();
    };
    Frags fa, fb;
    fetch_tok(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    issue(0, st0);
    fetch_tok(min(1, KT - 1));
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    issue(min(1, KT - 1), st1);
    fetch_tok(min(2, KT - 1));
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    issue(min(2, KT - 1), st2);
    fetch_tok(min(3, KT - 1));
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
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));

    // ---- the tile: element v of acc[mi][nj] on lane l is M row
    // tm*256 + 128 rw + 32 nj + l%32, N columns tn*256 + 64 fw + 32 mi + 8 (v/4) + 4 (l/32) + 0..3.
    // It leaves through LDS in two passes of 128 M rows, pass p holding the
    // rows of the wavefronts with rw = p: their block nj goes to stage buffer
    // nj as 32 rows of 256 fp32 (16-byte chunk c of row r at physical chunk
    // c ^ r), then every wavefront stores 16 whole 1 KiB rows, one row per
    // instruction.  A group of one chunk writes
    // its gradient directly; otherwise the chunk's partial goes to the
    // partial buffer for wgrad_reduce.
    __syncthreads();   // every wavefront is done with the operand stages
    const bool single = a.g.tile_off[tg.grp + 1] - a.g.tile_off[tg.grp] == 1;
    auto stq = [&](int q) -> char* { return q == 0 ? st0 : q == 1 ? st1 : q == 2 ? st2 : st3; };
    const int n0 = tn * TN + 4 * lane;       // this lane's 4 columns in the store phase
    const bool col_ok = n0 < N;
    float* dst_base;
    int64_t pitch;
    if (!single) {
        dst_base = a.partial + (int64_t)ck * M * N + n0;
        pitch = N;
    } else if (n0 < a.split) {
        dst_base = (shared ? a.out0_sh : a.out0 + (int64_t)tg.grp * M * a.split) + n0;
        pitch = a.split;
    } else {
        const int w = N - a.split;
        dst_base = (shared ? a.out1_sh : a.out1 + (int64_t)tg.grp * M * w) + (n0 - a.split);
        pitch = w;
    }
    const int rl = lane & 31;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        if (pass) __syncthreads();           // the previous pass's rows are read
        if (rw == pass) {
#pragma unroll
            for (int nj = 0; nj < 4; ++nj)
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                    for (int vg = 0; vg < 4; ++vg) {
                        const int c = 16 * fw + 8 * mi + 2 * vg + (lane >> 5);
                        const f32x16_t& v = acc[mi][nj];
                        *(float4*)(stq(nj) + rl * 1024 + ((c ^ rl) << 4)) =
                            make_float4(v[4 * vg], v[4 * vg + 1], v[4 * vg + 2], v[4 * vg + 3]);
                    }
        }
        __syncthreads();
        // wavefront w: rows 16 (w % 2) .. +15 of stage buffer w / 2
        char* const sq = stq(wave >> 1);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = 16 * (wave & 1) + i;
            const float4 row = *(const float4*)(sq + r * 1024 + ((lane ^ r) << 4));
            const int m = tm * TM + 128 * pass + 32 * (wave >> 1) + r;
            if (col_ok && m < M) *(float4*)(dst_base + (int64_t)m * pitch) = row;
        }
    }
}

// out[grp][m][n] = sum over the group's chunks c (ascending) of
// partial[c][m][n] for groups of several chunks (zero for a group without
// rows; one-chunk groups are written by the GEMM); columns n < split go to out0 ([M, split] per group),
// the rest to out1 ([M, N - split] per group); the shared group writes
// out0_sh / out1_sh.  Four columns per thread.
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(const float* __restrict__ partial,
                                                          const int32_t* __restrict__ chunk_off,
                                                          int E, int M, int N, int split,
                                                          float* __restrict__ out0,
                                                          float* __restrict__ out1,
                                                          float* __restrict__ out0_sh,
                                                          float* __restrict__ out1_sh) {
    const int grp = blockIdx.y;
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= (int64_t)M * N) return;
    const int m = (int)(e / N), n = (int)(e - (int64_t)m * N);
    const int c0 = chunk_off[grp], c1 = chunk_off[grp + 1];
    if (c1 - c0 == 1) return;              // written directly by its only chunk
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c = c0; c < c1; ++c) {
        const float4 v = *(const float4*)(partial + ((int64_t)c * M + m) * N + n);
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    const bool sh = grp == E;
    if (n < split) {
        float* d = sh ? out0_sh : out0 + (int64_t)grp * M * split;
        *(float4*)(d + (int64_t)m * split + n) = s;
    } else {
        const int w = N - split;
        float* d = sh ? out1_sh : out1 + (int64_t)grp * M * w;
        *(float4*)(d + (int64_t)m * w + n - split) = s;
    }
}

__global__ void zero_fill_kernel(uint32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

}  // namespace

int64_t wgrad_chunks_upper(int64_t R, int G, int KC) { return (R + KC - 1) / KC + G; }

int wgrad_chunk_rows(int64_t R, int D, int F) {
    // about three rounds of workgroups over the 256 CUs for the W1/W3
    // gradient, chunks of 512 .. kWgradChunkRows rows (multiples of 256)
    const int64_t tiles = (int64_t)((D + TM - 1) / TM) * ((2 * F + TN - 1) / TN);
    const int64_t want = (R * tiles + 3 * 256 - 1) / (3 * 256);
    const int64_t kc = (want + 255) / 256 * 256;
    return (int)(kc < 512 ? 512 : kc > KC_MAX ? KC_MAX : kc);
}

hipError_t launch_zero_fill(void* p, int64_t bytes, hipStream_t s) {
    const int n = (int)(bytes / 4);
    if (n <= 0) return hipSuccess;
    zero_fill_kernel<<<(n + 255) / 256, 256, 0, s>>>((uint32_t*)p, n);
    return hipGetLastError();
}

hipError_t launch_wgrad_bf16(const GroupArgs& chunks, int KC, const void* am, bool gather_m,
                             const void* bn, bool gather_n, int M, int N, float* partial,
                             const void* zeros, int split, float* out0, float* out1,
                             float* out0_sh, float* out1_sh, int64_t R, hipStream_t s) {
    if (KC % BK || KC > KC_MAX || M % 64 || N % 64) return hipErrorInvalidValue;
    if (R <= 0) return hipSuccess;
    WgradArgs a{chunks, (const uint16_t*)am, (const uint16_t*)bn, M, N, KC,
                (M + TM - 1) / TM, (N + TN - 1) / TN, partial, (const uint16_t*)zeros,
                split, out0, out1, out0_sh, out1_sh};
    const int64_t blocks = wgrad_chunks_upper(R, chunks.G, KC) * a.m_tiles * a.n_tiles;
    const unsigned grid = grid_for_work(blocks);
    if (gather_m && gather_n) wgrad_bf16_kernel<true, true><<<grid, NT, 0, s>>>(a);
    else if (gather_m) wgrad_bf16_kernel<true, false><<<grid, NT, 0, s>>>(a);
    else if (gather_n) wgrad_bf16_kernel<false, true><<<grid, NT, 0, s>>>(a);
    else wgrad_bf16_kernel<false, false><<<grid, NT, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_wgrad_reduce(const float* partial, const GroupArgs& chunks, int M, int N, int split,
                               float* out0, float* out1, float* out0_sh, float* out1_sh,
                               hipStream_t s) {
    if (M % 64 || N % 64) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(((int64_t)M * N / 4 + 255) / 256), (unsigned)chunks.G);
    wgrad_reduce_kernel<<<grid, 256, 0, s>>>(partial, chunks.tile_off, chunks.E, M, N, split, out0,
                                             out1, out0_sh, out1_sh);
    return hipGetLastError();
}

}  // namespace moe
