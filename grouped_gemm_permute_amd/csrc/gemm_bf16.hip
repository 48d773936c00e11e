// gemm_bf16.hip -- grouped GEMMs of the expert FFN on gfx950 bf16 MFMA.
//
// Two kernels share one tile engine:
//
//  up_swiglu:  for every row p of every group (routed experts in sorted
//              order, then the shared expert on all tokens),
//                g = x[tok(p)] . W1[grp],  u = x[tok(p)] . W3[grp]   (fp32 accumulate)
//                h[p] = bf16(silu(g) * u)
//              x rows are gathered straight from the token matrix while the
//              A tile is loaded, and W1 and W3 columns of the same output
//              column sit in one workgroup tile, so g and u never leave the
//              registers.  This is the fused gate/up/SiLU-multiply grouped
//              GEMM of "Triton MoE Kernels & Memory Checkpointing" (Part A,
//              sections 6 and 10.1) with fp32 SiLU and a single cast of the
//              product to the storage type.
//  down:       Y[p] = h[p] . W2[grp]   (fp32 accumulate, fp32 out), the per
//              expert W2 product of the same page's section 10.3 step 4.
//
// Tile engine: 256 threads (4 wavefronts, 2 x 2), workgroup tile 256 rows x
// 256 MFMA columns, K step 64, double-buffered LDS (2 x 64 KiB), one wave
// tile 128 x 128 = 4 x 4 v_mfma_f32_32x32x16_bf16 accumulators.  Global
// loads of the next K step are issued before the MFMAs of the current one.
// Weights are stored [K][N] (N contiguous); MFMA wants 8 consecutive K per
// lane, so each thread loads an 8 x 8 (K x N) block and transposes it in
// registers before writing K-contiguous rows to LDS.  LDS rows are 128 B;
// their 16-byte chunks are XOR-swizzled with (row ^ row/8) & 7 so that both
// the MFMA operand reads and the transposed writes spread over the banks.
//
// Row tiles never cross a group: group g owns tiles tile_off[g] ..
// tile_off[g+1]-1 (computed by the permute on the device), the grid is sized
// by the host from an upper bound, and workgroups past tile_off[G] exit, so
// no host synchronisation is needed.  Rows past a group's end are clamped
// to its last row on load and never stored.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr int BM = kBf16TileRows;   // 256 rows per tile
constexpr int BN = 256;             // MFMA columns per tile (up: 128 g + 128 u)
constexpr int BK = 64;
constexpr int NT = 256;
constexpr int KCH = BK / 8;         // 16-byte chunks per LDS row
constexpr int TILE_CHUNKS = BM * KCH;  // chunks of one A (or B) tile in LDS

static_assert(BM == 256 && BN == 256 && BK == 64 && NT == 256, "index math below assumes these");

__device__ __forceinline__ int swz(int row, int c) { return row * KCH + (c ^ ((row ^ (row >> 3)) & 7)); }

// Round-to-nearest-even fp32 -> bf16 bits.
__device__ __forceinline__ uint16_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
// contiguous range of logical tiles so neighbours share L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
    const int x = bid & 7, i = bid >> 3;
    const int per = nblk >> 3, rem = nblk & 7;
    return x * per + min(x, rem) + i;
}

struct GemmArgs {
    GroupArgs g;
    const uint16_t* a;        // up: x [T, D]; down: h [R, F]
    const uint16_t* b0;       // up: W1 [E, D, F]; down: W2 [E, F, D]
    const uint16_t* b1;       // up: W3; down: unused
    const uint16_t* bs0;      // shared expert: up Ws1, down Ws2
    const uint16_t* bs1;      // up Ws3
    void* out;                // up: h bf16 [R, F]; down: Y fp32 [R, D]
    int D, F;
    int n_tiles;              // column tiles
};

template <bool UP>
__global__ __launch_bounds__(NT, 1) void grouped_gemm_bf16_kernel(const GemmArgs a) {
    __shared__ u32x4_t lds[2 * 2 * TILE_CHUNKS];   // [buf][A, B][row][chunk] = 128 KiB

    const int K = UP ? a.D : a.F;      // reduction length
    const int N = UP ? a.F : a.D;      // output columns
    const int ldb = N;                 // weight row stride (elements)

    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int mt = bid / a.n_tiles, nt = bid - mt * a.n_tiles;
    const int32_t* tile_off = a.g.tile_off;
    if (mt >= tile_off[a.g.G]) return;
    int grp = 0;
    {
        int lo = 0, hi = a.g.G - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tile_off[mid] <= mt) lo = mid; else hi = mid - 1;
        }
        grp = lo;
    }
    const bool shared = grp >= a.g.E;
    const int64_t grp_row0 = shared ? a.g.S : (int64_t)a.g.offsets[grp];
    const int64_t grp_rows = shared ? a.g.T : (int64_t)(a.g.offsets[grp + 1] - a.g.offsets[grp]);
    const int64_t tile_r0 = grp_row0 + (int64_t)(mt - tile_off[grp]) * BM;
    const int valid_rows = (int)min((int64_t)BM, grp_row0 + grp_rows - tile_r0);
    if (valid_rows <= 0) return;       // only if tile_off disagrees with offsets

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- A rows this thread loads: rows (tid>>3) + 32 i, chunk tid & 7.
    const int ca = tid & 7;
    const uint16_t* a_ptr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = min((tid >> 3) + 32 * i, valid_rows - 1);
        const int64_t p = tile_r0 + r;
        int64_t src_row;
        if (UP) src_row = p < a.g.S ? (int64_t)(a.g.perm[p] / a.g.k) : p - a.g.S;
        else src_row = p;
        a_ptr[i] = a.a + src_row * (int64_t)K + ca * 8;
    }

    // ---- B block this thread loads: K rows 8 kb .. 8 kb + 7, 8 columns.
    const int nb = tid & 31, kb = tid >> 5;
    const uint16_t* b_ptr;
    {
        int col;
        const uint16_t* base;
        const int64_t gstride = (int64_t)a.D * a.F;
        if (UP) {
            // LDS B row R = 8 nb + i: half = R / 128, kind = (R / 64) & 1 (0: W1, 1: W3)
            const int half = nb >> 4, kind = (nb >> 3) & 1;
            col = nt * (BN / 2) + half * 64 + (nb & 7) * 8;
            if (shared) base = kind ? a.bs1 : a.bs0;
            else base = (kind ? a.b1 : a.b0) + grp * gstride;
        } else {
            col = nt * BN + nb * 8;
            base = shared ? a.bs0 : a.b0 + grp * gstride;
        }
        if (col >= N) col = 0;                   // past the last column: load a valid one, never stored
        b_ptr = base + (int64_t)(kb * 8) * ldb + col;
    }

    u32x4_t ra[8], rb[8];
    auto load_global = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) ra[i] = *(const u32x4_t*)(a_ptr[i] + k0);
#pragma unroll
        for (int j = 0; j < 8; ++j) rb[j] = *(const u32x4_t*)(b_ptr + (int64_t)(k0 + j) * ldb);
    };
    auto store_lds = [&](int buf) {
        u32x4_t* As = lds + buf * 2 * TILE_CHUNKS;
        u32x4_t* Bs = As + TILE_CHUNKS;
#pragma unroll
        for (int i = 0; i < 8; ++i) As[swz((tid >> 3) + 32 * i, ca)] = ra[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) {          // column i of the 8 x 8 block, K ascending
            const int dw = i >> 1;
            u32x4_t o;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint32_t lo = rb[2 * m][dw], hi = rb[2 * m + 1][dw];
                o[m] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
            }
            Bs[swz(8 * nb + i, kb)] = o;
        }
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) acc[mi][nj] = f32x16_t{};

    const int KT = K / BK;
    load_global(0);
    store_lds(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) load_global((kt + 1) * BK);
        const u32x4_t* As = lds + buf * 2 * TILE_CHUNKS;
        const u32x4_t* Bs = As + TILE_CHUNKS;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int c = ks * 2 + (lane >> 5);
            bf16x8_t af[4], bfr[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                af[mi] = __builtin_bit_cast(bf16x8_t, As[swz(wm * 128 + mi * 32 + (lane & 31), c)]);
#pragma unroll
            for (int nj = 0; nj < 4; ++nj)
                bfr[nj] = __builtin_bit_cast(bf16x8_t, Bs[swz(wn * 128 + nj * 32 + (lane & 31), c)]);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int nj = 0; nj < 4; ++nj)
                    acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[nj],
                                                                          acc[mi][nj], 0, 0, 0);
        }
        if (kt + 1 < KT) store_lds(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue.  Accumulator element v of lane l holds column l % 32 and
    // row 8 (v / 4) + 4 (l / 32) + v % 4 of its 32 x 32 block.
    const int rbase = wm * 128 + 4 * (lane >> 5);
    if (UP) {
        uint16_t* h = (uint16_t*)a.out;
#pragma unroll
        for (int nj = 0; nj < 2; ++nj) {
            const int col = nt * (BN / 2) + wn * 64 + nj * 32 + (lane & 31);
            if (col >= N) continue;
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = rbase + mi * 32 + 8 * (v >> 2) + (v & 3);
                    if (r < valid_rows) {
                        const float g = acc[mi][nj][v], u = acc[mi][nj + 2][v];
                        const float hv = g / (1.0f + __expf(-g)) * u;
                        h[(tile_r0 + r) * (int64_t)N + col] = bf16_rne(hv);
                    }
                }
        }
    } else {
        float* Y = (float*)a.out;
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) {
            const int col = nt * BN + wn * 128 + nj * 32 + (lane & 31);
            if (col >= N) continue;
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = rbase + mi * 32 + 8 * (v >> 2) + (v & 3);
                    if (r < valid_rows) Y[(tile_r0 + r) * (int64_t)N + col] = acc[mi][nj][v];
                }
        }
    }
}

int m_tiles_upper(const GroupArgs& g) {
    const int64_t rows = g.S + (g.G > g.E ? g.T : 0);
    return (int)((rows + BM - 1) / BM) + g.G;
}

}  // namespace

hipError_t launch_up_swiglu_bf16(const GroupArgs& g, const void* x, const void* W1, const void* W3,
                                 const void* Ws1, const void* Ws3, void* h, int D, int F,
                                 hipStream_t s) {
    GemmArgs a{g, (const uint16_t*)x, (const uint16_t*)W1, (const uint16_t*)W3,
               (const uint16_t*)Ws1, (const uint16_t*)Ws3, h, D, F, (F + BN / 2 - 1) / (BN / 2)};
    const int64_t blocks = (int64_t)m_tiles_upper(g) * a.n_tiles;
    grouped_gemm_bf16_kernel<true><<<(unsigned)blocks, NT, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_down_bf16(const GroupArgs& g, const void* h, const void* W2, const void* Ws2,
                            float* Y, int D, int F, hipStream_t s) {
    GemmArgs a{g, (const uint16_t*)h, (const uint16_t*)W2, nullptr, (const uint16_t*)Ws2, nullptr,
               Y, D, F, (D + BN - 1) / BN};
    const int64_t blocks = (int64_t)m_tiles_upper(g) * a.n_tiles;
    grouped_gemm_bf16_kernel<false><<<(unsigned)blocks, NT, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
