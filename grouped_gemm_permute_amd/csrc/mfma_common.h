// mfma_common.h -- device helpers shared by the bf16 MFMA kernels
// (gemm_bf16.hip, fused_bf16.hip).  Internal to libmoe_ffn.so.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace mfma {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) short s16x8_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// 16-byte-chunk swizzles (index of a chunk within its LDS row).
// K-contiguous rows of 8 chunks (128 B): conflict-free ds_read_b128 over 16
// consecutive rows.
__device__ __forceinline__ int swz8(int row) { return (row ^ (row >> 3)) & 7; }
// K-contiguous rows of 16 chunks (256 B).
__device__ __forceinline__ int swz16(int row) { return (row ^ (row >> 4)) & 15; }
// [K][N] rows read with ds_read_b64_tr_b16: the 4 rows one 16-lane group
// reads land 64 bytes apart in the banks.
__device__ __forceinline__ int swz_tr(int k) { return 4 * (k & 3); }

// Two fp32 values -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// silu(g) * u in fp32 with the hardware exp2 and reciprocal (about 1 ulp each):
// g * (1 / (1 + 2^(-g log2 e))) * u.  g -> -inf gives -0, g -> +inf gives g.
__device__ __forceinline__ float silu_mul(float g, float u) {
    const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
// contiguous range of logical tiles so neighbours share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
    const int x = bid & 7, i = bid >> 3;
    const int per = nblk >> 3, rem = nblk & 7;
    return x * per + min(x, rem) + i;
}

// The same for a grid sized from an upper bound on the tile count: the
// `work` tiles that exist (known only on the device) are spread evenly over
// the XCDs, each XCD taking a contiguous range; returns -1 for a workgroup
// with no tile.  The grid must hold at least 8 * ceil(work / 8) workgroups
// (grid_for_work).
__device__ __forceinline__ int xcd_remap_work(int bid, int work) {
    const int x = bid & 7, i = bid >> 3;
    const int per = work >> 3, rem = work & 7;
    if (i >= per + (x < rem ? 1 : 0)) return -1;
    return x * per + min(x, rem) + i;
}

// 16 bytes per lane global -> LDS; the wavefront's 64 lanes fill 1 KiB of
// LDS starting at `lds` (wave-uniform), lane i at lds + 16 i.
__device__ __forceinline__ void load_lds16(const void* g, char* lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds, 16, 0, 0);
}

// The same with the non-temporal cache policy: for data read once per use
// that should not displace reused lines from the L2.
__device__ __forceinline__ void load_lds16_nt(const void* g, char* lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds, 16, 0, 2);
}

// s_waitcnt immediate (gfx9 encoding): at most vm vector-memory and lgkm
// LDS/scalar operations of this wavefront outstanding (vm up to 63, lgkm up
// to 15; 15 leaves the LDS counter unchecked).
constexpr int waitcnt_imm(int vm, int lgkm) {
    return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

// Wait until this wavefront's global_load_lds transfers (vector memory) have
// landed; LDS and scalar counters untouched.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Four bf16 of column R, rows k .. k+3 of a [K][N] LDS tile, per lane of a
// 16-lane group (see the callers for the lane -> address mapping).
__device__ __forceinline__ s16x4_t read_tr(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
}

__device__ __forceinline__ bf16x8_t cat_bf16(s16x4_t lo, s16x4_t hi) {
    const s16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
}

// Owner of row tile mt among the G groups: tile_off is non-decreasing, so the
// owner is (number of groups g < G with tile_off[g] <= mt) - 1.  One vector
// load of 64 entries per step and a ballot; the owner's tile start and row
// range come back through readlane (no dependent load chain).  Every lane of
// the wavefront must call it; requires mt < tile_off[G].
struct TileGroup {
    int grp;
    int64_t row0;     // first row of the group in the row space
    int64_t rows;     // rows of the group
    int64_t tile_r0;  // first row of tile mt
    int valid_rows;   // rows of tile mt that exist (<= tile_rows)
};

// The group table's first 64 entries (tile starts, row ranges), one group
// per lane.  The loads need nothing but the table, so a kernel can issue them
// at entry, beside the read that decides its tile.
struct GroupBlock {
    int to, o0, o1;
};

__device__ __forceinline__ GroupBlock load_group_block(const GroupArgs& ga, int base, int lane) {
    const int g = base + lane;
    const bool in = g < ga.G;
    GroupBlock b;
    b.to = in ? ga.tile_off[g] : 0x7fffffff;
    b.o0 = (in && g < ga.E) ? ga.offsets[g] : 0;
    b.o1 = (in && g < ga.E) ? ga.offsets[g + 1] : 0;
    return b;
}

// first: load_group_block(ga, 0, lane); later 64-group blocks are loaded here.
__device__ __forceinline__ TileGroup find_tile_group(const GroupArgs& ga, int mt, int tile_rows,
                                                     int lane, const GroupBlock& first) {
    int grp = 0, tile0 = 0, o0v = 0, o1v = 0;
    for (int base = 0; base < ga.G; base += 64) {
        const GroupBlock b = base == 0 ? first : load_group_block(ga, base, lane);
        const int n = __popcll(__ballot(b.to <= mt));
        if (n == 0) break;                  // owner is the last group of the previous block
        grp = base + n - 1;
        tile0 = __builtin_amdgcn_readlane(b.to, n - 1);
        o0v = __builtin_amdgcn_readlane(b.o0, n - 1);
        o1v = __builtin_amdgcn_readlane(b.o1, n - 1);
        if (n < 64) break;
    }
    TileGroup t;
    t.grp = grp;
    const bool shared = grp >= ga.E;
    t.row0 = shared ? ga.S : (int64_t)o0v;
    t.rows = shared ? ga.T : (int64_t)(o1v - o0v);
    t.tile_r0 = t.row0 + (int64_t)(mt - tile0) * tile_rows;
    t.valid_rows = (int)min((int64_t)tile_rows, t.row0 + t.rows - t.tile_r0);
    return t;
}

__device__ __forceinline__ TileGroup find_tile_group(const GroupArgs& ga, int mt, int tile_rows,
                                                     int lane) {
    return find_tile_group(ga, mt, tile_rows, lane, load_group_block(ga, 0, lane));
}

}  // namespace mfma
}  // namespace moe
