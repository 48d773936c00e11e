// permute_device.h -- device side of the stable counting sort of the
// slots by expert id (see permute.hip), shared by the permute kernels and
// by the small-chunk up GEMM that sorts in one of its own workgroups.
// Internal to libmoe_ffn.so.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace permute_dev {

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Lanes of this wavefront whose key equals this lane's key.  Every lane of
// the wavefront must call it.  Keys are in [0, 2^nbits).
__device__ __forceinline__ uint64_t match_peers(int key, int nbits) {
    uint64_t peers = ~0ull;
    for (int b = 0; b < nbits; ++b) {
        const int bit = (key >> b) & 1;
        const uint64_t m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    return peers;
}

__device__ __forceinline__ int key_of(const int32_t* idx, int64_t s, int64_t S, int E) {
    if (s >= S) return E + 1;                        // past the end: no slot
    const int32_t e = idx[s];
    return (e >= 0 && e < E) ? e : E;                // E: invalid id
}

struct TileSpec {
    int rows;          // tile height
    int32_t* off;      // [E+2] row-tile prefix, or null
};

// Serial prefix sums by one thread: counts/offsets/err and up to two row-tile
// prefixes from cnt[0..E].
__device__ inline void finish_scan(const int32_t* cnt, int E, TileSpec ta, TileSpec tb,
                            int64_t shared_rows, int32_t* counts, int32_t* offsets, int32_t* err,
                            int32_t* run) {
    int32_t acc = 0, tiles_a = 0, tiles_b = 0;
    for (int e = 0; e < E; ++e) {
        const int32_t c = cnt[e];
        counts[e] = c;
        offsets[e] = acc;
        ta.off[e] = tiles_a;
        if (tb.off) tb.off[e] = tiles_b;
        if (run) run[e] = acc;
        acc += c;
        tiles_a += (c + ta.rows - 1) / ta.rows;
        if (tb.off) tiles_b += (c + tb.rows - 1) / tb.rows;
    }
    offsets[E] = acc;
    ta.off[E] = tiles_a;
    ta.off[E + 1] = tiles_a + (int32_t)((shared_rows + ta.rows - 1) / ta.rows);
    if (tb.off) {
        tb.off[E] = tiles_b;
        tb.off[E + 1] = tiles_b + (int32_t)((shared_rows + tb.rows - 1) / tb.rows);
    }
    err[0] = cnt[E];
}

// Rank the slots [c0, c0 + blockDim) of one chunk and scatter them; key is
// this thread's key_of(idx, c0 + threadIdx.x, end, E), loaded by the caller
// (so that a block's loads can all be in flight at once).
// run[e]: next free position of expert e; wcnt [nwaves][E] zeroed on entry
// and on exit.
// Slots at or past `end` are not part of this chunk; S bounds every write.
template <int NT>
__device__ inline void scatter_chunk(int key, int64_t c0, int64_t end, int64_t S, int E, int nbits,
                                     int32_t* run, int32_t* wcnt, int32_t* perm, int32_t* inv) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / 64;
    const int64_t s = c0 + tid;
    const uint64_t peers = match_peers(key, nbits);
    const int rank = __popcll(peers & ((1ull << lane) - 1ull));
    if (rank == 0 && key < E) wcnt[wave * E + key] = __popcll(peers);
    __syncthreads();
    if (key < E) {
        // the counts of the wavefronts below: all loads issued at once
        int32_t pos = run[key] + rank;
#pragma unroll
        for (int w = 0; w < NW - 1; ++w) {
            const int32_t c = wcnt[w * E + key];
            pos += w < wave ? c : 0;
        }
        if (pos >= 0 && pos < S) {     // always true for a consistent histogram
            perm[pos] = (int32_t)s;
            inv[s] = pos;
        }
    } else if (s < end) {
        inv[s] = -1;
    }
    __syncthreads();
    for (int e = tid; e < E; e += NT) {
        int32_t tot = 0;
        for (int w = 0; w < NW; ++w) {
            tot += wcnt[w * E + e];
            wcnt[w * E + e] = 0;
        }
        run[e] += tot;
    }
    __syncthreads();
}

__device__ __forceinline__ int key_bits(int E) { return 32 - __clz(E + 1); }


// The whole counting sort in one workgroup of NT threads: histogram (LDS
// atomics), prefix sums by one thread, then the slots in chunks of NT in
// slot order, each ranked with ballots.  LDS scratch from the caller:
// cnt [E + 1], run [E], wcnt [(NT / 64) E].
template <int NT>
__device__ void permute_one_workgroup(const int32_t* idx, int64_t S, int E, TileSpec ta, TileSpec tb,
                                      int64_t shared_rows, int32_t* counts, int32_t* offsets,
                                      int32_t* perm, int32_t* inv, int32_t* err, int32_t* cnt,
                                      int32_t* run, int32_t* wcnt) {
    constexpr int KPT = (int)(kPermuteSingleMax / NT);   // slots per thread (S <= kPermuteSingleMax)
    static_assert(KPT * NT == kPermuteSingleMax, "whole chunks");
    const int tid = threadIdx.x;
    // every key of this thread, loaded once, all in flight together
    int keys[KPT];
#pragma unroll
    for (int q = 0; q < KPT; ++q) keys[q] = key_of(idx, (int64_t)q * NT + tid, S, E);
    for (int e = tid; e <= E; e += NT) cnt[e] = 0;
    for (int i = tid; i < (NT / 64) * E; i += NT) wcnt[i] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < KPT; ++q)
        if (keys[q] <= E) atomicAdd(&cnt[keys[q]], 1);
    __syncthreads();
    if (tid == 0) finish_scan(cnt, E, ta, tb, shared_rows, counts, offsets, err, run);
    __syncthreads();
    const int nbits = key_bits(E);
#pragma unroll
    for (int q = 0; q < KPT; ++q)
        if ((int64_t)q * NT < S)
            scatter_chunk<NT>(keys[q], (int64_t)q * NT, S, S, E, nbits, run, wcnt, perm, inv);
    const int32_t valid = (int32_t)(S - cnt[E]);
    for (int64_t p = valid + tid; p < S; p += NT) perm[p] = -1;
}

}  // namespace permute_dev
}  // namespace moe
