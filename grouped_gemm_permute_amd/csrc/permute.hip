// permute.hip -- expert_permute: stable counting sort of the flattened
// (token, choice) slots by expert id.
//
// The dispatch of "Triton MoE Kernels & Memory Checkpointing" (Part A,
// section 10.3, steps 1-2) flattens the router's top-k ids to slots,
// stable-argsorts them by expert so each expert's rows are contiguous, and
// takes per-expert counts (bincount) and start offsets (cumulative sum);
// "Chinchilla scaling, MoE, and fused Triton kernels" (section "PyTorch MoE
// implementation") adds the inverse permutation used by the combine.  Here
// the argsort is a counting sort, which yields the same unique stable order:
//
//   histogram   counts[e] = #{s : idx[s] == e}      (order-free, LDS atomics)
//   scan        offsets = exclusive prefix of counts; tile_off = prefix of
//               ceil(counts/tile_rows) plus one shared group
//   scatter     perm[offsets[e] + #{s' < s : idx[s'] == e}] = s, inv[s] = that
//
// The in-order rank #{s' < s : idx[s'] == e} never depends on atomic timing:
// inside a wavefront it is the popcount of the lanes below with the same key
// (found with one ballot per key bit), across wavefronts and slot blocks it
// is a prefix sum in (expert, block) order.
//
// Small problems run as one workgroup.  Larger ones take per-block
// histograms first; then, while the histogram table is small, every scatter
// block scans the small histogram table itself (two launches), and beyond
// that one scan workgroup turns the table into start positions between the
// two (three launches).
#include "moe_internal.h"
#include "permute_device.h"

namespace moe {
namespace {

using namespace permute_dev;

constexpr int kSingleThreads = 512;
// One thread per slot of a block: the block ranks its slots in one pass
// (scan_scatter 1.2-1.5 us faster at 8192 and 65536 slots than 256 threads
// walking four chunks, each a chain of barriers).
constexpr int kScatterThreads = 1024;
constexpr int kScanThreads = 1024;
constexpr int kBlockChunks = kPermuteBlockSlots / kScatterThreads;   // scatter chunks per block
static_assert(kBlockChunks * kScatterThreads == kPermuteBlockSlots, "whole chunks per block");
// Largest histogram table, (E+1) x nblocks entries, that every scatter block
// re-reads itself instead of a separate scan launch.
constexpr int64_t kFusedScanEntries = 8192;

__global__ __launch_bounds__(kSingleThreads) void permute_single_kernel(
    const int32_t* __restrict__ idx, int64_t S, int E, TileSpec ta, TileSpec tb, int64_t shared_rows,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, int32_t* __restrict__ err) {
    __shared__ int32_t cnt[kMaxExperts + 1];
    __shared__ int32_t run[kMaxExperts];
    __shared__ int32_t wcnt[(kSingleThreads / 64) * kMaxExperts];
    permute_one_workgroup<kSingleThreads>(idx, S, E, ta, tb, shared_rows, counts, offsets, perm, inv,
                                          err, cnt, run, wcnt);
}

// hist[e * nb + b] = slots of block b with key e (e == E: invalid ids).
__global__ __launch_bounds__(kScatterThreads) void permute_hist_kernel(
    const int32_t* __restrict__ idx, int64_t S, int E, int32_t* __restrict__ hist) {
    __shared__ int32_t cnt[kMaxExperts + 1];
    const int tid = threadIdx.x, b = blockIdx.x, nb = gridDim.x;
    for (int e = tid; e <= E; e += kScatterThreads) cnt[e] = 0;
    __syncthreads();
    const int64_t lo = (int64_t)b * kPermuteBlockSlots;
    const int64_t hi = min(S, lo + kPermuteBlockSlots);
    for (int64_t s = lo + tid; s < hi; s += kScatterThreads) atomicAdd(&cnt[key_of(idx, s, S, E)], 1);
    __syncthreads();
    for (int e = tid; e <= E; e += kScatterThreads) hist[(int64_t)e * nb + b] = cnt[e];
}

// Turns hist into per-(expert, block) start positions and writes the
// per-expert results.  One thread per expert row; each row is read in
// batches of 16 independent loads (two passes: totals, then exclusive
// prefixes plus the expert's start).
__global__ __launch_bounds__(kScanThreads) void permute_scan_kernel(
    int32_t* __restrict__ hist, int nb, int64_t S, int E, TileSpec ta, TileSpec tb,
    int64_t shared_rows, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ err) {
    constexpr int B = 16;
    __shared__ int32_t cnt[kMaxExperts + 1];
    __shared__ int32_t start[kMaxExperts];
    const int tid = threadIdx.x;
    for (int e = tid; e <= E; e += kScanThreads) {
        const int32_t* row = hist + (int64_t)e * nb;
        int32_t sum = 0;
        for (int b0 = 0; b0 < nb; b0 += B) {
            int32_t v[B];
#pragma unroll
            for (int i = 0; i < B; ++i) v[i] = b0 + i < nb ? row[b0 + i] : 0;
#pragma unroll
            for (int i = 0; i < B; ++i) sum += v[i];
        }
        cnt[e] = sum;
    }
    __syncthreads();
    if (tid == 0) finish_scan(cnt, E, ta, tb, shared_rows, counts, offsets, err, start);
    __syncthreads();
    for (int e = tid; e < E; e += kScanThreads) {
        int32_t* row = hist + (int64_t)e * nb;
        int32_t run = start[e];
        for (int b0 = 0; b0 < nb; b0 += B) {
            int32_t v[B];
#pragma unroll
            for (int i = 0; i < B; ++i) v[i] = b0 + i < nb ? row[b0 + i] : 0;
#pragma unroll
            for (int i = 0; i < B; ++i) {
                if (b0 + i < nb) row[b0 + i] = run;
                run += v[i];
            }
        }
    }
    const int32_t valid = (int32_t)(S - cnt[E]);
    for (int64_t p = valid + tid; p < S; p += kScanThreads) perm[p] = -1;
}

__global__ __launch_bounds__(kScatterThreads) void permute_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t S, int E, const int32_t* __restrict__ hist,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    __shared__ int32_t run[kMaxExperts];
    __shared__ int32_t wcnt[(kScatterThreads / 64) * kMaxExperts];
    const int tid = threadIdx.x, b = blockIdx.x, nb = gridDim.x;
    const int64_t lo = (int64_t)b * kPermuteBlockSlots;
    const int64_t hi = min(S, lo + kPermuteBlockSlots);
    int keys[kBlockChunks];
#pragma unroll
    for (int q = 0; q < kBlockChunks; ++q) keys[q] = key_of(idx, lo + q * kScatterThreads + tid, hi, E);
    for (int e = tid; e < E; e += kScatterThreads) run[e] = hist[(int64_t)e * nb + b];
    for (int i = tid; i < (kScatterThreads / 64) * E; i += kScatterThreads) wcnt[i] = 0;
    __syncthreads();
    const int nbits = key_bits(E);
#pragma unroll
    for (int q = 0; q < kBlockChunks; ++q)
        if (lo + q * kScatterThreads < hi)
            scatter_chunk<kScatterThreads>(keys[q], lo + q * kScatterThreads, hi, S, E, nbits, run,
                                           wcnt, perm, inv);
}

// Scan and scatter in one launch.  Block b reads the histogram table
// (E+1) x nb, forms per-expert totals and the counts of blocks before b,
// takes its start position per expert (offset of the expert plus the slots
// of that expert in earlier blocks) and scatters its slots.  Block 0 also
// writes counts, offsets, the tile prefixes, the error count and the -1
// tail of perm.
// The table may be finer than the scatter blocks: sub columns per block
// (column c covers slots [c * kPermuteBlockSlots / sub, ...)), as the
// router writes it.
__global__ __launch_bounds__(kScatterThreads) void permute_scan_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t S, int E, const int32_t* __restrict__ hist, int sub,
    TileSpec ta, TileSpec tb, int64_t shared_rows, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    int32_t* __restrict__ err) {
    __shared__ int32_t tot[kMaxExperts + 1];
    __shared__ int32_t run[kMaxExperts + 1];
    __shared__ int32_t wcnt[(kScatterThreads / 64) * kMaxExperts];
    const int tid = threadIdx.x, b = blockIdx.x, nb = gridDim.x;
    // this block's keys first: their loads overlap the table scan below
    const int64_t lo = (int64_t)b * kPermuteBlockSlots;
    const int64_t hi = min(S, lo + kPermuteBlockSlots);
    int keys[kBlockChunks];
#pragma unroll
    for (int q = 0; q < kBlockChunks; ++q) keys[q] = key_of(idx, lo + q * kScatterThreads + tid, hi, E);
    for (int e = tid; e <= E; e += kScatterThreads) tot[e] = run[e] = 0;
    for (int i = tid; i < (kScatterThreads / 64) * E; i += kScatterThreads) wcnt[i] = 0;
    __syncthreads();
    const int ncol = nb * sub;
    const int n = (E + 1) * ncol;
    for (int i = tid; i < n; i += kScatterThreads) {
        const int e = i / ncol, bb = i - e * ncol;
        const int32_t v = hist[i];
        if (v) {
            atomicAdd(&tot[e], v);
            if (bb < b * sub) atomicAdd(&run[e], v);
        }
    }
    __syncthreads();
    if (tid == 0) {
        int32_t acc = 0;
        for (int e = 0; e < E; ++e) {
            run[e] += acc;
            acc += tot[e];
        }
        if (b == 0) finish_scan(tot, E, ta, tb, shared_rows, counts, offsets, err, nullptr);
    }
    __syncthreads();
    if (b == 0) {
        const int32_t valid = (int32_t)(S - tot[E]);
        for (int64_t p = valid + tid; p < S; p += kScatterThreads) perm[p] = -1;
    }
    const int nbits = key_bits(E);
#pragma unroll
    for (int q = 0; q < kBlockChunks; ++q)
        if (lo + q * kScatterThreads < hi)
            scatter_chunk<kScatterThreads>(keys[q], lo + q * kScatterThreads, hi, S, E, nbits, run,
                                           wcnt, perm, inv);
}

}  // namespace

hipError_t launch_permute(const int32_t* idx, int64_t S, int E, int tile_rows, int64_t shared_rows,
                          int32_t* counts, int32_t* offsets, int32_t* tile_off, int32_t* perm,
                          int32_t* inv, int32_t* err, int32_t* hist, int nblocks, hipStream_t s,
                          int tile_rows2, int32_t* tile_off2) {
    const TileSpec ta{tile_rows, tile_off}, tb{tile_rows2 > 0 ? tile_rows2 : 1, tile_off2};
    if (nblocks == 0) {
        permute_single_kernel<<<1, kSingleThreads, 0, s>>>(idx, S, E, ta, tb, shared_rows, counts,
                                                           offsets, perm, inv, err);
        return hipGetLastError();
    }
    permute_hist_kernel<<<nblocks, kScatterThreads, 0, s>>>(idx, S, E, hist);
    if ((int64_t)(E + 1) * nblocks <= kFusedScanEntries) {
        permute_scan_scatter_kernel<<<nblocks, kScatterThreads, 0, s>>>(
            idx, S, E, hist, 1, ta, tb, shared_rows, counts, offsets, perm, inv, err);
        return hipGetLastError();
    }
    permute_scan_kernel<<<1, kScanThreads, 0, s>>>(hist, nblocks, S, E, ta, tb, shared_rows,
                                                   counts, offsets, perm, err);
    permute_scatter_kernel<<<nblocks, kScatterThreads, 0, s>>>(idx, S, E, hist, perm, inv);
    return hipGetLastError();
}

}  // namespace moe

namespace moe {

bool permute_fine_ok(int64_t S, int E, int sub) {
    const int nb = permute_hist_blocks(S);
    return nb > 0 && (int64_t)(E + 1) * nb * sub <= kFusedScanEntries;
}

hipError_t launch_permute_from_hist(const int32_t* idx, int64_t S, int E, int tile_rows,
                                    int64_t shared_rows, int32_t* counts, int32_t* offsets,
                                    int32_t* tile_off, int32_t* perm, int32_t* inv, int32_t* err,
                                    const int32_t* hist, int sub, hipStream_t s, int tile_rows2,
                                    int32_t* tile_off2) {
    const TileSpec ta{tile_rows, tile_off}, tb{tile_rows2 > 0 ? tile_rows2 : 1, tile_off2};
    const int nb = permute_hist_blocks(S);
    permute_scan_scatter_kernel<<<nb, kScatterThreads, 0, s>>>(idx, S, E, hist, sub, ta, tb,
                                                               shared_rows, counts, offsets, perm,
                                                               inv, err);
    return hipGetLastError();
}

}  // namespace moe
