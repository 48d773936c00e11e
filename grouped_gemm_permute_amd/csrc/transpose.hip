// transpose.hip -- batched bf16 matrix transpose through LDS.
//
// The backward's transposed-weight products (dh' = dy W2^T and the per-row
// dx = dg W1^T + du W3^T) run on the same grouped GEMM engine as the
// forward, which streams [K, N] weight tiles; this kernel lays W2 out as
// [E, D, F] and W1, W3 as one stacked [E, 2F, D] once per backward call.
//
// 64 x 64 tiles, 256 threads.  Thread t reads 16 bytes (8 consecutive
// columns) of two consecutive rows 2 (t / 8), +1, pairs the two rows'
// elements of each column into one 32-bit word -- two consecutive elements
// of that column's output row -- and writes the 8 words to LDS; after the
// barrier it reads 16 bytes (8 elements) of an output row and stores them.
// LDS holds the output tile as 64 rows of 32 words, word w of row R at
// R * 32 + (w ^ 8 ((R / 8) % 4)): the 64 lanes of a write land on distinct
// banks pairwise, and a read's four words stay contiguous and aligned.
// A batch past the contiguous ones can come from a separate matrix (the
// shared expert's), so one launch covers the experts and the shared expert.
#include "moe_bwd_internal.h"

namespace moe {
namespace {

constexpr int TS = 64;

__device__ __forceinline__ int swz(int R) { return 8 * ((R >> 3) & 3); }

__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src,
                                                            const uint16_t* __restrict__ src_extra,
                                                            int64_t nsrc, int rows, int cols,
                                                            uint16_t* __restrict__ dst,
                                                            int64_t dst_batch_stride, int dst_ld,
                                                            int dst_row0) {
    __shared__ __attribute__((aligned(16))) uint32_t tw[TS * TS / 2];
    const int tid = threadIdx.x;
    const int c0 = blockIdx.x * TS, r0 = blockIdx.y * TS;
    const int64_t b = blockIdx.z;
    const uint16_t* s = b < nsrc ? src + b * rows * (int64_t)cols : src_extra;
    const int rp = tid >> 3, cc = tid & 7;
    const uint4 va = *(const uint4*)(s + (int64_t)(r0 + 2 * rp) * cols + c0 + 8 * cc);
    const uint4 vb = *(const uint4*)(s + (int64_t)(r0 + 2 * rp + 1) * cols + c0 + 8 * cc);
    const uint32_t wa[4] = {va.x, va.y, va.z, va.w}, wb[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // columns 8 cc + 2 i (low halves) and 8 cc + 2 i + 1 (high halves);
        // in each word row 2 rp is the low half, row 2 rp + 1 the high half
        const int R0 = 8 * cc + 2 * i, R1 = R0 + 1;
        tw[R0 * 32 + (rp ^ swz(R0))] = (wa[i] & 0xffffu) | (wb[i] << 16);
        tw[R1 * 32 + (rp ^ swz(R1))] = (wa[i] >> 16) | (wb[i] & 0xffff0000u);
    }
    __syncthreads();
    uint16_t* d = dst + b * dst_batch_stride;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int idx = tid + 256 * pass, R = idx >> 3, q = idx & 7;
        const uint4 v = *(const uint4*)(tw + R * 32 + ((4 * q) ^ swz(R)));
        *(uint4*)(d + (int64_t)(dst_row0 + c0 + R) * dst_ld + r0 + 8 * q) = v;
    }
}

}  // namespace

hipError_t launch_transpose_bf16(const void* src, int64_t batches, int rows, int cols, void* dst,
                                 int64_t dst_batch_stride, int dst_ld, int dst_row0, hipStream_t s,
                                 const void* src_extra) {
    if (rows % TS || cols % TS || batches < 0) return hipErrorInvalidValue;
    const int64_t nb = batches + (src_extra ? 1 : 0);
    if (nb == 0 || rows == 0 || cols == 0) return hipSuccess;
    const dim3 grid((unsigned)(cols / TS), (unsigned)(rows / TS), (unsigned)nb);
    transpose_bf16_kernel<<<grid, 256, 0, s>>>((const uint16_t*)src, (const uint16_t*)src_extra,
                                                batches, rows, cols, (uint16_t*)dst,
                                                dst_batch_stride, dst_ld, dst_row0);
    return hipGetLastError();
}

}  // namespace moe
