// transpose.hip -- batched bf16 matrix transpose through LDS.
//
// The backward's transposed-weight products (dh' = dy W2^T and the per-row
// dx = dg W1^T + du W3^T) run on the same grouped GEMM engine as the
// forward, which streams [K, N] weight tiles; this kernel lays W2 out as
// [E, D, F] and W1, W3 as one stacked [E, 2F, D] once per backward call.
//
// 64 x 64 tiles, 256 threads: each thread reads 16 bytes (8 consecutive
// columns of one row) into LDS, then writes 16 bytes (8 consecutive rows of
// one column) of the transposed tile.  LDS rows are padded by 2 elements so
// the column reads of one wavefront spread over the banks.
#include "moe_bwd_internal.h"

namespace moe {
namespace {

constexpr int TS = 64;
constexpr int PAD = TS + 2;

__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src, int rows,
                                                            int cols, uint16_t* __restrict__ dst,
                                                            int64_t dst_batch_stride, int dst_ld,
                                                            int dst_row0) {
    __shared__ uint16_t tile[TS][PAD];
    const int tid = threadIdx.x;
    const int c0 = blockIdx.x * TS, r0 = blockIdx.y * TS;
    const int64_t b = blockIdx.z;
    const uint16_t* s = src + b * rows * (int64_t)cols;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int r = tid / 8 + 32 * pass, c = (tid % 8) * 8;
        const uint4 v = *(const uint4*)(s + (int64_t)(r0 + r) * cols + c0 + c);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            tile[r][c + 2 * i] = (uint16_t)(w[i] & 0xffff);
            tile[r][c + 2 * i + 1] = (uint16_t)(w[i] >> 16);
        }
    }
    __syncthreads();
    uint16_t* d = dst + b * dst_batch_stride;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int c = tid / 8 + 32 * pass, r = (tid % 8) * 8;
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = (uint32_t)tile[r + 2 * i][c] | ((uint32_t)tile[r + 2 * i + 1][c] << 16);
        *(uint4*)(d + (int64_t)(dst_row0 + c0 + c) * dst_ld + r0 + r) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

}  // namespace

hipError_t launch_transpose_bf16(const void* src, int64_t batches, int rows, int cols, void* dst,
                                 int64_t dst_batch_stride, int dst_ld, int dst_row0, hipStream_t s) {
    if (rows % TS || cols % TS || batches < 0) return hipErrorInvalidValue;
    if (batches == 0 || rows == 0 || cols == 0) return hipSuccess;
    const dim3 grid((unsigned)(cols / TS), (unsigned)(rows / TS), (unsigned)batches);
    transpose_bf16_kernel<<<grid, 256, 0, s>>>((const uint16_t*)src, rows, cols, (uint16_t*)dst,
                                                dst_batch_stride, dst_ld, dst_row0);
    return hipGetLastError();
}

}  // namespace moe
