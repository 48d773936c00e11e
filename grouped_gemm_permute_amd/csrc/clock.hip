// clock.hip -- measurement helpers.  moe_device_clock_sample: the
// engine clock the kernels actually ran at, for pricing a launch against
// the MFMA peak at that clock (compute units x clock x dense bf16 FLOPs per
// CU per cycle) as well as against the nominal peak.
//
// Each one-wavefront workgroup reads where it runs (HW_REG_XCC_ID: the XCD;
// HW_REG_HW_ID bits 8-15: shader engine, array and compute unit within it),
// the shader-clock cycle counter (s_memtime) and the constant 100 MHz
// counter (s_memrealtime).  Cycle counters of different units are not
// comparable with each other (they start at different times), so the host
// pairs two samples by compute unit.
//
// moe_stream_read: the HBM read rate a plain streaming kernel reaches on
// this part, the yardstick for kernels bound by reading their operands once
// (the small-chunk forward streams its experts' weights).
#include <hip/hip_runtime.h>

#include "moe_ffn.h"

#include <stdint.h>

namespace {

__global__ __launch_bounds__(64) void clock_sample_kernel(int64_t* out) {
    if (threadIdx.x != 0) return;
    uint32_t xcc, hw;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    const uint64_t cyc = __builtin_amdgcn_s_memtime();
    const uint64_t rt = __builtin_amdgcn_s_memrealtime();
    out[3 * blockIdx.x] = (int64_t)(((xcc & 15u) << 16) | ((hw >> 8) & 0xffu));
    out[3 * blockIdx.x + 1] = (int64_t)cyc;
    out[3 * blockIdx.x + 2] = (int64_t)rt;
}

// Every thread keeps eight 16-byte reads in flight per pass, the grid
// striding over the buffer; each workgroup's xor of what it read goes to
// sink[blockIdx] (so no load can be elided).  The loads are non-temporal
// (nothing is re-read): 6.8 TB/s at 192 workgroups against 6.2 TB/s with
// the default policy, measured.
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
constexpr int kReadThreads = 512;
constexpr int kReadUnroll = 8;
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4* __restrict__ src,
                                                                    int64_t n16, uint32_t* sink) {
    __shared__ uint32_t red[kReadThreads / 64];
    const int64_t stride = (int64_t)gridDim.x * kReadThreads;
    uint32_t acc = 0;
    int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
    for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
        uint4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) {
            const u32x4 t = __builtin_nontemporal_load((const u32x4*)(src + i + u * stride));
            v[u] = make_uint4(t[0], t[1], t[2], t[3]);
        }
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int w = 0; w < kReadThreads / 64; ++w) r ^= red[w];
        sink[blockIdx.x] = r;
    }
}

}  // namespace

extern "C" moe_status moe_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks,
                                      hipStream_t stream) {
    if (!src || !sink || bytes == 0 || bytes % 16 != 0 || ((uintptr_t)src % 16) != 0 ||
        ((uintptr_t)sink % 4) != 0 || blocks < 1 || blocks > 65536)
        return MOE_ERR_INVALID_ARG;
    (void)hipGetLastError();
    stream_read_kernel<<<blocks, kReadThreads, 0, stream>>>((const uint4*)src, (int64_t)(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" moe_status moe_device_clock_sample(int64_t* out, int blocks, hipStream_t stream) {
    if (!out || blocks < 1 || blocks > 1024 || ((uintptr_t)out % 8) != 0) return MOE_ERR_INVALID_ARG;
    (void)hipGetLastError();
    clock_sample_kernel<<<blocks, 64, 0, stream>>>(out);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
