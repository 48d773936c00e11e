// clock.hip -- measurement helper behind moe_device_clock_sample: the
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

}  // namespace

extern "C" moe_status moe_device_clock_sample(int64_t* out, int blocks, hipStream_t stream) {
    if (!out || blocks < 1 || blocks > 1024 || ((uintptr_t)out % 8) != 0) return MOE_ERR_INVALID_ARG;
    (void)hipGetLastError();
    clock_sample_kernel<<<blocks, 64, 0, stream>>>(out);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
