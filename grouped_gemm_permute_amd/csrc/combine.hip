// combine.hip -- unpermute and weighted combine.
//
//   y[t] = Ysh[t] + sum_{j=0}^{k-1} w[t,j] * Y[inv[t*k + j]]
//
// "Chinchilla scaling, MoE, and fused Triton kernels" (section "PyTorch MoE
// implementation") gathers each token's k expert rows through the inverse
// permutation and sums them weighted; "Triton MoE Kernels & Memory
// Checkpointing" (Part A, section 10.3 step 4) scales by the routing weight
// after W2 and adds the result back into the token's row.  Here the k terms
// are added in j order, starting from the shared expert's row (or 0), in
// fp32, and rounded once to the output type, so the result does not depend
// on scheduling (no scatter atomics).  Slots with inv = -1 (invalid ids)
// add nothing.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int NT = 256;

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// One thread per (token, 4 consecutive columns).
template <bool BF16>
__global__ __launch_bounds__(NT) void combine_kernel(const float* __restrict__ Y,
                                                    const int32_t* __restrict__ inv,
                                                    const float* __restrict__ w, void* __restrict__ y,
                                                    int64_t T, int D, int k, int has_shared) {
    const int cg = (D + 3) / 4;
    const int64_t gid = (int64_t)blockIdx.x * NT + threadIdx.x;
    if (gid >= T * cg) return;
    const int64_t t = gid / cg;
    const int c = (int)(gid - t * cg) * 4;
    const int64_t S = T * k;
    const bool vec = (c + 4 <= D) && (D % 4 == 0);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (has_shared) {
        const float* ys = Y + (S + t) * D + c;
        if (vec) {
            const float4 v = *(const float4*)ys;
            acc[0] = v.x; acc[1] = v.y; acc[2] = v.z; acc[3] = v.w;
        } else {
            for (int i = 0; i < 4 && c + i < D; ++i) acc[i] = ys[i];
        }
    }
    for (int j = 0; j < k; ++j) {
        const int32_t p = inv[t * k + j];
        if (p < 0 || p >= S) continue;      // invalid slot (p == -1)
        const float wt = w[t * k + j];
        const float* yr = Y + (int64_t)p * D + c;
        if (vec) {
            const float4 v = *(const float4*)yr;
            acc[0] = fmaf(wt, v.x, acc[0]);
            acc[1] = fmaf(wt, v.y, acc[1]);
            acc[2] = fmaf(wt, v.z, acc[2]);
            acc[3] = fmaf(wt, v.w, acc[3]);
        } else {
            for (int i = 0; i < 4 && c + i < D; ++i) acc[i] = fmaf(wt, yr[i], acc[i]);
        }
    }
    if (BF16) {
        uint16_t* out = (uint16_t*)y + t * D + c;
        if (vec) {
            const uint32_t lo = bf16_rne(acc[0]) | ((uint32_t)bf16_rne(acc[1]) << 16);
            const uint32_t hi = bf16_rne(acc[2]) | ((uint32_t)bf16_rne(acc[3]) << 16);
            *(uint2*)out = make_uint2(lo, hi);
        } else {
            for (int i = 0; i < 4 && c + i < D; ++i) out[i] = bf16_rne(acc[i]);
        }
    } else {
        float* out = (float*)y + t * D + c;
        for (int i = 0; i < 4 && c + i < D; ++i) out[i] = acc[i];
    }
}

}  // namespace

hipError_t launch_combine(const float* Y, const int32_t* inv, const float* w, void* y, int64_t T,
                          int D, int k, bool has_shared, bool out_bf16, hipStream_t s) {
    const int64_t threads = T * ((D + 3) / 4);
    const unsigned blocks = (unsigned)((threads + NT - 1) / NT);
    if (out_bf16)
        combine_kernel<true><<<blocks, NT, 0, s>>>(Y, inv, w, y, T, D, k, has_shared);
    else
        combine_kernel<false><<<blocks, NT, 0, s>>>(Y, inv, w, y, T, D, k, has_shared);
    return hipGetLastError();
}

}  // namespace moe
