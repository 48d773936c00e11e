// combine.hip -- unpermute and weighted combine.
//
//   y[t] = Y[S + t] + sum_{j=0}^{k-1} topk_w[t, j] * Y[inv[t*k + j]]
//
// where Y holds every row's expert output (the down GEMM's result) and row
// S + t is the shared expert's output for token t (absent without a shared
// expert, weight 1).
// "Chinchilla scaling, MoE, and fused Triton kernels" (section "PyTorch MoE
// implementation") gathers each token's k expert rows through the inverse
// permutation and sums them weighted; "Triton MoE Kernels & Memory
// Checkpointing" (Part A, section 10.3 step 4) scales by the routing weight
// after W2 and adds the result back into the token's row.  Here each term
// is scaled and added in fp32 (one fused multiply-add per term) in j order,
// starting from the shared row (or 0), and rounded once to the output
// type, so the result does not depend on scheduling (no scatter atomics).
// Slots with inv = -1 (invalid ids) add nothing.  topk_w == nullptr means
// weight 1 on every slot (the backward's gather of dx rows).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int NT = 256;
constexpr int KPRE = 4;   // top-k up to this many: all loads issued up front

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// bf16: one thread per (token, 8 consecutive columns); D % 8 == 0 (the bf16
// path requires D % 64 == 0), all accesses 16 bytes.
__global__ __launch_bounds__(NT) void combine_bf16_kernel(const uint16_t* __restrict__ Y,
                                                         const int32_t* __restrict__ inv,
                                                         const float* __restrict__ topk_w,
                                                         uint16_t* __restrict__ y, int64_t T, int D,
                                                         int k, int has_shared) {
    const int cg = D / 8;
    const int64_t gid = (int64_t)blockIdx.x * NT + threadIdx.x;
    if (gid >= T * cg) return;
    const int64_t t = gid / cg;
    const int c = (int)(gid - t * cg) * 8;
    const int64_t S = T * k;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto add4 = [&](const uint4 v, float wt) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = fmaf(wt, bf16_lo(w[i]), acc[2 * i]);
            acc[2 * i + 1] = fmaf(wt, bf16_hi(w[i]), acc[2 * i + 1]);
        }
    };
    auto add = [&](const uint16_t* src, float wt) { add4(*(const uint4*)src, wt); };
    if (k <= KPRE) {
        // every slot's row index and weight first, then every row, all in
        // flight at once; the sum runs in the same order as below
        int32_t p[KPRE];
        float wt[KPRE];
#pragma unroll
        for (int j = 0; j < KPRE; ++j) {
            p[j] = j < k ? inv[t * k + j] : -1;
            wt[j] = j < k && topk_w ? topk_w[t * k + j] : 1.f;
        }
        uint4 v[KPRE];
        const uint4 vs = has_shared ? *(const uint4*)(Y + (S + t) * D + c) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < KPRE; ++j) {
            const bool ok = p[j] >= 0 && p[j] < S;      // invalid slot (p == -1) adds nothing
            v[j] = ok ? *(const uint4*)(Y + (int64_t)p[j] * D + c) : make_uint4(0, 0, 0, 0);
        }
        if (has_shared) add4(vs, 1.f);
#pragma unroll
        for (int j = 0; j < KPRE; ++j)
            if (p[j] >= 0 && p[j] < S) add4(v[j], wt[j]);
    } else {
        if (has_shared) add(Y + (S + t) * D + c, 1.f);
        for (int j = 0; j < k; ++j) {
            const int32_t p = inv[t * k + j];
            if (p < 0 || p >= S) continue;      // invalid slot (p == -1)
            add(Y + (int64_t)p * D + c, topk_w ? topk_w[t * k + j] : 1.f);
        }
    }
    *(uint4*)(y + t * D + c) = make_uint4(pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]),
                                          pack_bf16(acc[4], acc[5]), pack_bf16(acc[6], acc[7]));
}

// fp32: one thread per (token, column).
__global__ __launch_bounds__(NT) void combine_f32_kernel(const float* __restrict__ Y,
                                                        const int32_t* __restrict__ inv,
                                                        const float* __restrict__ topk_w,
                                                        float* __restrict__ y, int64_t T, int D,
                                                        int k, int has_shared) {
    const int64_t gid = (int64_t)blockIdx.x * NT + threadIdx.x;
    if (gid >= T * D) return;
    const int64_t t = gid / D;
    const int c = (int)(gid - t * D);
    const int64_t S = T * k;
    float acc = has_shared ? Y[(S + t) * D + c] : 0.f;
    for (int j = 0; j < k; ++j) {
        const int32_t p = inv[t * k + j];
        if (p < 0 || p >= S) continue;
        acc = fmaf(topk_w ? topk_w[t * k + j] : 1.f, Y[(int64_t)p * D + c], acc);
    }
    y[t * D + c] = acc;
}

}  // namespace

hipError_t launch_combine(const void* Y, const int32_t* inv, const float* topk_w, void* y,
                          int64_t T, int D, int k, bool has_shared, bool bf16, hipStream_t s) {
    if (bf16) {
        const int64_t threads = T * (D / 8);
        combine_bf16_kernel<<<(unsigned)((threads + NT - 1) / NT), NT, 0, s>>>(
            (const uint16_t*)Y, inv, topk_w, (uint16_t*)y, T, D, k, has_shared);
    } else {
        const int64_t threads = T * D;
        combine_f32_kernel<<<(unsigned)((threads + NT - 1) / NT), NT, 0, s>>>(
            (const float*)Y, inv, topk_w, (float*)y, T, D, k, has_shared);
    }
    return hipGetLastError();
}

}  // namespace moe
