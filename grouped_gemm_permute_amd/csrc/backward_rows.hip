// backward_rows.hip -- the backward pass of the routed SwiGLU MoE layer as
// plain kernels: one thread per output element, fp32 accumulation, for both
// storage types (fp32, and bf16 with fp32 arithmetic).  Their reduction
// loops are unrolled so that a thread's loads go out together (the FMA
// order, and so every result, is that of the plain loop).
//
// The vector-Jacobian product follows the autograd contract of "Triton MoE
// Kernels & Memory Checkpointing" (Part A, section 8): the gate and up
// products are recomputed from x rather than saved, their gradients are the
// upstream gradient times the derivative of silu(g) * u, and the weight
// gradients are outer products of those gradients with the layer inputs;
// the W2 stage and the routing weights follow from the same chain rule on
// the down projection and the weighted combine of the same page's section
// 10.3.  Per sorted row p (expert grp, token tok(p), routing weight w; w = 1
// on shared rows):
//
//   gate_up:  g, u = x[tok] W1[grp], x[tok] W3[grp]
//   dh:       dh' = dy[tok] W2[grp]^T,  h = silu(g) u,  partial dy.o = dh' . h,
//             dh = w dh',  dg = dh u silu'(g),  du = dh silu(g),  hw = w h
//   dx_rows:  dxr[p] = dg W1[grp]^T + du W3[grp]^T
//   dw13:     [dW1 | dW3][grp] = sum_p x[tok(p)]^T [dg | du][p]
//   dw2:      dW2[grp] = sum_p hw[p]^T dy[tok(p)]
//   dtopk:    dtopk_w[slot] = sum of the partial dy.o of the slot's row
//
// and dx[t] is the unweighted combine of dxr over the token's rows.
// silu'(z) = s (1 + z (1 - s)) with s = 1 / (1 + e^-z).
#include "moe_bwd_internal.h"

namespace moe {
namespace {

constexpr int NT = 128;

template <typename T> __device__ __forceinline__ float ld(const T* p, int64_t i);
template <> __device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);
}
template <typename T> __device__ __forceinline__ void st(T* p, int64_t i, float v);
template <> __device__ __forceinline__ void st<float>(float* p, int64_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void st<uint16_t>(uint16_t* p, int64_t i, float v) {
    p[i] = __builtin_bit_cast(uint16_t, (__bf16)v);      // round to nearest even
}

// Group of row p (E for shared rows), or -1 for a row left unused by
// invalid ids.
__device__ __forceinline__ int group_of(const GroupArgs& g, int64_t p) {
    if (p >= g.S) return g.E;
    if (p >= g.offsets[g.E]) return -1;
    int lo = 0, hi = g.E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (g.offsets[mid] <= p) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ int64_t token_of(const GroupArgs& g, int grp, int64_t p) {
    return grp == g.E ? p - g.S : (int64_t)(g.perm[p] / g.k);
}

template <typename T>
__global__ __launch_bounds__(NT) void gate_up_kernel(BwdArgs a, const T* __restrict__ x,
                                                     const T* __restrict__ W1, const T* __restrict__ W3,
                                                     const T* __restrict__ Ws1, const T* __restrict__ Ws3,
                                                     T* __restrict__ gu) {
    const int64_t p = blockIdx.x;
    const int f = blockIdx.y * NT + threadIdx.x;
    const int D = a.D, F = a.F;
    if (f >= F) return;
    const int grp = group_of(a.g, p);
    if (grp < 0) return;
    const bool sh = grp == a.g.E;
    const T* w1 = sh ? Ws1 : W1 + (int64_t)grp * D * F;
    const T* w3 = sh ? Ws3 : W3 + (int64_t)grp * D * F;
    const int64_t xo = token_of(a.g, grp, p) * D;
    float g = 0.f, u = 0.f;
#pragma unroll 16
    for (int d = 0; d < D; ++d) {
        const float xv = ld(x, xo + d);
        g = fmaf(xv, ld(w1, (int64_t)d * F + f), g);
        u = fmaf(xv, ld(w3, (int64_t)d * F + f), u);
    }
    st(gu, p * 2 * F + f, g);
    st(gu, p * 2 * F + F + f, u);
}

// One wavefront per (row, block of kBwdDwBlock columns).
template <typename T>
__global__ __launch_bounds__(kBwdDwBlock) void dh_kernel(BwdArgs a, const T* __restrict__ dy,
                                                         const T* __restrict__ W2,
                                                         const T* __restrict__ Ws2,
                                                         const T* __restrict__ gu,
                                                         T* __restrict__ dgu, T* __restrict__ hw,
                                                         float* __restrict__ dwpart) {
    const int64_t p = blockIdx.x;
    const int f = blockIdx.y * kBwdDwBlock + threadIdx.x;
    const int D = a.D, F = a.F;
    const int grp = group_of(a.g, p);
    if (grp < 0) return;                        // uniform over the block (one row)
    const bool sh = grp == a.g.E;
    const bool valid = f < F;
    const T* w2 = sh ? Ws2 : W2 + (int64_t)grp * F * D;
    const int64_t yo = token_of(a.g, grp, p) * D;
    float dhp = 0.f;
    if (valid)
#pragma unroll 16
        for (int d = 0; d < D; ++d) dhp = fmaf(ld(dy, yo + d), ld(w2, (int64_t)f * D + d), dhp);
    const float w = sh ? 1.f : a.topk_w[a.g.perm[p]];
    float prod = 0.f;
    if (valid) {
        const float g = ld(gu, p * 2 * F + f), u = ld(gu, p * 2 * F + F + f);
        const float s = 1.f / (1.f + expf(-g));
        const float act = g * s;
        const float h = act * u;
        prod = dhp * h;
        const float dh = w * dhp;
        st(dgu, p * 2 * F + f, dh * u * (s * (1.f + g * (1.f - s))));
        st(dgu, p * 2 * F + F + f, dh * act);
        st(hw, p * F + f, w * h);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) prod += __shfl_xor(prod, off);
    if (threadIdx.x == 0) dwpart[p * gridDim.y + blockIdx.y] = prod;
}

template <typename T>
__global__ __launch_bounds__(NT) void dx_rows_kernel(BwdArgs a, const T* __restrict__ dgu,
                                                     const T* __restrict__ W1, const T* __restrict__ W3,
                                                     const T* __restrict__ Ws1, const T* __restrict__ Ws3,
                                                     T* __restrict__ dxr) {
    const int64_t p = blockIdx.x;
    const int d = blockIdx.y * NT + threadIdx.x;
    const int D = a.D, F = a.F;
    if (d >= D) return;
    const int grp = group_of(a.g, p);
    if (grp < 0) return;
    const bool sh = grp == a.g.E;
    const T* w1 = (sh ? Ws1 : W1 + (int64_t)grp * D * F) + (int64_t)d * F;
    const T* w3 = (sh ? Ws3 : W3 + (int64_t)grp * D * F) + (int64_t)d * F;
    const int64_t ro = p * 2 * F;
    float acc = 0.f;
#pragma unroll 16
    for (int f = 0; f < F; ++f) acc = fmaf(ld(dgu, ro + f), ld(w1, f), acc);
#pragma unroll 16
    for (int f = 0; f < F; ++f) acc = fmaf(ld(dgu, ro + F + f), ld(w3, f), acc);
    st(dxr, p * D + d, acc);
}

// Rows [p0, p1) of group grp.
__device__ __forceinline__ void group_rows(const GroupArgs& g, int grp, int64_t& p0, int64_t& p1) {
    if (grp == g.E) { p0 = g.S; p1 = g.S + g.T; }
    else { p0 = g.offsets[grp]; p1 = g.offsets[grp + 1]; }
}

template <typename T>
__global__ __launch_bounds__(NT) void dw13_kernel(BwdArgs a, const T* __restrict__ x,
                                                  const T* __restrict__ dgu, float* __restrict__ dW1,
                                                  float* __restrict__ dW3, float* __restrict__ dWs1,
                                                  float* __restrict__ dWs3) {
    const int grp = blockIdx.y;
    const int D = a.D, F = a.F;
    const int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
    if (i >= (int64_t)D * 2 * F) return;
    const int d = (int)(i / (2 * F)), c = (int)(i - (int64_t)d * 2 * F);
    int64_t p0, p1;
    group_rows(a.g, grp, p0, p1);
    float acc = 0.f;
#pragma unroll 8
    for (int64_t p = p0; p < p1; ++p)
        acc = fmaf(ld(x, token_of(a.g, grp, p) * D + d), ld(dgu, p * 2 * F + c), acc);
    const bool sh = grp == a.g.E;
    if (c < F) (sh ? dWs1 : dW1 + (int64_t)grp * D * F)[(int64_t)d * F + c] = acc;
    else (sh ? dWs3 : dW3 + (int64_t)grp * D * F)[(int64_t)d * F + c - F] = acc;
}

template <typename T>
__global__ __launch_bounds__(NT) void dw2_kernel(BwdArgs a, const T* __restrict__ hw,
                                                 const T* __restrict__ dy, float* __restrict__ dW2,
                                                 float* __restrict__ dWs2) {
    const int grp = blockIdx.y;
    const int D = a.D, F = a.F;
    const int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
    if (i >= (int64_t)F * D) return;
    const int f = (int)(i / D), d = (int)(i - (int64_t)f * D);
    int64_t p0, p1;
    group_rows(a.g, grp, p0, p1);
    float acc = 0.f;
#pragma unroll 8
    for (int64_t p = p0; p < p1; ++p)
        acc = fmaf(ld(hw, p * F + f), ld(dy, token_of(a.g, grp, p) * D + d), acc);
    (grp == a.g.E ? dWs2 : dW2 + (int64_t)grp * F * D)[i] = acc;
}

__global__ __launch_bounds__(NT) void dtopk_kernel(int64_t S, int nb, const int32_t* __restrict__ inv,
                                                   const float* __restrict__ dwpart,
                                                   float* __restrict__ dtopk_w) {
    const int64_t s = (int64_t)blockIdx.x * NT + threadIdx.x;
    if (s >= S) return;
    const int32_t p = inv[s];
    float acc = 0.f;
    if (p >= 0 && p < S)
        for (int b = 0; b < nb; ++b) acc += dwpart[(int64_t)p * nb + b];
    dtopk_w[s] = acc;
}

int64_t rows(const GroupArgs& g) { return g.S + (g.G > g.E ? g.T : 0); }

}  // namespace

#define MOE_BWD_DISPATCH(a, ...)                                               \
    do {                                                                       \
        if ((a).bf16) { using T = uint16_t; __VA_ARGS__; }                     \
        else { using T = float; __VA_ARGS__; }                                 \
    } while (0)

hipError_t launch_bwd_gate_up(const BwdArgs& a, const void* x, const void* W1, const void* W3,
                              const void* Ws1, const void* Ws3, void* gu, hipStream_t s) {
    const dim3 grid((unsigned)rows(a.g), (unsigned)((a.F + NT - 1) / NT));
    MOE_BWD_DISPATCH(a, gate_up_kernel<T><<<grid, NT, 0, s>>>(a, (const T*)x, (const T*)W1,
                                                              (const T*)W3, (const T*)Ws1,
                                                              (const T*)Ws3, (T*)gu));
    return hipGetLastError();
}

hipError_t launch_bwd_dh(const BwdArgs& a, const void* dy, const void* W2, const void* Ws2,
                         const void* gu, void* dgu, void* hw, float* dwpart, hipStream_t s) {
    const dim3 grid((unsigned)rows(a.g), (unsigned)bwd_dw_blocks(a.F));
    MOE_BWD_DISPATCH(a, dh_kernel<T><<<grid, kBwdDwBlock, 0, s>>>(a, (const T*)dy, (const T*)W2,
                                                                  (const T*)Ws2, (const T*)gu,
                                                                  (T*)dgu, (T*)hw, dwpart));
    return hipGetLastError();
}

hipError_t launch_bwd_dx_rows(const BwdArgs& a, const void* dgu, const void* W1, const void* W3,
                              const void* Ws1, const void* Ws3, void* dxr, hipStream_t s) {
    const dim3 grid((unsigned)rows(a.g), (unsigned)((a.D + NT - 1) / NT));
    MOE_BWD_DISPATCH(a, dx_rows_kernel<T><<<grid, NT, 0, s>>>(a, (const T*)dgu, (const T*)W1,
                                                              (const T*)W3, (const T*)Ws1,
                                                              (const T*)Ws3, (T*)dxr));
    return hipGetLastError();
}

hipError_t launch_bwd_dw13(const BwdArgs& a, const void* x, const void* dgu, float* dW1,
                           float* dW3, float* dWs1, float* dWs3, hipStream_t s) {
    const dim3 grid((unsigned)(((int64_t)a.D * 2 * a.F + NT - 1) / NT), (unsigned)a.g.G);
    MOE_BWD_DISPATCH(a, dw13_kernel<T><<<grid, NT, 0, s>>>(a, (const T*)x, (const T*)dgu, dW1, dW3,
                                                           dWs1, dWs3));
    return hipGetLastError();
}

hipError_t launch_bwd_dw2(const BwdArgs& a, const void* hw, const void* dy, float* dW2,
                          float* dWs2, hipStream_t s) {
    const dim3 grid((unsigned)(((int64_t)a.F * a.D + NT - 1) / NT), (unsigned)a.g.G);
    MOE_BWD_DISPATCH(a, dw2_kernel<T><<<grid, NT, 0, s>>>(a, (const T*)hw, (const T*)dy, dW2, dWs2));
    return hipGetLastError();
}

hipError_t launch_bwd_dtopk(const BwdArgs& a, const int32_t* inv, const float* dwpart,
                            float* dtopk_w, hipStream_t s) {
    const int64_t S = a.g.S;
    if (S == 0) return hipSuccess;
    dtopk_kernel<<<(unsigned)((S + NT - 1) / NT), NT, 0, s>>>(S, bwd_dw_blocks(a.F), inv, dwpart,
                                                             dtopk_w);
    return hipGetLastError();
}

}  // namespace moe
