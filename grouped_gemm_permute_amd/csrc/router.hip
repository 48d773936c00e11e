// router.hip -- top-k routing in front of the permute.
//
// The router of "Chinchilla scaling, MoE, and fused Triton kernels" (section
// "PyTorch MoE implementation"): logits = x gate_w, the k largest logits of
// each token, and routing weights that are the softmax over those k logits.
// Equal logits are taken in ascending expert order (the page leaves ties to
// torch.topk).  Arithmetic is fp32: products of the stored values summed in
// fp32, the softmax in fp32.
//
// When it feeds the permute directly, the kernel also counts each slot's
// expert: workgroup c owns the slots of histogram column c (kRouterSub
// columns per permute block of kPermuteBlockSlots slots), routes the tokens
// those slots belong to and writes the column, so the permute's own
// histogram launch and the [T, E] logits never exist.  A token whose slots
// straddle two columns is routed by both workgroups, with identical
// results.
//
// One wavefront routes one token: lane l accumulates the partial logits of
// all experts over the 8-element chunks l, l + 64, ... of the token's row
// (gate_w is held in LDS as fp32 [E, D]), a reduce-scatter over the 64
// lanes (recursive halving) completes the logits, and the k winners are
// found by k wavefront-wide argmax rounds (larger value, then lower expert).
#include "mfma_common.h"
#include "moe_router_internal.h"

#include <math.h>

namespace moe {
namespace {

constexpr int RT = 1024;                    // 16 wavefronts: many tokens in flight per CU
constexpr int TOKENS_PER_WG = 64;           // without a histogram

__device__ __forceinline__ float bf16_at(const uint16_t* p, int64_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);
}

template <bool BF16, int EMAX>
__global__ __launch_bounds__(RT) void router_kernel(const void* __restrict__ xv,
                                                   const void* __restrict__ gv, int64_t T, int D,
                                                   int E, int k, int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w,
                                                   int32_t* __restrict__ hist, int ncols,
                                                   int64_t slots_per_col) {
    __shared__ __attribute__((aligned(16))) float gw[kRouterMaxGateElems];
    __shared__ int32_t cnt[kRouterMaxExperts + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // gw[e * D + d] = gate_w[d][e]: lanes reading consecutive d of one
    // expert touch consecutive banks
    for (int i = tid; i < D * E; i += RT) {
        const int d = i / E, e = i - d * E;
        gw[e * D + d] = BF16 ? bf16_at((const uint16_t*)gv, i) : ((const float*)gv)[i];
    }
    for (int e = tid; e <= E; e += RT) cnt[e] = 0;
    __syncthreads();

    const int64_t S = T * k;
    int64_t s_lo = 0, s_hi = 0, t0, t1;
    if (hist) {
        s_lo = (int64_t)blockIdx.x * slots_per_col;
        s_hi = min(S, s_lo + slots_per_col);
        t0 = s_lo / k;
        t1 = s_hi > s_lo ? (s_hi + k - 1) / k : t0;
    } else {
        t0 = (int64_t)blockIdx.x * TOKENS_PER_WG;
        t1 = min(T, t0 + TOKENS_PER_WG);
    }
    const int nch = D / 8;
    for (int64_t t = t0 + wave; t < t1; t += RT / 64) {
        float acc[EMAX];
#pragma unroll
        for (int e = 0; e < EMAX; ++e) acc[e] = 0.f;
        for (int c = lane; c < nch; c += 64) {
            float xs[8];
            if (BF16) {
                const uint4 q = *(const uint4*)((const uint16_t*)xv + t * D + 8 * c);
                const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    xs[2 * i] = __uint_as_float(w[i] << 16);
                    xs[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
                }
            } else {
                const float4 a = *(const float4*)((const float*)xv + t * D + 8 * c);
                const float4 b = *(const float4*)((const float*)xv + t * D + 8 * c + 4);
                xs[0] = a.x; xs[1] = a.y; xs[2] = a.z; xs[3] = a.w;
                xs[4] = b.x; xs[5] = b.y; xs[6] = b.z; xs[7] = b.w;
            }
#pragma unroll
            for (int e = 0; e < EMAX; ++e) {
                if (e >= E) break;
                const float4 g0 = *(const float4*)(gw + e * D + 8 * c);
                const float4 g1 = *(const float4*)(gw + e * D + 8 * c + 4);
                float a = acc[e];
                a = fmaf(xs[0], g0.x, a); a = fmaf(xs[1], g0.y, a);
                a = fmaf(xs[2], g0.z, a); a = fmaf(xs[3], g0.w, a);
                a = fmaf(xs[4], g1.x, a); a = fmaf(xs[5], g1.y, a);
                a = fmaf(xs[6], g1.z, a); a = fmaf(xs[7], g1.w, a);
                acc[e] = a;
            }
        }
        // Complete the logits by recursive halving: at each of the first
        // log2(EMAX) steps a lane keeps the half of its experts selected by
        // one lane-index bit and adds the partner's copy of that half, then
        // plain butterfly steps finish the sum.  Lane l ends with the logit
        // of expert my_e (every lane of the same expert holds the same sum).
        constexpr int LOGE = EMAX == 8 ? 3 : EMAX == 16 ? 4 : EMAX == 32 ? 5 : 6;
        int my_e = 0;
#pragma unroll
        for (int st = 0; st < LOGE; ++st) {
            const int off = 32 >> st;
            const int half = EMAX >> (st + 1);            // experts kept after this step
            const bool upper = (lane & off) != 0;
#pragma unroll
            for (int i = 0; i < half; ++i) {
                const float lo = acc[i], hi = acc[i + half];
                const float send = upper ? lo : hi;       // the half the partner keeps
                const float keep = upper ? hi : lo;
                acc[i] = keep + __shfl_xor(send, off);
            }
            my_e += upper ? half : 0;
        }
        float v = acc[0];
#pragma unroll
        for (int off = 32 >> LOGE; off > 0; off >>= 1) v += __shfl_xor(v, off);
        float mine = my_e < E ? v : -INFINITY;
        // k argmax rounds: lane j keeps the j-th winner
        int my_sel = -1;
        float my_val = 0.f, top = 0.f;
        for (int j = 0; j < k; ++j) {
            float bv = mine;
            int bi = my_e < E ? my_e : 0x7fffffff;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                const float ov = __shfl_xor(bv, off);
                const int oi = __shfl_xor(bi, off);
                if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
            }
            if (j == 0) top = bv;
            if (lane == j) { my_sel = bi; my_val = bv; }
            if (my_e == bi) mine = -INFINITY;
        }
        // softmax over the k selected logits
        const float ex = lane < k ? expf(my_val - top) : 0.f;
        float sum = ex;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
        if (lane < k) {
            topk_idx[t * k + lane] = my_sel;
            topk_w[t * k + lane] = ex / sum;
            const int64_t s = t * k + lane;
            if (hist && s >= s_lo && s < s_hi) atomicAdd(&cnt[my_sel], 1);
        }
    }
    if (hist) {
        __syncthreads();
        for (int e = tid; e <= E; e += RT) hist[(int64_t)e * ncols + blockIdx.x] = cnt[e];
    }
}

// bf16 path on MFMA.  A wavefront takes 32 tokens: the MFMA's A operand is
// 32 token rows x 16 features (lane l: token l%32, features 8 (l/32) .. +7 of
// the step, read straight from x), its B operand 16 features x 32 experts
// from the gate matrix staged in LDS as bf16 [32 experts, D] (rows padded
// by 16 bytes against bank conflicts).  Rows E .. 31 are left as they are:
// they only feed the logit columns of experts E .. 31, which are never read
// (zeroing them cost 4.5 us of the 24 us kernel on 32768 tokens).  The 32 x 32
// fp32 logits go through LDS so that lane j < 32 holds token j's logits and
// selects its k experts serially.
constexpr int MT = 256;                            // 4 wavefronts
constexpr int MAX_D_MFMA = 2048;

template <int EMAX>
__global__ __launch_bounds__(MT) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ gate, int64_t T,
                                                        int D, int E, int k,
                                                        int32_t* __restrict__ topk_idx,
                                                        float* __restrict__ topk_w,
                                                        int32_t* __restrict__ hist, int ncols,
                                                        int64_t slots_per_col) {
    using namespace mfma;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int rowb = 2 * D + 16;                       // bytes per staged expert row
    char* gw = smem;                                   // [32][rowb]
    float* lg = (float*)(smem + 32 * rowb);            // [4 waves][32 tokens][33]
    int32_t* cnt = (int32_t*)(lg + 4 * 32 * 33);       // [E + 1]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t S = T * k;
    int64_t s_lo = 0, s_hi = 0, t0, t1;
    if (hist) {
        s_lo = (int64_t)blockIdx.x * slots_per_col;
        s_hi = min(S, s_lo + slots_per_col);
        t0 = s_lo / k;
        t1 = s_hi > s_lo ? (s_hi + k - 1) / k : t0;
    } else {
        t0 = (int64_t)blockIdx.x * 128;
        t1 = min(T, t0 + 128);
    }
    // The first 256 features of this wavefront's first token block do not
    // depend on the gate matrix: their loads go out before it is staged.
    u32x4_t pre[16];
    const bool has_pre = t0 + 32 * wave < t1 && D >= 256;
    if (has_pre) {
        const int64_t tr = min(t0 + 32 * wave + (lane & 31), T - 1);
        const uint16_t* xr = x + tr * D + 8 * (lane >> 5);
#pragma unroll
        for (int i = 0; i < 16; ++i) pre[i] = *(const u32x4_t*)(xr + 16 * i);
    }
    // stage: 16-byte loads of gate [D, E] (D * E is a multiple of 16),
    // each element stored to its expert row
    for (int i = tid; i < D * E / 8; i += MT) {
        const uint4 q = *(const uint4*)(gate + 8 * (int64_t)i);
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int f = 8 * i + j, d = f / E, e = f - d * E;
            *(uint16_t*)(gw + e * rowb + 2 * d) = (uint16_t)(j & 1 ? w[j >> 1] >> 16 : w[j >> 1] & 0xffff);
        }
    }
    for (int e = tid; e <= E; e += MT) cnt[e] = 0;
    __syncthreads();

    float* mylg = lg + wave * 32 * 33;
    for (int64_t tb = t0 + 32 * wave; tb < t1; tb += 128) {
        const int64_t tr = min(tb + (lane & 31), T - 1);
        const uint16_t* xr = x + tr * D + 8 * (lane >> 5);
        const char* gr = gw + (lane & 31) * rowb + 16 * (lane >> 5);
        f32x16_t acc = {};
        int k0 = 0;
        // 16 steps at a time: all 16 row loads in flight before the MFMAs
        for (; k0 + 256 <= D; k0 += 256) {
            u32x4_t a[16];
            const bool first = has_pre && k0 == 0 && tb == t0 + 32 * wave;
#pragma unroll
            for (int i = 0; i < 16; ++i) a[i] = first ? pre[i] : *(const u32x4_t*)(xr + k0 + 16 * i);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8_t, a[i]),
                    __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(gr + 2 * (k0 + 16 * i))), acc, 0, 0, 0);
        }
        for (; k0 < D; k0 += 16) {
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(xr + k0));
            const bf16x8_t b = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(gr + 2 * k0));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
        }
        // acc element v of lane l: token 8 (v/4) + 4 (l/32) + v%4, expert l%32
#pragma unroll
        for (int v = 0; v < 16; ++v)
            mylg[(8 * (v >> 2) + 4 * (lane >> 5) + (v & 3)) * 33 + (lane & 31)] = acc[v];
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));   // this wavefront's LDS writes done
        __builtin_amdgcn_wave_barrier();
        if (lane < 32 && tb + lane < t1) {
            const int64_t t = tb + lane;
            float l[EMAX];
#pragma unroll
            for (int e = 0; e < EMAX; ++e) l[e] = e < E ? mylg[lane * 33 + e] : -INFINITY;
            float top = 0.f, sum = 0.f;
            int sel[EMAX];
            float val[EMAX];
            for (int j = 0; j < k; ++j) {
                float bv = -INFINITY;
                int bi = 0;
#pragma unroll
                for (int e = 0; e < EMAX; ++e)
                    if (l[e] > bv) { bv = l[e]; bi = e; }    // first maximum: lower expert on ties
#pragma unroll
                for (int e = 0; e < EMAX; ++e)
                    if (e == bi) l[e] = -INFINITY;
#pragma unroll
                for (int jj = 0; jj < EMAX; ++jj)
                    if (jj == j) { sel[jj] = bi; val[jj] = bv; }
                if (j == 0) top = bv;
            }
#pragma unroll
            for (int jj = 0; jj < EMAX; ++jj)
                if (jj < k) sum += expf(val[jj] - top);
#pragma unroll
            for (int jj = 0; jj < EMAX; ++jj) {
                if (jj >= k) break;
                topk_idx[t * k + jj] = sel[jj];
                topk_w[t * k + jj] = expf(val[jj] - top) / sum;
                const int64_t s = t * k + jj;
                if (hist && s >= s_lo && s < s_hi) atomicAdd(&cnt[sel[jj]], 1);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    if (hist) {
        __syncthreads();
        for (int e = tid; e <= E; e += MT) hist[(int64_t)e * ncols + blockIdx.x] = cnt[e];
    }
}

template <bool BF16>
hipError_t launch_t(const void* x, const void* gw, int64_t T, int D, int E, int k, int32_t* idx,
                    float* w, int32_t* hist, dim3 grid, int ncols, int64_t spc, hipStream_t s) {
    if (E <= 8)
        router_kernel<BF16, 8><<<grid, RT, 0, s>>>(x, gw, T, D, E, k, idx, w, hist, ncols, spc);
    else if (E <= 16)
        router_kernel<BF16, 16><<<grid, RT, 0, s>>>(x, gw, T, D, E, k, idx, w, hist, ncols, spc);
    else if (E <= 32)
        router_kernel<BF16, 32><<<grid, RT, 0, s>>>(x, gw, T, D, E, k, idx, w, hist, ncols, spc);
    else
        router_kernel<BF16, 64><<<grid, RT, 0, s>>>(x, gw, T, D, E, k, idx, w, hist, ncols, spc);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const void* x, const void* gate_w, int64_t T, int D, int E, int k, bool bf16,
                         int32_t* topk_idx, float* topk_w, int32_t* hist, hipStream_t s) {
    if (E < 1 || E > kRouterMaxExperts || D % 8 || D * E > kRouterMaxGateElems || k < 1 || k > E)
        return hipErrorInvalidValue;
    if (T == 0) return hipSuccess;
    int ncols = 0;
    int64_t spc = 0;
    dim3 grid;
    if (hist) {
        ncols = permute_hist_blocks(T * k) * kRouterSub;
        spc = kPermuteBlockSlots / kRouterSub;
        grid = dim3((unsigned)ncols);
    } else {
        grid = dim3((unsigned)((T + TOKENS_PER_WG - 1) / TOKENS_PER_WG));
    }
    if (bf16 && E <= 32 && D % 16 == 0 && D <= MAX_D_MFMA) {
        if (!hist) grid = dim3((unsigned)((T + 127) / 128));
        const size_t lds = 32 * (size_t)(2 * D + 16) + 4 * 32 * 33 * 4 + 4 * (size_t)(E + 1);
        const uint16_t* xb = (const uint16_t*)x;
        const uint16_t* gb = (const uint16_t*)gate_w;
        if (E <= 8)
            router_mfma_kernel<8><<<grid, MT, lds, s>>>(xb, gb, T, D, E, k, topk_idx, topk_w, hist, ncols, spc);
        else if (E <= 16)
            router_mfma_kernel<16><<<grid, MT, lds, s>>>(xb, gb, T, D, E, k, topk_idx, topk_w, hist, ncols, spc);
        else
            router_mfma_kernel<32><<<grid, MT, lds, s>>>(xb, gb, T, D, E, k, topk_idx, topk_w, hist, ncols, spc);
        return hipGetLastError();
    }
    return bf16 ? launch_t<true>(x, gate_w, T, D, E, k, topk_idx, topk_w, hist, grid, ncols, spc, s)
                : launch_t<false>(x, gate_w, T, D, E, k, topk_idx, topk_w, hist, grid, ncols, spc, s);
}

}  // namespace moe
