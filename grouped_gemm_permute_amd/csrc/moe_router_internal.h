// moe_router_internal.h -- the top-k router and the permute entry it feeds.
// Internal to libmoe_ffn.so.
#pragma once

#include "moe_internal.h"

namespace moe {

// Router limits: experts handled per token in one wavefront, and the
// gate matrix held in LDS as fp32.
constexpr int kRouterMaxExperts = 64;
constexpr int kRouterMaxGateElems = 16384;     // D * E

// Histogram columns the router writes per permute block of
// kPermuteBlockSlots slots (each router workgroup counts the slots of one
// column).
constexpr int kRouterSub = 4;

// logits[t] = x[t] gate_w (fp32 accumulation); topk_idx[t] = the k largest
// logits' experts in descending order (equal logits: lower expert first);
// topk_w[t] = softmax over those k logits (fp32).  With hist != null the
// slots' expert counts go to hist[e * (nb * kRouterSub) + c] for the
// kRouterSub columns of each of the nb permute blocks (requires
// permute_fine_ok(T*k, E, kRouterSub)).  bf16: D % 8 == 0; fp32: D % 4 == 0.
hipError_t launch_router(const void* x, const void* gate_w, int64_t T, int D, int E, int k, bool bf16,
                         int32_t* topk_idx, float* topk_w, int32_t* hist, hipStream_t s);

// Whether the permute of S slots can take a histogram of sub columns per
// block straight into its scan-scatter launch.
bool permute_fine_ok(int64_t S, int E, int sub);

// The permute's scan and scatter from a histogram already in hist (sub
// columns per block), as launch_permute does after its histogram launch.
hipError_t launch_permute_from_hist(const int32_t* idx, int64_t S, int E, int tile_rows,
                                    int64_t shared_rows, int32_t* counts, int32_t* offsets,
                                    int32_t* tile_off, int32_t* perm, int32_t* inv, int32_t* err,
                                    const int32_t* hist, int sub, hipStream_t s, int tile_rows2,
                                    int32_t* tile_off2);

}  // namespace moe
