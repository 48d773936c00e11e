/*
 * moe_ffn.h -- C ABI of the MI355X (gfx950) top-k routed mixture-of-experts
 * SwiGLU feed-forward forward pass.
 *
 * The layer (one token t, k routed choices, optional always-on shared expert):
 *
 *   SwiGLU_e(v) = (silu(v . W1[e]) * (v . W3[e])) . W2[e],   silu(z) = z / (1 + exp(-z))
 *   y[t] = [shared] SwiGLU_sh(x[t]) + sum_{j=0}^{k-1} topk_w[t,j] * SwiGLU_{topk_idx[t,j]}(x[t])
 *
 * The expert is the SwiGLU block W2(silu(W1 x) * W3 x) with top-2-of-8
 * routing plus a shared expert ("Triton MoE Kernels & Memory
 * Checkpointing", Part A section 2); tokens are grouped by expert through a
 * stable sort of the flattened (token, choice) slots with per-expert counts
 * and start offsets (same page, section 10.3; "Chinchilla scaling, MoE, and
 * fused Triton kernels", section "PyTorch MoE implementation"), the experts
 * run as grouped matrix products, and the outputs are unpermuted and summed
 * with the routing weights (both pages, same sections).
 *
 * Conventions shared by every entry point:
 *  - The caller owns every buffer.  All data pointers are device pointers
 *    (HIP device memory of the current device); the library never allocates
 *    or frees memory.
 *  - Tensors are dense, row-major, with no padding between rows.
 *  - Work is enqueued on `stream` in order and returns without waiting for
 *    the device (no host synchronisation), except moe_ffn_get_device_error.
 *  - Argument errors are detected on the host before anything is enqueued;
 *    in that case nothing is launched and the outputs are untouched.
 *  - The library never falls back to a different algorithm or precision: a
 *    shape or variant it does not implement returns MOE_ERR_UNSUPPORTED.
 *  - Expert ids outside [0, E) are detected on the device: such a slot takes
 *    no sorted position (inv = -1), contributes nothing to y, and is counted
 *    in a flag that moe_ffn_get_device_error reads back.
 *  - Calls that share a workspace must not overlap in time (same stream, or
 *    ordered by events).
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size, k > E, unknown enum */
    MOE_ERR_UNSUPPORTED = 2,   /* valid but not implemented (e.g. D % 64 != 0 for bf16) */
    MOE_ERR_WORKSPACE = 3,     /* ws_bytes smaller than moe_ffn_workspace_size() */
    MOE_ERR_HIP = 4            /* a HIP launch or copy reported an error */
} moe_status;

typedef enum moe_dtype {
    MOE_F32 = 0,               /* x, weights, y in fp32; fp32 arithmetic throughout */
    MOE_BF16 = 1               /* x, weights, y in bf16; fp32 accumulation, h stored as bf16 */
} moe_dtype;

typedef enum moe_variant {
    MOE_VARIANT_UNFUSED = 0,   /* permute -> up+SwiGLU GEMM -> down GEMM -> combine */
    MOE_VARIANT_FUSED = 1      /* permute -> fused up-act-down (h kept on chip) -> combine;
                                  bf16 only, D % 128 == 0, D <= 1024, F % 128 == 0 */
} moe_variant;

/* Byte offsets of the pieces of a forward workspace (all 256-byte aligned).
 * Row space: R = T*k + (has_shared ? T : 0); sorted routed rows come first,
 * shared-expert row of token t is row T*k + t. */
typedef struct moe_ws_layout {
    size_t total;       /* bytes the workspace must hold */
    size_t err;         /* int32: number of slots with an out-of-range expert id (always 0) */
    size_t counts;      /* int32 [E] rows per expert */
    size_t offsets;     /* int32 [E+1] exclusive prefix sum of counts */
    size_t tile_off;    /* int32 [E+2] prefix sum of ceil(rows/tile_rows), shared group last */
    size_t tile_off64;  /* int32 [E+2] the same prefix for 64-row tiles (small-chunk down GEMM) */
    size_t perm;        /* int32 [T*k] sorted position -> slot t*k+j (-1 past the valid rows) */
    size_t inv;         /* int32 [T*k] slot -> sorted position (-1 for an invalid slot) */
    size_t hist;        /* int32 scratch of the multi-block permute */
    size_t h;           /* unfused: [R, F] silu(g)*u, dtype of the call.  fused: fp32
                           partial outputs [units][64][D] of the workgroups that share
                           out the tiles of the last, partial round of 256 (units <= 256) */
    size_t Y;           /* [R, D] per-row expert outputs (unweighted), dtype of the call */
    int32_t tile_rows;  /* row-tile height of the grouped GEMMs (tile_off's divisor) */
    int32_t hist_blocks;/* number of slot blocks of the multi-block permute (0: single block) */
    int32_t small_tiles;/* 1: the call uses the small-chunk kernels, chosen when the groups
                           average fewer than 256 rows: the up GEMM on tiles of tile_rows rows
                           (a multiple of 32 sized to hold a typical group), the down GEMM on
                           64-row tiles; 0: 256-row tiles */
} moe_ws_layout;

/* Human-readable name of a status code (static storage, never NULL). */
const char *moe_status_string(moe_status status);

/* Row-tile height the grouped GEMMs of (dtype, variant) use for large
 * groups (bf16 unfused: 256; fused: 64; fp32: 64).  Small groups use other
 * heights; moe_ffn_workspace_layout reports the value a given shape uses. */
int moe_ffn_tile_rows(moe_dtype dtype, moe_variant variant);

/*
 * Fill *layout for a forward call of these sizes.  Returns MOE_OK,
 * MOE_ERR_INVALID_ARG (layout NULL, T < 0, D/F/E <= 0, k < 1, k > E,
 * E > 1024, T*k + T >= 2^31, unknown enum) or MOE_ERR_UNSUPPORTED (see
 * moe_ffn_forward).
 */
moe_status moe_ffn_workspace_layout(int64_t T, int D, int F, int E, int k, int has_shared,
                                    moe_dtype dtype, moe_variant variant, moe_ws_layout *layout);

/* Workspace bytes a forward call of these sizes needs; 0 if the sizes are
 * invalid or unsupported. */
size_t moe_ffn_workspace_size(int64_t T, int D, int F, int E, int k, int has_shared,
                              moe_dtype dtype, moe_variant variant);

/*
 * Forward pass of the routed SwiGLU MoE layer.
 *
 *   x         [T, D]     dtype; token activations, 16-byte aligned
 *   topk_idx  [T, k]     int32; expert id of choice j of token t
 *   topk_w    [T, k]     fp32;  routing weight of that choice (used as given)
 *   W1, W3    [E, D, F]  dtype; gate and up projections (v . W1[e] is v's gate row)
 *   W2        [E, F, D]  dtype; down projection
 *   Ws1, Ws3  [D, F], Ws2 [F, D]  dtype; shared expert, all three NULL for none
 *   y         [T, D]     dtype; output, fully overwritten
 *   workspace device buffer of ws_bytes >= moe_ffn_workspace_size(), 256-byte aligned
 *
 * Stored results (bf16): per row, the gate and up products accumulate in
 * fp32, silu(g)*u is formed in fp32 and rounded once to bf16 (h); the down
 * product accumulates in fp32 and is rounded once to bf16 (Y); the combine
 * starts from the shared row (or 0), adds topk_w[t,j] * Y[row of slot t*k+j]
 * for j = 0..k-1 in that order as fp32 fused multiply-adds and rounds once
 * to the output dtype.  In fp32 every step stays fp32.  The summation
 * order does not depend on timing, so repeated calls give bitwise-identical
 * y.
 *
 * Returns MOE_OK; MOE_ERR_INVALID_ARG (null pointer, pointer misaligned,
 * sizes as in moe_ffn_workspace_layout, only some of Ws1/Ws3/Ws2 given);
 * MOE_ERR_UNSUPPORTED (bf16 with D or F not a multiple of 64; the fused
 * variant with fp32, D % 128 != 0, D > 1024 or F % 128 != 0);
 * MOE_ERR_WORKSPACE; MOE_ERR_HIP.
 *
 * Variants: MOE_VARIANT_UNFUSED writes h [R, F] to the workspace between
 * the up and down grouped GEMMs; MOE_VARIANT_FUSED ("Chinchilla scaling,
 * MoE, and fused Triton kernels", fused kernel sections) computes up,
 * SwiGLU and down per 64-token tile in one kernel and never stores h.
 * Tiles run whole in full rounds of 256 workgroups; each tile of the last,
 * partial round (all tiles when there are fewer than 256) has its F chunks
 * shared out over several workgroups (a power of two, at most one per
 * 256-column chunk, at most 256 in all) whose fp32 partial outputs a second
 * kernel sums in a fixed order before rounding Y to bf16.  Both
 * give results within the same tolerance of the exact layer; they are not
 * bitwise equal to each other (different accumulation blocking).
 * T == 0 returns MOE_OK and launches nothing.
 */
moe_status moe_ffn_forward(const void *x, const int32_t *topk_idx, const float *topk_w,
                           const void *W1, const void *W3, const void *W2,
                           const void *Ws1, const void *Ws3, const void *Ws2,
                           void *y, int64_t T, int D, int F, int E, int k,
                           moe_dtype dtype, moe_variant variant,
                           void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * moe_ffn_forward plus per-stage timing: the same call, which also records
 * events[0] before the permute, events[1] after it (back to back when the
 * small-chunk up GEMM does the counting sort itself: bf16, unfused, groups
 * averaging under 256 rows, T*k <= 4096, E <= 512), events[2] after the
 * up+SwiGLU GEMM (the fused variant: after its single up-act-down kernel),
 * events[3] after the down GEMM (fused: after the sum of the split tiles'
 * partial outputs) and
 * events[4] after the combine, all on `stream` (five caller-created
 * hipEvent_t).  For measuring
 * each kernel's duration inside a timed loop; results are identical to
 * moe_ffn_forward.  events == NULL behaves exactly like moe_ffn_forward.
 */
moe_status moe_ffn_forward_timed(const void *x, const int32_t *topk_idx, const float *topk_w,
                                 const void *W1, const void *W3, const void *W2,
                                 const void *Ws1, const void *Ws3, const void *Ws2,
                                 void *y, int64_t T, int D, int F, int E, int k,
                                 moe_dtype dtype, moe_variant variant,
                                 void *workspace, size_t ws_bytes, hipStream_t stream,
                                 hipEvent_t events[5]);

/*
 * moe_ffn_forward that also keeps, for the backward, each sorted row's gate
 * and up products: the "Triton MoE Kernels & Memory Checkpointing" autograd
 * contract (Part A, section 8) recomputes g = v W1 and u = v W3 in the
 * backward; keeping them instead trades their storage for that recompute
 * (moe_ffn_backward_cached takes them back).
 *
 *   gu  [R, 2F] dtype, caller-owned, 16-byte aligned, R = T*k (+ T with a
 *       shared expert): row p is sorted row p of the layer (the rows in the
 *       order of moe_expert_permute's perm, then the T shared rows), g in
 *       columns 0..F-1, u in F..2F-1, each the fp32 product rounded once to
 *       bf16 -- bitwise what the backward's own recompute produces.  Rows of
 *       invalid slots (positions >= offsets[E] among the routed rows) are not
 *       written.
 *
 * y is bitwise the y of moe_ffn_forward.  Only bf16 with
 * MOE_VARIANT_UNFUSED keeps g and u (the fused variant never stores the
 * up product, and the fp32 path has no bf16 rows): other dtypes or variants
 * return MOE_ERR_UNSUPPORTED.  Other arguments and errors as
 * moe_ffn_forward; gu NULL with T > 0 is MOE_ERR_INVALID_ARG.
 */
moe_status moe_ffn_forward_save_gu(const void *x, const int32_t *topk_idx, const float *topk_w,
                                   const void *W1, const void *W3, const void *W2,
                                   const void *Ws1, const void *Ws3, const void *Ws2,
                                   void *y, void *gu, int64_t T, int D, int F, int E, int k,
                                   moe_dtype dtype, moe_variant variant,
                                   void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * moe_ffn_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The library keeps one workspace of
 * MOE_NOALLOC_SCRATCH_BYTES per device in a file-scope device array, which
 * each GPU the library runs on holds until the process ends; the first call
 * on a device resolves its address (hipGetSymbolAddress), no call allocates
 * or frees memory.  The caller still passes the inputs and y.
 *
 * Arguments, results, variants and errors are those of moe_ffn_forward,
 * except that MOE_ERR_WORKSPACE means the call would need more than
 * MOE_NOALLOC_SCRATCH_BYTES of workspace (moe_ffn_workspace_size() of the
 * same sizes; for example the 4096-token layer at D 768, F 1536, E 8, top-2
 * with a shared expert needs 54 MiB, 32768 tokens need 433 MiB and are
 * refused).  The forward reads nothing from its workspace that the same call
 * has not written, so the array needs no clearing between calls.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last
 * call's contents: two calls that overlap in time on the same GPU (different
 * streams not ordered by events, or different host threads) race on it and
 * give undefined results.  moe_ffn_get_device_error cannot read this
 * workspace's invalid-slot count.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

moe_status moe_ffn_forward_noalloc(const void *x, const int32_t *topk_idx, const float *topk_w,
                                   const void *W1, const void *W3, const void *W2,
                                   const void *Ws1, const void *Ws3, const void *Ws2,
                                   void *y, int64_t T, int D, int F, int E, int k,
                                   moe_dtype dtype, moe_variant variant, hipStream_t stream);

/*
 * Expert permute alone: the stable counting sort of the T*k slots
 * s = t*k + j by expert id ("Triton MoE Kernels & Memory Checkpointing",
 * Part A section 10.3 steps 1-2: flatten, stable argsort, bincount and
 * cumulative sum), plus row-tile offsets for the grouped GEMMs.
 *
 *   topk_idx [T*k] int32 in; counts [E]; offsets [E+1] (exclusive starts,
 *   offsets[E] = number of valid slots); tile_off [E+2] (prefix sum of
 *   ceil(counts[e]/tile_rows), then one group of shared_rows rows);
 *   perm [T*k] sorted position -> slot, ascending by (expert, slot), -1 at
 *   positions >= offsets[E]; inv [T*k] slot -> position, -1 for invalid
 *   slots; err [1] number of invalid slots.  scratch: scratch_bytes >=
 *   moe_expert_permute_scratch_size(T, k, E) bytes, 4-byte aligned (may be
 *   NULL when that size is 0).
 *
 * Returns MOE_OK, MOE_ERR_INVALID_ARG (null outputs, T < 0, k < 1, E < 1,
 * E > 1024, tile_rows < 1, shared_rows < 0, T*k >= 2^31), MOE_ERR_WORKSPACE,
 * MOE_ERR_HIP.  T == 0 writes counts/offsets/tile_off/err and nothing else.
 */
moe_status moe_expert_permute(const int32_t *topk_idx, int64_t T, int k, int E, int tile_rows,
                              int64_t shared_rows, int32_t *counts, int32_t *offsets,
                              int32_t *tile_off, int32_t *perm, int32_t *inv, int32_t *err,
                              void *scratch, size_t scratch_bytes, hipStream_t stream);

/* Scratch bytes moe_expert_permute needs for these sizes (0 when it runs as
 * a single workgroup). */
size_t moe_expert_permute_scratch_size(int64_t T, int k, int E);

/*
 * Read the invalid-slot count of the last forward that used `workspace`.
 * Waits for `stream` to finish (the one synchronising call).  Returns
 * MOE_OK, MOE_ERR_INVALID_ARG (null argument) or MOE_ERR_HIP.
 */
moe_status moe_ffn_get_device_error(const void *workspace, hipStream_t stream, int32_t *out);

/*
 * Measurement helper, not part of the layer: launches `blocks` one-wavefront
 * workgroups on `stream`; workgroup b writes out[3b] = the compute unit it
 * ran on (XCD id * 65536 + the shader engine, array and CU bits of the
 * hardware id), out[3b+1] = the shader-clock cycle counter and out[3b+2] =
 * the constant 100 MHz counter.  Two samples taken around a timed region,
 * paired by compute unit, give the mean engine clock over the region:
 * (difference of cycle counters) / (difference of 100 MHz counters) * 100 MHz.
 *
 *   out     device int64 [3 * blocks], 8-byte aligned, caller-owned
 *   blocks  1 .. 1024 (1024 one-wavefront workgroups reach every CU)
 *
 * Returns MOE_OK, MOE_ERR_INVALID_ARG (null or misaligned out, blocks out of
 * range) or MOE_ERR_HIP.
 */
moe_status moe_device_clock_sample(int64_t *out, int blocks, hipStream_t stream);

/*
 * Measurement helper (not part of the layer): read `bytes` of device memory
 * once with a plain streaming kernel of `blocks` workgroups of 512 threads
 * on `stream` (each thread 16 bytes at a time, eight in flight,
 * non-temporal), so that the
 * read rate it reaches, timed by the caller, prices kernels bound by
 * reading their operands once against what this part delivers rather than
 * against the nominal 8 TB/s.  Workgroup b writes the xor of what it read
 * to sink[b].
 *
 *   src    device pointer, 16-byte aligned; bytes a positive multiple of 16
 *   sink   device uint32 [blocks], 4-byte aligned, caller-owned
 *   blocks 1 .. 65536
 *
 * Returns MOE_OK, MOE_ERR_INVALID_ARG or MOE_ERR_HIP.
 */
moe_status moe_stream_read(const void *src, size_t bytes, uint32_t *sink, int blocks,
                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * Router in front of the layer.
 *
 * The top-k router of "Chinchilla scaling, MoE, and fused Triton kernels"
 * (section "PyTorch MoE implementation"): logits = x gate_w, the k largest
 * logits of each token in descending order, and routing weights equal to
 * the softmax over those k logits.  Equal logits are taken in ascending
 * expert order.  Arithmetic is fp32 (products of the stored values summed
 * in fp32; fp32 softmax).
 * ------------------------------------------------------------------------ */

/*
 *   x         [T, D]  dtype, 16-byte aligned
 *   gate_w    [D, E]  dtype
 *   topk_idx  [T, k]  int32 out: expert of choice j (descending logit)
 *   topk_w    [T, k]  fp32 out: softmax over the token's k chosen logits
 *
 * Returns MOE_OK; MOE_ERR_INVALID_ARG (null or misaligned pointer, T < 0,
 * D <= 0, E < 1, k < 1, k > E, unknown dtype); MOE_ERR_UNSUPPORTED (E > 64,
 * D % 8 != 0 or D * E > 16384); MOE_ERR_HIP.  T == 0 launches nothing.
 */
moe_status moe_router_topk(const void *x, const void *gate_w, int64_t T, int D, int E, int k,
                           moe_dtype dtype, int32_t *topk_idx, float *topk_w, hipStream_t stream);

/*
 * moe_ffn_forward with the router in front: routes x with gate_w [D, E]
 * (as moe_router_topk), writes the routing to topk_idx / topk_w (caller
 * buffers, [T, k]) and computes y from it.  When the permute runs as more
 * than one block, the router also writes the permute's per-block expert
 * counts, so the permute starts at its scan (no separate histogram pass and
 * no [T, E] logits in memory).  Same workspace, variants, results and
 * errors as moe_ffn_forward, plus the router's MOE_ERR_UNSUPPORTED shapes.
 */
moe_status moe_ffn_forward_routed(const void *x, const void *gate_w,
                                  const void *W1, const void *W3, const void *W2,
                                  const void *Ws1, const void *Ws3, const void *Ws2,
                                  void *y, int32_t *topk_idx, float *topk_w,
                                  int64_t T, int D, int F, int E, int k,
                                  moe_dtype dtype, moe_variant variant,
                                  void *workspace, size_t ws_bytes, hipStream_t stream);

/* moe_ffn_forward_routed with the five stage events of
 * moe_ffn_forward_timed (events[1] follows the router and the permute). */
moe_status moe_ffn_forward_routed_timed(const void *x, const void *gate_w,
                                        const void *W1, const void *W3, const void *W2,
                                        const void *Ws1, const void *Ws3, const void *Ws2,
                                        void *y, int32_t *topk_idx, float *topk_w,
                                        int64_t T, int D, int F, int E, int k,
                                        moe_dtype dtype, moe_variant variant,
                                        void *workspace, size_t ws_bytes, hipStream_t stream,
                                        hipEvent_t events[5]);

/* ------------------------------------------------------------------------
 * Backward pass.
 *
 * The vector-Jacobian product of the layer for an incoming gradient dy:
 * the autograd contract of "Triton MoE Kernels & Memory Checkpointing"
 * (Part A, section 8) -- the gate and up products are recomputed from x
 * instead of being saved by the forward, their gradients are the upstream
 * gradient times the derivative of silu(g) * u, and the weight gradients
 * are the outer products of those gradients with the inputs -- extended by
 * the same chain rule through W2 and the weighted combine (same page,
 * section 10.3).  Per routed slot (token t, choice j, expert e, weight w):
 *
 *   g = x[t] W1[e], u = x[t] W3[e], h = silu(g) * u, o = h W2[e]
 *   dtopk_w[t,j] = dy[t] . o
 *   dh = w dy[t] W2[e]^T,  dg = dh * u * silu'(g),  du = dh * silu(g)
 *   dW2[e] += h^T (w dy[t]),  dW1[e] += x[t]^T dg,  dW3[e] += x[t]^T du
 *   dx[t]  += dg W1[e]^T + du W3[e]^T
 *
 * and the same with w = 1 and the shared weights for the shared expert.
 * ------------------------------------------------------------------------ */

/* Byte offsets of the pieces of a backward workspace (256-byte aligned);
 * rows as in the forward (R = T*k + T*[shared]). */
typedef struct moe_bwd_ws_layout {
    size_t total;       /* bytes the workspace must hold */
    size_t err, counts, offsets, tile_off;   /* the permute's, as forward */
    size_t chunk_off;   /* int32 [E+2] prefix of ceil(rows / chunk_rows), shared group last (bf16) */
    size_t perm, inv, hist;
    size_t gu;          /* [R, 2F] recomputed gate (columns 0..F-1) and up (F..2F-1), dtype of the call */
    size_t dgu;         /* [R, 2F] gradients of the gate and up products, dtype of the call */
    size_t hw;          /* [R, F]  w * h per row, dtype of the call */
    size_t dxr;         /* [R, D]  each row's contribution to dx, dtype of the call */
    size_t dwpart;      /* fp32 [R, ceil(F/64)] partial sums of dy . o per 64 columns */
    size_t w2t;         /* bf16 [E(+1), D, F] W2 (and Ws2) transposed; empty for fp32 */
    size_t w13t;        /* bf16 [E(+1), 2F, D] W1^T stacked over W3^T (and shared); empty for fp32 */
    size_t partial;     /* fp32 [chunks, D*2F] per-chunk dW1/dW3 partial sums, then [chunks, F*D] dW2's (bf16) */
    size_t zeros;       /* 256 zero bytes (bf16) */
    int32_t tile_rows;  /* row-tile height of tile_off */
    int32_t hist_blocks;/* slot blocks of the multi-block permute (0: single block) */
    int32_t chunk_rows; /* rows per weight-gradient chunk (bf16; 0 for fp32) */
} moe_bwd_ws_layout;

/* Fill *layout for a backward call of these sizes.  Returns MOE_OK,
 * MOE_ERR_INVALID_ARG or MOE_ERR_UNSUPPORTED under the same rules as
 * moe_ffn_workspace_layout (variant unfused). */
moe_status moe_ffn_backward_workspace_layout(int64_t T, int D, int F, int E, int k, int has_shared,
                                             moe_dtype dtype, moe_bwd_ws_layout *layout);

/* Backward workspace bytes; 0 if the sizes are invalid or unsupported. */
size_t moe_ffn_backward_workspace_size(int64_t T, int D, int F, int E, int k, int has_shared,
                                       moe_dtype dtype);

/*
 * Backward of moe_ffn_forward for the incoming gradient dy.
 *
 *   x, topk_idx, topk_w, W1, W3, W2, Ws1, Ws3, Ws2: the forward's inputs
 *                (same types, layouts and alignment rules; the shared
 *                weights all NULL for none)
 *   dy        [T, D]     dtype; gradient of the loss with respect to y
 *   dx        [T, D]     dtype; out, fully overwritten
 *   dW1, dW3  [E, D, F]  fp32; out, fully overwritten (zero for an expert no slot chose)
 *   dW2       [E, F, D]  fp32; out
 *   dWs1, dWs3 [D, F], dWs2 [F, D]  fp32; out, required exactly when the
 *                shared weights are given
 *   dtopk_w   [T, k]     fp32; out, dy[t] . o for each slot, 0 for an
 *                invalid slot
 *   workspace >= moe_ffn_backward_workspace_size() bytes, 256-byte aligned
 *
 * Precision: fp32 accumulation throughout.  bf16 calls store the recomputed
 * g and u, the gradients dg and du, w*h and the per-row dx contributions as
 * bf16 (round to nearest even) between kernels; the weight gradients and
 * dtopk_w are written in fp32.  Summation orders are fixed (no atomics), so
 * repeated calls give bitwise-identical results.  Slots with an
 * out-of-range id are counted in the error flag (moe_ffn_get_device_error)
 * and contribute nothing.
 *
 * Returns MOE_OK, MOE_ERR_INVALID_ARG (null or misaligned pointer, sizes
 * as in the forward, only some of the shared weights or their gradients
 * given), MOE_ERR_UNSUPPORTED (bf16 with D or F not a multiple of 64),
 * MOE_ERR_WORKSPACE, MOE_ERR_HIP.  With T == 0 the weight gradients are
 * written as zeros and nothing else is touched.
 */
moe_status moe_ffn_backward(const void *x, const int32_t *topk_idx, const float *topk_w,
                            const void *W1, const void *W3, const void *W2,
                            const void *Ws1, const void *Ws3, const void *Ws2,
                            const void *dy, void *dx, float *dW1, float *dW3, float *dW2,
                            float *dWs1, float *dWs3, float *dWs2, float *dtopk_w,
                            int64_t T, int D, int F, int E, int k, moe_dtype dtype,
                            void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * moe_ffn_backward plus per-stage timing: events[0] before the permute,
 * [1] after it, [2] after the weight transposes (bf16; none for fp32), [3]
 * after the gate/up recompute, [4] after the dh stage, [5] after the
 * per-row dx products, [6] after the W1/W3 gradient GEMM, [7] after the W2
 * gradient GEMM, [8] after the weight gradients' chunk reductions (bf16),
 * dtopk_w and the dx combine (nine caller-created hipEvent_t on `stream`).
 * events == NULL behaves exactly like moe_ffn_backward.
 */
moe_status moe_ffn_backward_timed(const void *x, const int32_t *topk_idx, const float *topk_w,
                                  const void *W1, const void *W3, const void *W2,
                                  const void *Ws1, const void *Ws3, const void *Ws2,
                                  const void *dy, void *dx, float *dW1, float *dW3, float *dW2,
                                  float *dWs1, float *dWs3, float *dWs2, float *dtopk_w,
                                  int64_t T, int D, int F, int E, int k, moe_dtype dtype,
                                  void *workspace, size_t ws_bytes, hipStream_t stream,
                                  hipEvent_t events[9]);

/*
 * moe_ffn_backward with the gate and up products taken from the forward
 * instead of recomputed ("Triton MoE Kernels & Memory Checkpointing",
 * Part A section 8: the recompute-versus-keep trade-off of the autograd
 * contract): gu is the [R, 2F] array moe_ffn_forward_save_gu wrote for the
 * same x, topk_idx, W1 and W3 (caller-owned, 16-byte aligned, read only).
 * The gate/up recompute launch is skipped; every other step is that of
 * moe_ffn_backward, and since gu holds bitwise what the recompute would
 * store, every gradient is bitwise the one moe_ffn_backward returns.  The
 * workspace is moe_ffn_backward_workspace_size() bytes, as for
 * moe_ffn_backward (its gate/up slot stays unused).  bf16 only (other
 * dtypes return MOE_ERR_UNSUPPORTED); gu NULL with T > 0 is
 * MOE_ERR_INVALID_ARG; other errors as moe_ffn_backward.
 */
moe_status moe_ffn_backward_cached(const void *x, const int32_t *topk_idx, const float *topk_w,
                                   const void *W1, const void *W3, const void *W2,
                                   const void *Ws1, const void *Ws3, const void *Ws2,
                                   const void *gu, const void *dy, void *dx, float *dW1,
                                   float *dW3, float *dW2, float *dWs1, float *dWs3, float *dWs2,
                                   float *dtopk_w, int64_t T, int D, int F, int E, int k,
                                   moe_dtype dtype, void *workspace, size_t ws_bytes,
                                   hipStream_t stream);

/* moe_ffn_backward_cached plus the nine events of moe_ffn_backward_timed
 * (events[2] and [3] back to back: no recompute launch between them). */
moe_status moe_ffn_backward_cached_timed(const void *x, const int32_t *topk_idx,
                                         const float *topk_w, const void *W1, const void *W3,
                                         const void *W2, const void *Ws1, const void *Ws3,
                                         const void *Ws2, const void *gu, const void *dy,
                                         void *dx, float *dW1, float *dW3, float *dW2,
                                         float *dWs1, float *dWs3, float *dWs2, float *dtopk_w,
                                         int64_t T, int D, int F, int E, int k, moe_dtype dtype,
                                         void *workspace, size_t ws_bytes, hipStream_t stream,
                                         hipEvent_t events[9]);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
