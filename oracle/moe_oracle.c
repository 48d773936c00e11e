/*
 * moe_oracle.c -- plain, slow, fp64 CPU oracle for the forward pass of a
 * top-k routed mixture-of-experts SwiGLU feed-forward layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no
 * code, header, table or constant with the HIP path, and the HIP path never
 * calls it.
 *
 * What it computes (the plain definition; every sum runs in fp64 in
 * ascending index order, no blocking, no fusion):
 *
 *   SwiGLU_e(v) = (silu(v . W1[e]) * (v . W3[e])) . W2[e],  silu(z) = z / (1 + exp(-z))
 *   y[t] = [shared] SwiGLU_sh(x[t]) + sum_{j=0}^{k-1} w[t,j] * SwiGLU_{idx[t,j]}(x[t])
 *
 * Sources (pages as published on the web):
 *  - "Triton MoE Kernels & Memory Checkpointing", Part A section 2: each
 *    expert is the SwiGLU block W2(silu(W1 x) * W3 x), every token goes to its
 *    top-2 of 8 routed experts plus one shared expert.
 *  - same page, section 10.2 (the CPU reference): a loop over experts that
 *    skips empty experts and evaluates each expert on its contiguous chunk
 *    of sorted rows.
 *  - same page, section 10.3 (the dispatch): flatten (token, choice) pairs
 *    to slots, stable-argsort the slots by expert id, per-expert counts by
 *    bincount and start offsets by cumulative sum; W2 per expert; scale by
 *    the routing weight after W2 and add back into the token's row.
 *  - "Chinchilla scaling, MoE, and fused Triton kernels", section "PyTorch
 *    MoE implementation": slot order t*k + j (reshape(-1)), stable argsort,
 *    bincount with minlength E, the inverse permutation inv[perm[p]] = p,
 *    and the weighted sum over the k choices of each token.
 *
 * Readings where the pages are silent or garbled:
 *  - weights are stored [E,D,F] for W1/W3 and [E,F,D] for W2, so the gate
 *    pre-activation is the row vector x times W1[e];
 *  - the activation is SwiGLU (silu of the W1 product times the W3 product);
 *    the second page's "silu(h) * h" is taken as a garbled single-matrix form;
 *  - the shared expert has weight 1 and the routing weights are used as given
 *    (no renormalisation);
 *  - combine order: start from the shared expert's row (or 0), then add
 *    w[t,j] * Y_j for j = 0 .. k-1;
 *  - an expert id outside [0, E) marks its slot invalid: the slot gets no
 *    sorted position (inv = -1), is not counted and contributes nothing; the
 *    function returns how many such slots it saw.
 *
 * Backward (moe_oracle_backward): the vector-Jacobian product of the same
 * layer for an incoming gradient dy, by the chain rule on the recomputed
 * forward, as "Triton MoE Kernels & Memory Checkpointing" (Part A, section 8)
 * does it: the gate and up products are recomputed, their gradients are the
 * upstream gradient times the derivative of silu(g) * u, and the weight
 * gradients are the outer products of those gradients with the inputs.
 * Per routed slot (token t, choice j, expert e, weight w = w[t,j]):
 *
 *   g = x W1[e],  u = x W3[e],  h = silu(g) * u,  o = h W2[e]
 *   dw[t,j]  = dy[t] . o                    (gradient of the routing weight)
 *   dh       = (w dy[t]) W2[e]^T
 *   dg       = dh * u * silu'(g),   silu'(z) = s (1 + z (1 - s)),  s = 1 / (1 + exp(-z))
 *   du       = dh * silu(g)
 *   dW2[e]  += h^T (w dy[t]),  dW1[e] += x^T dg,  dW3[e] += x^T du
 *   dx[t]   += dg W1[e]^T + du W3[e]^T
 *
 * and the same with w = 1 and the shared weights for the shared expert.
 * dx[t] accumulates the shared expert first, then j = 0 .. k-1; each weight
 * gradient accumulates tokens in ascending order (choices ascending).
 *
 * Build: gcc -O2 -fPIC -shared -ffp-contract=off -pthread (no -ffast-math).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* d silu / dz = s + z s (1 - s) with s the logistic sigmoid of z. */
static double dsilu(double z)
{
    const double s = 1.0 / (1.0 + exp(-z));
    return s * (1.0 + z * (1.0 - s));
}

/*
 * Counting sort of the flattened slots by expert id (stable).
 *   idx      [S]     expert id of slot s = t*k + j
 *   counts   [E]     number of valid slots per expert
 *   offsets  [E+1]   exclusive prefix sum of counts; offsets[E] = valid slots
 *   tile_off [E+2]   prefix sum of ceil(count/BM) over the E routed groups
 *                    followed by one shared group of shared_rows rows
 *   perm     [S]     sorted position -> slot, ascending (expert, slot);
 *                    positions >= offsets[E] are set to -1
 *   inv      [S]     slot -> sorted position, -1 for invalid slots
 * Returns the number of invalid slots.
 */
int64_t moe_oracle_permute(const int32_t *idx, int64_t S, int E, int BM, int64_t shared_rows,
                           int32_t *counts, int32_t *offsets, int32_t *tile_off,
                           int32_t *perm, int32_t *inv)
{
    int64_t bad = 0;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t s = 0; s < S; ++s) {
        int32_t e = idx[s];
        if (e >= 0 && e < E) counts[e] += 1;
        else bad += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];

    tile_off[0] = 0;
    for (int e = 0; e < E; ++e)
        tile_off[e + 1] = tile_off[e] + (int32_t)((counts[e] + BM - 1) / BM);
    tile_off[E + 1] = tile_off[E] + (int32_t)((shared_rows + BM - 1) / BM);

    /* Stable by construction: experts in ascending order, and within one
     * expert the slots in ascending order. */
    for (int64_t s = 0; s < S; ++s) inv[s] = -1;
    for (int64_t p = 0; p < S; ++p) perm[p] = -1;
    int64_t pos = 0;
    for (int e = 0; e < E; ++e)
        for (int64_t s = 0; s < S; ++s)
            if (idx[s] == e) {
                perm[pos] = (int32_t)s;
                inv[s] = (int32_t)pos;
                ++pos;
            }
    return bad;
}

/*
 * Gate and up products of one row and the gated activation:
 * g = xr W1, u = xr W3 (W1, W3 [D,F]), h = silu(g) * u, all of length F.
 */
static void gate_up_row(const double *xr, const double *W1, const double *W3, int64_t D,
                        int64_t F, double *g, double *u, double *h)
{
    for (int64_t f = 0; f < F; ++f) { g[f] = 0.0; u[f] = 0.0; }
    for (int64_t d = 0; d < D; ++d) {          /* g[f] = sum_d x[d] W1[d][f], d ascending */
        const double xd = xr[d];
        const double *w1 = W1 + d * F, *w3 = W3 + d * F;
        for (int64_t f = 0; f < F; ++f) {
            g[f] += xd * w1[f];
            u[f] += xd * w3[f];
        }
    }
    for (int64_t f = 0; f < F; ++f) h[f] = silu(g[f]) * u[f];
}

/*
 * One expert on one row: out[D] = SwiGLU(xr) with W1,W3 [D,F] and W2 [F,D].
 * h[F] receives silu(g)*u.  g and u are scratch of length F.
 */
static void swiglu_row(const double *xr, const double *W1, const double *W3, const double *W2,
                       int64_t D, int64_t F, double *g, double *u, double *h, double *out)
{
    gate_up_row(xr, W1, W3, D, F, g, u, h);
    for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
    for (int64_t f = 0; f < F; ++f) {          /* out[d] = sum_f h[f] W2[f][d], f ascending */
        const double hf = h[f];
        const double *w2 = W2 + f * D;
        for (int64_t d = 0; d < D; ++d) out[d] += hf * w2[d];
    }
}

typedef struct {
    /* problem */
    const double *x, *w, *W1, *W3, *W2, *Ws1, *Ws3, *Ws2;
    const int32_t *idx;
    int64_t T, D, F;
    int E, k;
    /* dense path */
    const int64_t *tokens;
    int64_t ntok;
    double *y;
    /* permuted path */
    const int32_t *perm, *offsets;
    int64_t S;
    double *h_out, *Y_out;     /* sorted-row results [S(+T), F] and [S(+T), D] */
    double *gu_out;            /* optional [S(+T), 2F]: g in columns 0..F-1, u in F..2F-1 */
    /* backward */
    const int32_t *groups;
    const double *dy;
    double *dx, *dW1, *dW3, *dW2, *dWs1, *dWs3, *dWs2, *dw;
    /* work split */
    int64_t lo, hi;
    int status;
} job_t;

/* Path (i): every listed token evaluated directly through its experts. */
static void *dense_worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const int64_t D = J->D, F = J->F;
    double *g = malloc(sizeof(double) * F), *u = malloc(sizeof(double) * F);
    double *h = malloc(sizeof(double) * F), *o = malloc(sizeof(double) * D);
    if (!g || !u || !h || !o) { J->status = -1; goto done; }
    for (int64_t i = J->lo; i < J->hi; ++i) {
        const int64_t t = J->tokens ? J->tokens[i] : i;
        const double *xr = J->x + t * D;
        double *yr = J->y + i * D;
        for (int64_t d = 0; d < D; ++d) yr[d] = 0.0;
        if (J->Ws1) {
            swiglu_row(xr, J->Ws1, J->Ws3, J->Ws2, D, F, g, u, h, o);
            for (int64_t d = 0; d < D; ++d) yr[d] = o[d];
        }
        for (int j = 0; j < J->k; ++j) {
            const int32_t e = J->idx[t * J->k + j];
            if (e < 0 || e >= J->E) continue;
            const double wt = J->w[t * J->k + j];
            swiglu_row(xr, J->W1 + (int64_t)e * D * F, J->W3 + (int64_t)e * D * F,
                       J->W2 + (int64_t)e * F * D, D, F, g, u, h, o);
            for (int64_t d = 0; d < D; ++d) yr[d] = yr[d] + wt * o[d];
        }
    }
done:
    free(g); free(u); free(h); free(o);
    return NULL;
}

static int run_jobs(job_t *base, int64_t n, int nthreads, void *(*fn)(void *))
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > n) nthreads = (int)(n > 0 ? n : 1);
    job_t *jobs = calloc((size_t)nthreads, sizeof(job_t));
    pthread_t *th = calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return -1; }
    int status = 0;
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = *base;
        jobs[i].lo = n * i / nthreads;
        jobs[i].hi = n * (i + 1) / nthreads;
        jobs[i].status = 0;
        if (nthreads > 1) pthread_create(&th[i], NULL, fn, &jobs[i]);
        else fn(&jobs[i]);
    }
    for (int i = 0; i < nthreads; ++i) {
        if (nthreads > 1) pthread_join(th[i], NULL);
        if (jobs[i].status) status = jobs[i].status;
    }
    free(jobs); free(th);
    return status;
}

/*
 * Path (i), dense brute force.  For each of the ntok listed tokens (or all T
 * when tokens == NULL, ntok = T) y[i] = shared + sum_j w * SwiGLU_e(x[t]).
 * Ws1/Ws3/Ws2 NULL means no shared expert.  Returns 0, or -1 on allocation
 * failure.
 */
int moe_oracle_forward_dense(const double *x, const int32_t *idx, const double *w,
                             const double *W1, const double *W3, const double *W2,
                             const double *Ws1, const double *Ws3, const double *Ws2,
                             int64_t T, int64_t D, int64_t F, int E, int k,
                             const int64_t *tokens, int64_t ntok, double *y, int nthreads)
{
    job_t J;
    memset(&J, 0, sizeof J);
    J.x = x; J.idx = idx; J.w = w; J.W1 = W1; J.W3 = W3; J.W2 = W2;
    J.Ws1 = Ws1; J.Ws3 = Ws3; J.Ws2 = Ws2;
    J.T = T; J.D = D; J.F = F; J.E = E; J.k = k;
    J.tokens = tokens; J.ntok = tokens ? ntok : T; J.y = y;
    return run_jobs(&J, J.ntok, nthreads, dense_worker);
}

/* Path (ii) stage: evaluate sorted rows [lo, hi) of the routed-plus-shared
 * row space.  Row p < S belongs to expert e with offsets[e] <= p <
 * offsets[e+1] and reads token perm[p] / k; row S + t is the shared expert on
 * token t. */
static void *sorted_worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const int64_t D = J->D, F = J->F;
    double *g = malloc(sizeof(double) * F), *u = malloc(sizeof(double) * F);
    if (!g || !u) { J->status = -1; goto done; }
    for (int64_t p = J->lo; p < J->hi; ++p) {
        const double *A1, *A3, *A2;
        int64_t t;
        if (p < J->S) {
            if (p >= J->offsets[J->E]) continue;          /* unused (invalid slots) */
            int e = 0;
            while (!(p < J->offsets[e + 1])) ++e;          /* the expert whose chunk holds p */
            A1 = J->W1 + (int64_t)e * D * F;
            A3 = J->W3 + (int64_t)e * D * F;
            A2 = J->W2 + (int64_t)e * F * D;
            t = J->perm[p] / J->k;
        } else {
            A1 = J->Ws1; A3 = J->Ws3; A2 = J->Ws2;
            t = p - J->S;
        }
        swiglu_row(J->x + t * D, A1, A3, A2, D, F, g, u, J->h_out + p * F, J->Y_out + p * D);
        if (J->gu_out) {
            double *r = J->gu_out + p * 2 * F;
            for (int64_t f = 0; f < F; ++f) { r[f] = g[f]; r[F + f] = u[f]; }
        }
    }
done:
    free(g); free(u);
    return NULL;
}

/*
 * Path (ii), the permuted evaluation in the pages' order: counting sort,
 * per-expert loop over sorted rows (empty experts do nothing), shared rows
 * appended after the S routed rows, then unpermute through inv and combine
 * in j order.  h_out [S + T*sh, F] and Y_out [S + T*sh, D] receive every
 * sorted row's h and W2 output (rows of invalid slots are left as zero);
 * gu_out [S + T*sh, 2F], when not NULL, receives the row's gate and up
 * products g = v W1, u = v W3 (columns 0..F-1 and F..2F-1), the values a
 * backward that caches them instead of recomputing them would keep.
 * perm/inv/counts/offsets are written to the caller's arrays
 * (sizes S, S, E, E+1).  Returns the number of invalid slots, or -1 on
 * allocation failure.
 */
int64_t moe_oracle_forward_permuted(const double *x, const int32_t *idx, const double *w,
                                    const double *W1, const double *W3, const double *W2,
                                    const double *Ws1, const double *Ws3, const double *Ws2,
                                    int64_t T, int64_t D, int64_t F, int E, int k,
                                    double *y, double *h_out, double *Y_out, double *gu_out,
                                    int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv,
                                    int nthreads)
{
    const int64_t S = T * k;
    const int has_sh = Ws1 != NULL;
    const int64_t rows = S + (has_sh ? T : 0);
    int32_t *tile_off = malloc(sizeof(int32_t) * (size_t)(E + 2));
    if (!tile_off) return -1;
    const int64_t bad = moe_oracle_permute(idx, S, E, 1, has_sh ? T : 0, counts, offsets,
                                           tile_off, perm, inv);
    free(tile_off);
    memset(h_out, 0, sizeof(double) * (size_t)(rows * F));
    memset(Y_out, 0, sizeof(double) * (size_t)(rows * D));
    if (gu_out) memset(gu_out, 0, sizeof(double) * (size_t)(rows * 2 * F));

    job_t J;
    memset(&J, 0, sizeof J);
    J.x = x; J.idx = idx; J.w = w; J.W1 = W1; J.W3 = W3; J.W2 = W2;
    J.Ws1 = Ws1; J.Ws3 = Ws3; J.Ws2 = Ws2;
    J.T = T; J.D = D; J.F = F; J.E = E; J.k = k;
    J.perm = perm; J.offsets = offsets; J.S = S; J.h_out = h_out; J.Y_out = Y_out;
    J.gu_out = gu_out;
    if (run_jobs(&J, rows, nthreads, sorted_worker)) return -1;

    /* Unpermute and combine: y[t] = Ysh[t] + sum_j w[t,j] * Y[inv[t*k+j]]. */
    for (int64_t t = 0; t < T; ++t) {
        double *yr = y + t * D;
        for (int64_t d = 0; d < D; ++d) yr[d] = has_sh ? Y_out[(S + t) * D + d] : 0.0;
        for (int j = 0; j < k; ++j) {
            const int32_t p = inv[t * k + j];
            if (p < 0) continue;
            const double wt = w[t * k + j];
            for (int64_t d = 0; d < D; ++d) yr[d] = yr[d] + wt * Y_out[(int64_t)p * D + d];
        }
    }
    return bad;
}

/*
 * Backward of one (token, expert) pair with routing weight wt (1 for the
 * shared expert).  xr, dyr: the token's rows [D].  Recomputes g, u, h (and
 * o when dw is wanted), then adds the pair's contributions to whichever of
 * dx_acc [D], dW1/dW3 [D,F], dW2 [F,D] and *dw are not NULL.  sc holds 6F
 * doubles of scratch.
 */
static void swiglu_row_backward(const double *xr, const double *dyr, double wt,
                                const double *W1, const double *W3, const double *W2,
                                int64_t D, int64_t F, double *sc, double *dx_acc,
                                double *dW1, double *dW3, double *dW2, double *dw)
{
    double *g = sc, *u = sc + F, *h = sc + 2 * F, *dh = sc + 3 * F, *dg = sc + 4 * F,
           *du = sc + 5 * F;
    gate_up_row(xr, W1, W3, D, F, g, u, h);
    if (dw) {                                    /* dw = dy . (h W2) */
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d) {
            double o = 0.0;
            for (int64_t f = 0; f < F; ++f) o += h[f] * W2[f * D + d];
            acc += dyr[d] * o;
        }
        *dw = acc;
    }
    for (int64_t f = 0; f < F; ++f) {            /* dh[f] = sum_d W2[f][d] (wt dy[d]) */
        const double *w2 = W2 + f * D;
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d) acc += w2[d] * (wt * dyr[d]);
        dh[f] = acc;
    }
    for (int64_t f = 0; f < F; ++f) {
        dg[f] = dh[f] * u[f] * dsilu(g[f]);
        du[f] = dh[f] * silu(g[f]);
    }
    if (dW2)
        for (int64_t f = 0; f < F; ++f)
            for (int64_t d = 0; d < D; ++d) dW2[f * D + d] += h[f] * (wt * dyr[d]);
    if (dW1)
        for (int64_t d = 0; d < D; ++d)
            for (int64_t f = 0; f < F; ++f) {
                dW1[d * F + f] += xr[d] * dg[f];
                dW3[d * F + f] += xr[d] * du[f];
            }
    if (dx_acc)
        for (int64_t d = 0; d < D; ++d) {
            const double *w1 = W1 + d * F, *w3 = W3 + d * F;
            double a1 = 0.0, a3 = 0.0;
            for (int64_t f = 0; f < F; ++f) {
                a1 += w1[f] * dg[f];
                a3 += w3[f] * du[f];
            }
            dx_acc[d] = dx_acc[d] + a1 + a3;
        }
}

/* Tokens [lo, hi): dx[t] and dw[t, :]. */
static void *bwd_token_worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const int64_t D = J->D, F = J->F;
    double *sc = malloc(sizeof(double) * 6 * F);
    if (!sc) { J->status = -1; return NULL; }
    for (int64_t t = J->lo; t < J->hi; ++t) {
        const double *xr = J->x + t * D, *dyr = J->dy + t * D;
        double *dxr = J->dx + t * D;
        for (int64_t d = 0; d < D; ++d) dxr[d] = 0.0;
        if (J->Ws1)
            swiglu_row_backward(xr, dyr, 1.0, J->Ws1, J->Ws3, J->Ws2, D, F, sc, dxr,
                                NULL, NULL, NULL, NULL);
        for (int j = 0; j < J->k; ++j) {
            const int32_t e = J->idx[t * J->k + j];
            double *dwp = J->dw + t * J->k + j;
            *dwp = 0.0;
            if (e < 0 || e >= J->E) continue;
            swiglu_row_backward(xr, dyr, J->w[t * J->k + j], J->W1 + (int64_t)e * D * F,
                                J->W3 + (int64_t)e * D * F, J->W2 + (int64_t)e * F * D, D, F,
                                sc, dxr, NULL, NULL, NULL, dwp);
        }
    }
    free(sc);
    return NULL;
}

/* Groups [lo, hi) of 0..E (E: the shared expert), or of the list J->groups
 * when given: the weight gradients. */
static void *bwd_expert_worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const int64_t D = J->D, F = J->F;
    double *sc = malloc(sizeof(double) * 6 * F);
    if (!sc) { J->status = -1; return NULL; }
    for (int64_t gi = J->lo; gi < J->hi; ++gi) {
        const int64_t grp = J->groups ? J->groups[gi] : gi;
        const int shared = grp == J->E;
        const double *A1 = shared ? J->Ws1 : J->W1 + grp * D * F;
        const double *A3 = shared ? J->Ws3 : J->W3 + grp * D * F;
        const double *A2 = shared ? J->Ws2 : J->W2 + grp * F * D;
        double *g1 = shared ? J->dWs1 : J->dW1 + grp * D * F;
        double *g3 = shared ? J->dWs3 : J->dW3 + grp * D * F;
        double *g2 = shared ? J->dWs2 : J->dW2 + grp * F * D;
        memset(g1, 0, sizeof(double) * (size_t)(D * F));
        memset(g3, 0, sizeof(double) * (size_t)(D * F));
        memset(g2, 0, sizeof(double) * (size_t)(F * D));
        for (int64_t t = 0; t < J->T; ++t)
            for (int j = 0; j < (shared ? 1 : J->k); ++j) {
                if (!shared && J->idx[t * J->k + j] != grp) continue;
                swiglu_row_backward(J->x + t * D, J->dy + t * D, shared ? 1.0 : J->w[t * J->k + j],
                                    A1, A3, A2, D, F, sc, NULL, g1, g3, g2, NULL);
            }
    }
    free(sc);
    return NULL;
}

/*
 * Backward of the layer for the incoming gradient dy [T,D]: dx [T,D],
 * dW1/dW3 [E,D,F], dW2 [E,F,D], dw [T,k] (0 for invalid slots) and, when
 * Ws1 is not NULL, dWs1/dWs3 [D,F] and dWs2 [F,D].  Returns 0, or -1 on
 * allocation failure.
 */
int moe_oracle_backward(const double *x, const int32_t *idx, const double *w,
                        const double *W1, const double *W3, const double *W2,
                        const double *Ws1, const double *Ws3, const double *Ws2,
                        const double *dy, int64_t T, int64_t D, int64_t F, int E, int k,
                        double *dx, double *dW1, double *dW3, double *dW2,
                        double *dWs1, double *dWs3, double *dWs2, double *dw, int nthreads)
{
    job_t J;
    memset(&J, 0, sizeof J);
    J.x = x; J.idx = idx; J.w = w; J.W1 = W1; J.W3 = W3; J.W2 = W2;
    J.Ws1 = Ws1; J.Ws3 = Ws3; J.Ws2 = Ws2;
    J.T = T; J.D = D; J.F = F; J.E = E; J.k = k;
    J.dy = dy; J.dx = dx; J.dW1 = dW1; J.dW3 = dW3; J.dW2 = dW2;
    J.dWs1 = dWs1; J.dWs3 = dWs3; J.dWs2 = dWs2; J.dw = dw;
    if (T > 0 && run_jobs(&J, T, nthreads, bwd_token_worker)) return -1;
    return run_jobs(&J, E + (Ws1 ? 1 : 0), nthreads, bwd_expert_worker);
}

/*
 * The weight gradients of the listed groups only (ngroups entries of
 * 0..E, E meaning the shared expert), as moe_oracle_backward computes them;
 * the other groups' gradients are not touched.  Returns 0, or -1 on
 * allocation failure.
 */
int moe_oracle_backward_groups(const double *x, const int32_t *idx, const double *w,
                               const double *W1, const double *W3, const double *W2,
                               const double *Ws1, const double *Ws3, const double *Ws2,
                               const double *dy, int64_t T, int64_t D, int64_t F, int E, int k,
                               const int32_t *groups, int ngroups,
                               double *dW1, double *dW3, double *dW2,
                               double *dWs1, double *dWs3, double *dWs2, int nthreads)
{
    job_t J;
    memset(&J, 0, sizeof J);
    J.x = x; J.idx = idx; J.w = w; J.W1 = W1; J.W3 = W3; J.W2 = W2;
    J.Ws1 = Ws1; J.Ws3 = Ws3; J.Ws2 = Ws2;
    J.T = T; J.D = D; J.F = F; J.E = E; J.k = k;
    J.dy = dy; J.dW1 = dW1; J.dW3 = dW3; J.dW2 = dW2;
    J.dWs1 = dWs1; J.dWs3 = dWs3; J.dWs2 = dWs2; J.groups = groups;
    return run_jobs(&J, ngroups, nthreads, bwd_expert_worker);
}
