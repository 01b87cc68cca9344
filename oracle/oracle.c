/*
 * CPU oracle for one tensor-parallel rank's share of a decode step.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file: only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg do. It shares no code, header, helper or
 * table with the HIP library; the two meet only through the byte arrays of
 * the seeded input generator.
 *
 * Plain C99, slow and obvious by design. Floating point:
 *   - bf16 inputs are widened exactly to double (a bf16 is the top half of an
 *     IEEE binary32, so the widening is a shift);
 *   - every product of two bf16 values is exact in double (8-bit significands
 *     give a 16-bit product), and the products are summed in double in
 *     ascending k; the double result is rounded once to float;
 *   - the ring-ordered reduction is done in float, one IEEE addition at a
 *     time, in the rank order fixed below. Build with -ffp-contract=off and
 *     without -ffast-math so the compiler neither fuses nor reassociates.
 *
 * Sources (the pages this follows):
 *   [P1] "Interconnects e clusters", llmdeepdive.com lesson 9.9,
 *        section "01 · Conceito".
 *   [P2] "Hosting Qwen on Blackwell", Perplexity blog (Bengali and Greek
 *        editions), sections "All-Reduce", "MoE Dispatch-Combine",
 *        "Expert Parallel".
 *
 * Parity pins (checked by the CPU tests) are listed per function. The MoE
 * routing step has no printed example on the pages; its pins are the
 * invariants named at oracle_moe_route.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- bf16 -- */

/* Exact widening: a bf16 bit pattern is the upper 16 bits of a binary32. */
static float bf16_bits_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a binary32 to bf16, nearest-even; NaN stays a (quiet) NaN. */
static uint16_t float_to_bf16_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lower = u & 0xffffu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u; /* carries into the exponent correctly, up to Inf */
    return (uint16_t)upper;
}

float oracle_bf16_to_f32(uint16_t h) { return bf16_bits_to_float(h); }
uint16_t oracle_f32_to_bf16(float f) { return float_to_bf16_bits(f); }

int oracle_abi_version(void) { return 1; }

/* ------------------------------------------------------ thread helper -- */

typedef void (*col_fn)(void* ctx, int64_t n_begin, int64_t n_end);

typedef struct {
    col_fn fn;
    void* ctx;
    int64_t n_begin, n_end;
} col_job;

static void* col_job_run(void* p)
{
    col_job* j = (col_job*)p;
    j->fn(j->ctx, j->n_begin, j->n_end);
    return NULL;
}

/* Split the output columns [0, n) into nthreads contiguous ranges. Each
 * output element is computed by exactly one thread, so the result does not
 * depend on the thread count. */
static void for_columns(col_fn fn, void* ctx, int64_t n, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n) nthreads = n > 0 ? (int)n : 1;
    if (nthreads == 1) {
        fn(ctx, 0, n);
        return;
    }
    pthread_t th[256];
    col_job jobs[256];
    int started[256];
    int64_t per = (n + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].n_begin = (int64_t)t * per < n ? (int64_t)t * per : n;
        jobs[t].n_end = (int64_t)(t + 1) * per < n ? (int64_t)(t + 1) * per : n;
        started[t] = pthread_create(&th[t], NULL, col_job_run, &jobs[t]) == 0;
        if (!started[t]) col_job_run(&jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        if (started[t]) pthread_join(th[t], NULL);
}

/* ------------------------------------------- row-parallel projection -- */

typedef struct {
    const uint16_t* x; /* [batch][ldx] bf16, columns [0, k) used */
    int64_t ldx;
    const uint16_t* w; /* [k][hidden] bf16, row-major */
    int64_t batch, k, hidden;
    double* y64;       /* [batch][hidden] or NULL */
    float* y32;        /* [batch][hidden] or NULL */
} partial_ctx;

static void partial_cols(void* p, int64_t n0, int64_t n1)
{
    partial_ctx* c = (partial_ctx*)p;
    int64_t width = n1 - n0;
    if (width <= 0) return;
    double* acc = (double*)malloc((size_t)width * sizeof(double));
    for (int64_t b = 0; b < c->batch; ++b) {
        for (int64_t n = 0; n < width; ++n) acc[n] = 0.0;
        /* y[b,n] = sum over k of x[b,k] * W[k,n]; for every n the terms are
         * added in ascending k, one rounding per addition, in double. */
        for (int64_t kk = 0; kk < c->k; ++kk) {
            double xv = (double)bf16_bits_to_float(c->x[b * c->ldx + kk]);
            const uint16_t* wrow = c->w + kk * c->hidden + n0;
            for (int64_t n = 0; n < width; ++n)
                acc[n] += xv * (double)bf16_bits_to_float(wrow[n]);
        }
        for (int64_t n = 0; n < width; ++n) {
            if (c->y64) c->y64[b * c->hidden + n0 + n] = acc[n];
            if (c->y32) c->y32[b * c->hidden + n0 + n] = (float)acc[n];
        }
    }
    free(acc);
}

/*
 * Row-parallel partial projection [P1, Conceito]: under tensor parallelism a
 * projection's weight matrix W[K, H] is split by rows over the ranks; rank r
 * holds rows K_r and computes p_r = x[:, K_r] . W[K_r, :], a partial result
 * that still has to be summed over ranks. With the whole of K this is the
 * unsharded projection y = x . W.
 *
 *   x   bf16 [batch][ldx], the first k columns are the rank's slice
 *   w   bf16 [k][hidden] row-major (the rank's rows of W)
 *   y64 double [batch][hidden] (optional), y32 float [batch][hidden]
 *       (optional, the double value rounded once, nearest-even)
 *
 * Pins: exact big-integer brute force on tiny shapes (y32 is the correctly
 * rounded exact sum up to the stated double error bound); the shard
 * partials sum to the unsharded product; one rank (N=1) is the full GEMV.
 */
void oracle_partial(const uint16_t* x, int64_t ldx, const uint16_t* w,
                    int64_t batch, int64_t k, int64_t hidden,
                    double* y64, float* y32, int nthreads)
{
    partial_ctx c = {x, ldx, w, batch, k, hidden, y64, y32};
    for_columns(partial_cols, &c, hidden, nthreads);
}

/* -------------------------------------------------- ring reduction -- */

/*
 * Ring all-reduce sum plus residual [P1, Conceito; P2, All-Reduce].
 *
 * The payload of one reduction is the flattened row-major [batch x hidden]
 * vector of `len` elements, split into n_ranks equal contiguous chunks of
 * C = len / n_ranks elements. In the reduce-scatter phase chunk c starts on
 * rank c and travels once round the ring, each rank adding its own partial
 * to the running sum it received, so chunk c is summed in the rank order
 * c, c+1, ..., c+N-1 (mod N). That takes N-1 steps; the all-gather phase
 * then copies the finished chunks round the ring in N-1 more steps and adds
 * nothing. The residual is added once, after the full sum:
 *
 *     s = p_c[i];  for j = 1..N-1: s = s + p_{(c+j) mod N}[i];
 *     out[i] = s + residual[i]                          (all in binary32)
 *
 * partials: float [n_ranks][len], rank-major. residual may alias out.
 * out_bf16 (optional) receives out rounded to bf16, nearest-even.
 * Returns 0, or -1 if n_ranks < 1 or n_ranks does not divide len.
 *
 * Pins: the IEEE vector p = (2^24, 1, -2^24, 1) at N=4 gives (1, 2, 2, 0)
 * per chunk under this start convention, which no other rank order gives;
 * N=1 is the identity plus residual; N=2 is p0 + p1 + residual; for small
 * integer partials every order is exact and the output is the exact sum.
 */
int oracle_ring_reduce(const float* partials, int32_t n_ranks, int64_t len,
                       const float* residual, float* out, uint16_t* out_bf16)
{
    if (n_ranks < 1 || len < 0 || len % n_ranks != 0) return -1;
    int64_t chunk = len / n_ranks;
    for (int64_t i = 0; i < len; ++i) {
        int32_t c = (int32_t)(i / chunk);
        volatile float s = partials[(int64_t)c * len + i];
        for (int32_t j = 1; j < n_ranks; ++j) {
            int32_t r = (c + j) % n_ranks;
            s = s + partials[(int64_t)r * len + i];
        }
        volatile float o = s + residual[i];
        out[i] = o;
        if (out_bf16) out_bf16[i] = float_to_bf16_bits(o);
    }
    return 0;
}

/* ------------------------------------------------------ wire bytes -- */

/*
 * Bytes a ring all-reduce puts on each rank's wire [P1, Conceito]:
 * 2(N-1)/N times the payload, i.e. N-1 reduce-scatter sends plus N-1
 * all-gather sends of one chunk of payload/N elements each.
 * Returns -1 if the payload does not split into N equal chunks.
 */
int64_t oracle_ring_wire_bytes_per_rank(int32_t n_ranks, int64_t payload_elems,
                                        int32_t elem_bytes)
{
    if (n_ranks < 1 || payload_elems % n_ranks != 0) return -1;
    int64_t chunk = payload_elems / n_ranks;
    return 2 * (int64_t)(n_ranks - 1) * chunk * elem_bytes;
}

/*
 * Total over all ranks [P2, All-Reduce]: every peer reduces one 1/N slice,
 * reading (N-1) * B/N bytes from the others, then broadcasts it, for
 * (N-1) * B * 2 reads and writes in all. The naive scheme, where one peer
 * reads everything from every other, moves N * (N-1) * B.
 */
int64_t oracle_split_allreduce_total_bytes(int32_t n_ranks, int64_t payload_bytes)
{
    if (n_ranks < 1) return -1;
    return (int64_t)(n_ranks - 1) * payload_bytes * 2;
}

int64_t oracle_naive_allreduce_total_bytes(int32_t n_ranks, int64_t payload_bytes)
{
    if (n_ranks < 1) return -1;
    return (int64_t)n_ranks * (n_ranks - 1) * payload_bytes;
}

/* ------------------------------------------------- layer stack -- */

/*
 * One rank's share of a decode step over a stack of layers [P1, Conceito]:
 * every layer has two reconciliation points, after the sequence-mixer's
 * output projection and after the FFN down projection, and at each the
 * rank's partial is all-reduced and the result added to the residual
 * stream before it goes on. The operations between the points are not
 * part of this path; each point's activation slice is an input.
 *
 *   x_attn  bf16 [L][batch][ka_r]      w_o    bf16 [L][ka_r][hidden]
 *   x_ffn   bf16 [L][batch][ki_r]      w_down bf16 [L][ki_r][hidden]
 *   slots   float [L][2][n_ranks][batch][hidden]: the other ranks' partials
 *           are inputs; this rank's entry is written (rounded once from
 *           double) and then reduced with them.
 *   hidden_state float [batch][hidden], in/out: h <- ring(slots) + h at each
 *           of the 2L points in order.
 * Returns 0, or -1 on bad sizes.
 */
int oracle_decode_layers(int32_t n_layers, int32_t n_ranks, int32_t rank,
                         int64_t batch, int64_t hidden, int64_t ka_r, int64_t ki_r,
                         const uint16_t* x_attn, const uint16_t* w_o,
                         const uint16_t* x_ffn, const uint16_t* w_down,
                         float* slots, float* hidden_state, int nthreads)
{
    if (n_layers < 0 || n_ranks < 1 || rank < 0 || rank >= n_ranks) return -1;
    int64_t len = batch * hidden;
    if (len % n_ranks != 0) return -1;
    for (int32_t l = 0; l < n_layers; ++l) {
        for (int point = 0; point < 2; ++point) {
            int64_t kr = point == 0 ? ka_r : ki_r;
            const uint16_t* x = point == 0 ? x_attn + (int64_t)l * batch * ka_r
                                           : x_ffn + (int64_t)l * batch * ki_r;
            const uint16_t* w = point == 0 ? w_o + (int64_t)l * ka_r * hidden
                                           : w_down + (int64_t)l * ki_r * hidden;
            float* slot = slots + ((int64_t)l * 2 + point) * n_ranks * len;
            oracle_partial(x, kr, w, batch, kr, hidden, NULL,
                           slot + (int64_t)rank * len, nthreads);
            if (oracle_ring_reduce(slot, n_ranks, len, hidden_state,
                                   hidden_state, NULL) != 0)
                return -1;
        }
    }
    return 0;
}

/* ------------------------------------------------------------- MoE -- */

/*
 * Top-k routing of decode tokens to experts [P2, Prefillers: each token is
 * sent to 8 of 128 experts]. The pages give only the top-8-of-128 choice
 * and a weighted combine; the reading taken here is the usual one:
 *   - probabilities = softmax over all experts of the token's logits
 *     (in double, shifted by the maximum);
 *   - the top_k experts by probability are selected (softmax is monotone,
 *     so this is the top_k by logit), ties going to the lower expert index;
 *   - with renorm != 0 the selected probabilities are divided by their sum,
 *     otherwise they are the plain softmax values;
 *   - per token the selection is listed in ascending expert index.
 *
 *   logits [tokens][experts] float; sel_expert [tokens][top_k] int32;
 *   sel_weight [tokens][top_k] double.
 * Pins: the selected logits dominate the unselected ones; ties resolve to
 * the lower index; renormalised weights sum to 1; top_k = experts gives the
 * full softmax.
 */
int oracle_moe_route(const float* logits, int32_t tokens, int32_t experts,
                     int32_t top_k, int32_t renorm, int32_t* sel_expert,
                     double* sel_weight)
{
    if (tokens < 0 || experts < 1 || top_k < 1 || top_k > experts) return -1;
    double* prob = (double*)malloc((size_t)experts * sizeof(double));
    unsigned char* taken = (unsigned char*)malloc((size_t)experts);
    for (int32_t t = 0; t < tokens; ++t) {
        const float* z = logits + (int64_t)t * experts;
        double zmax = z[0];
        for (int32_t e = 1; e < experts; ++e)
            if (z[e] > zmax) zmax = z[e];
        double denom = 0.0;
        for (int32_t e = 0; e < experts; ++e) {
            prob[e] = exp((double)z[e] - zmax);
            denom += prob[e];
        }
        for (int32_t e = 0; e < experts; ++e) {
            prob[e] /= denom;
            taken[e] = 0;
        }
        /* repeated arg-max: the first maximum found is the lowest index */
        for (int32_t s = 0; s < top_k; ++s) {
            int32_t best = -1;
            for (int32_t e = 0; e < experts; ++e)
                if (!taken[e] && (best < 0 || z[e] > z[best])) best = e;
            taken[best] = 1;
        }
        double sel_sum = 0.0;
        for (int32_t e = 0; e < experts; ++e)
            if (taken[e]) sel_sum += prob[e];
        int32_t s = 0;
        for (int32_t e = 0; e < experts; ++e) {
            if (!taken[e]) continue;
            sel_expert[(int64_t)t * top_k + s] = e;
            sel_weight[(int64_t)t * top_k + s] = renorm ? prob[e] / sel_sum : prob[e];
            ++s;
        }
    }
    free(taken);
    free(prob);
    return 0;
}

typedef struct {
    int32_t tokens, top_k, e_begin, e_end;
    const int32_t* sel_expert;
    const double* sel_weight;
    const uint16_t* u;   /* [tokens][top_k][moe_inter] bf16 */
    const uint16_t* w;   /* [e_end - e_begin][moe_inter][hidden] bf16 */
    int64_t moe_inter, hidden;
    double* part64;
    float* part32;
} moe_ctx;

static void moe_cols(void* p, int64_t n0, int64_t n1)
{
    moe_ctx* c = (moe_ctx*)p;
    int64_t width = n1 - n0;
    if (width <= 0) return;
    double* acc = (double*)malloc((size_t)width * sizeof(double));
    double* y = (double*)malloc((size_t)width * sizeof(double));
    for (int32_t t = 0; t < c->tokens; ++t) {
        for (int64_t n = 0; n < width; ++n) acc[n] = 0.0;
        /* the token's selection is in ascending expert order */
        for (int32_t s = 0; s < c->top_k; ++s) {
            int32_t e = c->sel_expert[(int64_t)t * c->top_k + s];
            if (e < c->e_begin || e >= c->e_end) continue;
            double g = c->sel_weight[(int64_t)t * c->top_k + s];
            const uint16_t* uv = c->u + ((int64_t)t * c->top_k + s) * c->moe_inter;
            const uint16_t* we = c->w + (int64_t)(e - c->e_begin) * c->moe_inter * c->hidden;
            for (int64_t n = 0; n < width; ++n) y[n] = 0.0;
            for (int64_t kk = 0; kk < c->moe_inter; ++kk) {
                double xv = (double)bf16_bits_to_float(uv[kk]);
                const uint16_t* wrow = we + kk * c->hidden + n0;
                for (int64_t n = 0; n < width; ++n)
                    y[n] += xv * (double)bf16_bits_to_float(wrow[n]);
            }
            for (int64_t n = 0; n < width; ++n) acc[n] += g * y[n];
        }
        for (int64_t n = 0; n < width; ++n) {
            if (c->part64) c->part64[(int64_t)t * c->hidden + n0 + n] = acc[n];
            if (c->part32) c->part32[(int64_t)t * c->hidden + n0 + n] = (float)acc[n];
        }
    }
    free(y);
    free(acc);
}

/*
 * Expert-parallel down projection and local combine [P2, MoE Dispatch-
 * Combine; Expert Parallel]: the rank holds experts [e_begin, e_end); for
 * each token it accumulates, over its selected experts that live on this
 * rank (ascending expert index), the routing weight times that expert's
 * down projection of the token's activation. The result is this rank's
 * partial, which the all-reduce over ranks then sums.
 *
 *   part[t, :] = sum_{s: e_begin <= sel_expert[t,s] < e_end}
 *                    sel_weight[t,s] * (u[t,s,:] . W_e)        (double)
 *
 *   u        bf16 [tokens][top_k][moe_inter]: one activation per selection
 *   w_local  bf16 [e_end-e_begin][moe_inter][hidden]
 *   part64 / part32 [tokens][hidden] (either may be NULL)
 * Pins: with all experts local the partial is the full combine; the
 * partials of all ranks sum to it; a single selection with weight 1 is the
 * dense projection of oracle_partial.
 */
int oracle_moe_partial(int32_t tokens, int32_t top_k, const int32_t* sel_expert,
                       const double* sel_weight, int32_t e_begin, int32_t e_end,
                       const uint16_t* u, const uint16_t* w_local,
                       int64_t moe_inter, int64_t hidden,
                       double* part64, float* part32, int nthreads)
{
    if (tokens < 0 || top_k < 1 || e_end < e_begin) return -1;
    moe_ctx c = {tokens, top_k, e_begin, e_end, sel_expert, sel_weight,
                 u, w_local, moe_inter, hidden, part64, part32};
    for_columns(moe_cols, &c, hidden, nthreads);
    return 0;
}

/* -------------------------------------- column-parallel up projection -- */

/*
 * Column-parallel FFN up projection with its activation [P1, Conceito:
 * under tensor parallelism the FFN's up projection is split over the ranks
 * the other way from its down projection, so rank r holds its columns of
 * the up projection and computes, with no reduction, its own slice of the
 * down projection's input]. The pages name no activation; the reading taken
 * is SwiGLU, with a gate and an up matrix split by the same columns:
 *
 *     g = x . W_gate,  u = x . W_up           (double, ascending k)
 *     a = silu(g) * u,  silu(z) = z / (1 + e^(-z))          (double)
 *     a_bf16 = bf16(float(a))       (nearest-even both times, as stored)
 *
 *   x              bf16 [batch][hidden]
 *   w_gate, w_up   bf16 [hidden][cols] row-major (the rank's columns)
 *   a64            double [batch][cols] (optional)
 *   a_bf16         bf16 bits [batch][cols] (optional)
 *
 * Pins: zero gate weights give a = 0 (silu(0) = 0); a 1x1 case gives
 * silu(1) = sigma(1) = 0.7310585786300049...; negating the gate weights
 * changes a by exactly g*u (silu(z) - silu(-z) = z), with g and u from
 * oracle_partial; a large gate gives a -> g*u.
 */
int oracle_gate_up_swiglu(const uint16_t* x, const uint16_t* w_gate, const uint16_t* w_up,
                          int64_t batch, int64_t hidden, int64_t cols, double* a64,
                          uint16_t* a_bf16, int nthreads)
{
    if (batch < 0 || hidden < 0 || cols < 0) return -1;
    size_t n = (size_t)(batch * cols);
    double* g = (double*)malloc((n ? n : 1) * sizeof(double));
    double* u = (double*)malloc((n ? n : 1) * sizeof(double));
    if (!g || !u) {
        free(g);
        free(u);
        return -1;
    }
    oracle_partial(x, hidden, w_gate, batch, hidden, cols, g, NULL, nthreads);
    oracle_partial(x, hidden, w_up, batch, hidden, cols, u, NULL, nthreads);
    for (size_t i = 0; i < n; ++i) {
        double silu = g[i] / (1.0 + exp(-g[i]));
        double a = silu * u[i];
        if (a64) a64[i] = a;
        if (a_bf16) a_bf16[i] = float_to_bf16_bits((float)a);
    }
    free(g);
    free(u);
    return 0;
}

/*
 * Column-parallel mixer input projection of one rank (lesson 9.9, Conceito:
 * the attention heads are split over the ranks by columns, so a rank
 * computes its heads' Q, K and V columns from the full hidden state, with no
 * reduction; "Hosting Qwen on Blackwell", Prefillers: with fewer key-value
 * heads than ranks the K and V columns are replicated, which only changes
 * which columns a rank holds):
 *     a[b, n] = sum_{h < hidden} x[b, h] * w[h, n]
 * the exact sum (oracle_partial's fp64 accumulation) rounded to bf16
 * nearest-even through binary32, as the activation is stored.
 *   x bf16 [batch][hidden], w bf16 [hidden][cols] (the rank's columns)
 *   a64 [batch][cols] (may be NULL), a_bf16 [batch][cols] (may be NULL)
 * Pins: a permutation matrix gives a column permutation of x (bits equal),
 * small-integer inputs give the exact integer sums of a brute-force loop,
 * and the columns of a wide matrix split into slices give the slices of the
 * wide result.
 */
int oracle_qkv_proj(const uint16_t* x, const uint16_t* w, int64_t batch, int64_t hidden,
                    int64_t cols, double* a64, uint16_t* a_bf16, int nthreads)
{
    if (batch < 0 || hidden < 0 || cols < 0) return -1;
    size_t n = (size_t)(batch * cols);
    double* y = (double*)malloc((n ? n : 1) * sizeof(double));
    if (!y) return -1;
    oracle_partial(x, hidden, w, batch, hidden, cols, y, NULL, nthreads);
    for (size_t i = 0; i < n; ++i) {
        if (a64) a64[i] = y[i];
        if (a_bf16) a_bf16[i] = float_to_bf16_bits((float)y[i]);
    }
    free(y);
    return 0;
}

/* ------------------------------------------ microscaled (MX) weights -- */

/*
 * Block-scaled weights [P2, Quantization]: the pages deploy their model with
 * its weights converted once, statically, to MXFP8, and weigh MXFP4 as well.
 * The pages give the format names only; the reading taken here is the
 * microscaling (MX) layout those names denote: the weights are cut into
 * blocks of 32 consecutive elements along K (the reduction dimension, rows
 * of W[K, H]), each block shares one 8-bit power-of-two scale
 * E (value 2^(E-127); E = 255 means NaN), and each element is a small float:
 *
 *   fmt 1, MXFP8: FP8 E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa
 *                 bits; no infinities; S.1111.111 is NaN; largest 448)
 *   fmt 2, MXFP4: FP4 E2M1 (sign, 2 exponent bits with bias 1, 1 mantissa
 *                 bit; no infinities or NaN; largest 6)
 *
 * A weight is element * 2^(E-127), held exactly in double here.
 */
#define MX_BLOCK 32

/* The value of one element code, from its sign, exponent and mantissa
 * fields. */
static double mx_elem_value(int fmt, unsigned code)
{
    if (fmt == 1) {
        const int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
        if (e == 15 && m == 7) return NAN;
        /* normal: (1 + m/8) 2^(e-7); subnormal (e = 0): (m/8) 2^-6 */
        const double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
        return s ? -v : v;
    } else {
        const int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
        /* normal: (1 + m/2) 2^(e-1); subnormal (e = 0): m/2 */
        const double v = e == 0 ? 0.5 * m : ldexp((double)(2 + m), e - 2);
        return s ? -v : v;
    }
}

double oracle_mx_element_value(int32_t fmt, uint32_t code)
{
    if (fmt != 1 && fmt != 2) return NAN;
    return mx_elem_value(fmt, code & (fmt == 1 ? 0xffu : 0xfu));
}

/* Exponent of the element format's largest binade (448 = 1.75 * 2^8,
 * 6 = 1.5 * 2^2). */
static int mx_emax(int fmt) { return fmt == 1 ? 8 : 2; }

/* Round v (already divided by the block's scale) to the nearest element
 * value: the non-negative codes are listed in increasing value, so the
 * candidates are the largest code not above |v| and the next one; a tie
 * goes to the even code (an even mantissa); |v| beyond the largest finite
 * value saturates to it. The sign of v is kept (so -0 for a negative v
 * that rounds to zero). */
static unsigned mx_round(int fmt, double v)
{
    const unsigned ncodes = fmt == 1 ? 0x7fu : 0x8u; /* finite non-negative codes */
    const double a = fabs(v);
    /* the largest code whose value is not above a (values increase with the
     * code): a binary search over [0, ncodes) */
    unsigned lo = 0, hi = ncodes;
    while (hi - lo > 1) {
        const unsigned mid = (lo + hi) / 2;
        if (mx_elem_value(fmt, mid) <= a) lo = mid;
        else hi = mid;
    }
    unsigned code = lo;
    if (lo + 1 < ncodes) {
        const double dl = a - mx_elem_value(fmt, lo), dh = mx_elem_value(fmt, lo + 1) - a;
        if (dh < dl || (dh == dl && (lo & 1u))) code = lo + 1;
    }
    return code | (signbit(v) ? (fmt == 1 ? 0x80u : 0x8u) : 0u);
}

/*
 * Static conversion of bf16 weights to an MX format, block by block:
 *   amax = max |w| over the block's 32 rows (one column);
 *   E = floor(log2(amax)) - emax + 127, clamped to [0, 254]  (so that
 *       amax / 2^(E-127) lies in the element format's top binade,
 *       [2^emax, 2^(emax+1)), unless clamped);
 *   E = 0 for an all-zero block; E = 255 (NaN) if the block holds a NaN or
 *       infinity, with every element code 0;
 *   element = mx_round(w / 2^(E-127)).
 * Layouts (K a multiple of 32):
 *   w      bf16 [K][H] row-major
 *   codes  fmt 1: uint8 [K][H], one E4M3 code per weight;
 *          fmt 2: uint8 [K/2][H], byte [kk][n] = code(2kk, n) | code(2kk+1, n) << 4
 *   scales uint8 [K/32][H], E of rows [32kb, 32kb+32) of column n
 * Returns 0, or 1 for a bad format or size.
 *
 * Pins: element values of every code (E4M3 against an independent
 * conversion library, E2M1 against the format's table of values); blocks
 * built from representable values round-trip exactly; the scaled block
 * maximum lands in the top binade; saturation and ties on hand-made
 * blocks; the quantisation error of each element is within half an element
 * spacing.
 */
int oracle_mx_quantize(int32_t fmt, const uint16_t* w, int64_t K, int64_t H, uint8_t* codes,
                       uint8_t* scales)
{
    if ((fmt != 1 && fmt != 2) || K < MX_BLOCK || K % MX_BLOCK || H < 1) return 1;
    if (fmt == 2) memset(codes, 0, (size_t)(K / 2 * H));
    for (int64_t kb = 0; kb < K / MX_BLOCK; ++kb)
        for (int64_t n = 0; n < H; ++n) {
            double amax = 0.0;
            int finite = 1;
            for (int i = 0; i < MX_BLOCK; ++i) {
                const double v = (double)bf16_bits_to_float(w[(kb * MX_BLOCK + i) * H + n]);
                if (!isfinite(v)) finite = 0;
                else if (fabs(v) > amax) amax = fabs(v);
            }
            unsigned E;
            if (!finite) {
                E = 255;
            } else if (amax == 0.0) {
                E = 0;
            } else {
                int e2;
                frexp(amax, &e2); /* amax = f 2^e2, f in [0.5, 1): floor(log2 amax) = e2 - 1 */
                const long se = (long)(e2 - 1) - mx_emax(fmt) + 127;
                E = se < 0 ? 0u : se > 254 ? 254u : (unsigned)se;
            }
            scales[kb * H + n] = (uint8_t)E;
            for (int i = 0; i < MX_BLOCK; ++i) {
                const int64_t k = kb * MX_BLOCK + i;
                const double v = (double)bf16_bits_to_float(w[k * H + n]);
                const unsigned c = E == 255 ? 0u : mx_round(fmt, ldexp(v, 127 - (int)E));
                if (fmt == 1)
                    codes[k * H + n] = (uint8_t)c;
                else
                    codes[(k / 2) * H + n] |= (uint8_t)(c << (k % 2 ? 4 : 0));
            }
        }
    return 0;
}

/* Weight (k, n) of an MX matrix, exactly. */
static double mx_weight(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t H,
                        int64_t k, int64_t n)
{
    const unsigned E = scales[(k / MX_BLOCK) * H + n];
    if (E == 255) return NAN;
    unsigned c;
    if (fmt == 1)
        c = codes[k * H + n];
    else
        c = (codes[(k / 2) * H + n] >> (k % 2 ? 4 : 0)) & 0xfu;
    return ldexp(mx_elem_value(fmt, c), (int)E - 127);
}

typedef struct {
    int fmt;
    const uint16_t* x;
    const uint8_t* codes;
    const uint8_t* scales;
    int64_t batch, k, hidden;
    double* y64;
    float* y32;
} mx_ctx;

static void mx_cols(void* p, int64_t n0, int64_t n1)
{
    mx_ctx* c = (mx_ctx*)p;
    for (int64_t b = 0; b < c->batch; ++b)
        for (int64_t n = n0; n < n1; ++n) {
            /* y[b,n] = sum over k of x[b,k] * W[k,n], ascending k, in double:
             * each product of a bf16 and an MX weight is exact */
            double acc = 0.0;
            for (int64_t kk = 0; kk < c->k; ++kk)
                acc += (double)bf16_bits_to_float(c->x[b * c->k + kk]) *
                       mx_weight(c->fmt, c->codes, c->scales, c->hidden, kk, n);
            if (c->y64) c->y64[b * c->hidden + n] = acc;
            if (c->y32) c->y32[b * c->hidden + n] = (float)acc;
        }
}

/*
 * The row-parallel partial projection [P1, Conceito] on MX weights:
 * p[b, n] = sum_k x[b, k] * W[k, n], with W decoded exactly from codes and
 * scales (layouts as oracle_mx_quantize), x bf16 [batch][K]; summed in
 * double, rounded once to float. Returns 0, or 1 for a bad format or size.
 *
 * Pins: with every scale 127 and every element a bf16 value it equals
 * oracle_partial on those values bit for bit; raising every scale by one
 * doubles every output exactly; exact big-rational brute force on tiny
 * shapes.
 */
int oracle_mx_partial(int32_t fmt, const uint16_t* x, int64_t batch, int64_t K, int64_t H,
                      const uint8_t* codes, const uint8_t* scales, double* y64, float* y32,
                      int nthreads)
{
    if ((fmt != 1 && fmt != 2) || K < MX_BLOCK || K % MX_BLOCK || H < 1 || batch < 1) return 1;
    mx_ctx c = {fmt, x, codes, scales, batch, K, H, y64, y32};
    for_columns(mx_cols, &c, H, nthreads);
    return 0;
}
