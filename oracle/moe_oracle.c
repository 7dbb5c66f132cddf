/*
 * moe_oracle.c -- plain, slow, scalar CPU oracle for the MoE token
 * permute / unpermute path and the fused chunk sort-and-pad / restore pair.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the
 * entry module and the CPU-baseline leg of the benchmark may load it.  The
 * product library never links, calls or includes anything from here, and
 * this file includes nothing from the product sources.
 *
 * Every function is the plain definition of its step, written as loops in
 * the order the pages describe, with no blocking, fusion or reordering:
 *
 *   oracle_row_id_map*      -- stable counting sort: per-expert counts, an
 *                              exclusive scan, then a cursor walk over the
 *                              (token, expert) pairs in token order.
 *   oracle_permute          -- bitwise row copies token -> destination rows.
 *   oracle_unpermute        -- fp32 fused multiply-adds of prob x row, in
 *                              top-k slot order, starting from +0, rounded
 *                              once to bf16.
 *   oracle_unpermute_bwd    -- act-grad scatter (fp32 product, then bf16)
 *                              and prob-grad row dot products (exact
 *                              products summed in fp64, rounded once).
 *   oracle_permute_bwd      -- slot-order fp32 sum of the k gradient rows.
 *   oracle_unpermute_ep     -- the same combine with experts split into EP
 *                              ranks: per-rank slot-order partials (optionally
 *                              rounded to bf16) added in rank order (fp32 or
 *                              fp64), then bf16.
 *   oracle_topk_softmax(_bwd) -- top-k selection + softmax router and its
 *                              gradient (fp64 arithmetic, rounded once).
 *   oracle_mask_row_id_map  -- TE mask-map form: [T][2E+1] per-token map
 *                              from a [T][E] routing mask, with dropping.
 *   oracle_mask_permute / oracle_mask_unpermute(_bwd)
 *                           -- the TE-order copies and combine on that map.
 *   oracle_permute_scaled / oracle_mask_permute_scaled
 *                           -- quantized (e.g. FP8) rows with their scale rows.
 *   oracle_chunk_map        -- padded destination -> source row map.
 *   oracle_sort_chunks_and_pad / oracle_unpad_and_restore_chunks
 *                           -- the two copies driven by that map.
 *
 * bf16 values travel as their 16-bit patterns (uint16_t).  The conversions
 * below are written from the IEEE 754 definitions: widening is exact, and
 * narrowing is round-to-nearest, ties-to-even on the 16 discarded bits.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math -fopenmp -shared
 * -fPIC.  -ffp-contract=off keeps every a*b+c that is not an explicit fmaf()
 * as two roundings.
 *
 * Threads: the per-token loops of the row copies, the combines and their
 * backwards run their tokens on OpenMP threads (oracle_set_threads).  Each
 * token's outputs are computed by one thread with the same scalar loop, and
 * no two tokens write the same output, so the results do not depend on the
 * thread count.  Those functions first check every slot in token order,
 * serially, and return the first error before any output is written.
 *
 * Parity unpinned at the bit level: the prob-grad dot products of
 * oracle_unpermute_bwd and oracle_mask_unpermute_bwd (the pages leave the
 * summation order open) and the router's softmax weights and gradients
 * (fp32 exponentials the pages do not fix).  Each is computed here in fp64
 * and rounded once; the GPU results are held to it within a stated bound.
 * The tests pin the dots to a numpy fp64 dot of the widened rows and the
 * router to a stable sort with a library softmax and its autograd.
 *
 * Return codes (all functions): 0 ok, otherwise one of the ORC_* values.
 * Outputs are unspecified after an error.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD_EXPERT 1   /* an expert index outside [0, E)               */
#define ORC_DUP_EXPERT 2   /* one expert twice in a token's routing        */
#define ORC_BAD_ARG 3      /* a size or shape argument out of range        */
#define ORC_BAD_ROW 4      /* a map entry pointing outside its buffer      */
#define ORC_BAD_CHUNKS 5   /* negative split size / order not a permutation */
#define ORC_OVERFLOW 6     /* tokens exceed the input capacity, or padded
                              groups exceed the output capacity            */
#define ORC_NO_MEM 7
#define ORC_BAD_ORDER 8    /* pair list not in non-decreasing token order  */

/* ---- bf16 <-> fp32, from the bfloat16 / IEEE 754 binary32 layouts ----- */

static float bf16_to_f32(uint16_t b)
{
    /* bf16 is the top half of a binary32: widening appends 16 zero bits. */
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t exponent = (u >> 23) & 0xffu;
    uint32_t mantissa = u & 0x7fffffu;
    if (exponent == 0xffu && mantissa != 0u) {
        /* NaN: keep sign and the upper payload bits, force the quiet bit. */
        return (uint16_t)((u >> 16) | 0x0040u);
    }
    uint32_t kept = u >> 16;          /* sign, exponent, 7 mantissa bits */
    uint32_t dropped = u & 0xffffu;   /* the 16 bits rounded away        */
    if (dropped > 0x8000u) {
        kept += 1u;                   /* above the halfway point: up     */
    } else if (dropped == 0x8000u) {
        if (kept & 1u) kept += 1u;    /* exactly halfway: to even        */
    }
    /* A carry out of the mantissa increments the exponent, which is the
       correct next representable value (up to +-Inf on overflow). */
    return (uint16_t)kept;
}

uint16_t oracle_f32_to_bf16(float f) { return f32_to_bf16_rne(f); }

/* Threads of the per-token loops (n < 1 keeps the current setting); returns
   the number the next such loop uses. */
int oracle_set_threads(int n)
{
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
}
float oracle_bf16_to_f32(uint16_t b) { return bf16_to_f32(b); }
float oracle_fmaf(float a, float b, float c) { return fmaf(a, b, c); }

/* ---- (1) row map: stable counting sort --------------------------------- */

/*
 * Core of the row map, over an explicit list of routed (token, expert)
 * pairs given in non-decreasing token order.
 *
 * d9d 0.1.0, permute_with_probs.py, make_row_id_map: the worked example in
 * its comments shows that after the second pass the destination rows run
 * expert-major (all rows of expert 0 first) and, inside one expert, in
 * ascending token order.  moe-ops README, "Why this library": the permute
 * is a counting sort (histogram + exclusive prefix sum).  That is exactly:
 *   count[e]   = number of pairs with expert e
 *   offset[e]  = count[0] + ... + count[e-1]         (exclusive scan)
 *   walking the pairs in token order, the next pair of expert e takes
 *   row offset[e] + (pairs of e already placed).
 * Output: row_id_map[e * T + t] = row, or -1 when t is not routed to e;
 *         expert_offsets[0..E] = the exclusive scan, expert_offsets[E] =
 *         number of pairs.
 */
int oracle_row_id_map_pairs(const int32_t *pair_token, const int32_t *pair_expert,
                            int64_t npairs, int T, int E,
                            int32_t *row_id_map, int32_t *expert_offsets)
{
    if (T < 0 || E < 1 || npairs < 0) return ORC_BAD_ARG;
    for (int64_t i = 0; i < npairs; i++) {
        if (pair_token[i] < 0 || pair_token[i] >= T) return ORC_BAD_ARG;
        if (pair_expert[i] < 0 || pair_expert[i] >= E) return ORC_BAD_EXPERT;
        if (i > 0 && pair_token[i] < pair_token[i - 1]) return ORC_BAD_ORDER;
    }
    int64_t *count = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    int64_t *cursor = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    if (!count || !cursor) { free(count); free(cursor); return ORC_NO_MEM; }

    for (int64_t i = 0; i < npairs; i++) count[pair_expert[i]] += 1;

    int64_t running = 0;
    for (int e = 0; e < E; e++) {
        expert_offsets[e] = (int32_t)running;
        cursor[e] = running;
        running += count[e];
    }
    expert_offsets[E] = (int32_t)running;

    for (int64_t i = 0; i < (int64_t)E * T; i++) row_id_map[i] = -1;

    int status = ORC_OK;
    for (int64_t i = 0; i < npairs; i++) {
        int t = pair_token[i];
        int e = pair_expert[i];
        int64_t slot = (int64_t)e * T + t;
        if (row_id_map[slot] != -1) { status = ORC_DUP_EXPERT; break; }
        row_id_map[slot] = (int32_t)cursor[e];
        cursor[e] += 1;
    }
    free(count);
    free(cursor);
    return status;
}

/*
 * Row map from top-k routing: topk_idx[t * k + j] is token t's j-th expert.
 * The pairs are (t, topk_idx[t][j]) for t ascending, then j ascending; with
 * the experts of one token distinct this is the same map as a stable argsort
 * of the flattened top-k index array (xtuner issue "permute different with
 * torch version", maintainer's reply).
 */
int oracle_row_id_map(const int32_t *topk_idx, int T, int k, int E,
                      int32_t *row_id_map, int32_t *expert_offsets)
{
    if (T < 0 || k < 1 || E < 1) return ORC_BAD_ARG;
    int64_t n = (int64_t)T * k;
    int32_t *pt = (int32_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int32_t));
    int32_t *pe = (int32_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int32_t));
    if (!pt || !pe) { free(pt); free(pe); return ORC_NO_MEM; }
    for (int t = 0; t < T; t++) {
        for (int j = 0; j < k; j++) {
            pt[(int64_t)t * k + j] = t;
            pe[(int64_t)t * k + j] = topk_idx[(int64_t)t * k + j];
        }
    }
    int status = oracle_row_id_map_pairs(pt, pe, n, T, E, row_id_map, expert_offsets);
    free(pt);
    free(pe);
    return status;
}

/* Destination row of token t's slot j, with bounds checks. */
static int slot_row(const int32_t *topk_idx, const int32_t *row_id_map,
                    int T, int k, int E, int64_t n_rows, int t, int j, int64_t *row)
{
    int e = topk_idx[(int64_t)t * k + j];
    if (e < 0 || e >= E) return ORC_BAD_EXPERT;
    int32_t r = row_id_map[(int64_t)e * T + t];
    if (r < 0 || (int64_t)r >= n_rows) return ORC_BAD_ROW;
    *row = r;
    return ORC_OK;
}

/* The first bad slot in token order, walking (t, j) as the loops below do. */
static int check_slots(const int32_t *topk_idx, const int32_t *row_id_map,
                       int T, int k, int E, int64_t n_rows)
{
    for (int t = 0; t < T; t++) {
        for (int j = 0; j < k; j++) {
            int64_t r;
            int s = slot_row(topk_idx, row_id_map, T, k, E, n_rows, t, j, &r);
            if (s) return s;
        }
    }
    return ORC_OK;
}

/* Destination row of a slot that check_slots has accepted. */
static int64_t dest_row(const int32_t *topk_idx, const int32_t *row_id_map, int T, int k,
                        int t, int j)
{
    return row_id_map[(int64_t)topk_idx[(int64_t)t * k + j] * T + t];
}

/* ---- (2) permute -------------------------------------------------------- */

/*
 * d9d permute_with_probs.py, _permute_kernel: each token's hidden row is
 * stored unchanged to every destination row it is routed to, and with
 * probabilities the token's probability for that expert is stored at the
 * same destination index.  (The kernel's zero-row rule for a probability of
 * exactly 0.0 serves mask-map padding and is not part of this path.)
 * out is [T*k][H] bf16 bits; out_probs [T*k] (may be NULL).
 */
int oracle_permute(const uint16_t *x, const float *probs, const int32_t *topk_idx,
                   const int32_t *row_id_map, int T, int H, int k, int E,
                   uint16_t *out, float *out_probs)
{
    if (T < 0 || H < 1 || k < 1 || E < 1) return ORC_BAD_ARG;
    int64_t n_rows = (int64_t)T * k;
    int status = check_slots(topk_idx, row_id_map, T, k, E, n_rows);
    if (status) return status;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++) {
        for (int j = 0; j < k; j++) {
            int64_t r = dest_row(topk_idx, row_id_map, T, k, t, j);
            for (int h = 0; h < H; h++) out[r * H + h] = x[(int64_t)t * H + h];
            if (probs && out_probs) out_probs[r] = probs[(int64_t)t * k + j];
        }
    }
    return ORC_OK;
}

/* ---- (4) unpermute combine ---------------------------------------------- */

/*
 * Megatron-core core.transformer.moe.batch_invariant,
 * unpermute_with_bf16_rank_partials (and _rank_tree_unpermute_kernel with
 * BF16_RANK_PARTIALS): per output element, an fp32 accumulator begins at
 * zero and takes one fused multiply-add per routed slot (probability times
 * the slot's row value), slots visited in the column order of the [tokens,
 * topk] routing; the final value is rounded once to bf16.  With a single EP
 * rank this is the whole combine.
 *   acc = +0.0f
 *   for j = 0 .. k-1:  acc = fmaf(p[t][j], float(in[r_j][h]), acc)
 *   out[t][h] = bf16_rne(acc)
 * probs == NULL means unit weights; fmaf(1, x, acc) is then exactly acc + x.
 * in is [n_rows][H] bf16 bits (n_rows = T*k normally).
 */
int oracle_unpermute(const uint16_t *in, const float *probs, const int32_t *topk_idx,
                     const int32_t *row_id_map, int T, int H, int k, int E,
                     int64_t n_rows, uint16_t *out)
{
    if (T < 0 || H < 1 || k < 1 || E < 1) return ORC_BAD_ARG;
    int status = check_slots(topk_idx, row_id_map, T, k, E, n_rows);
    if (status) return status;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++) {
        for (int h = 0; h < H; h++) {
            float acc = +0.0f;
            for (int j = 0; j < k; j++) {
                int64_t r = dest_row(topk_idx, row_id_map, T, k, t, j);
                float p = probs ? probs[(int64_t)t * k + j] : 1.0f;
                acc = fmaf(p, bf16_to_f32(in[r * H + h]), acc);
            }
            out[(int64_t)t * H + h] = f32_to_bf16_rne(acc);
        }
    }
    return ORC_OK;
}

/* ---- EP rank-ordered combine (one GPU) ----------------------------------- */

/*
 * binary64 -> bf16, round to nearest, ties to even, written from the
 * definition: the bf16 grid near |d| has quantum 2^(e-8) for |d| in
 * [2^(e-1), 2^e) (8 significant bits), never finer than the smallest bf16
 * subnormal 2^-133; round |d| / quantum to the nearest integer (ties to
 * even, nearbyint in the default rounding mode), scale back, and saturate
 * to infinity above the largest finite bf16.
 */
static uint16_t f64_to_bf16_rne(double d)
{
    if (isnan(d)) {
        float f = (float)d;
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        return (uint16_t)((u >> 16) | 0x0040u);
    }
    double a = fabs(d);
    double r;
    if (a == 0.0 || isinf(a)) {
        r = a;
    } else {
        int e;
        frexp(a, &e);                           /* a = m * 2^e, m in [0.5, 1) */
        int qexp = e - 8;
        if (qexp < -133) qexp = -133;
        double q = ldexp(1.0, qexp);
        r = nearbyint(a / q) * q;               /* a / q is exact (power of 2) */
        const double max_bf16 = ldexp(255.0, 120); /* 0x7F7F: (2 - 2^-7) * 2^127 */
        if (r > max_bf16) r = INFINITY;
    }
    float f = (float)(signbit(d) ? -r : r);     /* exact: r is on the bf16 grid */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

uint16_t oracle_f64_to_bf16(double d) { return f64_to_bf16_rne(d); }

/*
 * Megatron-core core.transformer.moe.batch_invariant: the loop reference
 * (_unpermute_loop) walks EP ranks in order and, inside a rank, the token's
 * slots in top-k order; in the BF16_RANK_PARTIALS form
 * (unpermute_with_bf16_rank_partials) a rank's slots build an fp32 partial
 * by fused multiply-adds from zero, and the partial is rounded to bf16
 * before the ranks are summed; CROSS_RANK_FP64 sums the ranks in fp64.  On one GPU the ranks are expert ranges: the E experts split into
 * ep_size equal ranges, rank(e) = e / (E / ep_size).
 *   total = 0 (fp32, or fp64)
 *   for rank = 0 .. ep_size-1:
 *       partial = +0.0f
 *       for j = 0 .. k-1 with rank(topk_idx[t][j]) == rank:
 *           partial = fmaf(p[t][j], in[r_j][h], partial)
 *       if bf16_partials: partial = bf16_rne(partial)
 *       total = total + partial
 *   out[t][h] = bf16_rne(total)
 * probs == NULL means unit weights.
 */
int oracle_unpermute_ep(const uint16_t *in, const float *probs, const int32_t *topk_idx,
                        const int32_t *row_id_map, int T, int H, int k, int E, int64_t n_rows,
                        int ep_size, int bf16_partials, int fp64_cross, uint16_t *out)
{
    if (T < 0 || H < 1 || k < 1 || E < 1 || ep_size < 1 || E % ep_size != 0) return ORC_BAD_ARG;
    int per_rank = E / ep_size;
    int status = check_slots(topk_idx, row_id_map, T, k, E, n_rows);
    if (status) return status;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++) {
        for (int h = 0; h < H; h++) {
            float total32 = 0.0f;
            double total64 = 0.0;
            for (int rank = 0; rank < ep_size; rank++) {
                float partial = +0.0f;
                for (int j = 0; j < k; j++) {
                    int64_t r = dest_row(topk_idx, row_id_map, T, k, t, j);
                    if (topk_idx[(int64_t)t * k + j] / per_rank != rank) continue;
                    float p = probs ? probs[(int64_t)t * k + j] : 1.0f;
                    partial = fmaf(p, bf16_to_f32(in[r * H + h]), partial);
                }
                if (bf16_partials) partial = bf16_to_f32(f32_to_bf16_rne(partial));
                if (fp64_cross)
                    total64 = total64 + (double)partial;
                else
                    total32 = total32 + partial;
            }
            out[(int64_t)t * H + h] = fp64_cross ? f64_to_bf16_rne(total64)
                                                 : f32_to_bf16_rne(total32);
        }
    }
    return ORC_OK;
}

/* ---- unpermute backward ------------------------------------------------- */

/*
 * d9d permute_with_probs.py, _unpermute_bwd_with_merging_probs_kernel:
 *   act grad:  d_in[r_j][h] = bf16(fp32(d_out[t][h]) * p[t][j])
 *              (an fp32 product rounded to fp32, then cast to bf16; there is
 *              no addition, so no fused operation),
 *   prob grad: d_probs[t][j] = sum_h float(fwd_in[r_j][h]) * float(d_out[t][h]).
 * Megatron batch_invariant, _rank_tree_unpermute_bwd_kernel: a permuted row
 * is owned by exactly one (token, slot) pair, hence one write per row in the
 * scatter.
 * The pages leave the order of the prob-grad sum open; here each product of
 * two bf16 values is exact in fp64 and the products are summed in fp64, with
 * one final rounding to fp32 (a tolerance covers any fp32 order).
 * probs == NULL: d_in[r_j] = d_out[t] bitwise and d_probs is not written.
 */
int oracle_unpermute_bwd(const uint16_t *d_out, const uint16_t *fwd_in, const float *probs,
                         const int32_t *topk_idx, const int32_t *row_id_map,
                         int T, int H, int k, int E, int64_t n_rows,
                         uint16_t *d_in, float *d_probs)
{
    if (T < 0 || H < 1 || k < 1 || E < 1) return ORC_BAD_ARG;
    int status = check_slots(topk_idx, row_id_map, T, k, E, n_rows);
    if (status) return status;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++) {
        for (int j = 0; j < k; j++) {
            int64_t r = dest_row(topk_idx, row_id_map, T, k, t, j);
            if (probs) {
                float p = probs[(int64_t)t * k + j];
                for (int h = 0; h < H; h++) {
                    float g = bf16_to_f32(d_out[(int64_t)t * H + h]);
                    float prod = g * p;          /* one fp32 rounding */
                    d_in[r * H + h] = f32_to_bf16_rne(prod);
                }
                if (d_probs && fwd_in) {
                    double dot = 0.0;
                    for (int h = 0; h < H; h++) {
                        double a = (double)bf16_to_f32(fwd_in[r * H + h]);
                        double b = (double)bf16_to_f32(d_out[(int64_t)t * H + h]);
                        dot += a * b;
                    }
                    d_probs[(int64_t)t * k + j] = (float)dot;
                }
            } else {
                for (int h = 0; h < H; h++) d_in[r * H + h] = d_out[(int64_t)t * H + h];
            }
        }
    }
    return ORC_OK;
}

/* ---- permute backward --------------------------------------------------- */

/*
 * d9d permute_with_probs.py, _moe_permute_mask_map.backward: the permute's
 * gradient is the unweighted unpermute of the permuted gradient, and the
 * permuted-probability gradient is gathered back to each token's slots.
 *   d_x[t][h]        = bf16_rne(((+0 + g_0) + g_1) + ... + g_{k-1}),
 *                      g_j = float(d_out[r_j][h]), fp32, slot order
 *   d_probs[t][j]    = d_out_probs[r_j]
 */
int oracle_permute_bwd(const uint16_t *d_out, const float *d_out_probs, const int32_t *topk_idx,
                       const int32_t *row_id_map, int T, int H, int k, int E, int64_t n_rows,
                       uint16_t *d_x, float *d_probs)
{
    if (T < 0 || H < 1 || k < 1 || E < 1) return ORC_BAD_ARG;
    int status = check_slots(topk_idx, row_id_map, T, k, E, n_rows);
    if (status) return status;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++) {
        for (int h = 0; h < H; h++) {
            float acc = +0.0f;
            for (int j = 0; j < k; j++) {
                int64_t r = dest_row(topk_idx, row_id_map, T, k, t, j);
                acc = acc + bf16_to_f32(d_out[r * H + h]);
            }
            d_x[(int64_t)t * H + h] = f32_to_bf16_rne(acc);
        }
        if (d_out_probs && d_probs) {
            for (int j = 0; j < k; j++) {
                int64_t r = dest_row(topk_idx, row_id_map, T, k, t, j);
                d_probs[(int64_t)t * k + j] = d_out_probs[r];
            }
        }
    }
    return ORC_OK;
}

/* ---- fused top-k softmax router ------------------------------------------ */

/*
 * moe-ops README, "Fused Top-K Softmax": top-k selection and a softmax
 * over the selected logits; the fp32_routing option there keeps the weights
 * in fp32, otherwise they come in the activation dtype.  Per token:
 *   the k largest logits, in descending order, a tie going to the lower
 *   expert index (repeated selection of the maximum of the rest);
 *   w_j = exp(l_j - l_max) / sum_i exp(l_i - l_max) over the k selected,
 *   in fp64, rounded once to fp32 (prob_bytes 4) or bf16 (prob_bytes 2).
 * logits: [T][E] of elem_bytes 2 (bf16 bits) or 4 (fp32); NaN logits are
 * not supported.
 */
int oracle_topk_softmax(const void *logits, int elem_bytes, int T, int E, int k,
                        int32_t *topk_idx, void *probs, int prob_bytes)
{
    if (T < 0 || E < 1 || k < 1 || k > E || (elem_bytes != 2 && elem_bytes != 4) ||
        (prob_bytes != 2 && prob_bytes != 4))
        return ORC_BAD_ARG;
    char *taken = (char *)malloc((size_t)E);
    double *lv = (double *)malloc((size_t)k * sizeof(double));
    if (!taken || !lv) { free(taken); free(lv); return ORC_NO_MEM; }
    for (int t = 0; t < T; t++) {
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; j++) {
            int best = -1;
            double bv = 0.0;
            for (int e = 0; e < E; e++) {
                if (taken[e]) continue;
                double v = elem_bytes == 2
                               ? (double)bf16_to_f32(((const uint16_t *)logits)[(int64_t)t * E + e])
                               : (double)((const float *)logits)[(int64_t)t * E + e];
                if (best < 0 || v > bv) { best = e; bv = v; }
            }
            taken[best] = 1;
            topk_idx[(int64_t)t * k + j] = best;
            lv[j] = bv;
        }
        double sum = 0.0;
        for (int j = 0; j < k; j++) sum += exp(lv[j] - lv[0]);
        for (int j = 0; j < k; j++) {
            double w = exp(lv[j] - lv[0]) / sum;
            if (prob_bytes == 4)
                ((float *)probs)[(int64_t)t * k + j] = (float)w;
            else
                ((uint16_t *)probs)[(int64_t)t * k + j] = f64_to_bf16_rne(w);
        }
    }
    free(taken);
    free(lv);
    return ORC_OK;
}

/*
 * Gradient of the router weights w.r.t. the logits (same section: exact
 * softmax gradients scattered back to the logits): for the selected
 * experts, d_logits[t][e_j] = w_j * (d_probs[t][j] - sum_i w_i d_probs[t][i])
 * in fp64, rounded once to the output type; 0 for the experts not selected.
 * Weights and their gradients come as fp32 or bf16 (prob_bytes 4 or 2, read
 * exactly); d_logits is fp32 or bf16 (logit_bytes 4 or 2).
 */
static double load_real(const void *p, int bytes, int64_t i)
{
    return bytes == 4 ? (double)((const float *)p)[i]
                      : (double)bf16_to_f32(((const uint16_t *)p)[i]);
}

static void store_real(void *p, int bytes, int64_t i, double v)
{
    if (bytes == 4)
        ((float *)p)[i] = (float)v;
    else
        ((uint16_t *)p)[i] = f64_to_bf16_rne(v);
}

int oracle_topk_softmax_bwd(const void *d_probs, const void *probs, int prob_bytes,
                            const int32_t *topk_idx, int T, int E, int k, void *d_logits,
                            int logit_bytes)
{
    if (T < 0 || E < 1 || k < 1 || k > E || (prob_bytes != 2 && prob_bytes != 4) ||
        (logit_bytes != 2 && logit_bytes != 4))
        return ORC_BAD_ARG;
    for (int64_t i = 0; i < (int64_t)T * E; i++) store_real(d_logits, logit_bytes, i, 0.0);
    for (int t = 0; t < T; t++) {
        double dot = 0.0;
        for (int j = 0; j < k; j++)
            dot += load_real(probs, prob_bytes, (int64_t)t * k + j) *
                   load_real(d_probs, prob_bytes, (int64_t)t * k + j);
        for (int j = 0; j < k; j++) {
            int e = topk_idx[(int64_t)t * k + j];
            if (e < 0 || e >= E) return ORC_BAD_EXPERT;
            double w = load_real(probs, prob_bytes, (int64_t)t * k + j);
            double dp = load_real(d_probs, prob_bytes, (int64_t)t * k + j);
            store_real(d_logits, logit_bytes, (int64_t)t * E + e, w * (dp - dot));
        }
    }
    return ORC_OK;
}

/* ---- TE mask-map interop ------------------------------------------------ */

/*
 * d9d permute_with_probs.py (TransformerEngine mask-map permutation),
 * make_row_id_map and its worked example.  routing_map[t][e] != 0 routes
 * token t to expert e (mask_bytes 1 or 4).  Passes 1 and 2 give every routed
 * pair its destination row: rows run expert-major, tokens ascending inside
 * an expert.  Token dropping (moe_permute_with_probs, num_out_tokens: the
 * count of rows not dropped): a row at or beyond num_out is dropped and
 * becomes -1; num_out < 0 keeps every row.  Pass 3 then stores, per token,
 * its kept rows sorted descending in map[t][0..n), the matching experts in
 * map[t][E..E+n) and n in map[t][2E]; the entries the page leaves unused
 * are set to -1 here.  expert_offsets[e] = kept rows of experts below e.
 */
struct row_expert { int32_t row, expert; };

static int by_row_descending(const void *a, const void *b)
{
    const struct row_expert *x = (const struct row_expert *)a;
    const struct row_expert *y = (const struct row_expert *)b;
    return (x->row < y->row) - (x->row > y->row);
}

int oracle_mask_row_id_map(const void *routing_map, int mask_bytes, int T, int E, int num_out,
                           int32_t *map, int32_t *expert_offsets)
{
    if (T < 0 || E < 1 || (mask_bytes != 1 && mask_bytes != 4)) return ORC_BAD_ARG;
    const int64_t W = 2 * (int64_t)E + 1;
    int32_t *dense = (int32_t *)malloc(((size_t)T * E + 1) * sizeof(int32_t));
    struct row_expert *tok = (struct row_expert *)malloc((size_t)E * sizeof *tok);
    if (!dense || !tok) { free(dense); free(tok); return ORC_NO_MEM; }
    /* passes 1 and 2: the state [t][e] = destination row or -1 */
    int64_t row = 0;
    for (int e = 0; e < E; e++) {
        if (expert_offsets) expert_offsets[e] = (int32_t)(num_out >= 0 && row > num_out ? num_out : row);
        for (int t = 0; t < T; t++) {
            int routed = mask_bytes == 1
                             ? ((const uint8_t *)routing_map)[(int64_t)t * E + e] != 0
                             : ((const int32_t *)routing_map)[(int64_t)t * E + e] != 0;
            dense[(int64_t)t * E + e] = routed ? (int32_t)row++ : -1;
        }
    }
    if (expert_offsets) expert_offsets[E] = (int32_t)(num_out >= 0 && row > num_out ? num_out : row);
    /* dropping */
    if (num_out >= 0)
        for (int64_t i = 0; i < (int64_t)T * E; i++)
            if (dense[i] >= num_out) dense[i] = -1;
    /* pass 3: per token, the kept rows sorted descending with their experts */
    for (int t = 0; t < T; t++) {
        int n = 0;
        for (int e = 0; e < E; e++)
            if (dense[(int64_t)t * E + e] >= 0) {
                tok[n].row = dense[(int64_t)t * E + e];
                tok[n].expert = e;
                n++;
            }
        qsort(tok, (size_t)n, sizeof *tok, by_row_descending);
        int32_t *m = map + (int64_t)t * W;
        for (int64_t i = 0; i < W; i++) m[i] = -1;
        for (int i = 0; i < n; i++) {
            m[i] = tok[i].row;
            m[E + i] = tok[i].expert;
        }
        m[2 * E] = n;
    }
    free(dense);
    free(tok);
    return ORC_OK;
}

/* One slot of a token's mask map: its row (checked against n_rows) and expert. */
static int mask_slot(const int32_t *map, int E, int n_rows, int t, int i, int *row, int *expert)
{
    const int32_t *m = map + (int64_t)t * (2 * (int64_t)E + 1);
    *row = m[i];
    *expert = m[E + i];
    if (*expert < 0 || *expert >= E) return ORC_BAD_EXPERT;
    if (*row < 0 || *row >= n_rows) return ORC_BAD_ROW;
    return ORC_OK;
}

static int mask_count(const int32_t *map, int E, int t, int *n)
{
    *n = map[(int64_t)t * (2 * (int64_t)E + 1) + 2 * (int64_t)E];
    return (*n < 0 || *n > E) ? ORC_BAD_ROW : ORC_OK;
}

/*
 * Same page, _permute_kernel: each token row is copied to every row its map
 * lists.  With probs ([T][E] fp32) the row's prob goes to out_probs[row],
 * and a prob equal to zero marks a padded slot whose output row is zeros
 * instead of the token (the routing_map padding rule).  Output rows that no
 * map entry names are left as they were.
 */
int oracle_mask_permute(const uint16_t *x, const float *probs, const int32_t *map, int T, int H,
                        int E, int n_rows, uint16_t *out, float *out_probs)
{
    if (T < 0 || H < 0 || E < 1 || n_rows < 0) return ORC_BAD_ARG;
    for (int t = 0; t < T; t++) {
        int n, s = mask_count(map, E, t, &n);
        if (s) return s;
        for (int i = 0; i < n; i++) {
            int row, e;
            s = mask_slot(map, E, n_rows, t, i, &row, &e);
            if (s) return s;
            int zero_row = 0;
            if (probs) {
                float p = probs[(int64_t)t * E + e];
                if (out_probs) out_probs[row] = p;
                zero_row = p == 0.0f;
            }
            for (int h = 0; h < H; h++)
                out[(int64_t)row * H + h] = zero_row ? 0 : x[(int64_t)t * H + h];
        }
    }
    return ORC_OK;
}

/*
 * Same page, _unpermute_kernel: per token and element, an fp32 accumulator
 * from zero visits the token's rows in map order (descending rows); each
 * row is widened to fp32, multiplied by its merging prob (merging_probs
 * [T][E], when given; one fp32 rounding), then added (a second rounding);
 * the sum is rounded once to bf16.  With permuted_probs, unpermuted_probs
 * [T][E] holds permuted_probs[row] at each routed expert and 0 elsewhere.
 */
int oracle_mask_unpermute(const uint16_t *in, const float *merging_probs,
                          const float *permuted_probs, const int32_t *map, int T, int H, int E,
                          int n_rows, uint16_t *out, float *unpermuted_probs)
{
    if (T < 0 || H < 0 || E < 1 || n_rows < 0) return ORC_BAD_ARG;
    for (int t = 0; t < T; t++) {
        int n, s = mask_count(map, E, t, &n);
        if (s) return s;
        for (int i = 0; i < n; i++) {
            int row, e;
            s = mask_slot(map, E, n_rows, t, i, &row, &e);
            if (s) return s;
        }
        for (int h = 0; h < H; h++) {
            float acc = 0.0f;
            for (int i = 0; i < n; i++) {
                int row, e;
                mask_slot(map, E, n_rows, t, i, &row, &e);
                float v = bf16_to_f32(in[(int64_t)row * H + h]);
                if (merging_probs) v = v * merging_probs[(int64_t)t * E + e];
                acc = acc + v;
            }
            out[(int64_t)t * H + h] = f32_to_bf16_rne(acc);
        }
        if (unpermuted_probs) {
            for (int e = 0; e < E; e++) unpermuted_probs[(int64_t)t * E + e] = 0.0f;
            if (permuted_probs)
                for (int i = 0; i < n; i++) {
                    int row, e;
                    mask_slot(map, E, n_rows, t, i, &row, &e);
                    unpermuted_probs[(int64_t)t * E + e] = permuted_probs[row];
                }
        }
    }
    return ORC_OK;
}

/*
 * Same page, _unpermute_bwd_with_merging_probs_kernel: for each routed slot
 * of token t, d_in[row] = bf16(fp32(d_out[t] * merging_probs[t][e])), and
 * d_merging_probs[t][e] = sum_h fwd_in[row][h] * d_out[t][h] (fp64 here,
 * rounded once to fp32); the other experts of the row get 0.  Rows of d_in
 * that no map entry names are left as they were.
 */
int oracle_mask_unpermute_bwd(const uint16_t *d_out, const uint16_t *fwd_in,
                              const float *merging_probs, const int32_t *map, int T, int H, int E,
                              int n_rows, uint16_t *d_in, float *d_merging_probs)
{
    if (T < 0 || H < 0 || E < 1 || n_rows < 0 || !merging_probs) return ORC_BAD_ARG;
    for (int t = 0; t < T; t++) {
        int n, s = mask_count(map, E, t, &n);
        if (s) return s;
        if (d_merging_probs)
            for (int e = 0; e < E; e++) d_merging_probs[(int64_t)t * E + e] = 0.0f;
        for (int i = 0; i < n; i++) {
            int row, e;
            s = mask_slot(map, E, n_rows, t, i, &row, &e);
            if (s) return s;
            float p = merging_probs[(int64_t)t * E + e];
            double dot = 0.0;
            for (int h = 0; h < H; h++) {
                float g = bf16_to_f32(d_out[(int64_t)t * H + h]);
                float prod = g * p;
                d_in[(int64_t)row * H + h] = f32_to_bf16_rne(prod);
                dot += (double)bf16_to_f32(fwd_in[(int64_t)row * H + h]) * (double)g;
            }
            if (d_merging_probs) d_merging_probs[(int64_t)t * E + e] = (float)dot;
        }
    }
    return ORC_OK;
}

/* ---- quantized rows: data rows of any element size, scale rows alongside -- */

/*
 * d9d permute_with_probs.py, _permute_kernel with PERMUTE_SCALE and
 * permute_with_mask_map (scale, scale_hidden_dim): next to each token's data
 * row, the token's scale row is stored to the same destination index of a
 * permuted scale tensor.  Data rows are row_bytes bytes (an FP8 row of H
 * elements is H bytes) and are copied bitwise, so the FP8 encoding does not
 * enter; scale rows are scale_row_bytes bytes (0: no scales).
 * The top-k form routes by topk_idx / row_id_map[E][T] as oracle_permute;
 * the mask-map form by the per-token map, and with probs ([T][E] fp32) a zero
 * prob writes a zero data row while the scale row is still copied.  Rows no
 * route names are left as they were.
 */
static void copy_bytes(uint8_t *dst, const uint8_t *src, int64_t n)
{
    for (int64_t i = 0; i < n; i++) dst[i] = src[i];
}

int oracle_permute_scaled(const uint8_t *x, int64_t row_bytes, const uint8_t *scale,
                          int64_t scale_row_bytes, const float *probs, const int32_t *topk_idx,
                          const int32_t *row_id_map, int T, int k, int E, int64_t n_rows,
                          uint8_t *out, uint8_t *out_scale, float *out_probs)
{
    if (T < 0 || row_bytes < 1 || scale_row_bytes < 0 || k < 1 || E < 1 || n_rows < 0)
        return ORC_BAD_ARG;
    for (int t = 0; t < T; t++) {
        for (int j = 0; j < k; j++) {
            int64_t r;
            int s = slot_row(topk_idx, row_id_map, T, k, E, n_rows, t, j, &r);
            if (s) return s;
            copy_bytes(out + r * row_bytes, x + (int64_t)t * row_bytes, row_bytes);
            if (scale && out_scale && scale_row_bytes > 0)
                copy_bytes(out_scale + r * scale_row_bytes, scale + (int64_t)t * scale_row_bytes,
                           scale_row_bytes);
            if (probs && out_probs) out_probs[r] = probs[(int64_t)t * k + j];
        }
    }
    return ORC_OK;
}

int oracle_mask_permute_scaled(const uint8_t *x, int64_t row_bytes, const uint8_t *scale,
                               int64_t scale_row_bytes, const float *probs, const int32_t *map,
                               int T, int E, int n_rows, uint8_t *out, uint8_t *out_scale,
                               float *out_probs)
{
    if (T < 0 || row_bytes < 1 || scale_row_bytes < 0 || E < 1 || n_rows < 0)
        return ORC_BAD_ARG;
    for (int t = 0; t < T; t++) {
        int n, s = mask_count(map, E, t, &n);
        if (s) return s;
        for (int i = 0; i < n; i++) {
            int row, e;
            s = mask_slot(map, E, n_rows, t, i, &row, &e);
            if (s) return s;
            int zero_row = 0;
            if (probs) {
                float p = probs[(int64_t)t * E + e];
                if (out_probs) out_probs[row] = p;
                zero_row = p == 0.0f;
            }
            if (zero_row)
                for (int64_t b = 0; b < row_bytes; b++) out[(int64_t)row * row_bytes + b] = 0;
            else
                copy_bytes(out + (int64_t)row * row_bytes, x + (int64_t)t * row_bytes, row_bytes);
            if (scale && out_scale && scale_row_bytes > 0)
                copy_bytes(out_scale + (int64_t)row * scale_row_bytes,
                           scale + (int64_t)t * scale_row_bytes, scale_row_bytes);
        }
    }
    return ORC_OK;
}

/* ---- (3) fused chunk sort-and-pad / unpad-and-restore -------------------- */

/*
 * TransformerEngine PR "Fuse MoE chunk sorting and padding", Description,
 * Changes and Diagram.  Rank chunks arrive back to back in input order
 * (chunk c holds split_sizes[c] rows).  The explicit chunk order lists, for
 * each sorted position q, the input chunk sorted_idx[q]; R consecutive sorted
 * positions form one expert group g = q / R.  Inside a group the chunks are
 * laid back to back; the group is then zero-padded to a multiple of the
 * alignment A (an empty group takes no rows).  The map from padded
 * destination rows to source rows is kept for the restore and the
 * backward; destination rows with no source hold -1, including every row
 * past the last group up to the fixed output capacity.
 *   src_off[c]  = split_sizes[0] + ... + split_sizes[c-1]   (input order)
 *   n_g         = sum of split_sizes[sorted_idx[q]] over q in group g
 *   padded_g    = ceil(n_g / A) * A
 *   pad_off[g]  = padded_0 + ... + padded_{g-1};  padded_offsets = pad_off
 * Errors: order not a permutation of [0, C), a negative size, C % R != 0,
 * sum of sizes > N_cap, pad_off[G] > out_cap.
 */
int oracle_chunk_map(const int32_t *split_sizes, const int32_t *sorted_idx, int C, int R, int A,
                     int N_cap, int out_cap, int32_t *row_map, int32_t *padded_offsets)
{
    if (C < 1 || R < 1 || A < 1 || N_cap < 0 || out_cap < 0 || C % R != 0) return ORC_BAD_ARG;
    int G = C / R;
    int status = ORC_OK;
    int64_t *src_off = (int64_t *)calloc((size_t)C, sizeof(int64_t));
    int *seen = (int *)calloc((size_t)C, sizeof(int));
    if (!src_off || !seen) { free(src_off); free(seen); return ORC_NO_MEM; }

    int64_t total = 0;
    for (int c = 0; c < C; c++) {
        if (split_sizes[c] < 0) { status = ORC_BAD_CHUNKS; goto done; }
        src_off[c] = total;
        total += split_sizes[c];
    }
    for (int q = 0; q < C; q++) {
        int c = sorted_idx[q];
        if (c < 0 || c >= C || seen[c]) { status = ORC_BAD_CHUNKS; goto done; }
        seen[c] = 1;
    }
    if (total > N_cap) { status = ORC_OVERFLOW; goto done; }

    for (int d = 0; d < out_cap; d++) row_map[d] = -1;

    int64_t group_start = 0;
    for (int g = 0; g < G; g++) {
        padded_offsets[g] = (int32_t)group_start;
        int64_t d = group_start;          /* next destination row in group */
        for (int q = g * R; q < (g + 1) * R; q++) {
            int c = sorted_idx[q];
            for (int i = 0; i < split_sizes[c]; i++) {
                if (d >= out_cap) { status = ORC_OVERFLOW; goto done; }
                row_map[d] = (int32_t)(src_off[c] + i);
                d += 1;
            }
        }
        int64_t n_g = d - group_start;
        int64_t padded = ((n_g + A - 1) / A) * A;
        group_start += padded;
        if (group_start > out_cap) { status = ORC_OVERFLOW; goto done; }
    }
    padded_offsets[G] = (int32_t)group_start;

done:
    free(src_off);
    free(seen);
    return status;
}

/*
 * Sort-and-pad copy (same PR): out[d] = in[row_map[d]] for mapped rows and
 * all-zero bits for padding rows; the probabilities move with the tokens.
 * elem_bytes / prob_bytes give the element sizes (copies are bitwise).
 */
static int pad_copy(const uint8_t *in, const uint8_t *probs, int elem_bytes, int prob_bytes,
                    int N_cap, int H, const int32_t *row_map, int out_cap,
                    uint8_t *out, uint8_t *out_probs)
{
    int64_t row_bytes = (int64_t)H * elem_bytes;
    for (int d = 0; d < out_cap; d++) {
        int32_t s = row_map[d];
        if (s >= N_cap) return ORC_BAD_ROW;
        if (s >= 0) {
            memcpy(out + d * row_bytes, in + (int64_t)s * row_bytes, (size_t)row_bytes);
            if (probs && out_probs)
                memcpy(out_probs + (int64_t)d * prob_bytes, probs + (int64_t)s * prob_bytes,
                       (size_t)prob_bytes);
        } else {
            memset(out + d * row_bytes, 0, (size_t)row_bytes);
            if (probs && out_probs) memset(out_probs + (int64_t)d * prob_bytes, 0, (size_t)prob_bytes);
        }
    }
    return ORC_OK;
}

/*
 * Unpad-and-restore copy (same PR): every mapped padded row goes back to its
 * source row; padding rows are dropped.  Rows of the restored buffer that no
 * chunk covers (from the token total up to N_cap) are all-zero bits.
 * A map that does not belong to these split sizes (say, one saved for an
 * earlier, larger routing) can name a source row at or past the token total;
 * such an entry is dropped and reported as ORC_BAD_ROW, and the output is
 * still defined: the zero tail, and every other mapped row copied.
 */
static int restore_copy(const uint8_t *in, const uint8_t *probs, int elem_bytes, int prob_bytes,
                        const int32_t *row_map, int64_t n_act, int out_cap, int H, int N_cap,
                        uint8_t *out, uint8_t *out_probs)
{
    int64_t row_bytes = (int64_t)H * elem_bytes;
    for (int64_t s = n_act; s < N_cap; s++) {
        memset(out + s * row_bytes, 0, (size_t)row_bytes);
        if (probs && out_probs) memset(out_probs + s * prob_bytes, 0, (size_t)prob_bytes);
    }
    int status = ORC_OK;
    for (int d = 0; d < out_cap; d++) {
        int32_t s = row_map[d];
        if (s < 0) continue;
        if (s >= n_act) { status = ORC_BAD_ROW; continue; }
        memcpy(out + (int64_t)s * row_bytes, in + (int64_t)d * row_bytes, (size_t)row_bytes);
        if (probs && out_probs)
            memcpy(out_probs + (int64_t)s * prob_bytes, probs + (int64_t)d * prob_bytes,
                   (size_t)prob_bytes);
    }
    return status;
}

static int check_elem(int elem_bytes, int prob_bytes)
{
    if (elem_bytes != 2 && elem_bytes != 4) return ORC_BAD_ARG;
    if (prob_bytes != 2 && prob_bytes != 4) return ORC_BAD_ARG;
    return ORC_OK;
}

int oracle_sort_chunks_and_pad(const void *in, const void *probs, int elem_bytes, int prob_bytes,
                               int N_cap, int H, const int32_t *split_sizes,
                               const int32_t *sorted_idx, int C, int R, int A, int out_cap,
                               void *out, void *out_probs, int32_t *row_map,
                               int32_t *padded_offsets)
{
    int s = check_elem(elem_bytes, prob_bytes);
    if (s || H < 1) return s ? s : ORC_BAD_ARG;
    s = oracle_chunk_map(split_sizes, sorted_idx, C, R, A, N_cap, out_cap, row_map, padded_offsets);
    if (s) return s;
    return pad_copy((const uint8_t *)in, (const uint8_t *)probs, elem_bytes, prob_bytes, N_cap, H,
                    row_map, out_cap, (uint8_t *)out, (uint8_t *)out_probs);
}

int oracle_unpad_and_restore_chunks(const void *in, const void *probs, int elem_bytes,
                                    int prob_bytes, const int32_t *row_map,
                                    const int32_t *split_sizes, int C, int out_cap, int H,
                                    int N_cap, void *out, void *out_probs)
{
    int s = check_elem(elem_bytes, prob_bytes);
    if (s || H < 1 || C < 1) return s ? s : ORC_BAD_ARG;
    int64_t n_act = 0;
    for (int c = 0; c < C; c++) {
        if (split_sizes[c] < 0) return ORC_BAD_CHUNKS;
        n_act += split_sizes[c];
    }
    if (n_act > N_cap) return ORC_OVERFLOW;
    return restore_copy((const uint8_t *)in, (const uint8_t *)probs, elem_bytes, prob_bytes,
                        row_map, n_act, out_cap, H, N_cap, (uint8_t *)out, (uint8_t *)out_probs);
}

/*
 * Backwards (same PR, Changes: padding rows hold zeros and pass no gradient
 * back).  The sort-and-pad copy is a row permutation plus zero rows, so
 * its gradient is the restore applied to the padded gradient (padding-row
 * gradients are dropped); the restore's gradient is the pad copy applied to
 * the restored gradient (padding rows get zero gradient).
 */
int oracle_sort_chunks_and_pad_bwd(const void *d_out, const void *d_out_probs, int elem_bytes,
                                   int prob_bytes, const int32_t *row_map,
                                   const int32_t *split_sizes, int C, int out_cap, int H,
                                   int N_cap, void *d_in, void *d_in_probs)
{
    return oracle_unpad_and_restore_chunks(d_out, d_out_probs, elem_bytes, prob_bytes, row_map,
                                           split_sizes, C, out_cap, H, N_cap, d_in, d_in_probs);
}

int oracle_unpad_and_restore_chunks_bwd(const void *d_out, const void *d_out_probs,
                                        int elem_bytes, int prob_bytes, const int32_t *row_map,
                                        int out_cap, int H, int N_cap, void *d_in,
                                        void *d_in_probs)
{
    int s = check_elem(elem_bytes, prob_bytes);
    if (s || H < 1) return s ? s : ORC_BAD_ARG;
    return pad_copy((const uint8_t *)d_out, (const uint8_t *)d_out_probs, elem_bytes, prob_bytes,
                    N_cap, H, row_map, out_cap, (uint8_t *)d_in, (uint8_t *)d_in_probs);
}
