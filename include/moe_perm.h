/*
 * moe_perm.h -- C ABI of the MI355X (gfx950) MoE token permute / unpermute
 * library: routing row map, permute, fixed-order unpermute, fused chunk
 * sort-and-pad / unpad-and-restore, and the backward of each.
 *
 * Sources of the operations (cited by page title and section):
 *   [TE-mask]   d9d 0.1.0 wheel, d9d/kernel/moe/permute_with_probs.py (a copy
 *               of TransformerEngine's mask-map permutation): make_row_id_map
 *               and its worked example, _permute_kernel, _unpermute_kernel,
 *               _unpermute_bwd_with_merging_probs_kernel, the two autograd
 *               functions and moe_permute_with_probs (num_out_tokens).
 *   [MCORE-BI]  Megatron-core API docs, core.transformer.moe.batch_invariant:
 *               unpermute_with_bf16_rank_partials, _rank_tree_unpermute_kernel,
 *               _rank_tree_unpermute_bwd_kernel, _unpermute_loop.
 *   [MOE-OPS]   moe-ops 0.1.0 README: "Why this library", "Routing
 *               permute / unpermute" and "Fused Top-K Softmax".
 *   [XTUNER]    xtuner issue "permute different with torch version".
 *   [TE-3509]   TransformerEngine PR "[PyTorch] Fuse MoE chunk sorting and
 *               padding": Description, Changes, Validation, Diagram.
 *
 * Conventions shared by every call
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees or synchronises; each call enqueues its
 *     kernels on `stream` and returns.  No call reads device memory from the
 *     host, so every call can be captured in a hipGraph; sizes read on the
 *     device (routing, chunk sizes) may change between graph replays.
 *   - bf16 tensors are passed as `void*` holding 16-bit bf16 patterns,
 *     row-major and contiguous.  Probabilities are fp32 unless stated.
 *   - Index tensors are int32.  Row offsets are computed in 64 bits.
 *   - Rows whose byte size is a multiple of 16 and whose base pointers are
 *     16-byte aligned move as 16-byte vectors; otherwise an element-wise path
 *     runs (same results).  Pointers must at least be aligned to their
 *     element size (MOE_ERR_ALIGN otherwise).
 *   - Host-side argument checks run before any HIP call and return a status
 *     code; a non-zero return means nothing was enqueued.
 *   - Data-dependent faults that only the device can see (an expert index
 *     out of range, a repeated expert in one token, a map entry out of range,
 *     bad chunk metadata, a capacity overflow) never cause an out-of-bounds
 *     access: the offending element is skipped and, when `dev_status` is
 *     non-NULL, the matching MOE_DEV_* bit is OR-ed into *dev_status (an int32
 *     in device memory the caller zeroes beforehand).  Outputs are then
 *     unspecified.
 *   - num_tokens == 0 (or n_cap == 0) is valid: outputs that still have a
 *     defined value (expert_offsets) are written, nothing else is touched.
 *   - Calls on one stream are ordered; calls that write the same buffers from
 *     different streams race.
 */
#ifndef MOE_PERM_H
#define MOE_PERM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_PERM_API __attribute__((visibility("default")))

/* Host-side status codes returned by every call. */
enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL                     */
    MOE_ERR_SHAPE = 2,       /* a size argument is out of range/inconsistent   */
    MOE_ERR_ALIGN = 3,       /* a pointer is not aligned to its element size   */
    MOE_ERR_UNSUPPORTED = 4, /* a size beyond what the kernels support         */
    MOE_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required     */
    MOE_ERR_HIP = 6          /* a kernel launch failed (hipGetLastError)       */
};

/* Device-side status bits OR-ed into *dev_status. */
#define MOE_DEV_BAD_EXPERT 0x1 /* top-k index outside [0, num_experts)         */
#define MOE_DEV_DUP_EXPERT 0x2 /* one expert twice in a token's top-k          */
#define MOE_DEV_BAD_ROW 0x4    /* row_id_map / row_map entry outside its range */
#define MOE_DEV_BAD_CHUNKS 0x8 /* negative split size or order not a permutation */
#define MOE_DEV_OVERFLOW 0x10  /* tokens exceed n_cap or padded rows exceed out_cap */

/* Largest supported sizes (MOE_ERR_UNSUPPORTED beyond). */
#define MOE_MAX_EXPERTS 2048
#define MOE_MAX_TOPK 64
#define MOE_MAX_CHUNKS 2048

/* Name of a host status code (static string, never NULL). */
MOE_PERM_API const char *moe_status_string(int status);

/* ------------------------------------------------------------------------ *
 * (1) Routing row map -- stable counting sort.
 *
 * [TE-mask] make_row_id_map and its worked example: per expert, count the
 * routed tokens per token block, exclusive-scan the counts in expert-major
 * order, and give each routed (token, expert) pair the row
 *     expert_offsets[e] + (number of tokens t' < t also routed to e).
 * [MOE-OPS] "Routing permute / unpermute": a counting sort (histogram plus
 * exclusive prefix sums), O(T*k).  [XTUNER]: the same rows as a stable
 * argsort of the flattened top-k indices -- the single convention here.
 *
 *   topk_idx        [num_tokens][topk] int32, token t's experts in slot order;
 *                   the experts of one token must be distinct.
 *   row_id_map      out [num_experts][num_tokens] int32: destination row of
 *                   (t, e), or -1 when t is not routed to e.  Rows are
 *                   expert-major, tokens ascending inside an expert, and
 *                   cover [0, num_tokens*topk) exactly once.
 *   expert_offsets  out [num_experts + 1] int32: exclusive scan of the
 *                   per-expert counts; expert_offsets[E] = num_tokens*topk.
 *   dev_status      optional; MOE_DEV_BAD_EXPERT, MOE_DEV_DUP_EXPERT.
 *   workspace       device scratch of at least
 *                   moe_make_row_id_map_workspace_bytes(...) bytes, 256-byte
 *                   aligned; contents need no initialisation.
 * Limits: 1 <= topk <= min(num_experts, MOE_MAX_TOPK),
 *         num_experts <= MOE_MAX_EXPERTS, num_tokens*topk < 2^31.
 * ------------------------------------------------------------------------ */
MOE_PERM_API size_t moe_make_row_id_map_workspace_bytes(int num_tokens, int topk,
                                                        int num_experts);
MOE_PERM_API int moe_make_row_id_map(const int32_t *topk_idx, int num_tokens, int topk,
                                     int num_experts, int32_t *row_id_map,
                                     int32_t *expert_offsets, int32_t *dev_status,
                                     void *workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Row map without a workspace argument, for callers that cannot allocate
 * device memory: code being captured into a hipGraph, tight serving loops,
 * harnesses that forbid allocation.  Same arguments (minus the workspace),
 * checks and results as moe_make_row_id_map.  The scratch is a fixed array
 * of MOE_NOALLOC_SCRATCH_BYTES in the library's device data: one copy per
 * GPU, held until the process ends; this call allocates and frees nothing.
 *   MOE_ERR_WORKSPACE  when moe_make_row_id_map_workspace_bytes(...) exceeds
 *                      MOE_NOALLOC_SCRATCH_BYTES (about 0.14 * num_tokens *
 *                      num_experts bytes are needed: e.g. 65536 tokens with
 *                      up to 896 experts fit).
 *   MOE_ERR_HIP        when the array's device address cannot be looked up.
 * Every call on one GPU uses that GPU's array: two calls that can run at the
 * same time on one GPU (unordered streams) race and give unspecified maps.
 * The array needs no clearing (each call writes every scratch byte it reads).
 * The first call on a device looks up the array's address (a host call, no
 * stream work); make it once before capturing a graph.
 * ------------------------------------------------------------------------ */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
MOE_PERM_API int moe_make_row_id_map_noalloc(const int32_t *topk_idx, int num_tokens, int topk,
                                             int num_experts, int32_t *row_id_map,
                                             int32_t *expert_offsets, int32_t *dev_status,
                                             hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * (2) Permute -- gather-copy of each token row to its top-k rows.
 *
 * [TE-mask] _permute_kernel: a token's hidden row is stored unchanged to each
 * destination row it is routed to; with probabilities, the slot's
 * probability is stored at the same destination index.
 *   out[r(t,j)][:]  = x[t][:]          (bitwise)
 *   out_probs[r(t,j)] = probs[t][j]    (when both pointers are non-NULL)
 * with r(t,j) = row_id_map[topk_idx[t][j]][t].
 *
 *   x          [num_tokens][hidden] bf16.
 *   probs      [num_tokens][topk] fp32 or NULL.
 *   out        [num_out_rows][hidden] bf16; num_out_rows must equal
 *              num_tokens*topk (no token dropping).
 *   out_probs  [num_out_rows] fp32 or NULL.
 *   dev_status optional; MOE_DEV_BAD_EXPERT, MOE_DEV_BAD_ROW.
 * ------------------------------------------------------------------------ */
MOE_PERM_API int moe_permute(const void *x, const float *probs, const int32_t *topk_idx,
                             const int32_t *row_id_map, int num_tokens, int hidden,
                             int topk, int num_experts, int num_out_rows, void *out,
                             float *out_probs, int32_t *dev_status, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * (4) Unpermute -- token-owned, fixed-order combine.
 *
 * [MCORE-BI] unpermute_with_bf16_rank_partials / _rank_tree_unpermute_kernel
 * with BF16_RANK_PARTIALS, on a single EP rank: an output token is the sum
 * of its routed rows, each scaled by its probability, accumulated in fp32
 * with one fused multiply-add per slot, slots taken in top-k order, the
 * accumulator starting at zero; the sum is rounded once to bf16:
 *   acc = +0.0f; for j in 0..topk-1: acc = fmaf(probs[t][j], in[r(t,j)][h], acc)
 *   out[t][h] = bf16_round_nearest_even(acc)
 * probs == NULL uses unit weights (identical to plain fp32 adds).
 * [MOE-OPS] "Why this library": a gather-add that writes each output once, no
 * atomics.  Results are bitwise reproducible and independent of launch shape.
 *
 *   in         [num_in_rows][hidden] bf16, num_in_rows == num_tokens*topk.
 *   probs      [num_tokens][topk] fp32 or NULL.
 *   out        [num_tokens][hidden] bf16.
 *   dev_status optional; MOE_DEV_BAD_EXPERT, MOE_DEV_BAD_ROW.
 * ------------------------------------------------------------------------ */
MOE_PERM_API int moe_unpermute(const void *in, const float *probs, const int32_t *topk_idx,
                               const int32_t *row_id_map, int num_tokens, int hidden,
                               int topk, int num_experts, int num_in_rows, void *out,
                               int32_t *dev_status, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Unpermute with an EP rank-ordered combine, on one GPU.
 *
 * [MCORE-BI] unpermute / _unpermute_loop (contributions added by EP rank,
 * then by top-k slot), _rank_tree_unpermute_kernel with BF16_RANK_PARTIALS
 * and CROSS_RANK_FP64, unpermute_with_bf16_rank_partials.  The experts split
 * into ep_size equal ranges; rank(e) = e / (num_experts / ep_size):
 *   total = 0                                   (fp32, or fp64 with
 *                                                MOE_EP_FP64_CROSS)
 *   for rank = 0 .. ep_size-1:
 *     partial = +0.0f
 *     for j in slot order with rank(topk_idx[t][j]) == rank:
 *       partial = fmaf(probs[t][j], in[r(t,j)][h], partial)
 *     if MOE_EP_BF16_PARTIALS: partial = bf16_rne(partial)
 *     total += partial
 *   out[t][h] = bf16_rne(total)                 (fp64 -> bf16 rounded once)
 * ep_size == 1 gives the same bits as moe_unpermute.  The gradient of this
 * combine (rounding steps taken as identity) is the one moe_unpermute_bwd
 * computes.  Arguments as moe_unpermute, plus ep_size (a divisor of
 * num_experts) and flags.
 * ------------------------------------------------------------------------ */
#define MOE_EP_BF16_PARTIALS 0x1
#define MOE_EP_FP64_CROSS 0x2
MOE_PERM_API int moe_unpermute_ep(const void *in, const float *probs, const int32_t *topk_idx,
                                  const int32_t *row_id_map, int num_tokens, int hidden,
                                  int topk, int num_experts, int num_in_rows, int ep_size,
                                  int flags, void *out, int32_t *dev_status,
                                  hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Unpermute backward.
 *
 * [TE-mask] _unpermute_bwd_with_merging_probs_kernel; [MCORE-BI]
 * _rank_tree_unpermute_bwd_kernel (one writer per permuted row):
 *   d_in[r(t,j)][h] = bf16(fp32(d_out[t][h]) * probs[t][j])  (fp32 product,
 *                                                            then bf16 RNE)
 *   d_probs[t][j]   = sum_h fp32(fwd_in[r(t,j)][h]) * fp32(d_out[t][h])
 * The order of the prob-grad sum is not fixed by the pages; here it is an
 * fp32 blocked tree that depends only on the call's sizes (through the
 * launch shape chosen for them: a call moving more than 256 MiB computes the
 * sums in a launch of their own), so results are bitwise reproducible.
 * With probs == NULL, d_in[r(t,j)] = d_out[t] bitwise and d_probs must be
 * NULL.  fwd_in may be NULL only when d_probs is NULL.
 *
 *   d_out   [num_tokens][hidden] bf16 (gradient of the unpermute output).
 *   fwd_in  [num_rows][hidden] bf16 (the unpermute's forward input).
 *   d_in    [num_rows][hidden] bf16, num_rows == num_tokens*topk.
 *   d_probs [num_tokens][topk] fp32 or NULL.
 * ------------------------------------------------------------------------ */
MOE_PERM_API int moe_unpermute_bwd(const void *d_out, const void *fwd_in, const float *probs,
                                   const int32_t *topk_idx, const int32_t *row_id_map,
                                   int num_tokens, int hidden, int topk, int num_experts,
                                   int num_rows, void *d_in, float *d_probs,
                                   int32_t *dev_status, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Permute backward.
 *
 * [TE-mask] _moe_permute_mask_map.backward: the gradient of the permute is
 * the unweighted unpermute of the permuted gradient, and the permuted-prob
 * gradient is gathered back to the token's slots:
 *   d_x[t][h]     = bf16_rne(sum over j in slot order, fp32, from +0, of
 *                            d_out[r(t,j)][h])
 *   d_probs[t][j] = d_out_probs[r(t,j)]      (when both are non-NULL)
 *
 *   d_out        [num_rows][hidden] bf16, num_rows == num_tokens*topk.
 *   d_out_probs  [num_rows] fp32 or NULL.
 *   d_x          [num_tokens][hidden] bf16.
 *   d_probs      [num_tokens][topk] fp32 or NULL.
 * ------------------------------------------------------------------------ */
MOE_PERM_API int moe_permute_bwd(const void *d_out, const float *d_out_probs,
                                 const int32_t *topk_idx, const int32_t *row_id_map,
                                 int num_tokens, int hidden, int topk, int num_experts,
                                 int num_rows, void *d_x, float *d_probs,
                                 int32_t *dev_status, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Fused top-k softmax router (the step before the row map).
 *
 * [MOE-OPS] "Fused Top-K Softmax": top-k selection and softmax in one kernel;
 * with the fp32_routing option the weights are fp32, without it they come
 * in the activation dtype (here: prob_bytes 4 or 2).  The backward gives the
 * exact softmax gradient scattered back to the logits.
 *   topk_idx[t][0..k): the k largest logits of token t in descending order, a
 *                      tie going to the lower expert index.
 *   probs[t][j]      = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k
 *                      selected logits, computed in fp32 and stored as fp32
 *                      (prob_bytes 4) or rounded to nearest-even bf16
 *                      (prob_bytes 2).  The sum's order is the kernel's own,
 *                      so results match an exact softmax to a few fp32 ulp.
 *   logits  [num_tokens][num_experts], logit_bytes 2 (bf16) or 4 (fp32).
 *   Limits: 1 <= topk <= min(num_experts, MOE_MAX_TOPK), num_experts <=
 *   MOE_MAX_EXPERTS.  NaN logits rank below every number (values then
 *   unspecified; the indices stay distinct and in range).
 *   Buffers: device memory, owned by the caller, element-aligned.
 *
 * moe_topk_softmax_bwd: d_logits[t][e] = w_j (d_probs[t][j] - sum_i w_i
 * d_probs[t][i]) for e = topk_idx[t][j], +0 for experts not selected, in
 * fp32 arithmetic.  probs and d_probs [num_tokens][topk] of prob_bytes 4 or
 * 2; d_logits [num_tokens][num_experts] of logit_bytes 4 or 2 (bf16 rounded
 * to nearest-even).  A token's expert indices must be distinct.
 * dev_status: MOE_DEV_BAD_EXPERT for an index outside [0, num_experts).
 * ------------------------------------------------------------------------ */
MOE_PERM_API int moe_topk_softmax(const void *logits, int logit_bytes, int num_tokens,
                                  int num_experts, int topk, int32_t *topk_idx, void *probs,
                                  int prob_bytes, hipStream_t stream);
MOE_PERM_API int moe_topk_softmax_bwd(const void *d_probs, const void *probs, int prob_bytes,
                                      const int32_t *topk_idx, int num_tokens, int num_experts,
                                      int topk, void *d_logits, int logit_bytes,
                                      int32_t *dev_status, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * TransformerEngine mask-map form (interop for callers holding a routing
 * mask instead of top-k indices).
 *
 * [TE-mask] make_row_id_map: routing_map [num_tokens][num_experts], entry !=
 * 0 routes the token to the expert (mask_bytes 1: bool / uint8, or 4:
 * int32).  Destination rows are the same counting sort as
 * moe_make_row_id_map: expert-major, tokens ascending inside an expert.
 * [TE-mask] moe_permute_with_probs, num_out_tokens (the count of rows not
 * dropped): a row >= num_out_tokens is dropped; -1 keeps every row.
 * row_id_map [num_tokens][2*num_experts+1], per token t:
 *   [0, n)            its kept destination rows in descending order,
 *   [E, E + n)        the expert of each of those rows,
 *   [2E]              n;
 * every other entry is left unwritten (the page leaves them unused).
 * expert_offsets [E+1] (optional): kept rows of the experts below e; the
 * last entry is the number of kept rows.  Workspace as for the top-k map:
 * moe_make_mask_row_id_map_workspace_bytes(), 256-byte aligned.
 * ------------------------------------------------------------------------ */
MOE_PERM_API size_t moe_make_mask_row_id_map_workspace_bytes(int num_tokens, int num_experts);
MOE_PERM_API int moe_make_mask_row_id_map(const void *routing_map, int mask_bytes,
                                          int num_tokens, int num_experts, int num_out_tokens,
                                          int32_t *row_id_map, int32_t *expert_offsets,
                                          void *workspace, size_t workspace_bytes,
                                          hipStream_t stream);

/*
 * [TE-mask] _permute_kernel: out[row] = x[t] for each slot of token t's map
 * row.  With probs ([num_tokens][num_experts] fp32): out_probs[row] =
 * probs[t][e], and a prob equal to zero (+0 or -0) marks a padded slot
 * whose out row is written as zeros instead of x[t].  Rows of out that no
 * map entry names are not written.  Also the backward of the unpermute
 * without merging probs (d_in = this gather-copy of d_out).
 *   x [num_tokens][hidden] bf16 (any 2-byte type without probs),
 *   out [num_out_rows][hidden], out_probs [num_out_rows] (optional).
 *   dev_status: MOE_DEV_BAD_EXPERT, MOE_DEV_BAD_ROW (a row outside
 *   [0, num_out_rows), or a count outside [0, E]).
 */
MOE_PERM_API int moe_permute_mask(const void *x, const float *probs, const int32_t *row_id_map,
                                  int num_tokens, int hidden, int num_experts, int num_out_rows,
                                  void *out, float *out_probs, int32_t *dev_status,
                                  hipStream_t stream);

/*
 * [TE-mask] _unpermute_kernel: per token and element, an fp32 accumulator
 * from +0 visits the token's rows in map order (descending rows); each row
 * is widened to fp32, multiplied by merging_probs[t][e] when given (one
 * fp32 rounding), then added (a second rounding); the sum is rounded to
 * nearest-even bf16.  This is TE's arithmetic, not the fused slot-order
 * combine of moe_unpermute.  With unpermuted_probs ([num_tokens][num_experts]
 * fp32, optional): permuted_probs[row] at each routed expert (0 when
 * permuted_probs is NULL), 0 elsewhere.  Without merging probs this is also
 * the backward of moe_permute_mask: d_x = this sum of d_out rows, and the
 * probs gradient is the unpermuted_probs of d_out_probs.
 *   in [num_in_rows][hidden] bf16, out [num_tokens][hidden] bf16.
 *   dev_status: MOE_DEV_BAD_EXPERT, MOE_DEV_BAD_ROW.
 */
MOE_PERM_API int moe_unpermute_mask(const void *in, const float *merging_probs,
                                    const float *permuted_probs, const int32_t *row_id_map,
                                    int num_tokens, int hidden, int num_experts, int num_in_rows,
                                    void *out, float *unpermuted_probs, int32_t *dev_status,
                                    hipStream_t stream);

/*
 * [TE-mask] _unpermute_bwd_with_merging_probs_kernel: for each slot of
 * token t (row, expert e), d_in[row] = bf16(fp32(d_out[t] * merging_probs
 * [t][e])), and d_merging_probs[t][e] = sum_h fwd_in[row][h] * d_out[t][h]
 * (fp32; its summation order is the kernel's own); the other experts of
 * the row get 0.  d_merging_probs (optional) needs fwd_in.  Rows of d_in no
 * map entry names are not written.
 *   dev_status: MOE_DEV_BAD_EXPERT, MOE_DEV_BAD_ROW.
 */
MOE_PERM_API int moe_unpermute_mask_bwd(const void *d_out, const void *fwd_in,
                                        const float *merging_probs, const int32_t *row_id_map,
                                        int num_tokens, int hidden, int num_experts,
                                        int num_rows, void *d_in, float *d_merging_probs,
                                        int32_t *dev_status, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Quantized rows (e.g. FP8) with per-row scale vectors moved alongside.
 *
 * [TE-mask] _permute_kernel with PERMUTE_SCALE, permute_with_mask_map
 * (scale, scale_hidden_dim): each token's scale row goes to the same
 * destination index of a permuted scale tensor as its data row.  Data rows
 * are `hidden` elements of elem_bytes (1: any FP8 encoding, 2, or 4) and
 * are copied bitwise, so the encoding does not enter; the routing, probs,
 * status bits and the mask-map form's zero-prob padding rule are those of
 * moe_permute / moe_permute_mask (the padding rule zeroes the data row only;
 * the scale row still moves).  The inputs this library is tested with are
 * OCP FP8 E4M3FN rows (gfx950's native FP8) with fp32 or E8M0 block scales.
 *   scale [num_tokens][scale_row_bytes bytes] (optional; NULL: no scales),
 *   out_scale [num_out_rows][scale_row_bytes bytes] (required with scale).
 * The backward of these permutes acts on bf16 gradients: moe_permute_bwd /
 * moe_unpermute_mask apply unchanged, and scales carry no gradient.
 * ------------------------------------------------------------------------ */
MOE_PERM_API int moe_permute_scaled(const void *x, int elem_bytes, const void *scale,
                                    int scale_row_bytes, const float *probs,
                                    const int32_t *topk_idx, const int32_t *row_id_map,
                                    int num_tokens, int hidden, int topk, int num_experts,
                                    int num_out_rows, void *out, void *out_scale,
                                    float *out_probs, int32_t *dev_status, hipStream_t stream);
MOE_PERM_API int moe_permute_mask_scaled(const void *x, int elem_bytes, const void *scale,
                                         int scale_row_bytes, const float *probs,
                                         const int32_t *row_id_map, int num_tokens, int hidden,
                                         int num_experts, int num_out_rows, void *out,
                                         void *out_scale, float *out_probs, int32_t *dev_status,
                                         hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * (3) Fused chunk sort-and-pad.
 *
 * [TE-3509] Description / Changes / Diagram: rank chunks are regrouped into
 * expert order and each expert group is zero-padded to an alignment, in one
 * copy that moves tokens and probabilities together; a padded
 * destination -> source row map is kept for the restore and the backward.
 * Chunk order and padding are explicit; routing metadata stays on the GPU;
 * the output size is fixed by the caller so graph replays can change the
 * routing; token counts are kernel arguments read on the device.
 *
 *   in           [n_cap][hidden] elements of elem_bytes (2: bf16/fp16,
 *                4: fp32), copied bitwise.  Chunk c occupies split_sizes[c]
 *                rows, chunks back to back in input order from row 0.
 *   probs        [n_cap] elements of prob_bytes (2 or 4), or NULL.  With
 *                n_cap == 0 it may be NULL even when out_probs is not (then
 *                out_probs is all zero).
 *   split_sizes  [num_chunks] int32, device.
 *   sorted_idx   [num_chunks] int32, device: input chunk at sorted position
 *                q.  Positions [g*R, (g+1)*R) form group g, R =
 *                chunks_per_group, G = num_chunks / R groups.
 *   align        group g takes padded_g = ceil(n_g / align) * align rows
 *                (an empty group takes none), n_g = its token count.
 *   out          [out_cap][hidden]: group g's chunks back to back from
 *                padded_offsets[g], then zero rows up to padded_offsets[g+1];
 *                rows from padded_offsets[G] to out_cap are zero.
 *   out_probs    [out_cap] or NULL (zero on padding rows).
 *   row_map      out [out_cap] int32: source row of each destination row,
 *                -1 for padding and tail rows.
 *   padded_offsets out [G + 1] int32: exclusive scan of padded_g.
 *   dev_status   optional; MOE_DEV_BAD_CHUNKS, MOE_DEV_OVERFLOW (then
 *                row_map is all -1 and out all zero).
 * Limits: num_chunks % chunks_per_group == 0, num_chunks <= MOE_MAX_CHUNKS,
 *         align >= 1.
 * ------------------------------------------------------------------------ */
MOE_PERM_API int moe_sort_chunks_and_pad(const void *in, const void *probs, int elem_bytes,
                                         int prob_bytes, int n_cap, int hidden,
                                         const int32_t *split_sizes, const int32_t *sorted_idx,
                                         int num_chunks, int chunks_per_group, int align,
                                         int out_cap, void *out, void *out_probs,
                                         int32_t *row_map, int32_t *padded_offsets,
                                         int32_t *dev_status, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * (3) Unpad and restore.
 *
 * [TE-3509] Description: padding is removed and the original order restored
 * in one copy, driven by the saved row map:
 *   out[row_map[d]] = in[d]   for every d with row_map[d] >= 0
 *   out[s] = 0                for s in [sum(split_sizes), n_cap)
 *
 *   in        [out_cap][hidden] (elem_bytes), probs [out_cap] or NULL
 *             (with out_cap == 0, NULL also when out_probs is not).
 *   row_map   [out_cap] from moe_sort_chunks_and_pad.
 *   split_sizes [num_chunks] device (gives the token total).
 *   out       [n_cap][hidden], out_probs [n_cap] or NULL.
 *   dev_status optional; MOE_DEV_BAD_ROW, MOE_DEV_BAD_CHUNKS, MOE_DEV_OVERFLOW.
 * A row_map entry at or past the token total (a map saved for other split
 * sizes) is dropped and sets MOE_DEV_BAD_ROW; the rest of out is still
 * written as above (the zero tail included).  Two entries naming the same
 * source row are outside the contract (a map from moe_sort_chunks_and_pad
 * never has them): that row then holds one of the two padded rows.
 * ------------------------------------------------------------------------ */
MOE_PERM_API int moe_unpad_and_restore_chunks(const void *in, const void *probs,
                                              int elem_bytes, int prob_bytes,
                                              const int32_t *row_map,
                                              const int32_t *split_sizes, int num_chunks,
                                              int out_cap, int hidden, int n_cap, void *out,
                                              void *out_probs, int32_t *dev_status,
                                              hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Chunk backwards.  [TE-3509] Changes: padding rows hold zeros and pass no
 * gradient back.
 *   moe_sort_chunks_and_pad_bwd: gradient of the sort-and-pad w.r.t. its
 *     input = the restore applied to the padded gradient (padding-row
 *     gradients are dropped, rows past the token total are zero).
 *   moe_unpad_and_restore_chunks_bwd: gradient of the restore w.r.t. the
 *     padded buffer = the pad copy applied to the restored gradient
 *     (padding rows get zero gradient).
 * Arguments as in the forward calls they mirror (the gradient of the
 * probs may likewise be NULL when its tensor has no rows).
 * ------------------------------------------------------------------------ */
MOE_PERM_API int moe_sort_chunks_and_pad_bwd(const void *d_out, const void *d_out_probs,
                                             int elem_bytes, int prob_bytes,
                                             const int32_t *row_map,
                                             const int32_t *split_sizes, int num_chunks,
                                             int out_cap, int hidden, int n_cap, void *d_in,
                                             void *d_in_probs, int32_t *dev_status,
                                             hipStream_t stream);
MOE_PERM_API int moe_unpad_and_restore_chunks_bwd(const void *d_out, const void *d_out_probs,
                                                  int elem_bytes, int prob_bytes,
                                                  const int32_t *row_map, int out_cap,
                                                  int hidden, int n_cap, void *d_in,
                                                  void *d_in_probs, int32_t *dev_status,
                                                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PERM_H */
