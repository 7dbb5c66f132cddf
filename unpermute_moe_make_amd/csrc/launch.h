// Internal launchers: one per kernel family.  Arguments are already checked
// by the C ABI layer (api.hip); these only pick launch shapes and enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// A per-row side vector (quantization scales) moved along with its data row.
struct SideRows {
  const uint8_t *src;   // [rows][bytes]
  uint8_t *dst;         // [out rows][bytes]
  int64_t bytes;        // bytes per row
  int words;            // 1: copy 4-byte words (bytes % 4 == 0, both bases aligned);
                        // 2: 16-byte units as well (bytes % 16 == 0, bases 16-aligned)
};

// Row map (stable counting sort).
size_t rowmap_workspace_bytes(int T, int k, int E);
hipError_t launch_rowmap(const int32_t *topk_idx, int T, int k, int E, int32_t *row_id_map,
                         int32_t *expert_offsets, int32_t *dev_status, void *ws,
                         hipStream_t s);

// Token-row kernels.  `vec` selects the 16-byte path (rows of 8-element
// vectors, 16-byte aligned) or the element path.
hipError_t launch_permute(const void *x, const float *probs, const int32_t *topk_idx,
                          const int32_t *row_id_map, int T, int H, int k, int E, int n_rows,
                          void *out, float *out_probs, int32_t *dev_status, bool vec,
                          hipStream_t s);
hipError_t launch_combine(const void *in, const float *probs, const int32_t *topk_idx,
                          const int32_t *row_id_map, int T, int H, int k, int E, int n_rows,
                          void *out, const float *gather_src, float *gather_dst,
                          int32_t *dev_status, bool vec, hipStream_t s);
hipError_t launch_combine_ep(const void *in, const float *probs, const int32_t *topk_idx,
                             const int32_t *row_id_map, int T, int H, int k, int E, int n_rows,
                             int ep_size, bool bf16_partials, bool fp64_cross, void *out,
                             int32_t *dev_status, bool vec, hipStream_t s);
hipError_t launch_combine_bwd(const void *d_out, const void *fwd_in, const float *probs,
                              const int32_t *topk_idx, const int32_t *row_id_map, int T, int H,
                              int k, int E, int n_rows, void *d_in, float *d_probs,
                              int32_t *dev_status, bool vec, hipStream_t s);

// Rows of any element size (quantized rows) with optional side rows
// (their scales): row_bytes per data row, moved in unit_bytes units.
hipError_t launch_permute_rows(const void *x, int64_t row_bytes, int unit_bytes,
                               const float *probs, const int32_t *topk_idx,
                               const int32_t *row_id_map, int T, int k, int E, int n_rows,
                               void *out, float *out_probs, const SideRows &side,
                               int32_t *dev_status, hipStream_t s);
hipError_t launch_mask_permute_rows(const void *x, int64_t row_bytes, int unit_bytes,
                                    const float *probs, const int32_t *map, int T, int E,
                                    int n_rows, void *out, float *out_probs,
                                    const SideRows &side, int32_t *dev_status, hipStream_t s);

// TransformerEngine mask-map form: map builder and its row kernels.
size_t maskmap_workspace_bytes(int T, int E);
hipError_t launch_maskmap(const void *routing_map, int mask_bytes, int T, int E, int num_out,
                          int32_t *map, int32_t *expert_offsets, void *ws, hipStream_t s);
hipError_t launch_mask_permute(const void *x, const float *probs, const int32_t *map, int T,
                               int H, int E, int n_rows, void *out, float *out_probs,
                               int32_t *dev_status, bool vec, hipStream_t s);
hipError_t launch_mask_unpermute(const void *in, const float *merging_probs,
                                 const float *permuted_probs, const int32_t *map, int T, int H,
                                 int E, int n_rows, void *out, float *unpermuted_probs,
                                 int32_t *dev_status, bool vec, hipStream_t s);
hipError_t launch_mask_unpermute_bwd(const void *d_out, const void *fwd_in,
                                     const float *merging_probs, const int32_t *map, int T,
                                     int H, int E, int n_rows, void *d_in,
                                     float *d_merging_probs, int32_t *dev_status, bool vec,
                                     hipStream_t s);

// Fused top-k softmax router and its gradient.
hipError_t launch_topk_softmax(const void *logits, int logit_bytes, int T, int E, int k,
                               int32_t *topk_idx, void *probs, int prob_bytes, hipStream_t s);
hipError_t launch_topk_softmax_bwd(const void *d_probs, const void *probs, int prob_bytes,
                                   const int32_t *topk_idx, int T, int E, int k, void *d_logits,
                                   int logit_bytes, int32_t *dev_status, hipStream_t s);

// Chunk map and the two chunk copies.  unit_bytes is 16, 4 or 2; the row
// length in units is row_units.
hipError_t launch_chunk_map(const int32_t *split_sizes, const int32_t *sorted_idx, int C, int R,
                            int A, int n_cap, int out_cap, int32_t *row_map,
                            int32_t *padded_offsets, int32_t *dev_status, hipStream_t s);
hipError_t launch_pad_copy(const void *in, const void *probs, int prob_bytes, int unit_bytes,
                           int64_t row_units, int n_cap, const int32_t *row_map, int out_cap,
                           void *out, void *out_probs, int32_t *dev_status, hipStream_t s);
// The map and the pad copy of one sort-and-pad call: one fused launch for a
// small destination, else the map and the pad copy.
hipError_t launch_sort_and_pad(const void *in, const void *probs, int prob_bytes, int unit_bytes,
                               int64_t row_units, const int32_t *split_sizes,
                               const int32_t *sorted_idx, int C, int R, int A, int n_cap,
                               int out_cap, void *out, void *out_probs, int32_t *row_map,
                               int32_t *padded_offsets, int32_t *dev_status, hipStream_t s);
hipError_t launch_restore_copy(const void *in, const void *probs, int prob_bytes, int unit_bytes,
                               int64_t row_units, const int32_t *row_map,
                               const int32_t *split_sizes, int C, int out_cap, int n_cap,
                               void *out, void *out_probs, int32_t *dev_status, hipStream_t s);

}  // namespace moe
