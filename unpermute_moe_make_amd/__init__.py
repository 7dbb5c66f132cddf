"""MI355X-native MoE token permute / unpermute path.

Hand-written HIP kernels for gfx950 behind a C ABI (include/moe_perm.h),
with a thin ctypes binding whose functions carry the C names:

  moe_make_row_id_map                 stable counting-sort routing row map
  moe_make_row_id_map_noalloc         the same with the library's fixed scratch
  moe_permute / moe_permute_bwd       row scatter-copy and its gradient
  moe_unpermute / moe_unpermute_bwd   fixed slot-order FMA combine, gradient
  moe_unpermute_ep                    the combine with EP rank-ordered partials
  moe_topk_softmax(_bwd)              fused top-k softmax router, gradient
  moe_make_mask_row_id_map            TE mask-map form: [T, 2E+1] map from a mask
  moe_permute_mask / moe_unpermute_mask(_bwd)  TE-order copies and combine
  moe_permute_scaled / moe_permute_mask_scaled quantized (FP8) rows + scales
  moe_sort_chunks_and_pad(_bwd)       fused chunk regroup + zero padding
  moe_unpad_and_restore_chunks(_bwd)  the matching restore

Importing the package loads libmoeperm.so and fails loudly if it is missing.
"""
from ._binding import (  # noqa: F401
    DEV_BAD_CHUNKS,
    DEV_BAD_EXPERT,
    DEV_BAD_ROW,
    DEV_DUP_EXPERT,
    DEV_OVERFLOW,
    EP_BF16_PARTIALS,
    EP_FP64_CROSS,
    EXPORTED,
    MoeError,
    library_path,
    moe_make_row_id_map,
    moe_make_row_id_map_noalloc,
    moe_make_row_id_map_workspace_bytes,
    moe_make_mask_row_id_map,
    moe_make_mask_row_id_map_workspace_bytes,
    moe_permute_mask,
    moe_permute_mask_scaled,
    moe_permute_scaled,
    moe_unpermute_mask,
    moe_unpermute_mask_bwd,
    moe_permute,
    moe_permute_bwd,
    moe_sort_chunks_and_pad,
    moe_topk_softmax,
    moe_topk_softmax_bwd,
    moe_sort_chunks_and_pad_bwd,
    moe_unpad_and_restore_chunks,
    moe_unpad_and_restore_chunks_bwd,
    moe_unpermute,
    moe_unpermute_bwd,
    moe_unpermute_ep,
)
