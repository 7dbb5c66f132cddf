// C ABI of the MoE permute library: host-side argument checks, then the
// launches.  Every check runs before the first HIP call, so a rejected call
// touches neither the device nor the HIP runtime.  Nothing here allocates,
// frees, synchronises or reads device memory.
#include <stdint.h>

#include <atomic>

#include "launch.h"
#include "moe_perm.h"

namespace {

inline bool aligned(const void *p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Checks shared by the token-row calls.
int check_rows(int T, int H, int k, int E, int n_rows) {
  if (T < 0 || H < 1 || k < 1 || E < 1) return MOE_ERR_SHAPE;
  if (k > E) return MOE_ERR_SHAPE;
  if (k > MOE_MAX_TOPK || E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * k > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)n_rows != (int64_t)T * k) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// 16-byte path when every bf16 row pointer is 16-byte aligned and the row is
// a whole number of 16-byte vectors.
bool vec_ok(int H, const void *a, const void *b, const void *c = nullptr) {
  if (H % 8 != 0) return false;
  if (!aligned(a, 16) || !aligned(b, 16)) return false;
  if (c != nullptr && !aligned(c, 16)) return false;
  return true;
}

int check_chunk_elems(int elem_bytes, int prob_bytes, const void *a, const void *b,
                      const void *pa, const void *pb) {
  if (elem_bytes != 2 && elem_bytes != 4) return MOE_ERR_UNSUPPORTED;
  if ((pa != nullptr || pb != nullptr) && prob_bytes != 2 && prob_bytes != 4)
    return MOE_ERR_UNSUPPORTED;
  if (!aligned(a, (uintptr_t)elem_bytes) || !aligned(b, (uintptr_t)elem_bytes))
    return MOE_ERR_ALIGN;
  if (pa != nullptr && !aligned(pa, (uintptr_t)prob_bytes)) return MOE_ERR_ALIGN;
  if (pb != nullptr && !aligned(pb, (uintptr_t)prob_bytes)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

// Unit of a chunk row: 16 bytes when the rows and pointers allow it.
int chunk_unit(int elem_bytes, int H, const void *a, const void *b) {
  const int64_t row_bytes = (int64_t)H * elem_bytes;
  if (row_bytes % 16 == 0 && aligned(a, 16) && aligned(b, 16)) return 16;
  return elem_bytes;
}

// Largest unit (16, 4, 2 or 1 bytes) that divides a row and aligns both bases.
int row_unit(int64_t row_bytes, const void *a, const void *b) {
  for (int u : {16, 4, 2}) {
    if (row_bytes % u == 0 && aligned(a, (uintptr_t)u) && aligned(b, (uintptr_t)u)) return u;
  }
  return 1;
}

// Side rows (scales) of a scaled permute; 0 on success.
int side_rows(const void *scale, int scale_row_bytes, void *out_scale, moe::SideRows *side) {
  side->src = static_cast<const uint8_t *>(scale);
  side->dst = static_cast<uint8_t *>(out_scale);
  side->bytes = scale != nullptr ? scale_row_bytes : 0;
  side->words = scale_row_bytes % 16 == 0 && aligned(scale, 16) && aligned(out_scale, 16) ? 2
                : scale_row_bytes % 4 == 0 && aligned(scale, 4) && aligned(out_scale, 4) ? 1
                                                                                          : 0;
  if (scale == nullptr) return MOE_OK;
  if (scale_row_bytes < 1) return MOE_ERR_SHAPE;
  if (out_scale == nullptr) return MOE_ERR_NULL;
  return MOE_OK;
}

}  // namespace

extern "C" {

MOE_PERM_API const char *moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size argument is out of range or inconsistent";
    case MOE_ERR_ALIGN: return "a pointer is not aligned to its element size";
    case MOE_ERR_UNSUPPORTED: return "a size beyond what the kernels support";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "a kernel launch failed";
    default: return "unknown status";
  }
}

MOE_PERM_API size_t moe_make_row_id_map_workspace_bytes(int num_tokens, int topk,
                                                        int num_experts) {
  if (num_tokens < 0 || topk < 1 || num_experts < 1) return 0;
  return moe::rowmap_workspace_bytes(num_tokens, topk, num_experts);
}

namespace {

// Checks of the row map calls, before any HIP call.
int check_row_id_map(const int32_t *topk_idx, int T, int k, int E, const int32_t *row_id_map,
                     const int32_t *expert_offsets, const int32_t *dev_status) {
  if (T < 0 || k < 1 || E < 1 || k > E) return MOE_ERR_SHAPE;
  if (k > MOE_MAX_TOPK || E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * k > INT32_MAX || (int64_t)T * E > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (expert_offsets == nullptr) return MOE_ERR_NULL;
  if (T > 0 && (topk_idx == nullptr || row_id_map == nullptr)) return MOE_ERR_NULL;
  if (!aligned(topk_idx, 4) || !aligned(row_id_map, 4) || !aligned(expert_offsets, 4) ||
      !aligned(dev_status, 4))
    return MOE_ERR_ALIGN;
  return MOE_OK;
}

}  // namespace

MOE_PERM_API int moe_make_row_id_map(const int32_t *topk_idx, int num_tokens, int topk,
                                     int num_experts, int32_t *row_id_map,
                                     int32_t *expert_offsets, int32_t *dev_status,
                                     void *workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  const int T = num_tokens, k = topk, E = num_experts;
  const int st = check_row_id_map(topk_idx, T, k, E, row_id_map, expert_offsets, dev_status);
  if (st) return st;
  if (T > 0) {
    const size_t need = moe::rowmap_workspace_bytes(T, k, E);
    if (workspace == nullptr || workspace_bytes < need) return MOE_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return MOE_ERR_ALIGN;
  }
  return hip_status(moe::launch_rowmap(topk_idx, T, k, E, row_id_map, expert_offsets,
                                       dev_status, workspace, stream));
}

// Scratch of the allocation-free row map: a file-scope device array, one copy
// per GPU in the library's device data.  On the host `noalloc_scratch` names a
// host-side stand-in, not device memory, so kernels get the address that
// hipGetSymbolAddress returns for the current device, looked up on the
// device's first call and kept.
static __device__ __align__(256) unsigned char noalloc_scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_noalloc_scratch[kMaxScratchDevices];

int noalloc_scratch_ptr(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return MOE_ERR_UNSUPPORTED;
  void *p = g_noalloc_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch)) != hipSuccess || p == nullptr)
      return MOE_ERR_HIP;
    g_noalloc_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return MOE_OK;
}

}  // namespace

MOE_PERM_API int moe_make_row_id_map_noalloc(const int32_t *topk_idx, int num_tokens, int topk,
                                             int num_experts, int32_t *row_id_map,
                                             int32_t *expert_offsets, int32_t *dev_status,
                                             hipStream_t stream) {
  const int T = num_tokens, k = topk, E = num_experts;
  int st = check_row_id_map(topk_idx, T, k, E, row_id_map, expert_offsets, dev_status);
  if (st) return st;
  void *ws = nullptr;
  if (T > 0) {
    if (moe::rowmap_workspace_bytes(T, k, E) > MOE_NOALLOC_SCRATCH_BYTES)
      return MOE_ERR_WORKSPACE;
    st = noalloc_scratch_ptr(&ws);
    if (st) return st;
  }
  return hip_status(moe::launch_rowmap(topk_idx, T, k, E, row_id_map, expert_offsets,
                                       dev_status, ws, stream));
}

MOE_PERM_API int moe_permute(const void *x, const float *probs, const int32_t *topk_idx,
                             const int32_t *row_id_map, int num_tokens, int hidden, int topk,
                             int num_experts, int num_out_rows, void *out, float *out_probs,
                             int32_t *dev_status, hipStream_t stream) {
  const int T = num_tokens, H = hidden, k = topk, E = num_experts;
  int st = check_rows(T, H, k, E, num_out_rows);
  if (st) return st;
  if (T == 0) return MOE_OK;
  if (!x || !topk_idx || !row_id_map || !out) return MOE_ERR_NULL;
  if (out_probs != nullptr && probs == nullptr) return MOE_ERR_NULL;
  if (!aligned(x, 2) || !aligned(out, 2) || !aligned(probs, 4) || !aligned(out_probs, 4) ||
      !aligned(topk_idx, 4) || !aligned(row_id_map, 4) || !aligned(dev_status, 4))
    return MOE_ERR_ALIGN;
  return hip_status(moe::launch_permute(x, probs, topk_idx, row_id_map, T, H, k, E,
                                        num_out_rows, out, out_probs, dev_status,
                                        vec_ok(H, x, out), stream));
}

MOE_PERM_API int moe_unpermute(const void *in, const float *probs, const int32_t *topk_idx,
                               const int32_t *row_id_map, int num_tokens, int hidden, int topk,
                               int num_experts, int num_in_rows, void *out,
                               int32_t *dev_status, hipStream_t stream) {
  const int T = num_tokens, H = hidden, k = topk, E = num_experts;
  int st = check_rows(T, H, k, E, num_in_rows);
  if (st) return st;
  if (T == 0) return MOE_OK;
  if (!in || !topk_idx || !row_id_map || !out) return MOE_ERR_NULL;
  if (!aligned(in, 2) || !aligned(out, 2) || !aligned(probs, 4) || !aligned(topk_idx, 4) ||
      !aligned(row_id_map, 4) || !aligned(dev_status, 4))
    return MOE_ERR_ALIGN;
  return hip_status(moe::launch_combine(in, probs, topk_idx, row_id_map, T, H, k, E,
                                        num_in_rows, out, nullptr, nullptr, dev_status,
                                        vec_ok(H, in, out), stream));
}

MOE_PERM_API int moe_unpermute_ep(const void *in, const float *probs, const int32_t *topk_idx,
                                  const int32_t *row_id_map, int num_tokens, int hidden,
                                  int topk, int num_experts, int num_in_rows, int ep_size,
                                  int flags, void *out, int32_t *dev_status,
                                  hipStream_t stream) {
  const int T = num_tokens, H = hidden, k = topk, E = num_experts;
  int st = check_rows(T, H, k, E, num_in_rows);
  if (st) return st;
  if (ep_size < 1 || E % ep_size != 0) return MOE_ERR_SHAPE;
  if (flags & ~(MOE_EP_BF16_PARTIALS | MOE_EP_FP64_CROSS)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!in || !topk_idx || !row_id_map || !out) return MOE_ERR_NULL;
  if (!aligned(in, 2) || !aligned(out, 2) || !aligned(probs, 4) || !aligned(topk_idx, 4) ||
      !aligned(row_id_map, 4) || !aligned(dev_status, 4))
    return MOE_ERR_ALIGN;
  return hip_status(moe::launch_combine_ep(
      in, probs, topk_idx, row_id_map, T, H, k, E, num_in_rows, ep_size,
      (flags & MOE_EP_BF16_PARTIALS) != 0, (flags & MOE_EP_FP64_CROSS) != 0, out, dev_status,
      vec_ok(H, in, out), stream));
}

MOE_PERM_API int moe_unpermute_bwd(const void *d_out, const void *fwd_in, const float *probs,
                                   const int32_t *topk_idx, const int32_t *row_id_map,
                                   int num_tokens, int hidden, int topk, int num_experts,
                                   int num_rows, void *d_in, float *d_probs,
                                   int32_t *dev_status, hipStream_t stream) {
  const int T = num_tokens, H = hidden, k = topk, E = num_experts;
  int st = check_rows(T, H, k, E, num_rows);
  if (st) return st;
  if (T == 0) return MOE_OK;
  if (!d_out || !topk_idx || !row_id_map || !d_in) return MOE_ERR_NULL;
  if (d_probs != nullptr && (probs == nullptr || fwd_in == nullptr)) return MOE_ERR_NULL;
  if (!aligned(d_out, 2) || !aligned(fwd_in, 2) || !aligned(d_in, 2) || !aligned(probs, 4) ||
      !aligned(d_probs, 4) || !aligned(topk_idx, 4) || !aligned(row_id_map, 4) ||
      !aligned(dev_status, 4))
    return MOE_ERR_ALIGN;
  if (probs == nullptr) {
    // Unweighted combine: its gradient is the plain row scatter of d_out.
    return hip_status(moe::launch_permute(d_out, nullptr, topk_idx, row_id_map, T, H, k, E,
                                          num_rows, d_in, nullptr, dev_status,
                                          vec_ok(H, d_out, d_in), stream));
  }
  const bool vec = vec_ok(H, d_out, d_in, fwd_in);
  return hip_status(moe::launch_combine_bwd(d_out, d_probs ? fwd_in : nullptr, probs, topk_idx,
                                            row_id_map, T, H, k, E, num_rows, d_in, d_probs,
                                            dev_status, vec, stream));
}

MOE_PERM_API int moe_permute_bwd(const void *d_out, const float *d_out_probs,
                                 const int32_t *topk_idx, const int32_t *row_id_map,
                                 int num_tokens, int hidden, int topk, int num_experts,
                                 int num_rows, void *d_x, float *d_probs, int32_t *dev_status,
                                 hipStream_t stream) {
  const int T = num_tokens, H = hidden, k = topk, E = num_experts;
  int st = check_rows(T, H, k, E, num_rows);
  if (st) return st;
  if (T == 0) return MOE_OK;
  if (!d_out || !topk_idx || !row_id_map || !d_x) return MOE_ERR_NULL;
  if (d_probs != nullptr && d_out_probs == nullptr) return MOE_ERR_NULL;
  if (!aligned(d_out, 2) || !aligned(d_x, 2) || !aligned(d_out_probs, 4) ||
      !aligned(d_probs, 4) || !aligned(topk_idx, 4) || !aligned(row_id_map, 4) ||
      !aligned(dev_status, 4))
    return MOE_ERR_ALIGN;
  return hip_status(moe::launch_combine(d_out, nullptr, topk_idx, row_id_map, T, H, k, E,
                                        num_rows, d_x, d_probs ? d_out_probs : nullptr, d_probs,
                                        dev_status, vec_ok(H, d_out, d_x), stream));
}

MOE_PERM_API int moe_permute_scaled(const void *x, int elem_bytes, const void *scale,
                                    int scale_row_bytes, const float *probs,
                                    const int32_t *topk_idx, const int32_t *row_id_map,
                                    int num_tokens, int hidden, int topk, int num_experts,
                                    int num_out_rows, void *out, void *out_scale,
                                    float *out_probs, int32_t *dev_status, hipStream_t stream) {
  const int T = num_tokens, H = hidden, k = topk, E = num_experts;
  int st = check_rows(T, H, k, E, num_out_rows);
  if (st) return st;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !topk_idx || !row_id_map || !out) return MOE_ERR_NULL;
  if (out_probs != nullptr && probs == nullptr) return MOE_ERR_NULL;
  moe::SideRows side;
  st = side_rows(scale, scale_row_bytes, out_scale, &side);
  if (st) return st;
  if (!aligned(x, (uintptr_t)elem_bytes) || !aligned(out, (uintptr_t)elem_bytes) ||
      !aligned(probs, 4) || !aligned(out_probs, 4) || !aligned(topk_idx, 4) ||
      !aligned(row_id_map, 4) || !aligned(dev_status, 4))
    return MOE_ERR_ALIGN;
  const int64_t row_bytes = (int64_t)H * elem_bytes;
  return hip_status(moe::launch_permute_rows(x, row_bytes, row_unit(row_bytes, x, out), probs,
                                             topk_idx, row_id_map, T, k, E, num_out_rows, out,
                                             out_probs, side, dev_status, stream));
}

MOE_PERM_API size_t moe_make_mask_row_id_map_workspace_bytes(int num_tokens, int num_experts) {
  if (num_tokens < 0 || num_experts < 1) return 0;
  return moe::maskmap_workspace_bytes(num_tokens, num_experts);
}

MOE_PERM_API int moe_make_mask_row_id_map(const void *routing_map, int mask_bytes,
                                          int num_tokens, int num_experts, int num_out_tokens,
                                          int32_t *row_id_map, int32_t *expert_offsets,
                                          void *workspace, size_t workspace_bytes,
                                          hipStream_t stream) {
  const int T = num_tokens, E = num_experts;
  if (T < 0 || E < 1 || num_out_tokens < -1) return MOE_ERR_SHAPE;
  if (E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  if (mask_bytes != 1 && mask_bytes != 4) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * E > INT32_MAX || (int64_t)T * (2 * (int64_t)E + 1) > INT32_MAX)
    return MOE_ERR_UNSUPPORTED;
  if (T > 0 && (routing_map == nullptr || row_id_map == nullptr)) return MOE_ERR_NULL;
  if (!aligned(routing_map, (uintptr_t)mask_bytes) || !aligned(row_id_map, 4) ||
      !aligned(expert_offsets, 4))
    return MOE_ERR_ALIGN;
  if (T > 0) {
    const size_t need = moe::maskmap_workspace_bytes(T, E);
    if (workspace == nullptr || workspace_bytes < need) return MOE_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return MOE_ERR_ALIGN;
  }
  return hip_status(moe::launch_maskmap(routing_map, mask_bytes, T, E, num_out_tokens,
                                        row_id_map, expert_offsets, workspace, stream));
}

// Checks shared by the mask-map row calls.
static int check_mask_rows(int T, int H, int E, int n_rows) {
  if (T < 0 || H < 1 || E < 1 || n_rows < 0) return MOE_ERR_SHAPE;
  if (E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * E > INT32_MAX || (int64_t)T * (2 * (int64_t)E + 1) > INT32_MAX)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

MOE_PERM_API int moe_permute_mask(const void *x, const float *probs, const int32_t *row_id_map,
                                  int num_tokens, int hidden, int num_experts, int num_out_rows,
                                  void *out, float *out_probs, int32_t *dev_status,
                                  hipStream_t stream) {
  const int T = num_tokens, H = hidden, E = num_experts;
  int st = check_mask_rows(T, H, E, num_out_rows);
  if (st) return st;
  if (T == 0) return MOE_OK;
  if (!x || !row_id_map || (num_out_rows > 0 && !out)) return MOE_ERR_NULL;
  if (out_probs != nullptr && probs == nullptr) return MOE_ERR_NULL;
  if (!aligned(x, 2) || !aligned(out, 2) || !aligned(probs, 4) || !aligned(out_probs, 4) ||
      !aligned(row_id_map, 4) || !aligned(dev_status, 4))
    return MOE_ERR_ALIGN;
  return hip_status(moe::launch_mask_permute(x, probs, row_id_map, T, H, E, num_out_rows, out,
                                             out_probs, dev_status, vec_ok(H, x, out), stream));
}

MOE_PERM_API int moe_permute_mask_scaled(const void *x, int elem_bytes, const void *scale,
                                         int scale_row_bytes, const float *probs,
                                         const int32_t *row_id_map, int num_tokens, int hidden,
                                         int num_experts, int num_out_rows, void *out,
                                         void *out_scale, float *out_probs, int32_t *dev_status,
                                         hipStream_t stream) {
  const int T = num_tokens, H = hidden, E = num_experts;
  int st = check_mask_rows(T, H, E, num_out_rows);
  if (st) return st;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !row_id_map || (num_out_rows > 0 && !out)) return MOE_ERR_NULL;
  if (out_probs != nullptr && probs == nullptr) return MOE_ERR_NULL;
  moe::SideRows side;
  st = side_rows(scale, scale_row_bytes, out_scale, &side);
  if (st) return st;
  if (!aligned(x, (uintptr_t)elem_bytes) || !aligned(out, (uintptr_t)elem_bytes) ||
      !aligned(probs, 4) || !aligned(out_probs, 4) || !aligned(row_id_map, 4) ||
      !aligned(dev_status, 4))
    return MOE_ERR_ALIGN;
  const int64_t row_bytes = (int64_t)H * elem_bytes;
  return hip_status(moe::launch_mask_permute_rows(x, row_bytes, row_unit(row_bytes, x, out),
                                                  probs, row_id_map, T, E, num_out_rows, out,
                                                  out_probs, side, dev_status, stream));
}

MOE_PERM_API int moe_unpermute_mask(const void *in, const float *merging_probs,
                                    const float *permuted_probs, const int32_t *row_id_map,
                                    int num_tokens, int hidden, int num_experts, int num_in_rows,
                                    void *out, float *unpermuted_probs, int32_t *dev_status,
                                    hipStream_t stream) {
  const int T = num_tokens, H = hidden, E = num_experts;
  int st = check_mask_rows(T, H, E, num_in_rows);
  if (st) return st;
  if (T == 0) return MOE_OK;
  if (!row_id_map || !out || (num_in_rows > 0 && !in)) return MOE_ERR_NULL;
  if (permuted_probs != nullptr && unpermuted_probs == nullptr) return MOE_ERR_NULL;
  if (!aligned(in, 2) || !aligned(out, 2) || !aligned(merging_probs, 4) ||
      !aligned(permuted_probs, 4) || !aligned(unpermuted_probs, 4) ||
      !aligned(row_id_map, 4) || !aligned(dev_status, 4))
    return MOE_ERR_ALIGN;
  const bool vec = in != nullptr ? vec_ok(H, in, out) : vec_ok(H, out, out);
  return hip_status(moe::launch_mask_unpermute(in, merging_probs, permuted_probs, row_id_map, T,
                                               H, E, num_in_rows, out, unpermuted_probs,
                                               dev_status, vec, stream));
}

MOE_PERM_API int moe_unpermute_mask_bwd(const void *d_out, const void *fwd_in,
                                        const float *merging_probs, const int32_t *row_id_map,
                                        int num_tokens, int hidden, int num_experts,
                                        int num_rows, void *d_in, float *d_merging_probs,
                                        int32_t *dev_status, hipStream_t stream) {
  const int T = num_tokens, H = hidden, E = num_experts;
  int st = check_mask_rows(T, H, E, num_rows);
  if (st) return st;
  if (T == 0) return MOE_OK;
  if (!d_out || !merging_probs || !row_id_map || (num_rows > 0 && !d_in)) return MOE_ERR_NULL;
  if (d_merging_probs != nullptr && num_rows > 0 && fwd_in == nullptr) return MOE_ERR_NULL;
  if (!aligned(d_out, 2) || !aligned(fwd_in, 2) || !aligned(d_in, 2) ||
      !aligned(merging_probs, 4) || !aligned(d_merging_probs, 4) || !aligned(row_id_map, 4) ||
      !aligned(dev_status, 4))
    return MOE_ERR_ALIGN;
  const void *d_in_or = d_in != nullptr ? d_in : d_out;
  const bool vec = vec_ok(H, d_out, d_in_or, d_merging_probs ? fwd_in : nullptr);
  return hip_status(moe::launch_mask_unpermute_bwd(d_out, fwd_in, merging_probs, row_id_map, T,
                                                   H, E, num_rows, d_in, d_merging_probs,
                                                   dev_status, vec, stream));
}

MOE_PERM_API int moe_topk_softmax(const void *logits, int logit_bytes, int num_tokens,
                                  int num_experts, int topk, int32_t *topk_idx, void *probs,
                                  int prob_bytes, hipStream_t stream) {
  const int T = num_tokens, E = num_experts, k = topk;
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_SHAPE;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if ((logit_bytes != 2 && logit_bytes != 4) || (prob_bytes != 2 && prob_bytes != 4))
    return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * E > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !probs) return MOE_ERR_NULL;
  if (!aligned(logits, (uintptr_t)logit_bytes) || !aligned(topk_idx, 4) ||
      !aligned(probs, (uintptr_t)prob_bytes))
    return MOE_ERR_ALIGN;
  return hip_status(moe::launch_topk_softmax(logits, logit_bytes, T, E, k, topk_idx, probs,
                                             prob_bytes, stream));
}

MOE_PERM_API int moe_topk_softmax_bwd(const void *d_probs, const void *probs, int prob_bytes,
                                      const int32_t *topk_idx, int num_tokens, int num_experts,
                                      int topk, void *d_logits, int logit_bytes,
                                      int32_t *dev_status, hipStream_t stream) {
  const int T = num_tokens, E = num_experts, k = topk;
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_SHAPE;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if ((logit_bytes != 2 && logit_bytes != 4) || (prob_bytes != 2 && prob_bytes != 4))
    return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * E > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!d_probs || !probs || !topk_idx || !d_logits) return MOE_ERR_NULL;
  if (!aligned(d_probs, (uintptr_t)prob_bytes) || !aligned(probs, (uintptr_t)prob_bytes) ||
      !aligned(topk_idx, 4) || !aligned(d_logits, (uintptr_t)logit_bytes) ||
      !aligned(dev_status, 4))
    return MOE_ERR_ALIGN;
  return hip_status(moe::launch_topk_softmax_bwd(d_probs, probs, prob_bytes, topk_idx, T, E, k,
                                                 d_logits, logit_bytes, dev_status, stream));
}

MOE_PERM_API int moe_sort_chunks_and_pad(const void *in, const void *probs, int elem_bytes,
                                         int prob_bytes, int n_cap, int hidden,
                                         const int32_t *split_sizes, const int32_t *sorted_idx,
                                         int num_chunks, int chunks_per_group, int align,
                                         int out_cap, void *out, void *out_probs,
                                         int32_t *row_map, int32_t *padded_offsets,
                                         int32_t *dev_status, hipStream_t stream) {
  const int C = num_chunks, R = chunks_per_group, H = hidden;
  if (n_cap < 0 || out_cap < 0 || H < 1 || C < 1 || R < 1 || align < 1) return MOE_ERR_SHAPE;
  if (C % R != 0) return MOE_ERR_SHAPE;
  if (C > MOE_MAX_CHUNKS) return MOE_ERR_UNSUPPORTED;
  if (!split_sizes || !sorted_idx || !padded_offsets) return MOE_ERR_NULL;
  if (out_cap > 0 && (!out || !row_map)) return MOE_ERR_NULL;
  if (n_cap > 0 && !in) return MOE_ERR_NULL;
  // with no source rows an empty probs tensor may be NULL; no kernel reads it
  if (out_probs != nullptr && probs == nullptr && n_cap > 0) return MOE_ERR_NULL;
  int st = check_chunk_elems(elem_bytes, prob_bytes, in, out, probs, out_probs);
  if (st) return st;
  if (!aligned(split_sizes, 4) || !aligned(sorted_idx, 4) || !aligned(row_map, 4) ||
      !aligned(padded_offsets, 4) || !aligned(dev_status, 4))
    return MOE_ERR_ALIGN;
  const int unit = chunk_unit(elem_bytes, H, in, out);
  const int64_t row_units = (int64_t)H * elem_bytes / unit;
  return hip_status(moe::launch_sort_and_pad(in, out_probs ? probs : nullptr, prob_bytes, unit,
                                             row_units, split_sizes, sorted_idx, C, R, align,
                                             n_cap, out_cap, out, out_probs, row_map,
                                             padded_offsets, dev_status, stream));
}

namespace {
int restore_common(const void *in, const void *probs, int elem_bytes, int prob_bytes,
                   const int32_t *row_map, const int32_t *split_sizes, int C, int out_cap, int H,
                   int n_cap, void *out, void *out_probs, int32_t *dev_status,
                   hipStream_t stream) {
  if (n_cap < 0 || out_cap < 0 || H < 1 || C < 1) return MOE_ERR_SHAPE;
  if (C > MOE_MAX_CHUNKS) return MOE_ERR_UNSUPPORTED;
  if (!split_sizes) return MOE_ERR_NULL;
  if (out_cap > 0 && (!in || !row_map)) return MOE_ERR_NULL;
  if (n_cap > 0 && !out) return MOE_ERR_NULL;
  if (out_probs != nullptr && probs == nullptr && out_cap > 0) return MOE_ERR_NULL;
  int st = check_chunk_elems(elem_bytes, prob_bytes, in, out, probs, out_probs);
  if (st) return st;
  if (!aligned(split_sizes, 4) || !aligned(row_map, 4) || !aligned(dev_status, 4))
    return MOE_ERR_ALIGN;
  const int unit = chunk_unit(elem_bytes, H, in, out);
  const int64_t row_units = (int64_t)H * elem_bytes / unit;
  return hip_status(moe::launch_restore_copy(in, out_probs ? probs : nullptr, prob_bytes, unit,
                                             row_units, row_map, split_sizes, C, out_cap, n_cap,
                                             out, out_probs, dev_status, stream));
}
}  // namespace

MOE_PERM_API int moe_unpad_and_restore_chunks(const void *in, const void *probs, int elem_bytes,
                                              int prob_bytes, const int32_t *row_map,
                                              const int32_t *split_sizes, int num_chunks,
                                              int out_cap, int hidden, int n_cap, void *out,
                                              void *out_probs, int32_t *dev_status,
                                              hipStream_t stream) {
  return restore_common(in, probs, elem_bytes, prob_bytes, row_map, split_sizes, num_chunks,
                        out_cap, hidden, n_cap, out, out_probs, dev_status, stream);
}

MOE_PERM_API int moe_sort_chunks_and_pad_bwd(const void *d_out, const void *d_out_probs,
                                             int elem_bytes, int prob_bytes,
                                             const int32_t *row_map, const int32_t *split_sizes,
                                             int num_chunks, int out_cap, int hidden, int n_cap,
                                             void *d_in, void *d_in_probs, int32_t *dev_status,
                                             hipStream_t stream) {
  return restore_common(d_out, d_out_probs, elem_bytes, prob_bytes, row_map, split_sizes,
                        num_chunks, out_cap, hidden, n_cap, d_in, d_in_probs, dev_status,
                        stream);
}

MOE_PERM_API int moe_unpad_and_restore_chunks_bwd(const void *d_out, const void *d_out_probs,
                                                  int elem_bytes, int prob_bytes,
                                                  const int32_t *row_map, int out_cap,
                                                  int hidden, int n_cap, void *d_in,
                                                  void *d_in_probs, int32_t *dev_status,
                                                  hipStream_t stream) {
  const int H = hidden;
  if (n_cap < 0 || out_cap < 0 || H < 1) return MOE_ERR_SHAPE;
  if (out_cap > 0 && (!d_in || !row_map)) return MOE_ERR_NULL;
  if (n_cap > 0 && out_cap > 0 && !d_out) return MOE_ERR_NULL;
  if (d_in_probs != nullptr && d_out_probs == nullptr && n_cap > 0) return MOE_ERR_NULL;
  int st = check_chunk_elems(elem_bytes, prob_bytes, d_out, d_in, d_out_probs, d_in_probs);
  if (st) return st;
  if (!aligned(row_map, 4) || !aligned(dev_status, 4)) return MOE_ERR_ALIGN;
  const int unit = chunk_unit(elem_bytes, H, d_out, d_in);
  const int64_t row_units = (int64_t)H * elem_bytes / unit;
  return hip_status(moe::launch_pad_copy(d_out, d_in_probs ? d_out_probs : nullptr, prob_bytes,
                                         unit, row_units, n_cap, row_map, out_cap, d_in,
                                         d_in_probs, dev_status, stream));
}

}  // extern "C"
