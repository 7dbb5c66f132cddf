// Token-row kernels on the TransformerEngine mask-map form (d9d
// permute_with_probs.py): the permute (_permute_kernel, with the prob == 0
// padding rule), the unpermute (_unpermute_kernel: rows visited in map
// order, each multiplied by its merging prob and then added in fp32, one
// bf16 rounding; optional [T][E] unpermuted probs) and the unpermute
// backward with merging probs (_unpermute_bwd_with_merging_probs_kernel).
//
// The map row of token t is [rows (n) | unused | experts (n) | unused | n],
// width 2E+1.  A token may be routed to any number of experts, so the
// kernels resolve its slots into LDS 64 at a time.  Otherwise the design is
// that of the top-k row kernels: one workgroup per token row (slice), 16-byte
// units, every load of a batch in flight before the arithmetic.
#include "common.h"
#include "launch.h"
#include "rows.h"

namespace moe {
namespace {

// Streaming policy of the permute on calls larger than kStreamBytes (bit 0:
// non-temporal loads, bit 1: non-temporal stores), as for the top-k permute.
#ifndef MOE_MASK_PERMUTE_STREAM
#define MOE_MASK_PERMUTE_STREAM 2
#endif


constexpr int kSlotChunk = 64;   // slots resolved into LDS at a time
constexpr int kBatch = 8;        // rows loaded together in the combine

// The token's slot count; bad counts become 0 and set a status bit.
__device__ __forceinline__ int mask_count(const int32_t *__restrict__ mrow, int E, int *bad) {
  const int n = mrow[2 * E];
  if (n < 0 || n > E) {
    *bad |= MOE_DEV_BAD_ROW;
    return 0;
  }
  return n;
}

// Slot i of the token: its row (or -1 with a status bit) and expert.
__device__ __forceinline__ int64_t mask_slot(const int32_t *__restrict__ mrow, int E, int n_rows,
                                             int i, int *expert, int *bad) {
  const int e = mrow[E + i];
  const int r = mrow[i];
  *expert = e;
  if ((unsigned)e >= (unsigned)E) {
    *bad |= MOE_DEV_BAD_EXPERT;
    return -1;
  }
  if ((unsigned)r >= (unsigned)n_rows) {
    *bad |= MOE_DEV_BAD_ROW;
    return -1;
  }
  return r;
}

// Slot check of map entries read ahead of the count: the row, or -1 with a
// status bit (as mask_slot).
__device__ __forceinline__ int64_t checked_slot(int e, int r, int E, int n_rows, int *bad) {
  if ((unsigned)e >= (unsigned)E) {
    *bad |= MOE_DEV_BAD_EXPERT;
    return -1;
  }
  if ((unsigned)r >= (unsigned)n_rows) {
    *bad |= MOE_DEV_BAD_ROW;
    return -1;
  }
  return r;
}

// out[row] = x[t] for each slot; with probs, out_probs[row] = probs[t][e]
// and a zero prob writes a zero row.
// SIDE: also move each token's side row (quantization scales) to the same
// destinations, padded slots included.
template <typename U, int VPT, int NTM, bool SIDE>
__global__ __launch_bounds__(kRowThreads) void mask_permute_kernel(
    const U *__restrict__ x, const float *__restrict__ probs, const int32_t *__restrict__ map,
    int T, int64_t V, int E, int n_rows, U *__restrict__ out, float *__restrict__ out_probs,
    SideRows side, int32_t *__restrict__ dev_status, int ahead) {
  __shared__ int64_t srow[kSlotChunk];
  __shared__ int szero[kSlotChunk];
  const int64_t tb = spill_block();
  if (tb >= T) return;  // a workgroup past the last token
  const int t = (int)tb;
  const int64_t c0 = (int64_t)blockIdx.y * blockDim.x * VPT + threadIdx.x;
  const int32_t *mrow = map + (int64_t)t * (2 * (int64_t)E + 1);

  U v[VPT];
  const U *xr = x + (int64_t)t * V;
#pragma unroll
  for (int i = 0; i < VPT; i++) {
    const int64_t c = c0 + (int64_t)i * blockDim.x;
    if (c < V) v[i] = ld_row<(NTM & 1) != 0>(xr + c);
  }
  SideCache sc{};
  if (SIDE && blockIdx.y == 0) sc = load_side_row(side, t);
  U zero;
  zero = U{};
  int bad = 0;
  const int n = mask_count(mrow, E, &bad);
  for (int j0 = 0; j0 < n; j0 += kSlotChunk) {
    const int nj = min(kSlotChunk, n - j0);
    if ((int)threadIdx.x < nj) {
      int e;
      const int64_t r = mask_slot(mrow, E, n_rows, j0 + threadIdx.x, &e, &bad);
      int z = 0;
      if (probs != nullptr && r >= 0) {
        // A streaming call reads the probs past the caches: at 16384 tokens
        // x 256 experts the [T][E] probs (16.8 MB, one line per slot) would
        // otherwise push part of the token rows out of the Infinity Cache
        // between back-to-back calls (357 us warm against 361-363).
        const float p = ld_row<NTM != 0>(probs + (int64_t)t * E + e);
        z = p == 0.0f;
        if (blockIdx.y == 0 && out_probs != nullptr) out_probs[r] = p;
      }
      srow[threadIdx.x] = r;
      szero[threadIdx.x] = z;
    }
    __syncthreads();
    for (int j = 0; j < nj; j++) {
      const int64_t r = srow[j];
      if (r < 0) continue;
      const bool z = szero[j] != 0;
      U *orow = out + r * V;
#pragma unroll
      for (int i = 0; i < VPT; i++) {
        const int64_t c = c0 + (int64_t)i * blockDim.x;
        if (c < V) st_row<(NTM & 2) != 0>(z ? zero : v[i], orow + c);
      }
      if (SIDE && blockIdx.y == 0) store_side_row(side, sc, t, r);
    }
    // Before the next chunk overwrites the slots in LDS.  Only then: a
    // barrier after the last stores, which no later LDS access needs, holds
    // every wave until the slowest has issued its stores (the 16384 x 7168
    // top-8 mask permute took 415-420 us cold with it, 392-394 without).
    if (j0 + kSlotChunk < n) __syncthreads();
  }
  // A streaming call prefetches this slice of a later token's row after its
  // stores, as the top-k permute does.
  if constexpr (NTM != 0 && !SIDE) {
    const int64_t s0 = (int64_t)blockIdx.y * blockDim.x * VPT;
    keep_loaded(prefetch_lines<U, VPT>(
        (int64_t)t + ahead < T ? x + (int64_t)(t + ahead) * V : nullptr, s0,
        min(V, s0 + (int64_t)blockDim.x * VPT), xr + s0));
  }
  if (blockIdx.y == 0) report(dev_status, bad);
}

// out[t] = bf16(sum over slots in map order of (in[row] * p)), the product
// and the sum each rounded in fp32 (MERGE), or of in[row] alone.  With
// unpermuted_probs, row t of it gets permuted_probs[row] at each routed
// expert (0 when permuted_probs is NULL) and 0 elsewhere.
template <int EPV, int VPT, bool NT, bool MERGE>
__global__ __launch_bounds__(kRowThreads) void mask_unpermute_kernel(
    const typename Bf16Unit<EPV>::T *__restrict__ in, const float *__restrict__ merging_probs,
    const float *__restrict__ permuted_probs, const int32_t *__restrict__ map, int T, int64_t V,
    int E, int n_rows, typename Bf16Unit<EPV>::T *__restrict__ out,
    float *__restrict__ unpermuted_probs, int32_t *__restrict__ dev_status) {
  using Unit = Bf16Unit<EPV>;
  using U = typename Unit::T;
  __shared__ int64_t srow[kSlotChunk];
  __shared__ float sp[kSlotChunk];
  __shared__ float sup[MOE_MAX_EXPERTS];
  const int64_t tb = spill_block();
  if (tb >= T) return;  // a workgroup past the last token
  const int t = (int)tb;
  const int64_t c0 = (int64_t)blockIdx.y * blockDim.x * VPT + threadIdx.x;
  const int32_t *mrow = map + (int64_t)t * (2 * (int64_t)E + 1);
  const bool scatter = unpermuted_probs != nullptr && blockIdx.y == 0;
  if (scatter)
    for (int e = threadIdx.x; e < E; e += blockDim.x) sup[e] = 0.0f;
  __syncthreads();

  float acc[VPT][EPV];
#pragma unroll
  for (int i = 0; i < VPT; i++)
#pragma unroll
    for (int e = 0; e < EPV; e++) acc[i][e] = 0.0f;

  int bad = 0;
  const int n = mask_count(mrow, E, &bad);
  for (int j0 = 0; j0 < n; j0 += kSlotChunk) {
    const int nj = min(kSlotChunk, n - j0);
    if ((int)threadIdx.x < nj) {
      int e;
      const int64_t r = mask_slot(mrow, E, n_rows, j0 + threadIdx.x, &e, &bad);
      srow[threadIdx.x] = r;
      if (MERGE) sp[threadIdx.x] = r >= 0 ? merging_probs[(int64_t)t * E + e] : 0.0f;
      if (scatter && r >= 0) sup[e] = permuted_probs != nullptr ? permuted_probs[r] : 0.0f;
    }
    __syncthreads();
    for (int jb = 0; jb < nj; jb += kBatch) {
      U vals[kBatch][VPT];
#pragma unroll
      for (int jj = 0; jj < kBatch; jj++) {
        const int64_t r = jb + jj < nj ? srow[jb + jj] : -1;
#pragma unroll
        for (int i = 0; i < VPT; i++) {
          const int64_t c = c0 + (int64_t)i * blockDim.x;
          vals[jj][i] = (r >= 0 && c < V) ? ld_row<NT>(in + r * V + c) : Unit::zero();
        }
      }
#pragma unroll
      for (int jj = 0; jj < kBatch; jj++) {
        if (jb + jj >= nj) break;
        const float p = MERGE ? sp[jb + jj] : 1.0f;
#pragma unroll
        for (int i = 0; i < VPT; i++) {
          float f[EPV];
          Unit::unpack(vals[jj][i], f);
#pragma unroll
          for (int e = 0; e < EPV; e++) {
            const float term = MERGE ? f[e] * p : f[e];   // rounded before the add
            acc[i][e] = acc[i][e] + term;
          }
        }
      }
    }
    if (j0 + kSlotChunk < n) __syncthreads();   // slots in LDS reused by the next chunk
  }

  U *orow = out + (int64_t)t * V;
#pragma unroll
  for (int i = 0; i < VPT; i++) {
    const int64_t c = c0 + (int64_t)i * blockDim.x;
    if (c < V) st_row<NT>(Unit::pack(acc[i]), orow + c);
  }
  if (scatter)
    for (int e = threadIdx.x; e < E; e += blockDim.x)
      unpermuted_probs[(int64_t)t * E + e] = sup[e];
  if (blockIdx.y == 0) report(dev_status, bad);
}

// d_in[row] = bf16(d_out[t] * p) per slot (one fp32 rounding, then bf16);
// d_merging_probs[t][e] = sum_h fwd_in[row][h] * d_out[t][h] at routed
// experts (a fixed per-lane fmaf chain, then a fixed tree), 0 elsewhere.
// With the probs gradient the workgroup walks the whole row in passes.
template <int EPV, int VPT, bool NT, int MAXT>
__global__ __launch_bounds__(MAXT) void mask_unpermute_bwd_kernel(
    const typename Bf16Unit<EPV>::T *__restrict__ d_out,
    const typename Bf16Unit<EPV>::T *__restrict__ fwd_in,
    const float *__restrict__ merging_probs, const int32_t *__restrict__ map, int T, int64_t V,
    int E, int n_rows, typename Bf16Unit<EPV>::T *__restrict__ d_in,
    float *__restrict__ d_merging_probs, int32_t *__restrict__ dev_status) {
  using Unit = Bf16Unit<EPV>;
  using U = typename Unit::T;
  __shared__ int64_t srow[kSlotChunk];
  __shared__ float sp[kSlotChunk];
  __shared__ int se[kSlotChunk];
  __shared__ float sred[MAXT / kWave][kBatch];
  __shared__ float sdp[MOE_MAX_EXPERTS];
  __shared__ float spr[MOE_MAX_EXPERTS];
  const int64_t tb = spill_block();
  if (tb >= T) return;  // a workgroup past the last token
  const int t = (int)tb;
  const int64_t pass = (int64_t)blockDim.x * VPT;
  const int64_t stride = pass * gridDim.y;
  const int64_t cfirst = (int64_t)blockIdx.y * pass + threadIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  const int32_t *mrow = map + (int64_t)t * (2 * (int64_t)E + 1);
  const U *grow = d_out + (int64_t)t * V;
  // First pass of the token's upstream gradient, issued before the slots are
  // resolved (as in the top-k backward): its read overlaps the map reads.
  U graw[VPT];
#pragma unroll
  for (int i = 0; i < VPT; i++) {
    const int64_t c = cfirst + (int64_t)i * blockDim.x;
    graw[i] = c < V ? ld_row<NT>(grow + c) : Unit::zero();
  }
  // The map entries of the first 64 slots and the token's merging-prob row
  // are read together, before the slot count is known, and the probs go to
  // LDS: one round trip to memory instead of four chained ones (count, expert,
  // row, prob), which with one 16-wave workgroup per CU showed in the cold
  // time (16384 x 7168 top-8: 725 us against 738).
  int e_ahead = 0, r_ahead = 0;
  if ((int)threadIdx.x < min(E, kSlotChunk)) {
    e_ahead = mrow[E + threadIdx.x];
    r_ahead = mrow[threadIdx.x];
  }
  const float p_own = (int)threadIdx.x < E ? merging_probs[(int64_t)t * E + threadIdx.x] : 0.0f;
  if ((int)threadIdx.x < E) spr[threadIdx.x] = p_own;
  for (int e = threadIdx.x + blockDim.x; e < E; e += blockDim.x)
    spr[e] = merging_probs[(int64_t)t * E + e];
  int bad = 0;
  const int n = mask_count(mrow, E, &bad);
  const bool want_dot = d_merging_probs != nullptr;
  if (want_dot)
    for (int e = threadIdx.x; e < E; e += blockDim.x) sdp[e] = 0.0f;
  __syncthreads();

  for (int j0 = 0; j0 < n; j0 += kSlotChunk) {
    const int nj = min(kSlotChunk, n - j0);
    if ((int)threadIdx.x < nj) {
      int e;
      int64_t r;
      if (j0 == 0) {
        e = e_ahead;
        r = checked_slot(e, r_ahead, E, n_rows, &bad);
      } else {
        r = mask_slot(mrow, E, n_rows, j0 + threadIdx.x, &e, &bad);
      }
      srow[threadIdx.x] = r;
      se[threadIdx.x] = r >= 0 ? e : -1;
      sp[threadIdx.x] = r >= 0 ? spr[e] : 0.0f;
    }
    __syncthreads();
    for (int jb = 0; jb < nj; jb += kBatch) {
      float part[kBatch];
#pragma unroll
      for (int jj = 0; jj < kBatch; jj++) part[jj] = 0.0f;
      for (int64_t cb = cfirst; cb < V; cb += stride) {
        if (!(j0 == 0 && jb == 0 && cb == cfirst)) {
#pragma unroll
          for (int i = 0; i < VPT; i++) {
            const int64_t c = cb + (int64_t)i * blockDim.x;
            graw[i] = c < V ? ld_row<NT>(grow + c) : Unit::zero();
          }
        }
        U fin[kBatch][VPT];
        if (want_dot) {
#pragma unroll
          for (int jj = 0; jj < kBatch; jj++) {
            const int64_t r = jb + jj < nj ? srow[jb + jj] : -1;
#pragma unroll
            for (int i = 0; i < VPT; i++) {
              const int64_t c = cb + (int64_t)i * blockDim.x;
              fin[jj][i] = (r >= 0 && c < V) ? ld_row<NT>(fwd_in + r * V + c) : Unit::zero();
            }
          }
        }
        float g[VPT][EPV];
#pragma unroll
        for (int i = 0; i < VPT; i++) Unit::unpack(graw[i], g[i]);
#pragma unroll
        for (int jj = 0; jj < kBatch; jj++) {
          if (jb + jj >= nj) break;
          const int64_t r = srow[jb + jj];
          const float p = sp[jb + jj];
#pragma unroll
          for (int i = 0; i < VPT; i++) {
            const int64_t c = cb + (int64_t)i * blockDim.x;
            float prod[EPV];
#pragma unroll
            for (int e = 0; e < EPV; e++) prod[e] = g[i][e] * p;
            if (r >= 0 && c < V) st_row<NT>(Unit::pack(prod), d_in + r * V + c);
            if (want_dot) {
              float f[EPV];
              Unit::unpack(fin[jj][i], f);
#pragma unroll
              for (int e = 0; e < EPV; e++) part[jj] = __builtin_fmaf(f[e], g[i][e], part[jj]);
            }
          }
        }
      }
      if (want_dot) {
#pragma unroll
        for (int jj = 0; jj < kBatch; jj++) {
          const float s = wave_sum(part[jj]);
          if (lane == 0) sred[wv][jj] = s;
        }
        __syncthreads();
        if ((int)threadIdx.x < kBatch && jb + (int)threadIdx.x < nj) {
          const int e = se[jb + threadIdx.x];
          float s = 0.0f;
          for (int w = 0; w < nwaves; w++) s += sred[w][threadIdx.x];
          if (e >= 0) sdp[e] = s;
        }
        __syncthreads();
      }
    }
    // slots in LDS reused by the next chunk; sdp was last written before the
    // barrier that ends each batch with want_dot
    if (j0 + kSlotChunk < n) __syncthreads();
  }
  if (want_dot)
    for (int e = threadIdx.x; e < E; e += blockDim.x)
      d_merging_probs[(int64_t)t * E + e] = sdp[e];
  if (blockIdx.y == 0) report(dev_status, bad);
}

template <typename U, int NTM, bool SIDE>
void mask_permute_dispatch(const void *x, const float *probs, const int32_t *map, int T,
                           int64_t V, int E, int n_rows, void *out, float *out_probs,
                           const SideRows &side, int32_t *st, hipStream_t s) {
  RowShape sh = row_shape_vpt(V, 2, kRowThreads);   // as the top-k permute
  if (sh.threads == 0) sh = row_shape(V, true);
  const dim3 grid = spill_grid(T, sh.ysplit), block(sh.threads);
  const U *xp = static_cast<const U *>(x);
  U *op = static_cast<U *>(out);
#define MOE_MASK_PERMUTE(VPTV)                                                                 \
  hipLaunchKernelGGL((mask_permute_kernel<U, VPTV, NTM, SIDE>), grid, block, 0, s, xp, probs, \
                     map, T, V, E, n_rows, op, out_probs, side, st, prefetch_ahead(sh.threads))
  switch (sh.vpt) {
    case 1: MOE_MASK_PERMUTE(1); break;
    case 2: MOE_MASK_PERMUTE(2); break;
    default: MOE_MASK_PERMUTE(4); break;
  }
#undef MOE_MASK_PERMUTE
}

template <int EPV, bool NT>
void mask_unpermute_dispatch(const void *in, const float *mp, const float *pp,
                             const int32_t *map, int T, int64_t V, int E, int n_rows, void *out,
                             float *up, int32_t *st, hipStream_t s) {
  using U = typename Bf16Unit<EPV>::T;
  // (two units per lane on 128 lanes was measured 6% slower for 4 KiB rows)
  const RowShape sh = row_shape(V, true);
  const dim3 grid = spill_grid(T, sh.ysplit), block(sh.threads);
  const U *ip = static_cast<const U *>(in);
  U *op = static_cast<U *>(out);
#define MOE_MASK_UNPERMUTE(VPTV, MERGE)                                                        \
  hipLaunchKernelGGL((mask_unpermute_kernel<EPV, VPTV, NT, MERGE>), grid, block, 0, s, ip, mp, \
                     pp, map, T, V, E, n_rows, op, up, st)
  if (mp != nullptr) {
    switch (sh.vpt) {
      case 1: MOE_MASK_UNPERMUTE(1, true); break;
      case 2: MOE_MASK_UNPERMUTE(2, true); break;
      default: MOE_MASK_UNPERMUTE(4, true); break;
    }
  } else {
    switch (sh.vpt) {
      case 1: MOE_MASK_UNPERMUTE(1, false); break;
      case 2: MOE_MASK_UNPERMUTE(2, false); break;
      default: MOE_MASK_UNPERMUTE(4, false); break;
    }
  }
#undef MOE_MASK_UNPERMUTE
}

template <int EPV, bool NT>
void mask_unpermute_bwd_dispatch(const void *d_out, const void *fwd_in, const float *mp,
                                 const int32_t *map, int T, int64_t V, int E, int n_rows,
                                 void *d_in, float *dmp, int32_t *st, hipStream_t s) {
  using U = typename Bf16Unit<EPV>::T;
  const U *gp = static_cast<const U *>(d_out);
  const U *fp = static_cast<const U *>(fwd_in);
  U *dp = static_cast<U *>(d_in);
  // One unit per lane on up to 1024 lanes when the row fits, as the top-k
  // unpermute backward.
  const RowShape wide = row_shape_vpt(V, 1, 1024);
  if (wide.threads > kRowThreads) {
    hipLaunchKernelGGL((mask_unpermute_bwd_kernel<EPV, 1, NT, 1024>), spill_grid(T, 1),
                       dim3(wide.threads), 0, s, gp, fp, mp, map, T, V, E, n_rows, dp, dmp, st);
    return;
  }
  const RowShape sh = row_shape(V, dmp == nullptr);
  const dim3 grid = spill_grid(T, sh.ysplit), block(sh.threads);
#define MOE_MASK_BWD(VPTV)                                                                      \
  hipLaunchKernelGGL((mask_unpermute_bwd_kernel<EPV, VPTV, NT, kRowThreads>), grid, block, 0, s, \
                     gp, fp, mp, map, T, V, E, n_rows, dp, dmp, st)
  switch (sh.vpt) {
    case 1: MOE_MASK_BWD(1); break;
    case 2: MOE_MASK_BWD(2); break;
    default: MOE_MASK_BWD(4); break;
  }
#undef MOE_MASK_BWD
}

// ------------------------------------ unpermute backward in two launches --

// As the top-k backward: a streaming call with merging-prob gradients runs as
// a gather of dot products and then a scaled scatter, one pattern per launch.

// d_in[row] = bf16(fp32(d_out[t]) * merging_probs[t][e]) for each slot: the
// mask permute's shape and source prefetch, one product per element.
template <int VPT, int NTM>
__global__ __launch_bounds__(kRowThreads) void mask_scale_scatter_kernel(
    const v4u *__restrict__ d_out, const float *__restrict__ merging_probs,
    const int32_t *__restrict__ map, int T, int64_t V, int E, int n_rows,
    v4u *__restrict__ d_in, int32_t *__restrict__ dev_status, int ahead) {
  using Unit = Bf16Unit<8>;
  __shared__ int64_t srow[kSlotChunk];
  __shared__ float sp[kSlotChunk];
  const int64_t tb = spill_block();
  if (tb >= T) return;  // a workgroup past the last token
  const int t = (int)tb;
  const int64_t s0 = (int64_t)blockIdx.y * blockDim.x * VPT;
  const int32_t *mrow = map + (int64_t)t * (2 * (int64_t)E + 1);
  const v4u *grow = d_out + (int64_t)t * V;
  v4u v[VPT];
#pragma unroll
  for (int i = 0; i < VPT; i++) {
    const int64_t c = s0 + threadIdx.x + (int64_t)i * blockDim.x;
    v[i] = c < V ? ld_row<(NTM & 1) != 0>(grow + c) : Unit::zero();
  }
  int bad = 0;
  const int n = mask_count(mrow, E, &bad);
  for (int j0 = 0; j0 < n; j0 += kSlotChunk) {
    const int nj = min(kSlotChunk, n - j0);
    if ((int)threadIdx.x < nj) {
      int e;
      const int64_t r = mask_slot(mrow, E, n_rows, j0 + threadIdx.x, &e, &bad);
      srow[threadIdx.x] = r;
      sp[threadIdx.x] = r >= 0 ? ld_row<NTM != 0>(merging_probs + (int64_t)t * E + e) : 0.0f;
    }
    __syncthreads();
    for (int j = 0; j < nj; j++) {
      const int64_t r = srow[j];
      if (r < 0) continue;
      const float p = sp[j];
      v4u *orow = d_in + r * V;
#pragma unroll
      for (int i = 0; i < VPT; i++) {
        const int64_t c = s0 + threadIdx.x + (int64_t)i * blockDim.x;
        float f[8];
        Unit::unpack(v[i], f);
#pragma unroll
        for (int e = 0; e < 8; e++) f[e] = f[e] * p;   // one fp32 rounding
        if (c < V) st_row<(NTM & 2) != 0>(Unit::pack(f), orow + c);
      }
    }
    if (j0 + kSlotChunk < n) __syncthreads();   // slots in LDS reused by the next chunk
  }
  if constexpr (NTM != 0)   // as in the permute
    keep_loaded(prefetch_lines<v4u, VPT>(
        (int64_t)t + ahead < T ? d_out + (int64_t)(t + ahead) * V : nullptr, s0,
        min(V, s0 + (int64_t)blockDim.x * VPT), grow + s0));
  if (blockIdx.y == 0) report(dev_status, bad);
}

// d_merging_probs[t][e] = <fwd_in[row], d_out[t]> at the routed experts, 0
// elsewhere: the dot products of the mask backward with nothing stored but
// the prob row.  Per lane an fmaf chain over its units and their elements
// in order, then a fixed wave tree and the waves in order.  The row is one
// pass of the workgroup.
template <int VPT, int NTM, int MAXT>
__global__ __launch_bounds__(MAXT) void mask_dot_gather_kernel(
    const v4u *__restrict__ d_out, const v4u *__restrict__ fwd_in,
    const int32_t *__restrict__ map, int T, int64_t V, int E, int n_rows,
    float *__restrict__ d_merging_probs, int32_t *__restrict__ dev_status) {
  using Unit = Bf16Unit<8>;
  __shared__ int64_t srow[kSlotChunk];
  __shared__ int se[kSlotChunk];
  __shared__ float sred[MAXT / kWave][kBatch];
  __shared__ float sdp[MOE_MAX_EXPERTS];
  const int64_t tb = spill_block();
  if (tb >= T) return;  // a workgroup past the last token
  const int t = (int)tb;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  const int32_t *mrow = map + (int64_t)t * (2 * (int64_t)E + 1);
  // plain loads of the upstream gradient: the scatter launched next reads it
  v4u g[VPT];
#pragma unroll
  for (int i = 0; i < VPT; i++) {
    const int64_t c = (int64_t)threadIdx.x + (int64_t)i * blockDim.x;
    g[i] = c < V ? d_out[(int64_t)t * V + c] : Unit::zero();
  }
  // the first chunk's map entries read with the count, as in the fused kernel
  int e_ahead = 0, r_ahead = 0;
  if ((int)threadIdx.x < min(E, kSlotChunk)) {
    e_ahead = mrow[E + threadIdx.x];
    r_ahead = mrow[threadIdx.x];
  }
  int bad = 0;
  const int n = mask_count(mrow, E, &bad);
  for (int e = threadIdx.x; e < E; e += blockDim.x) sdp[e] = 0.0f;
  __syncthreads();

  for (int j0 = 0; j0 < n; j0 += kSlotChunk) {
    const int nj = min(kSlotChunk, n - j0);
    if ((int)threadIdx.x < nj) {
      int e;
      int64_t r;
      if (j0 == 0) {
        e = e_ahead;
        r = checked_slot(e, r_ahead, E, n_rows, &bad);
      } else {
        r = mask_slot(mrow, E, n_rows, j0 + threadIdx.x, &e, &bad);
      }
      srow[threadIdx.x] = r;
      se[threadIdx.x] = r >= 0 ? e : -1;
    }
    __syncthreads();
    for (int jb = 0; jb < nj; jb += kBatch) {
      v4u vals[kBatch][VPT];
#pragma unroll
      for (int jj = 0; jj < kBatch; jj++) {
        const int64_t r = jb + jj < nj ? srow[jb + jj] : -1;
#pragma unroll
        for (int i = 0; i < VPT; i++) {
          const int64_t c = (int64_t)threadIdx.x + (int64_t)i * blockDim.x;
          vals[jj][i] = (r >= 0 && c < V) ? ld_row<(NTM & 1) != 0>(fwd_in + r * V + c)
                                          : Unit::zero();
        }
      }
#pragma unroll
      for (int jj = 0; jj < kBatch; jj++) {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < VPT; i++) {
          float f[8], gf[8];
          Unit::unpack(vals[jj][i], f);
          Unit::unpack(g[i], gf);
#pragma unroll
          for (int e = 0; e < 8; e++) part = __builtin_fmaf(f[e], gf[e], part);
        }
        const float sum = wave_sum(part);
        if (lane == 0) sred[wv][jj] = sum;
      }
      __syncthreads();
      if ((int)threadIdx.x < kBatch && jb + (int)threadIdx.x < nj) {
        float sum = 0.0f;
        for (int w = 0; w < nwaves; w++) sum += sred[w][threadIdx.x];
        const int e = se[jb + threadIdx.x];
        if (e >= 0) sdp[e] = sum;
      }
      // sred reused by the next batch; also ends this chunk's reads of the
      // slots and orders the sdp writes before the row is written out
      __syncthreads();
    }
  }
  // A streaming call stores the prob-gradient row past the caches: left
  // there (16.8 MB at 16384 tokens x 256 experts) it pushed part of d_out,
  // which the scatter launched next reads, out of the Infinity Cache (the
  // backward took 688-690 us warm and 697 cold, 664-666 and 686-689 with
  // these stores and the scatter's prob reads streamed).
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    st_row<NTM != 0>(sdp[e], d_merging_probs + (int64_t)t * E + e);
  report(dev_status, bad);
}

template <int NTM>
void mask_scale_scatter_dispatch(const void *d_out, const float *mp, const int32_t *map, int T,
                                 int64_t V, int E, int n_rows, void *d_in, int32_t *st,
                                 hipStream_t s) {
  RowShape sh = row_shape_vpt(V, 2, kRowThreads);   // as the mask permute
  if (sh.threads == 0) sh = row_shape(V, true);
  const dim3 grid = spill_grid(T, sh.ysplit), block(sh.threads);
  const v4u *gp = static_cast<const v4u *>(d_out);
  v4u *dp = static_cast<v4u *>(d_in);
#define MOE_MASK_SCATTER(VPTV)                                                                 \
  hipLaunchKernelGGL((mask_scale_scatter_kernel<VPTV, NTM>), grid, block, 0, s, gp, mp, map, T, \
                     V, E, n_rows, dp, st, prefetch_ahead(sh.threads))
  switch (sh.vpt) {
    case 1: MOE_MASK_SCATTER(1); break;
    case 2: MOE_MASK_SCATTER(2); break;
    default: MOE_MASK_SCATTER(4); break;
  }
#undef MOE_MASK_SCATTER
}

// sh: one pass over the row; more than kRowThreads lanes only with one unit
// per lane.
template <int NTM>
void mask_dot_gather_dispatch(const RowShape &sh, const void *d_out, const void *fwd_in,
                              const int32_t *map, int T, int64_t V, int E, int n_rows,
                              float *dmp, int32_t *st, hipStream_t s) {
  const dim3 grid = spill_grid(T, 1), block(sh.threads);
  const v4u *gp = static_cast<const v4u *>(d_out);
  const v4u *fp = static_cast<const v4u *>(fwd_in);
  if (sh.threads > kRowThreads) {
    hipLaunchKernelGGL((mask_dot_gather_kernel<1, NTM, 1024>), grid, block, 0, s, gp, fp, map, T,
                       V, E, n_rows, dmp, st);
    return;
  }
#define MOE_MASK_DOT(VPTV)                                                                     \
  hipLaunchKernelGGL((mask_dot_gather_kernel<VPTV, NTM, kRowThreads>), grid, block, 0, s, gp, \
                     fp, map, T, V, E, n_rows, dmp, st)
  switch (sh.vpt) {
    case 1: MOE_MASK_DOT(1); break;
    case 2: MOE_MASK_DOT(2); break;
    default: MOE_MASK_DOT(4); break;
  }
#undef MOE_MASK_DOT
}

}  // namespace

hipError_t launch_mask_permute(const void *x, const float *probs, const int32_t *map, int T,
                               int H, int E, int n_rows, void *out, float *out_probs,
                               int32_t *dev_status, bool vec, hipStream_t s) {
  const SideRows none{nullptr, nullptr, 0, 0};
  const bool stream = 2ll * H * ((int64_t)n_rows + T) > kStreamBytes;
  if (vec && stream)
    mask_permute_dispatch<v4u, MOE_MASK_PERMUTE_STREAM, false>(x, probs, map, T, H / 8, E, n_rows,
                                                               out, out_probs, none, dev_status,
                                                               s);
  else if (vec)
    mask_permute_dispatch<v4u, 0, false>(x, probs, map, T, H / 8, E, n_rows, out, out_probs,
                                         none, dev_status, s);
  else
    mask_permute_dispatch<uint16_t, 0, false>(x, probs, map, T, H, E, n_rows, out, out_probs,
                                              none, dev_status, s);
  return hipGetLastError();
}

hipError_t launch_mask_permute_rows(const void *x, int64_t row_bytes, int unit_bytes,
                                    const float *probs, const int32_t *map, int T, int E,
                                    int n_rows, void *out, float *out_probs,
                                    const SideRows &side, int32_t *dev_status, hipStream_t s) {
  const int64_t V = row_bytes / unit_bytes;
  const bool stream = row_bytes * ((int64_t)n_rows + T) > kStreamBytes;
#define MOE_MASK_ROWS(UT)                                                                      \
  if (stream)                                                                                  \
    mask_permute_dispatch<UT, MOE_MASK_PERMUTE_STREAM, true>(x, probs, map, T, V, E, n_rows,   \
                                                             out, out_probs, side, dev_status, \
                                                             s);                               \
  else                                                                                         \
    mask_permute_dispatch<UT, 0, true>(x, probs, map, T, V, E, n_rows, out, out_probs, side,   \
                                       dev_status, s);                                         \
  break
  switch (unit_bytes) {
    case 16: MOE_MASK_ROWS(v4u);
    case 4: MOE_MASK_ROWS(uint32_t);
    case 2: MOE_MASK_ROWS(uint16_t);
    default: MOE_MASK_ROWS(uint8_t);
  }
#undef MOE_MASK_ROWS
  return hipGetLastError();
}

hipError_t launch_mask_unpermute(const void *in, const float *merging_probs,
                                 const float *permuted_probs, const int32_t *map, int T, int H,
                                 int E, int n_rows, void *out, float *unpermuted_probs,
                                 int32_t *dev_status, bool vec, hipStream_t s) {
  const bool stream = 2ll * H * ((int64_t)n_rows + T) > kStreamBytes;
  if (vec && stream)
    mask_unpermute_dispatch<8, true>(in, merging_probs, permuted_probs, map, T, H / 8, E, n_rows,
                                     out, unpermuted_probs, dev_status, s);
  else if (vec)
    mask_unpermute_dispatch<8, false>(in, merging_probs, permuted_probs, map, T, H / 8, E,
                                      n_rows, out, unpermuted_probs, dev_status, s);
  else
    mask_unpermute_dispatch<1, false>(in, merging_probs, permuted_probs, map, T, H, E, n_rows,
                                      out, unpermuted_probs, dev_status, s);
  return hipGetLastError();
}

hipError_t launch_mask_unpermute_bwd(const void *d_out, const void *fwd_in,
                                     const float *merging_probs, const int32_t *map, int T,
                                     int H, int E, int n_rows, void *d_in,
                                     float *d_merging_probs, int32_t *dev_status, bool vec,
                                     hipStream_t s) {
  const bool stream =
      2ll * H * ((int64_t)n_rows * (d_merging_probs ? 2 : 1) + T) > kStreamBytes;
  if (vec) {
    // As the top-k backward: the activation gradient alone is the scaled
    // scatter (16384 x 7168 top-8: 363 us warm and 392 cold against 446 and
    // 448 fused; 4096 x 2048 top-6: 19.9 / 22.6 against 20.3 / 25.4); a
    // streaming call with prob gradients is the dot products, then the
    // scatter.
    const int64_t V = H / 8;
    const bool stream_rows = 2ll * H * ((int64_t)n_rows + T) > kStreamBytes;
    if (d_merging_probs == nullptr) {
      if (stream_rows)
        mask_scale_scatter_dispatch<MOE_MASK_PERMUTE_STREAM>(d_out, merging_probs, map, T, V, E,
                                                             n_rows, d_in, dev_status, s);
      else
        mask_scale_scatter_dispatch<0>(d_out, merging_probs, map, T, V, E, n_rows, d_in,
                                       dev_status, s);
      return hipGetLastError();
    }
    if (MOE_BWD_SPLIT && stream && d_merging_probs != nullptr) {
      RowShape ds = row_shape_vpt(V, 1, 1024);
      if (ds.threads == 0) ds = gather_shape(V);
      if (ds.ysplit == 1) {
        mask_dot_gather_dispatch<1>(ds, d_out, fwd_in, map, T, V, E, n_rows, d_merging_probs,
                                    dev_status, s);
        mask_scale_scatter_dispatch<MOE_MASK_PERMUTE_STREAM>(d_out, merging_probs, map, T, V, E,
                                                             n_rows, d_in, dev_status, s);
        return hipGetLastError();
      }
    }
  }
  if (vec && stream)
    mask_unpermute_bwd_dispatch<8, true>(d_out, fwd_in, merging_probs, map, T, H / 8, E, n_rows,
                                         d_in, d_merging_probs, dev_status, s);
  else if (vec)
    mask_unpermute_bwd_dispatch<8, false>(d_out, fwd_in, merging_probs, map, T, H / 8, E,
                                          n_rows, d_in, d_merging_probs, dev_status, s);
  else
    mask_unpermute_bwd_dispatch<1, false>(d_out, fwd_in, merging_probs, map, T, H, E, n_rows,
                                          d_in, d_merging_probs, dev_status, s);
  return hipGetLastError();
}

}  // namespace moe
