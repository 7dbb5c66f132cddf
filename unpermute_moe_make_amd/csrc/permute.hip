// Token-row kernels: permute (row scatter-copy), the fixed-order combine
// (unpermute, and permute backward), and the unpermute backward.
//
// gfx950 design.  One workgroup owns one token (and, for very long rows, a
// slice of it: grid.y).  The first `k` lanes resolve the token's k
// destination rows r_j = row_id_map[topk_idx[t][j]][t] (and its k weights)
// into LDS, lane j with two dependent loads; meanwhile every lane has
// already issued its loads of the token's own row where the kernel needs it.
// Each lane then moves VPT 16-byte vectors per row, all loads of a lane in
// flight before its first store (a combine wave keeps VPT * k KiB of
// gathers outstanding).  Row offsets are
// 64-bit.  There is no LDS tiling of the rows themselves: each byte is read
// once and written once, and HBM bandwidth is the bound.
//
// Numerics of the combine (Megatron-core batch_invariant,
// unpermute_with_bf16_rank_partials): per element acc = +0, then
// acc = fmaf(p_j, x_j, acc) for j = 0..k-1 in slot order, then one
// round-to-nearest-even to bf16.  The chain is per element, so the result
// does not depend on the launch shape.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "rows.h"

namespace moe {
namespace {

constexpr int kMaxTopk = MOE_MAX_TOPK;
// Streaming policy of calls larger than kStreamBytes, per kernel (bit 0:
// non-temporal loads, bit 1: non-temporal stores); build-time tuning.
#ifndef MOE_PERMUTE_STREAM
#define MOE_PERMUTE_STREAM 2
#endif
#ifndef MOE_COMBINE_STREAM
#define MOE_COMBINE_STREAM 3
#endif
#ifndef MOE_COMBINE_BWD_STREAM
#define MOE_COMBINE_BWD_STREAM 3
#endif
// Units per lane of the permute when a row fits one pass; build-time tuning.
#ifndef MOE_PERMUTE_VPT
#define MOE_PERMUTE_VPT 2
#endif
// Largest workgroup of the unpermute backward's one-unit-per-lane shape.
constexpr int kBwdThreads = 1024;

// Resolve the token's slots into LDS.  Returns status bits of this lane.
__device__ __forceinline__ int resolve_slots(const int32_t *__restrict__ topk_idx,
                                             const int32_t *__restrict__ row_id_map, int t,
                                             int T, int k, int E, int n_rows,
                                             int64_t *__restrict__ srow) {
  int bad = 0;
  const int j = threadIdx.x;
  if (j < k) {
    const int e = topk_idx[(int64_t)t * k + j];
    int64_t r = -1;
    if ((unsigned)e >= (unsigned)E) {
      bad |= MOE_DEV_BAD_EXPERT;
    } else {
      const int rr = row_id_map[(int64_t)e * T + t];
      if ((unsigned)rr >= (unsigned)n_rows)
        bad |= MOE_DEV_BAD_ROW;
      else
        r = rr;
    }
    srow[j] = r;
  }
  return bad;
}

// ---------------------------------------------------------------- permute --

// SIDE: also move each token's side row (quantization scales) to the same
// destinations.
template <typename U, int VPT, int NTM, bool SIDE>
__global__ __launch_bounds__(kRowThreads) void permute_kernel(
    const U *__restrict__ x, const float *__restrict__ probs,
    const int32_t *__restrict__ topk_idx, const int32_t *__restrict__ row_id_map, int T,
    int64_t V, int k, int E, int n_rows, U *__restrict__ out, float *__restrict__ out_probs,
    SideRows side, int32_t *__restrict__ dev_status, int ahead) {
  __shared__ int64_t srow[kMaxTopk];
  const int64_t tb = spill_block();
  if (tb >= T) return;  // a workgroup past the last token
  const int t = (int)tb;
  const int64_t c0 = (int64_t)blockIdx.y * blockDim.x * VPT + threadIdx.x;

  // The token's own row: issue the loads before resolving the slots.
  U v[VPT];
  const U *xr = x + (int64_t)t * V;
#pragma unroll
  for (int i = 0; i < VPT; i++) {
    const int64_t c = c0 + (int64_t)i * blockDim.x;
    if (c < V) v[i] = ld_row<(NTM & 1) != 0>(xr + c);
  }
  SideCache sc{};
  if (SIDE && blockIdx.y == 0) sc = load_side_row(side, t);
  const int bad = resolve_slots(topk_idx, row_id_map, t, T, k, E, n_rows, srow);
  if (blockIdx.y == 0 && threadIdx.x < k) {
    report(dev_status, bad);
    const int64_t r = srow[threadIdx.x];
    if (r >= 0 && out_probs != nullptr) out_probs[r] = probs[(int64_t)t * k + threadIdx.x];
  }
  __syncthreads();

  for (int j = 0; j < k; j++) {
    const int64_t r = srow[j];
    if (r < 0) continue;
    U *orow = out + r * V;
#pragma unroll
    for (int i = 0; i < VPT; i++) {
      const int64_t c = c0 + (int64_t)i * blockDim.x;
      if (c < V) st_row<(NTM & 2) != 0>(v[i], orow + c);
    }
    if (SIDE && blockIdx.y == 0) store_side_row(side, sc, t, r);
  }
  // A streaming call then prefetches this slice of a later token's row.
  // Issued after the stores: before a loop of stores alone the compiler
  // waits for every load in flight (gfx9 counts stores and loads on one
  // counter), so an earlier prefetch held up this token's stores (cold
  // 16384 x 7168 permute: 398 us with the prefetch before the stores, 385
  // after them, 420 without).  Not with side rows: on the FP8 permute of
  // that size (4-wave workgroups) it made the cold call slower at every
  // distance, 201-211 us from 1024 to 8192 tokens ahead against 195
  // (issued before the stores: 213 against 197).
  if constexpr (NTM != 0 && !SIDE) {
    const int64_t s0 = (int64_t)blockIdx.y * blockDim.x * VPT;
    keep_loaded(prefetch_lines<U, VPT>(
        (int64_t)t + ahead < T ? x + (int64_t)(t + ahead) * V : nullptr, s0,
        min(V, s0 + (int64_t)blockDim.x * VPT), xr + s0));
  }
}

// ---------------------------------------------------------------- combine --

// out[t] = bf16(fma chain over slots of p_j * in[r_j]); probs == NULL -> 1.
// KB = slots loaded per batch (all of them when k <= 8).  Optionally gathers
// gather_dst[t][j] = gather_src[r_j] (permute backward of the probs).
template <int EPV, int VPT, int KB, int NTM>
__global__ __launch_bounds__(kRowThreads) void combine_kernel(
    const typename Bf16Unit<EPV>::T *__restrict__ in, const float *__restrict__ probs,
    const int32_t *__restrict__ topk_idx, const int32_t *__restrict__ row_id_map, int T,
    int64_t V, int k, int E, int n_rows, typename Bf16Unit<EPV>::T *__restrict__ out,
    const float *__restrict__ gather_src, float *__restrict__ gather_dst,
    int32_t *__restrict__ dev_status) {
  using Unit = Bf16Unit<EPV>;
  using U = typename Unit::T;
  __shared__ int64_t srow[kMaxTopk];
  __shared__ float sp[kMaxTopk];
  const int64_t tb = spill_block();
  if (tb >= T) return;  // a workgroup past the last token
  const int t = (int)tb;
  const int64_t c0 = (int64_t)blockIdx.y * blockDim.x * VPT + threadIdx.x;

  const int bad = resolve_slots(topk_idx, row_id_map, t, T, k, E, n_rows, srow);
  if (threadIdx.x < k) {
    sp[threadIdx.x] = probs != nullptr ? probs[(int64_t)t * k + threadIdx.x] : 1.0f;
    if (blockIdx.y == 0) {
      report(dev_status, bad);
      if (gather_dst != nullptr) {
        const int64_t r = srow[threadIdx.x];
        gather_dst[(int64_t)t * k + threadIdx.x] = r >= 0 ? gather_src[r] : 0.0f;
      }
    }
  }
  __syncthreads();

  float acc[VPT][EPV];
#pragma unroll
  for (int i = 0; i < VPT; i++)
#pragma unroll
    for (int e = 0; e < EPV; e++) acc[i][e] = 0.0f;

  for (int j0 = 0; j0 < k; j0 += KB) {
    U vals[KB][VPT];
    // All loads of the batch first.
#pragma unroll
    for (int jj = 0; jj < KB; jj++) {
      const int j = j0 + jj;
      const int64_t r = (j < k) ? srow[j] : -1;
#pragma unroll
      for (int i = 0; i < VPT; i++) {
        const int64_t c = c0 + (int64_t)i * blockDim.x;
        vals[jj][i] = (r >= 0 && c < V) ? ld_row<(NTM & 1) != 0>(in + r * V + c) : Unit::zero();
      }
    }
    // Then the fused multiply-adds, strictly in slot order.
#pragma unroll
    for (int jj = 0; jj < KB; jj++) {
      const int j = j0 + jj;
      if (j < k) {
        const float p = sp[j];
#pragma unroll
        for (int i = 0; i < VPT; i++) {
          float f[EPV];
          Unit::unpack(vals[jj][i], f);
#pragma unroll
          for (int e = 0; e < EPV; e++) acc[i][e] = __builtin_fmaf(p, f[e], acc[i][e]);
        }
      }
    }
  }

  U *orow = out + (int64_t)t * V;
#pragma unroll
  for (int i = 0; i < VPT; i++) {
    const int64_t c = c0 + (int64_t)i * blockDim.x;
    if (c < V) st_row<(NTM & 2) != 0>(Unit::pack(acc[i]), orow + c);
  }
}

// ------------------------------------------------ EP rank-ordered combine --

// Megatron-core batch_invariant unpermute with experts split into EP ranks
// (rank(e) = e / per_rank): per rank, the fp32 fmaf chain of its slots in
// slot order from zero (optionally rounded to bf16); the partials are added
// in rank order from zero (fp32, or fp64 when FP64), then rounded to bf16.
// Ranks without slots contribute +0, which cannot change a sum that started
// from +0, so only the ranks present in the token are visited.  The slots
// are ordered by (rank, slot) once per token in LDS, each slot computing its
// own place in parallel and whether it is the last slot of its rank.  That
// order is the same for every lane of the token, so the walk over it
// branches on scalars: the partial is rounded and added to the total only at
// the last slot of each rank.  (Evaluated at every slot and kept by a
// select, as the compiler did with a per-lane branch, the rounding, the fp64
// conversion and add ran k times per element: 387 us against 381 warm on
// the 16384 x 7168 top-8 combine with 8 ranks in fp64.)
template <int EPV, int VPT, bool NT, bool FP64, bool BF16P>
__global__ __launch_bounds__(kRowThreads) void combine_ep_kernel(
    const typename Bf16Unit<EPV>::T *__restrict__ in, const float *__restrict__ probs,
    const int32_t *__restrict__ topk_idx, const int32_t *__restrict__ row_id_map, int T,
    int64_t V, int k, int E, int n_rows, int per_rank,
    typename Bf16Unit<EPV>::T *__restrict__ out, int32_t *__restrict__ dev_status) {
  using Unit = Bf16Unit<EPV>;
  using U = typename Unit::T;
  using Acc = typename std::conditional<FP64, double, float>::type;
  // Slots loaded per batch.  Measured on the 16384 x 7168 top-8 combine with
  // 8 ranks: batches of 4 give 347 us warm and cold in both cross-rank
  // precisions, against 379 / 385 (fp64) and 355 / 359 (fp32) with all 8
  // slots in flight (batches of 2 alike).  The plain combine is the other
  // way round (all slots at once, 354 against 372 in batches of 4).
  constexpr int KB = 4;
  __shared__ int64_t srow[kMaxTopk];
  __shared__ float sp[kMaxTopk];
  __shared__ int srank[kMaxTopk];
  __shared__ int sorder[kMaxTopk];
  __shared__ int slast[kMaxTopk];
  const int64_t tb = spill_block();
  if (tb >= T) return;  // a workgroup past the last token
  const int t = (int)tb;
  const int64_t c0 = (int64_t)blockIdx.y * blockDim.x * VPT + threadIdx.x;

  const int bad = resolve_slots(topk_idx, row_id_map, t, T, k, E, n_rows, srow);
  if (threadIdx.x < k) {
    const int j = threadIdx.x;
    sp[j] = probs != nullptr ? probs[(int64_t)t * k + j] : 1.0f;
    const int e = topk_idx[(int64_t)t * k + j];
    srank[j] = ((unsigned)e < (unsigned)E) ? e / per_rank : 0;
    if (blockIdx.y == 0) report(dev_status, bad);
  }
  __syncthreads();
  if (threadIdx.x < k) {
    // slot j's place in (rank, slot) order is the number of slots before it;
    // it ends its rank when no later slot has the same rank
    const int j = threadIdx.x;
    const int rj = srank[j];
    int pos = 0;
    bool last = true;
    for (int i = 0; i < k; i++) {
      const int ri = srank[i];
      pos += (ri < rj || (ri == rj && i < j)) ? 1 : 0;
      if (ri == rj && i > j) last = false;
    }
    sorder[pos] = j;
    slast[pos] = last ? 1 : 0;
  }
  __syncthreads();

  Acc total[VPT][EPV];
  float acc[VPT][EPV];
#pragma unroll
  for (int i = 0; i < VPT; i++)
#pragma unroll
    for (int e = 0; e < EPV; e++) {
      total[i][e] = (Acc)0;
      acc[i][e] = 0.0f;
    }
  for (int s0 = 0; s0 < k; s0 += KB) {
    U vals[KB][VPT];
#pragma unroll
    for (int ss = 0; ss < KB; ss++) {
      const int s = s0 + ss;
      const int64_t r = (s < k) ? srow[sorder[s]] : -1;
#pragma unroll
      for (int i = 0; i < VPT; i++) {
        const int64_t c = c0 + (int64_t)i * blockDim.x;
        vals[ss][i] = (r >= 0 && c < V) ? ld_row<NT>(in + r * V + c) : Unit::zero();
      }
    }
#pragma unroll
    for (int ss = 0; ss < KB; ss++) {
      const int s = s0 + ss;
      if (s >= k) break;
      const int j = __builtin_amdgcn_readfirstlane(sorder[s]);
      const float p = sp[j];
#pragma unroll
      for (int i = 0; i < VPT; i++) {
        float f[EPV];
        Unit::unpack(vals[ss][i], f);
#pragma unroll
        for (int e = 0; e < EPV; e++) acc[i][e] = __builtin_fmaf(p, f[e], acc[i][e]);
      }
      if (__builtin_amdgcn_readfirstlane(slast[s]) != 0) {
#pragma unroll
        for (int i = 0; i < VPT; i++)
#pragma unroll
          for (int e = 0; e < EPV; e++) {
            const float part = BF16P ? round_to_bf16(acc[i][e]) : acc[i][e];
            total[i][e] = total[i][e] + (Acc)part;
            acc[i][e] = 0.0f;
          }
      }
    }
  }
  U *orow = out + (int64_t)t * V;
#pragma unroll
  for (int i = 0; i < VPT; i++) {
    float res[EPV];
#pragma unroll
    for (int e = 0; e < EPV; e++) {
      if constexpr (FP64)
        res[e] = f64_to_f32_odd(total[i][e]);   // the pack below rounds it to bf16
      else
        res[e] = total[i][e];
    }
    const int64_t c = c0 + (int64_t)i * blockDim.x;
    if (c < V) st_row<NT>(Unit::pack(res), orow + c);
  }
}

// ----------------------------------------------------- unpermute backward --

// d_in[r_j] = bf16(fp32(d_out[t]) * p_j); d_probs[t][j] = <fwd_in[r_j], d_out[t]>.
// A workgroup walks its row slice in passes of blockDim*VPT units.  When
// d_probs is written the grid must not split rows (gridDim.y == 1), so the
// workgroup sees the whole row and reduces each slot's dot product itself.
template <int EPV, int VPT, int KB, int NTM, int MAXT>
__global__ __launch_bounds__(MAXT) void combine_bwd_kernel(
    const typename Bf16Unit<EPV>::T *__restrict__ d_out,
    const typename Bf16Unit<EPV>::T *__restrict__ fwd_in, const float *__restrict__ probs,
    const int32_t *__restrict__ topk_idx, const int32_t *__restrict__ row_id_map, int T,
    int64_t V, int k, int E, int n_rows, typename Bf16Unit<EPV>::T *__restrict__ d_in,
    float *__restrict__ d_probs, int32_t *__restrict__ dev_status) {
  using Unit = Bf16Unit<EPV>;
  using U = typename Unit::T;
  __shared__ int64_t srow[kMaxTopk];
  __shared__ float sp[kMaxTopk];
  __shared__ float sred[MAXT / kWave][KB];
  const int64_t tb = spill_block();
  if (tb >= T) return;  // a workgroup past the last token
  const int t = (int)tb;
  const int64_t pass = (int64_t)blockDim.x * VPT;
  const int64_t stride = pass * gridDim.y;
  const int64_t cfirst = (int64_t)blockIdx.y * pass + threadIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  const U *grow = d_out + (int64_t)t * V;

  // First pass of the token's upstream gradient, issued before the slots.
  U graw[VPT];
#pragma unroll
  for (int i = 0; i < VPT; i++) {
    const int64_t c = cfirst + (int64_t)i * blockDim.x;
    graw[i] = c < V ? ld_row<(NTM & 1) != 0>(grow + c) : Unit::zero();
  }
  const int bad = resolve_slots(topk_idx, row_id_map, t, T, k, E, n_rows, srow);
  if (threadIdx.x < k) {
    sp[threadIdx.x] = probs[(int64_t)t * k + threadIdx.x];
    if (blockIdx.y == 0) report(dev_status, bad);
  }
  __syncthreads();

  const bool want_dot = d_probs != nullptr;
  for (int j0 = 0; j0 < k; j0 += KB) {
    float part[KB];
#pragma unroll
    for (int jj = 0; jj < KB; jj++) part[jj] = 0.0f;

    for (int64_t cb = cfirst; cb < V; cb += stride) {
      if (!(j0 == 0 && cb == cfirst)) {
#pragma unroll
        for (int i = 0; i < VPT; i++) {
          const int64_t c = cb + (int64_t)i * blockDim.x;
          graw[i] = c < V ? ld_row<(NTM & 1) != 0>(grow + c) : Unit::zero();
        }
      }
      U fin[KB][VPT];
      if (want_dot) {
#pragma unroll
        for (int jj = 0; jj < KB; jj++) {
          const int j = j0 + jj;
          const int64_t r = (j < k) ? srow[j] : -1;
#pragma unroll
          for (int i = 0; i < VPT; i++) {
            const int64_t c = cb + (int64_t)i * blockDim.x;
            fin[jj][i] = (r >= 0 && c < V) ? ld_row<(NTM & 1) != 0>(fwd_in + r * V + c)
                                           : Unit::zero();
          }
        }
      }
      float g[VPT][EPV];
#pragma unroll
      for (int i = 0; i < VPT; i++) Unit::unpack(graw[i], g[i]);
#pragma unroll
      for (int jj = 0; jj < KB; jj++) {
        const int j = j0 + jj;
        if (j >= k) continue;
        const int64_t r = srow[j];
        const float p = sp[j];
#pragma unroll
        for (int i = 0; i < VPT; i++) {
          const int64_t c = cb + (int64_t)i * blockDim.x;
          float prod[EPV];
#pragma unroll
          for (int e = 0; e < EPV; e++) prod[e] = g[i][e] * p;  // one fp32 rounding
          if (r >= 0 && c < V) st_row<(NTM & 2) != 0>(Unit::pack(prod), d_in + r * V + c);
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
      for (int jj = 0; jj < KB; jj++) {
        const float s = wave_sum(part[jj]);
        if (lane == 0) sred[wv][jj] = s;
      }
      __syncthreads();
      if ((int)threadIdx.x < KB && j0 + (int)threadIdx.x < k) {
        float s = 0.0f;
        for (int w = 0; w < nwaves; w++) s += sred[w][threadIdx.x];
        d_probs[(int64_t)t * k + j0 + threadIdx.x] = s;
      }
      if (j0 + KB < k) __syncthreads();   // sred reused by the next batch
    }
  }
}

// ------------------------------------ unpermute backward in two launches --

// When the row fits one workgroup pass, the backward of the weighted
// unpermute runs as two kernels of the library's two access patterns: a
// gather that only reads (the prob-gradient dot products), then a scatter
// that reads one row per token and writes k (the activation gradient).  Fused, one
// kernel interleaves 1.88 GB of gathers with 1.88 GB of scattered stores
// (16384 x 7168 top-8), which the memory system serves more slowly than the
// two streams one after the other.

// d_probs[t][j] = <fwd_in[r_j], d_out[t]>: each lane runs an fmaf chain over
// its units and their elements in order; the lanes of a wave are then summed
// by a fixed DPP tree, and the waves in order.  All KB slots' loads are in
// flight before the arithmetic, as in the unpermute.
template <int VPT, int KB, int NTM, int MAXT>
__global__ __launch_bounds__(MAXT) void dot_gather_kernel(
    const v4u *__restrict__ d_out, const v4u *__restrict__ fwd_in,
    const int32_t *__restrict__ topk_idx, const int32_t *__restrict__ row_id_map, int T,
    int64_t V, int k, int E, int n_rows, float *__restrict__ d_probs,
    int32_t *__restrict__ dev_status) {
  using Unit = Bf16Unit<8>;
  __shared__ int64_t srow[kMaxTopk];
  __shared__ float sred[MAXT / kWave][KB];
  const int64_t tb = spill_block();
  if (tb >= T) return;  // a workgroup past the last token
  const int t = (int)tb;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;

  // The token's upstream gradient, issued before the slots are resolved;
  // always a plain load, so the scatter launched next finds it cached.
  v4u g[VPT];
#pragma unroll
  for (int i = 0; i < VPT; i++) {
    const int64_t c = (int64_t)threadIdx.x + (int64_t)i * blockDim.x;
    g[i] = c < V ? d_out[(int64_t)t * V + c] : Unit::zero();
  }
  const int bad = resolve_slots(topk_idx, row_id_map, t, T, k, E, n_rows, srow);
  if (threadIdx.x < k) report(dev_status, bad);
  __syncthreads();

  for (int j0 = 0; j0 < k; j0 += KB) {
    v4u vals[KB][VPT];
#pragma unroll
    for (int jj = 0; jj < KB; jj++) {
      const int j = j0 + jj;
      const int64_t r = (j < k) ? srow[j] : -1;
#pragma unroll
      for (int i = 0; i < VPT; i++) {
        const int64_t c = (int64_t)threadIdx.x + (int64_t)i * blockDim.x;
        vals[jj][i] = (r >= 0 && c < V) ? ld_row<(NTM & 1) != 0>(fwd_in + r * V + c)
                                        : Unit::zero();
      }
    }
    float part[KB];
#pragma unroll
    for (int jj = 0; jj < KB; jj++) {
      part[jj] = 0.0f;
#pragma unroll
      for (int i = 0; i < VPT; i++) {
        float f[8], gf[8];
        Unit::unpack(vals[jj][i], f);
        Unit::unpack(g[i], gf);
#pragma unroll
        for (int e = 0; e < 8; e++) part[jj] = __builtin_fmaf(f[e], gf[e], part[jj]);
      }
    }
#pragma unroll
    for (int jj = 0; jj < KB; jj++) {
      const float sum = wave_sum(part[jj]);
      if (lane == 0) sred[wv][jj] = sum;
    }
    __syncthreads();
    if ((int)threadIdx.x < KB && j0 + (int)threadIdx.x < k) {
      float sum = 0.0f;
      for (int w = 0; w < nwaves; w++) sum += sred[w][threadIdx.x];
      d_probs[(int64_t)t * k + j0 + threadIdx.x] = sum;
    }
    if (j0 + KB < k) __syncthreads();   // sred reused by the next batch
  }
}

// d_in[r_j] = bf16(fp32(d_out[t]) * p_j): the permute's shape and source
// prefetch, with one fp32 product and one rounding per element.
template <int VPT, int NTM>
__global__ __launch_bounds__(kRowThreads) void scale_scatter_kernel(
    const v4u *__restrict__ d_out, const float *__restrict__ probs,
    const int32_t *__restrict__ topk_idx, const int32_t *__restrict__ row_id_map, int T,
    int64_t V, int k, int E, int n_rows, v4u *__restrict__ d_in,
    int32_t *__restrict__ dev_status, int ahead) {
  using Unit = Bf16Unit<8>;
  __shared__ int64_t srow[kMaxTopk];
  __shared__ float sp[kMaxTopk];
  const int64_t tb = spill_block();
  if (tb >= T) return;  // a workgroup past the last token
  const int t = (int)tb;
  const int64_t s0 = (int64_t)blockIdx.y * blockDim.x * VPT;
  const v4u *grow = d_out + (int64_t)t * V;
  v4u v[VPT];
#pragma unroll
  for (int i = 0; i < VPT; i++) {
    const int64_t c = s0 + threadIdx.x + (int64_t)i * blockDim.x;
    v[i] = c < V ? ld_row<(NTM & 1) != 0>(grow + c) : Unit::zero();
  }
  const int bad = resolve_slots(topk_idx, row_id_map, t, T, k, E, n_rows, srow);
  if (threadIdx.x < k) {
    sp[threadIdx.x] = probs[(int64_t)t * k + threadIdx.x];
    if (blockIdx.y == 0) report(dev_status, bad);
  }
  __syncthreads();

  for (int j = 0; j < k; j++) {
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
  if constexpr (NTM != 0)   // as in the permute
    keep_loaded(prefetch_lines<v4u, VPT>(
        (int64_t)t + ahead < T ? d_out + (int64_t)(t + ahead) * V : nullptr, s0,
        min(V, s0 + (int64_t)blockDim.x * VPT), grow + s0));
}

template <int VPT, int NTM, int MAXT = kRowThreads>
void dot_gather_k(const RowShape &sh, int T, const void *d_out, const void *fwd_in,
                  const int32_t *topk_idx, const int32_t *row_id_map, int64_t V, int k, int E,
                  int n_rows, float *d_probs, int32_t *st, hipStream_t s) {
  const dim3 grid = spill_grid(T, 1), block(sh.threads);
  const v4u *gp = static_cast<const v4u *>(d_out);
  const v4u *fp = static_cast<const v4u *>(fwd_in);
#define MOE_DOT(KBV)                                                                           \
  hipLaunchKernelGGL((dot_gather_kernel<VPT, KBV, NTM, MAXT>), grid, block, 0, s, gp, fp,     \
                     topk_idx, row_id_map, T, V, k, E, n_rows, d_probs, st)
  switch (k) {
    case 1: MOE_DOT(1); break;
    case 2: MOE_DOT(2); break;
    case 3: MOE_DOT(3); break;
    case 4: MOE_DOT(4); break;
    case 5: MOE_DOT(5); break;
    case 6: MOE_DOT(6); break;
    case 7: MOE_DOT(7); break;
    default: MOE_DOT(8); break;
  }
#undef MOE_DOT
}

template <int NTM>
void scale_scatter_dispatch(const void *d_out, const float *probs, const int32_t *topk_idx,
                            const int32_t *row_id_map, int T, int64_t V, int k, int E,
                            int n_rows, void *d_in, int32_t *st, hipStream_t s) {
  RowShape sh = row_shape_vpt(V, MOE_PERMUTE_VPT, kRowThreads);   // as the permute
  if (sh.threads == 0) sh = row_shape(V, true);
  const dim3 grid = spill_grid(T, sh.ysplit), block(sh.threads);
  const v4u *gp = static_cast<const v4u *>(d_out);
  v4u *dp = static_cast<v4u *>(d_in);
#define MOE_SCATTER(VPTV)                                                                      \
  hipLaunchKernelGGL((scale_scatter_kernel<VPTV, NTM>), grid, block, 0, s, gp, probs, topk_idx, \
                     row_id_map, T, V, k, E, n_rows, dp, st, prefetch_ahead(sh.threads))
  switch (sh.vpt) {
    case 1: MOE_SCATTER(1); break;
    case 2: MOE_SCATTER(2); break;
    default: MOE_SCATTER(4); break;
  }
#undef MOE_SCATTER
}

// sh: one pass over the row (ysplit 1); more than kRowThreads lanes only
// with one unit per lane.
template <int NTM>
void dot_gather_dispatch(const RowShape &sh, const void *d_out, const void *fwd_in,
                         const int32_t *topk_idx, const int32_t *row_id_map, int T, int64_t V,
                         int k, int E, int n_rows, float *d_probs, int32_t *st, hipStream_t s) {
  if (sh.threads > kRowThreads) {
    dot_gather_k<1, NTM, kBwdThreads>(sh, T, d_out, fwd_in, topk_idx, row_id_map, V, k, E, n_rows,
                                      d_probs, st, s);
    return;
  }
  switch (sh.vpt) {
    case 1: dot_gather_k<1, NTM>(sh, T, d_out, fwd_in, topk_idx, row_id_map, V, k, E, n_rows, d_probs, st, s); break;
    case 2: dot_gather_k<2, NTM>(sh, T, d_out, fwd_in, topk_idx, row_id_map, V, k, E, n_rows, d_probs, st, s); break;
    default: dot_gather_k<4, NTM>(sh, T, d_out, fwd_in, topk_idx, row_id_map, V, k, E, n_rows, d_probs, st, s); break;
  }
}

template <typename U, int NTM, bool SIDE>
hipError_t permute_dispatch(const void *x, const float *probs, const int32_t *topk_idx,
                            const int32_t *row_id_map, int T, int64_t V, int k, int E,
                            int n_rows, void *out, float *out_probs, const SideRows &side,
                            int32_t *dev_status, hipStream_t s) {
  // two units per lane when a row fits one pass (measured: a 4 KiB row moves
  // faster with 128 lanes than with 256)
  RowShape sh = row_shape_vpt(V, MOE_PERMUTE_VPT, kRowThreads);
  if (sh.threads == 0) sh = row_shape(V, true);
  const dim3 grid = spill_grid(T, sh.ysplit), block(sh.threads);
  const U *xp = static_cast<const U *>(x);
  U *op = static_cast<U *>(out);
#define MOE_PERMUTE(VPTV)                                                                     \
  hipLaunchKernelGGL((permute_kernel<U, VPTV, NTM, SIDE>), grid, block, 0, s, xp, probs,       \
                     topk_idx, row_id_map, T, V, k, E, n_rows, op, out_probs, side, dev_status, \
                     prefetch_ahead(sh.threads))
  switch (sh.vpt) {
    case 1: MOE_PERMUTE(1); break;
    case 2: MOE_PERMUTE(2); break;
    default: MOE_PERMUTE(4); break;
  }
#undef MOE_PERMUTE
  return hipGetLastError();
}

template <int EPV, int VPT, int NTM>
void combine_k(const RowShape &sh, int T, const void *in, const float *probs,
               const int32_t *topk_idx, const int32_t *row_id_map, int64_t V, int k, int E,
               int n_rows, void *out, const float *gsrc, float *gdst, int32_t *st,
               hipStream_t s) {
  using U = typename Bf16Unit<EPV>::T;
  const dim3 grid = spill_grid(T, sh.ysplit), block(sh.threads);
  const U *ip = static_cast<const U *>(in);
  U *op = static_cast<U *>(out);
#define MOE_COMBINE(KBV)                                                                     \
  hipLaunchKernelGGL((combine_kernel<EPV, VPT, KBV, NTM>), grid, block, 0, s, ip, probs, topk_idx, \
                     row_id_map, T, V, k, E, n_rows, op, gsrc, gdst, st)
  switch (k) {
    case 1: MOE_COMBINE(1); break;
    case 2: MOE_COMBINE(2); break;
    case 3: MOE_COMBINE(3); break;
    case 4: MOE_COMBINE(4); break;
    case 5: MOE_COMBINE(5); break;
    case 6: MOE_COMBINE(6); break;
    case 7: MOE_COMBINE(7); break;
    default: MOE_COMBINE(8); break;
  }
#undef MOE_COMBINE
}

template <int EPV, int VPT, int NTM, int MAXT = kRowThreads>
void combine_bwd_k(const RowShape &sh, int T, const void *d_out, const void *fwd_in,
                   const float *probs, const int32_t *topk_idx, const int32_t *row_id_map,
                   int64_t V, int k, int E, int n_rows, void *d_in, float *d_probs, int32_t *st,
                   hipStream_t s) {
  using U = typename Bf16Unit<EPV>::T;
  const dim3 grid = spill_grid(T, sh.ysplit), block(sh.threads);
  const U *gp = static_cast<const U *>(d_out);
  const U *fp = static_cast<const U *>(fwd_in);
  U *dp = static_cast<U *>(d_in);
#define MOE_COMBINE_BWD(KBV)                                                                  \
  hipLaunchKernelGGL((combine_bwd_kernel<EPV, VPT, KBV, NTM, MAXT>), grid, block, 0, s, gp, fp, \
                     probs, topk_idx, row_id_map, T, V, k, E, n_rows, dp, d_probs, st)
  switch (k) {
    case 1: MOE_COMBINE_BWD(1); break;
    case 2: MOE_COMBINE_BWD(2); break;
    case 3: MOE_COMBINE_BWD(3); break;
    case 4: MOE_COMBINE_BWD(4); break;
    case 5: MOE_COMBINE_BWD(5); break;
    case 6: MOE_COMBINE_BWD(6); break;
    case 7: MOE_COMBINE_BWD(7); break;
    default: MOE_COMBINE_BWD(8); break;
  }
#undef MOE_COMBINE_BWD
}

template <int EPV, int NTM>
void combine_dispatch(const void *in, const float *probs, const int32_t *topk_idx,
                      const int32_t *row_id_map, int T, int64_t V, int k, int E, int n_rows,
                      void *out, const float *gsrc, float *gdst, int32_t *st, hipStream_t s) {
  // two units per lane when a row fits one pass, as in the permute (measured:
  // the 4 KiB-row unpermute and permute backward 2% faster than 256 x 1)
  const RowShape sh = gather_shape(V);
  switch (sh.vpt) {
    case 1: combine_k<EPV, 1, NTM>(sh, T, in, probs, topk_idx, row_id_map, V, k, E, n_rows, out, gsrc, gdst, st, s); break;
    case 2: combine_k<EPV, 2, NTM>(sh, T, in, probs, topk_idx, row_id_map, V, k, E, n_rows, out, gsrc, gdst, st, s); break;
    default: combine_k<EPV, 4, NTM>(sh, T, in, probs, topk_idx, row_id_map, V, k, E, n_rows, out, gsrc, gdst, st, s); break;
  }
}

template <int EPV, int NTM>
void combine_bwd_dispatch(const void *d_out, const void *fwd_in, const float *probs,
                          const int32_t *topk_idx, const int32_t *row_id_map, int T, int64_t V,
                          int k, int E, int n_rows, void *d_in, float *d_probs, int32_t *st,
                          hipStream_t s) {
  // One unit per lane and up to kBwdThreads lanes when the row fits (measured:
  // the 7168-wide rows run 3% faster as 896 lanes than as 448 x 2).
  const RowShape wide = row_shape_vpt(V, 1, kBwdThreads);
  if (wide.threads > kRowThreads) {
    combine_bwd_k<EPV, 1, NTM, kBwdThreads>(wide, T, d_out, fwd_in, probs, topk_idx, row_id_map,
                                            V, k, E, n_rows, d_in, d_probs, st, s);
    return;
  }
  // The prob-grad reduction needs the whole row in one workgroup; rows
  // longer than one pass are then walked in several passes.
  const RowShape sh = row_shape(V, d_probs == nullptr);
  switch (sh.vpt) {
    case 1: combine_bwd_k<EPV, 1, NTM>(sh, T, d_out, fwd_in, probs, topk_idx, row_id_map, V, k, E, n_rows, d_in, d_probs, st, s); break;
    case 2: combine_bwd_k<EPV, 2, NTM>(sh, T, d_out, fwd_in, probs, topk_idx, row_id_map, V, k, E, n_rows, d_in, d_probs, st, s); break;
    default: combine_bwd_k<EPV, 4, NTM>(sh, T, d_out, fwd_in, probs, topk_idx, row_id_map, V, k, E, n_rows, d_in, d_probs, st, s); break;
  }
}

template <int EPV, bool NT, bool FP64, bool BF16P>
void combine_ep_dispatch(const void *in, const float *probs, const int32_t *topk_idx,
                         const int32_t *row_id_map, int T, int64_t V, int k, int E, int n_rows,
                         int per_rank, void *out, int32_t *st, hipStream_t s) {
  using U = typename Bf16Unit<EPV>::T;
  const U *ip = static_cast<const U *>(in);
  U *op = static_cast<U *>(out);
  // (one unit per lane on up to 1024 lanes, and two units per lane on 128
  // lanes for 4 KiB rows, were measured slower here)
  const RowShape sh = row_shape(V, true);
  const dim3 grid = spill_grid(T, sh.ysplit), block(sh.threads);
#define MOE_EP(VPTV)                                                                          \
  hipLaunchKernelGGL((combine_ep_kernel<EPV, VPTV, NT, FP64, BF16P>), grid, block, 0, s,      \
                     ip, probs, topk_idx, row_id_map, T, V, k, E, n_rows, per_rank, op, st)
  switch (sh.vpt) {
    case 1: MOE_EP(1); break;
    case 2: MOE_EP(2); break;
    default: MOE_EP(4); break;
  }
#undef MOE_EP
}

}  // namespace

hipError_t launch_permute(const void *x, const float *probs, const int32_t *topk_idx,
                          const int32_t *row_id_map, int T, int H, int k, int E, int n_rows,
                          void *out, float *out_probs, int32_t *dev_status, bool vec,
                          hipStream_t s) {
  const SideRows none{nullptr, nullptr, 0, 0};
  const int64_t bytes = 2ll * H * ((int64_t)n_rows + T);
  if (vec && bytes > kStreamBytes)
    return permute_dispatch<v4u, MOE_PERMUTE_STREAM, false>(x, probs, topk_idx, row_id_map, T,
                                                            H / 8, k, E, n_rows, out, out_probs,
                                                            none, dev_status, s);
  if (vec)
    return permute_dispatch<v4u, 0, false>(x, probs, topk_idx, row_id_map, T, H / 8, k, E,
                                           n_rows, out, out_probs, none, dev_status, s);
  return permute_dispatch<uint16_t, 0, false>(x, probs, topk_idx, row_id_map, T, H, k, E,
                                              n_rows, out, out_probs, none, dev_status, s);
}

hipError_t launch_permute_rows(const void *x, int64_t row_bytes, int unit_bytes,
                               const float *probs, const int32_t *topk_idx,
                               const int32_t *row_id_map, int T, int k, int E, int n_rows,
                               void *out, float *out_probs, const SideRows &side,
                               int32_t *dev_status, hipStream_t s) {
  const int64_t V = row_bytes / unit_bytes;
  const bool stream = row_bytes * ((int64_t)n_rows + T) > kStreamBytes;
#define MOE_PERMUTE_ROWS(UT)                                                                  \
  return stream ? permute_dispatch<UT, MOE_PERMUTE_STREAM, true>(                             \
                      x, probs, topk_idx, row_id_map, T, V, k, E, n_rows, out, out_probs,     \
                      side, dev_status, s)                                                    \
                : permute_dispatch<UT, 0, true>(x, probs, topk_idx, row_id_map, T, V, k, E,   \
                                                n_rows, out, out_probs, side, dev_status, s)
  switch (unit_bytes) {
    case 16: MOE_PERMUTE_ROWS(v4u);
    case 4: MOE_PERMUTE_ROWS(uint32_t);
    case 2: MOE_PERMUTE_ROWS(uint16_t);
    default: MOE_PERMUTE_ROWS(uint8_t);
  }
#undef MOE_PERMUTE_ROWS
}

hipError_t launch_combine(const void *in, const float *probs, const int32_t *topk_idx,
                          const int32_t *row_id_map, int T, int H, int k, int E, int n_rows,
                          void *out, const float *gather_src, float *gather_dst,
                          int32_t *dev_status, bool vec, hipStream_t s) {
  // Gathered rows in, dense rows out: both stream when the call is large.
  const int64_t bytes = 2ll * H * ((int64_t)n_rows + T);
  if (vec && bytes > kStreamBytes)
    combine_dispatch<8, MOE_COMBINE_STREAM>(in, probs, topk_idx, row_id_map, T, H / 8, k, E, n_rows, out,
                              gather_src, gather_dst, dev_status, s);
  else if (vec)
    combine_dispatch<8, 0>(in, probs, topk_idx, row_id_map, T, H / 8, k, E, n_rows, out,
                               gather_src, gather_dst, dev_status, s);
  else
    combine_dispatch<1, 0>(in, probs, topk_idx, row_id_map, T, H, k, E, n_rows, out,
                               gather_src, gather_dst, dev_status, s);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const void *d_out, const void *fwd_in, const float *probs,
                              const int32_t *topk_idx, const int32_t *row_id_map, int T, int H,
                              int k, int E, int n_rows, void *d_in, float *d_probs,
                              int32_t *dev_status, bool vec, hipStream_t s) {
  const int64_t bytes = 2ll * H * ((int64_t)n_rows * (d_probs ? 2 : 1) + T);
  if (vec) {
    const int64_t V = H / 8;
    const bool stream_rows = 2ll * H * ((int64_t)n_rows + T) > kStreamBytes;
    if (d_probs == nullptr) {
      // The activation gradient alone is the scaled scatter (16384 x 7168
      // top-8: 344 us warm and 385 cold, against 447 and 411 for the fused
      // kernel without its dot products; 4096 x 2048 top-6: 19.9 / 21.5
      // against 20.6 / 25.7).
      if (stream_rows)
        scale_scatter_dispatch<MOE_PERMUTE_STREAM>(d_out, probs, topk_idx, row_id_map, T, V, k, E,
                                                   n_rows, d_in, dev_status, s);
      else
        scale_scatter_dispatch<0>(d_out, probs, topk_idx, row_id_map, T, V, k, E, n_rows, d_in,
                                  dev_status, s);
      return hipGetLastError();
    }
    // Streaming calls run as the dot products (one unit per lane on up to
    // 1024 lanes, d_out read with plain loads and the forward rows streamed),
    // then the scatter, which finds d_out in the Infinity Cache: 636-639 us
    // warm and 654-657 cold at 16384 x 7168 top-8, against 722 and 707
    // fused.  Scatter first: 684-688 / 677 (635-639 / 676 with the dot
    // kernel's plain d_out loads); two or four units per lane in the dot
    // kernel were slower.  Smaller calls keep the fused kernel: 35.3 us
    // against 39.3 split at 4096 x 2048 top-6, where the second launch and
    // the second read of d_out cost more.
    if (MOE_BWD_SPLIT && bytes > kStreamBytes) {
      RowShape ds = row_shape_vpt(V, 1, kBwdThreads);
      if (ds.threads == 0) ds = gather_shape(V);
      if (ds.ysplit == 1) {
        dot_gather_dispatch<MOE_COMBINE_STREAM>(ds, d_out, fwd_in, topk_idx, row_id_map, T, V, k,
                                                E, n_rows, d_probs, dev_status, s);
        scale_scatter_dispatch<MOE_PERMUTE_STREAM>(d_out, probs, topk_idx, row_id_map, T, V, k, E,
                                                   n_rows, d_in, dev_status, s);
        return hipGetLastError();
      }
    }
  }
  if (vec && bytes > kStreamBytes)
    combine_bwd_dispatch<8, MOE_COMBINE_BWD_STREAM>(d_out, fwd_in, probs, topk_idx, row_id_map,
                                                    T, H / 8, k, E, n_rows, d_in, d_probs,
                                                    dev_status, s);
  else if (vec)
    combine_bwd_dispatch<8, 0>(d_out, fwd_in, probs, topk_idx, row_id_map, T, H / 8, k, E,
                               n_rows, d_in, d_probs, dev_status, s);
  else
    combine_bwd_dispatch<1, 0>(d_out, fwd_in, probs, topk_idx, row_id_map, T, H, k, E, n_rows,
                               d_in, d_probs, dev_status, s);
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

hipError_t launch_combine_ep(const void *in, const float *probs, const int32_t *topk_idx,
                             const int32_t *row_id_map, int T, int H, int k, int E, int n_rows,
                             int ep_size, bool bf16_partials, bool fp64_cross, void *out,
                             int32_t *dev_status, bool vec, hipStream_t s) {
  const int per_rank = E / ep_size;
  const bool stream = 2ll * H * ((int64_t)n_rows + T) > kStreamBytes;
  const int64_t V = vec ? H / 8 : H;
#define MOE_EP_ARGS in, probs, topk_idx, row_id_map, T, V, k, E, n_rows, per_rank, out, dev_status, s
#define MOE_EP_VEC(FP64, BP)                                                                   \
  (stream ? combine_ep_dispatch<8, true, FP64, BP>(MOE_EP_ARGS)                               \
          : combine_ep_dispatch<8, false, FP64, BP>(MOE_EP_ARGS))
  if (vec) {
    if (fp64_cross)
      bf16_partials ? MOE_EP_VEC(true, true) : MOE_EP_VEC(true, false);
    else
      bf16_partials ? MOE_EP_VEC(false, true) : MOE_EP_VEC(false, false);
  } else {
    if (fp64_cross)
      bf16_partials ? combine_ep_dispatch<1, false, true, true>(MOE_EP_ARGS)
                    : combine_ep_dispatch<1, false, true, false>(MOE_EP_ARGS);
    else
      bf16_partials ? combine_ep_dispatch<1, false, false, true>(MOE_EP_ARGS)
                    : combine_ep_dispatch<1, false, false, false>(MOE_EP_ARGS);
  }
#undef MOE_EP_VEC
#undef MOE_EP_ARGS
  return hipGetLastError();
}

}  // namespace moe
