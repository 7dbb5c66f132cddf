// Fused chunk sort-and-pad and unpad-and-restore: one map kernel and two
// copy kernels (TransformerEngine PR "Fuse MoE chunk sorting and padding",
// Description, Changes and Diagram).
//
// Map.  Every map workgroup rebuilds the small chunk tables in LDS from the
// device-resident split sizes and chunk order (a few hundred integers) and
// then writes its own slice of the padded destination -> source row map by
// binary search, so the map costs one launch with no host round trip and no
// serial pass over the rows.  Every workgroup validates the metadata the
// same way; on bad metadata the whole map is -1 (so the copies write zeros)
// and workgroup 0 reports the error.
//
// Copies.  Both walk a flat index over (row, unit) with 16-byte units where
// the row allows, consecutive lanes on consecutive units, ILP units per lane
// loaded before any is stored.  The pad copy writes every destination row
// (zeros where the map is -1).  The restore scatters every mapped row back
// to its source and writes zeros to the rows past the token total, which it
// computes from the split sizes on the device.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kMapThreads = 512;
constexpr int kMapRowsPerBlock = 2048;
constexpr int kCopyThreads = 256;
constexpr int kCopyIlp = 4;

// In-place exclusive scan of n int64 values in LDS by one workgroup.
// Returns the total to every thread.  Contains barriers: call uniformly.
__device__ int64_t block_exclusive_scan(int64_t *a, int n, int64_t *wave_tot) {
  const int tid = threadIdx.x;
  const int nth = blockDim.x;
  const int per = (n + nth - 1) / nth;
  const int beg = min(n, tid * per);
  const int end = min(n, beg + per);
  int64_t sum = 0;
  for (int i = beg; i < end; i++) sum += a[i];
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  int64_t incl = sum;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int64_t v = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += v;
  }
  __syncthreads();  // callers may have just written a[]
  if (lane == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  int64_t base = 0;
  for (int i = 0; i < w; i++) base += wave_tot[i];
  int64_t run = base + incl - sum;
  for (int i = beg; i < end; i++) {
    const int64_t c = a[i];
    a[i] = run;
    run += c;
  }
  int64_t total = 0;
  for (int i = 0; i < nth / kWave; i++) total += wave_tot[i];
  __syncthreads();
  return total;
}

// Last index i in [lo, hi) with a[i] <= x, for non-decreasing a (a[lo] <= x).
__device__ __forceinline__ int last_le(const int64_t *a, int lo, int hi, int64_t x) {
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] <= x)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(kMapThreads) void chunk_map_kernel(
    const int32_t *__restrict__ split_sizes, const int32_t *__restrict__ sorted_idx, int C, int R,
    int A, int n_cap, int out_cap, int32_t *__restrict__ row_map,
    int32_t *__restrict__ padded_offsets, int32_t *__restrict__ dev_status) {
  const int G = C / R;
  extern __shared__ int64_t lds[];
  int64_t *src_off = lds;             // [C]   input-order exclusive scan
  int64_t *q_off = src_off + C;       // [C+1] sorted-order exclusive scan
  int64_t *g_pad = q_off + C + 1;     // [G+1] padded group starts
  int64_t *g_n = g_pad + G + 1;       // [G]   group token counts
  int32_t *order = (int32_t *)(g_n + G);  // [C]
  int32_t *seen = order + C;              // [C]
  __shared__ int64_t wave_tot[kMapThreads / kWave];
  __shared__ int bad_s;

  const int tid = threadIdx.x;
  if (tid == 0) bad_s = 0;
  for (int i = tid; i < C; i += kMapThreads) seen[i] = 0;
  __syncthreads();
  int bad = 0;
  for (int i = tid; i < C; i += kMapThreads) {
    const int s = split_sizes[i];
    const int c = sorted_idx[i];
    if (s < 0) bad |= MOE_DEV_BAD_CHUNKS;
    if (s > n_cap) bad |= MOE_DEV_OVERFLOW;
    src_off[i] = s < 0 ? 0 : s;
    order[i] = c;
    if ((unsigned)c >= (unsigned)C)
      bad |= MOE_DEV_BAD_CHUNKS;
    else
      atomicAdd(&seen[c], 1);
  }
  __syncthreads();
  for (int i = tid; i < C; i += kMapThreads)
    if (seen[i] != 1) bad |= MOE_DEV_BAD_CHUNKS;
  if (bad) atomicOr(&bad_s, bad);
  __syncthreads();
  bad = bad_s;

  for (int q = tid; q < C; q += kMapThreads) q_off[q] = bad ? 0 : src_off[order[q]];
  __syncthreads();
  // Scans are executed by every thread regardless of `bad` (barriers).
  const int64_t n_act = block_exclusive_scan(src_off, C, wave_tot);
  block_exclusive_scan(q_off, C, wave_tot);
  if (tid == 0) q_off[C] = n_act;
  __syncthreads();
  for (int g = tid; g < G; g += kMapThreads) {
    const int64_t n = q_off[(g + 1) * R] - q_off[g * R];
    g_n[g] = n;
    g_pad[g] = ((n + A - 1) / A) * A;
  }
  __syncthreads();
  const int64_t pad_total = block_exclusive_scan(g_pad, G, wave_tot);
  if (tid == 0) g_pad[G] = pad_total;
  if (!bad && (n_act > n_cap || pad_total > out_cap)) bad = MOE_DEV_OVERFLOW;
  __syncthreads();

  if (blockIdx.x == 0) {
    if (tid == 0) report(dev_status, bad);
    for (int g = tid; g <= G; g += kMapThreads) padded_offsets[g] = bad ? 0 : (int32_t)g_pad[g];
  }

  const int d0 = blockIdx.x * kMapRowsPerBlock;
  const int d1 = min(out_cap, d0 + kMapRowsPerBlock);
  for (int d = d0 + tid; d < d1; d += kMapThreads) {
    int32_t v = -1;
    if (!bad && d < pad_total) {
      const int g = last_le(g_pad, 0, G, d);
      const int64_t local = d - g_pad[g];
      if (local < g_n[g]) {
        const int64_t u = q_off[g * R] + local;   // position in sorted order
        const int q = last_le(q_off, g * R, (g + 1) * R, u);
        v = (int32_t)(src_off[order[q]] + (u - q_off[q]));
      }
    }
    row_map[d] = v;
  }
}

// NTS: stream the (dense, sequential) destination rows.
template <typename U, bool NTS>
__global__ __launch_bounds__(kCopyThreads) void pad_copy_kernel(
    const U *__restrict__ in, const uint8_t *__restrict__ probs, int prob_bytes, int64_t W,
    int n_cap, const int32_t *__restrict__ row_map, int out_cap, U *__restrict__ out,
    uint8_t *__restrict__ out_probs, int32_t *__restrict__ dev_status) {
  const int64_t total = (int64_t)out_cap * W;
  const int64_t base = (int64_t)blockIdx.x * kCopyThreads * kCopyIlp + threadIdx.x;
  U v[kCopyIlp];
  int bad = 0;
#pragma unroll
  for (int i = 0; i < kCopyIlp; i++) {
    const int64_t u = base + (int64_t)i * kCopyThreads;
    v[i] = zero_unit<U>();
    if (u < total) {
      const int64_t d = u / W;
      const int64_t c = u - d * W;
      const int32_t s = row_map[d];
      if (s >= n_cap) bad |= MOE_DEV_BAD_ROW;
      if (s >= 0 && s < n_cap) v[i] = ld_row<false>(in + (int64_t)s * W + c);
      if (c == 0 && out_probs != nullptr) {
        const bool ok = s >= 0 && s < n_cap;
        if (prob_bytes == 4)
          reinterpret_cast<uint32_t *>(out_probs)[d] =
              ok ? reinterpret_cast<const uint32_t *>(probs)[s] : 0u;
        else
          reinterpret_cast<uint16_t *>(out_probs)[d] =
              ok ? reinterpret_cast<const uint16_t *>(probs)[s] : (uint16_t)0;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kCopyIlp; i++) {
    const int64_t u = base + (int64_t)i * kCopyThreads;
    if (u < total) st_row<NTS>(v[i], out + u);
  }
  report(dev_status, bad);
}

// Token total of the chunk metadata, summed by one wave (every lane gets it).
__device__ __forceinline__ int64_t wave_total(const int32_t *__restrict__ sizes, int C) {
  const int lane = threadIdx.x & (kWave - 1);
  int64_t s = 0;
  for (int i = lane; i < C; i += kWave) s += sizes[i];
#pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) s += __shfl_xor(s, d, kWave);
  return s;
}

// Flat index over [0, max(out_cap, n_cap)) x W: unit (i, c) scatters padded
// row i (if mapped) and zero-fills restored row i (if past the token total).
// NTL: stream the (dense, sequential) padded source rows.
template <typename U, bool NTL>
__global__ __launch_bounds__(kCopyThreads) void restore_copy_kernel(
    const U *__restrict__ in, const uint8_t *__restrict__ probs, int prob_bytes, int64_t W,
    const int32_t *__restrict__ row_map, const int32_t *__restrict__ split_sizes, int C,
    int out_cap, int n_cap, U *__restrict__ out, uint8_t *__restrict__ out_probs,
    int32_t *__restrict__ dev_status) {
  const int64_t rows = max(out_cap, n_cap);
  const int64_t total = rows * W;
  const int64_t base = (int64_t)blockIdx.x * kCopyThreads * kCopyIlp + threadIdx.x;
  U v[kCopyIlp];
  int32_t dst[kCopyIlp];
  int bad = 0;
#pragma unroll
  for (int i = 0; i < kCopyIlp; i++) {
    const int64_t u = base + (int64_t)i * kCopyThreads;
    dst[i] = -1;
    if (u < total) {
      const int64_t d = u / W;
      const int64_t c = u - d * W;
      if (d < out_cap) {
        const int32_t s = row_map[d];
        if (s >= n_cap) bad |= MOE_DEV_BAD_ROW;
        if (s >= 0 && s < n_cap) {
          dst[i] = s;
          v[i] = ld_row<NTL>(in + u);
          if (c == 0 && out_probs != nullptr) {
            if (prob_bytes == 4)
              reinterpret_cast<uint32_t *>(out_probs)[s] =
                  reinterpret_cast<const uint32_t *>(probs)[d];
            else
              reinterpret_cast<uint16_t *>(out_probs)[s] =
                  reinterpret_cast<const uint16_t *>(probs)[d];
          }
        }
      }
    }
  }
  const int64_t n_act = wave_total(split_sizes, C);
  if (n_act > n_cap) bad |= MOE_DEV_OVERFLOW;
#pragma unroll
  for (int i = 0; i < kCopyIlp; i++) {
    const int64_t u = base + (int64_t)i * kCopyThreads;
    if (u < total) {
      const int64_t d = u / W;
      const int64_t c = u - d * W;
      if (dst[i] >= 0) st_row<false>(v[i], out + (int64_t)dst[i] * W + c);
      if (d >= n_act && d < n_cap) {
        st_row<false>(zero_unit<U>(), out + u);
        if (c == 0 && out_probs != nullptr) {
          if (prob_bytes == 4)
            reinterpret_cast<uint32_t *>(out_probs)[d] = 0u;
          else
            reinterpret_cast<uint16_t *>(out_probs)[d] = 0;
        }
      }
    }
  }
  report(dev_status, bad);
}

inline unsigned copy_blocks(int64_t units) {
  const int64_t per = (int64_t)kCopyThreads * kCopyIlp;
  return (unsigned)((units + per - 1) / per);
}

}  // namespace

hipError_t launch_chunk_map(const int32_t *split_sizes, const int32_t *sorted_idx, int C, int R,
                            int A, int n_cap, int out_cap, int32_t *row_map,
                            int32_t *padded_offsets, int32_t *dev_status, hipStream_t s) {
  const int G = C / R;
  const size_t lds = (size_t)(C + (C + 1) + (G + 1) + G) * sizeof(int64_t) +
                     (size_t)2 * C * sizeof(int32_t);
  const int blocks = out_cap > 0 ? (out_cap + kMapRowsPerBlock - 1) / kMapRowsPerBlock : 1;
  if (lds > 65536) {
    // Large chunk tables need more than the default 64 KiB of dynamic LDS
    // (gfx950 has 160 KiB per workgroup).
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&chunk_map_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(chunk_map_kernel, dim3(blocks), dim3(kMapThreads), lds, s, split_sizes,
                     sorted_idx, C, R, A, n_cap, out_cap, row_map, padded_offsets, dev_status);
  return hipGetLastError();
}

hipError_t launch_pad_copy(const void *in, const void *probs, int prob_bytes, int unit_bytes,
                           int64_t row_units, int n_cap, const int32_t *row_map, int out_cap,
                           void *out, void *out_probs, int32_t *dev_status, hipStream_t s) {
  const int64_t units = (int64_t)out_cap * row_units;
  if (units == 0) return hipSuccess;
  const dim3 grid(copy_blocks(units)), block(kCopyThreads);
  const auto *pp = static_cast<const uint8_t *>(probs);
  auto *op = static_cast<uint8_t *>(out_probs);
  const bool stream = units * 16 * 2 > kStreamBytes;
  switch (unit_bytes) {
    case 16:
      if (stream)
        hipLaunchKernelGGL((pad_copy_kernel<v4u, true>), grid, block, 0, s,
                           static_cast<const v4u *>(in), pp, prob_bytes, row_units, n_cap,
                           row_map, out_cap, static_cast<v4u *>(out), op, dev_status);
      else
        hipLaunchKernelGGL((pad_copy_kernel<v4u, false>), grid, block, 0, s,
                           static_cast<const v4u *>(in), pp, prob_bytes, row_units, n_cap,
                           row_map, out_cap, static_cast<v4u *>(out), op, dev_status);
      break;
    case 4:
      hipLaunchKernelGGL((pad_copy_kernel<uint32_t, false>), grid, block, 0, s,
                         static_cast<const uint32_t *>(in), pp, prob_bytes, row_units, n_cap,
                         row_map, out_cap, static_cast<uint32_t *>(out), op, dev_status);
      break;
    default:
      hipLaunchKernelGGL((pad_copy_kernel<uint16_t, false>), grid, block, 0, s,
                         static_cast<const uint16_t *>(in), pp, prob_bytes, row_units, n_cap,
                         row_map, out_cap, static_cast<uint16_t *>(out), op, dev_status);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_restore_copy(const void *in, const void *probs, int prob_bytes, int unit_bytes,
                               int64_t row_units, const int32_t *row_map,
                               const int32_t *split_sizes, int C, int out_cap, int n_cap,
                               void *out, void *out_probs, int32_t *dev_status, hipStream_t s) {
  const int64_t units = (int64_t)(out_cap > n_cap ? out_cap : n_cap) * row_units;
  if (units == 0) return hipSuccess;
  const dim3 grid(copy_blocks(units)), block(kCopyThreads);
  const auto *pp = static_cast<const uint8_t *>(probs);
  auto *op = static_cast<uint8_t *>(out_probs);
  const bool stream = ((int64_t)out_cap + n_cap) * row_units * 16 > kStreamBytes;
  switch (unit_bytes) {
    case 16:
      if (stream)
        hipLaunchKernelGGL((restore_copy_kernel<v4u, true>), grid, block, 0, s,
                           static_cast<const v4u *>(in), pp, prob_bytes, row_units, row_map,
                           split_sizes, C, out_cap, n_cap, static_cast<v4u *>(out), op,
                           dev_status);
      else
        hipLaunchKernelGGL((restore_copy_kernel<v4u, false>), grid, block, 0, s,
                           static_cast<const v4u *>(in), pp, prob_bytes, row_units, row_map,
                           split_sizes, C, out_cap, n_cap, static_cast<v4u *>(out), op,
                           dev_status);
      break;
    case 4:
      hipLaunchKernelGGL((restore_copy_kernel<uint32_t, false>), grid, block, 0, s,
                         static_cast<const uint32_t *>(in), pp, prob_bytes, row_units, row_map,
                         split_sizes, C, out_cap, n_cap, static_cast<uint32_t *>(out), op,
                         dev_status);
      break;
    default:
      hipLaunchKernelGGL((restore_copy_kernel<uint16_t, false>), grid, block, 0, s,
                         static_cast<const uint16_t *>(in), pp, prob_bytes, row_units, row_map,
                         split_sizes, C, out_cap, n_cap, static_cast<uint16_t *>(out), op,
                         dev_status);
      break;
  }
  return hipGetLastError();
}

}  // namespace moe
