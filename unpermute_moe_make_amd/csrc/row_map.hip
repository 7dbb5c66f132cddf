// Routing row map by a stable counting sort, in three launches.
//
// d9d permute_with_probs.py (TransformerEngine mask-map permutation),
// make_row_id_map: per-expert counts per token block, an exclusive scan of
// the counts in expert-major order, then each routed (token, expert) gets
// (expert base) + (its rank among the block's tokens routed to that expert).
// moe-ops README, "Routing permute / unpermute": histogram + exclusive prefix
// sums.  The result is rows expert-major, tokens ascending inside an expert.
//
// gfx950 design.  A block owns 256 tokens = 4 wavefronts x 64 lanes, and
// the routing of each 64-token wave tile is held as one 64-bit lane mask
// per expert: bit l of mask[w][e] says token 64*w + l of the block routes to
// expert e.  Building the masks with LDS atomic ORs is order-independent,
// and an OR that finds its bit already set exposes a repeated expert.  The
// stable in-tile rank of a routed token is then popcount(mask & lanes
// below), i.e. mbcnt -- no atomic arrival order decides any row.
//   count: masks -> workspace, per-(expert, block) counts.
//   scan:  one workgroup scans the E x nb counts (expert-major) into bases
//          and writes expert_offsets.
//   write: grid (blocks, expert groups); each wave writes 64 consecutive
//          row_id_map entries per expert (256-byte coalesced stores).
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kTokPerBlock = 256;     // 4 waves x 64 tokens
constexpr int kWavesPerBlock = kTokPerBlock / kWave;
constexpr int kExpertsPerWrite = 32;  // experts per write workgroup
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kTokPerBlock) void rowmap_count_kernel(
    const int32_t *__restrict__ topk_idx, int T, int k, int E, int nb,
    unsigned long long *__restrict__ masks, int32_t *__restrict__ counts,
    int32_t *__restrict__ dev_status) {
  extern __shared__ unsigned long long smask[];  // [4][E]
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  for (int i = tid; i < kWavesPerBlock * E; i += kTokPerBlock) smask[i] = 0ull;
  __syncthreads();

  const int t0 = b * kTokPerBlock;
  const int ntok = min(kTokPerBlock, T - t0);
  const int nflat = ntok * k;
  const int32_t *src = topk_idx + (int64_t)t0 * k;
  int bad = 0;
  // Flat, coalesced walk over the block's [ntok][k] indices.
  for (int f = tid; f < nflat; f += kTokPerBlock) {
    const int e = src[f];
    const int tl = f / k;
    if ((unsigned)e >= (unsigned)E) {
      bad |= MOE_DEV_BAD_EXPERT;
      continue;
    }
    const unsigned long long bit = 1ull << (tl & (kWave - 1));
    const unsigned long long old = atomicOr(&smask[(tl / kWave) * E + e], bit);
    if (old & bit) bad |= MOE_DEV_DUP_EXPERT;
  }
  report(dev_status, bad);
  __syncthreads();

  for (int e = tid; e < E; e += kTokPerBlock) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; w++) {
      const unsigned long long m = smask[w * E + e];
      masks[((int64_t)b * kWavesPerBlock + w) * E + e] = m;
      c += __popcll(m);
    }
    counts[(int64_t)e * nb + b] = c;
  }
}

// Exclusive scan of counts[E][nb] in expert-major order, in place; also
// expert_offsets[e] = base of (e, block 0) and expert_offsets[E] = total.
__global__ __launch_bounds__(kScanThreads) void rowmap_scan_kernel(
    int32_t *__restrict__ counts, int n, int nb, int E, int32_t *__restrict__ expert_offsets) {
  __shared__ int wave_tot[kScanThreads / kWave];
  const int tid = threadIdx.x;
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int beg = min(n, tid * per);
  const int end = min(n, beg + per);
  int sum = 0;
  for (int i = beg; i < end; i++) sum += counts[i];

  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  int incl = sum;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int v = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += v;
  }
  if (lane == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  int wbase = 0;
  for (int i = 0; i < w; i++) wbase += wave_tot[i];

  int run = wbase + incl - sum;
  int e = beg / nb;
  int b = beg - e * nb;
  for (int i = beg; i < end; i++) {
    const int c = counts[i];
    counts[i] = run;
    if (b == 0) expert_offsets[e] = run;
    run += c;
    if (++b == nb) {
      b = 0;
      e++;
    }
  }
  if (tid == kScanThreads - 1) expert_offsets[E] = wbase + incl;
}

__global__ __launch_bounds__(kTokPerBlock) void rowmap_write_kernel(
    const unsigned long long *__restrict__ masks, const int32_t *__restrict__ base, int T, int E,
    int nb, int32_t *__restrict__ row_id_map) {
  __shared__ unsigned long long smask[kWavesPerBlock][kExpertsPerWrite];
  __shared__ int32_t sbase[kWavesPerBlock][kExpertsPerWrite];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int e0 = blockIdx.y * kExpertsPerWrite;
  const int ne = min(kExpertsPerWrite, E - e0);
  if (tid < ne) {
    const int e = e0 + tid;
    int run = base[(int64_t)e * nb + b];
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; w++) {
      const unsigned long long m = masks[((int64_t)b * kWavesPerBlock + w) * E + e];
      smask[w][tid] = m;
      sbase[w][tid] = run;
      run += __popcll(m);
    }
  }
  __syncthreads();

  const int w = tid / kWave;
  const int lane = tid & (kWave - 1);
  const int t = b * kTokPerBlock + tid;
  if (t >= T) return;
  for (int i = 0; i < ne; i++) {
    const unsigned long long m = smask[w][i];
    // number of routed tokens below this lane in the wave tile
    const unsigned below = __builtin_amdgcn_mbcnt_hi(
        (unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
    const int v = ((m >> lane) & 1ull) ? sbase[w][i] + (int)below : -1;
    row_id_map[(int64_t)(e0 + i) * T + t] = v;
  }
}

__global__ void fill_kernel(int32_t *__restrict__ p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t rowmap_workspace_bytes(int T, int k, int E) {
  (void)k;
  const size_t nb = (size_t)((T + kTokPerBlock - 1) / kTokPerBlock);
  return align256(nb * kWavesPerBlock * (size_t)E * sizeof(unsigned long long)) +
         align256(nb * (size_t)E * sizeof(int32_t));
}

hipError_t launch_rowmap(const int32_t *topk_idx, int T, int k, int E, int32_t *row_id_map,
                         int32_t *expert_offsets, int32_t *dev_status, void *ws,
                         hipStream_t s) {
  if (T == 0) {
    hipLaunchKernelGGL(fill_kernel, dim3((E + 1 + 255) / 256), dim3(256), 0, s, expert_offsets,
                       E + 1, 0);
    return hipGetLastError();
  }
  const int nb = (T + kTokPerBlock - 1) / kTokPerBlock;
  auto *masks = reinterpret_cast<unsigned long long *>(ws);
  auto *counts = reinterpret_cast<int32_t *>(
      reinterpret_cast<char *>(ws) +
      align256((size_t)nb * kWavesPerBlock * E * sizeof(unsigned long long)));
  const size_t lds = (size_t)kWavesPerBlock * E * sizeof(unsigned long long);
  hipLaunchKernelGGL(rowmap_count_kernel, dim3(nb), dim3(kTokPerBlock), lds, s, topk_idx, T, k,
                     E, nb, masks, counts, dev_status);
  hipLaunchKernelGGL(rowmap_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, counts, E * nb, nb, E,
                     expert_offsets);
  hipLaunchKernelGGL(rowmap_write_kernel,
                     dim3(nb, (E + kExpertsPerWrite - 1) / kExpertsPerWrite),
                     dim3(kTokPerBlock), 0, s, masks, counts, T, E, nb, row_id_map);
  return hipGetLastError();
}

}  // namespace moe
