// Routing row map by a stable counting sort.
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
//
//   count:  masks -> workspace, per-(block, expert) counts [nb][E].
//   write:  each block derives its bases itself -- expert totals, their
//           exclusive scan, and the counts of the earlier blocks -- then
//           each wave writes 64 consecutive row_id_map entries per expert of
//           its expert group (256-byte coalesced stores).  Two launches.
//   With many blocks (long token counts) the per-block walk over all
//   earlier blocks would grow quadratically, so a column-scan kernel (one
//   workgroup per expert, a parallel scan over the blocks) computes the
//   bases once and the write kernel reads them: three launches.
//   With few entries (up to 4096 token slots) one launch does it all: each
//   workgroup counts every index itself (rowmap_single_kernel).
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kTokPerBlock = 256;  // 4 waves x 64 tokens
constexpr int kWavesPerBlock = kTokPerBlock / kWave;
// Build-time tuning: token blocks up to which the write kernel derives its
// bases itself (16384 tokens), and experts per write workgroup beyond 32
// blocks (measured: 16 and 32 alike at 16384 tokens, 64 slower).
#ifndef MOE_FUSED_MAX_BLOCKS
#define MOE_FUSED_MAX_BLOCKS 64
#endif
#ifndef MOE_WRITE_EPW_LARGE
#define MOE_WRITE_EPW_LARGE 16
#endif
constexpr int kFusedMaxBlocks = MOE_FUSED_MAX_BLOCKS;
constexpr int kWriteEpwLarge = MOE_WRITE_EPW_LARGE;
constexpr int kScanThreads = 256;
constexpr int kCountBatch = 8;     // topk indices loaded per lane before use
// One-launch map up to this many (token, slot) entries and experts, and the
// experts per workgroup there; build-time tuning (every workgroup counts all
// entries with LDS atomics, which costs more than the second launch it saves
// beyond about 4096 entries).
#ifndef MOE_SINGLE_MAX_ENTRIES
#define MOE_SINGLE_MAX_ENTRIES 4096
#endif
constexpr int kSingleMaxEntries = MOE_SINGLE_MAX_ENTRIES;
constexpr int kSingleMaxExperts = 512;
#ifndef MOE_SINGLE_EPW
#define MOE_SINGLE_EPW 4
#endif
// Experts per write workgroup: 8 while there are few token blocks (more
// workgroups to spread the map stores), 16 beyond (less repeated base
// derivation); chosen by measurement.
constexpr int kSmallBlocks = 32;

__global__ __launch_bounds__(kTokPerBlock) void rowmap_count_kernel(
    const int32_t *__restrict__ topk_idx, int T, int k, int E,
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
  // Flat, coalesced walk over the block's [ntok][k] indices, kCountBatch
  // loads of a lane in flight before its first LDS atomic (one memory
  // latency per batch rather than per index).
  for (int f0 = tid; f0 < nflat; f0 += kTokPerBlock * kCountBatch) {
    int ev[kCountBatch];
#pragma unroll
    for (int i = 0; i < kCountBatch; i++) {
      const int f = f0 + i * kTokPerBlock;
      ev[i] = f < nflat ? src[f] : 0;
    }
#pragma unroll
    for (int i = 0; i < kCountBatch; i++) {
      const int f = f0 + i * kTokPerBlock;
      if (f >= nflat) break;
      const int e = ev[i];
      const int tl = f / k;
      if ((unsigned)e >= (unsigned)E) {
        bad |= MOE_DEV_BAD_EXPERT;
        continue;
      }
      const unsigned long long bit = 1ull << (tl & (kWave - 1));
      const unsigned long long old = atomicOr(&smask[(tl / kWave) * E + e], bit);
      if (old & bit) bad |= MOE_DEV_DUP_EXPERT;
    }
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
    counts[(int64_t)b * E + e] = c;
  }
}

// Exclusive scan of n ints in LDS by the whole workgroup (any blockDim that
// is a multiple of 64); returns the total.  Contains barriers.
__device__ int block_scan_lds(int *a, int n, int *wave_tot) {
  const int tid = threadIdx.x;
  const int nth = blockDim.x;
  const int per = (n + nth - 1) / nth;
  const int beg = min(n, tid * per);
  const int end = min(n, beg + per);
  int sum = 0;
  for (int i = beg; i < end; i++) sum += a[i];
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const int incl = wave_inclusive_scan(sum);
  __syncthreads();
  if (lane == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; i++) base += wave_tot[i];
  int run = base + incl - sum;
  for (int i = beg; i < end; i++) {
    const int c = a[i];
    a[i] = run;
    run += c;
  }
  int total = 0;
  for (int i = 0; i < nth / kWave; i++) total += wave_tot[i];
  __syncthreads();
  return total;
}

// Column scan for long token counts: workgroup e turns counts[.][e] into
// the exclusive prefix over blocks (in place) and writes the expert total.
__global__ __launch_bounds__(kScanThreads) void rowmap_colscan_kernel(
    int32_t *__restrict__ counts, int nb, int E, int32_t *__restrict__ totals) {
  __shared__ int chunk[kScanThreads * 4];
  __shared__ int wave_tot[kScanThreads / kWave];
  const int e = blockIdx.x;
  int carry = 0;
  for (int b0 = 0; b0 < nb; b0 += kScanThreads * 4) {
    const int n = min(kScanThreads * 4, nb - b0);
    for (int i = threadIdx.x; i < n; i += kScanThreads) chunk[i] = counts[(int64_t)(b0 + i) * E + e];
    __syncthreads();
    const int tot = block_scan_lds(chunk, n, wave_tot);
    for (int i = threadIdx.x; i < n; i += kScanThreads)
      counts[(int64_t)(b0 + i) * E + e] = carry + chunk[i];
    carry += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) totals[e] = carry;
}

// The row_id_map entries of block b's tokens for experts [e0, e0+ne): lane =
// token; rank in its wave tile = routed tokens below it (mbcnt of the mask).
template <int EPW>
__device__ __forceinline__ void write_block_rows(
    const unsigned long long (*s_mask)[EPW], const int (*s_base)[EPW], int b, int e0, int ne,
    int T, int32_t *__restrict__ row_id_map) {
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int lane = tid & (kWave - 1);
  const int t = b * kTokPerBlock + tid;
  if (t >= T) return;
  for (int i = 0; i < ne; i++) {
    const unsigned long long m = s_mask[w][i];
    const unsigned below = __builtin_amdgcn_mbcnt_hi(
        (unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
    const int v = ((m >> lane) & 1ull) ? s_base[w][i] + (int)below : -1;
    row_id_map[(int64_t)(e0 + i) * T + t] = v;
  }
}

// FUSED: derive totals and the earlier-block prefix from counts[nb][E];
// otherwise counts already holds the prefix and totals the expert totals.
// Grid (nb, ceil(E / EPW)): block (b, y) writes the entries of experts
// [y*EPW, y*EPW+EPW) for the block's 256 tokens.
template <bool FUSED, int EPW>
__global__ __launch_bounds__(kTokPerBlock) void rowmap_write_kernel(
    const unsigned long long *__restrict__ masks, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ totals, int T, int E, int nb, int32_t *__restrict__ row_id_map,
    int32_t *__restrict__ expert_offsets) {
  extern __shared__ int s_off[];                         // [E] expert offsets
  __shared__ int s_pre[EPW];                             // rows of earlier blocks
  __shared__ int s_base[kWavesPerBlock][EPW];
  __shared__ unsigned long long s_mask[kWavesPerBlock][EPW];
  __shared__ int wave_tot[kTokPerBlock / kWave];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int e0 = blockIdx.y * EPW;
  const int ne = min(EPW, E - e0);

  // The block's own masks do not depend on the scan: load them first.
  unsigned long long mk[kWavesPerBlock];
  if (tid < ne) {
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; w++)
      mk[w] = masks[((int64_t)b * kWavesPerBlock + w) * E + e0 + tid];
  }
  for (int e = tid; e < E; e += kTokPerBlock) {
    int tot = 0, pre = 0;
    const bool mine = e >= e0 && e < e0 + ne;
    if (FUSED) {
#pragma unroll 16
      for (int b2 = 0; b2 < nb; b2++) {
        const int c = counts[(int64_t)b2 * E + e];
        tot += c;
        pre += (b2 < b) ? c : 0;
      }
    } else {
      tot = totals[e];
      if (mine) pre = counts[(int64_t)b * E + e];
    }
    s_off[e] = tot;
    if (mine) s_pre[e - e0] = pre;
  }
  __syncthreads();
  const int total = block_scan_lds(s_off, E, wave_tot);
  if (b == 0 && blockIdx.y == 0) {
    for (int e = tid; e < E; e += kTokPerBlock) expert_offsets[e] = s_off[e];
    if (tid == 0) expert_offsets[E] = total;
  }
  if (tid < ne) {
    const int e = e0 + tid;
    int run = s_off[e] + s_pre[tid];
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; w++) {
      s_mask[w][tid] = mk[w];
      s_base[w][tid] = run;
      run += __popcll(mk[w]);
    }
  }
  __syncthreads();
  write_block_rows<EPW>(s_mask, s_base, b, e0, ne, T, row_id_map);
}

// Short token ranges in one launch: every workgroup stages all T*k indices in
// LDS (as 16-bit experts) and counts them itself with LDS atomic adds -- the
// rows of every expert, and the rows of its own experts among the tokens
// before its block -- while the 64-bit lane masks of its own block give the
// in-tile ranks as above.  Counts and masks are order-free, so no arrival
// order decides a row.  Every workgroup reading all the indices is what
// bounds this path to kSingleMaxEntries.  (kdiv, kshift): floor(f / k) =
// (umulhi(kdiv, f) + f) >> kshift for every flat index f < 2^32.
template <int EPW>
__global__ __launch_bounds__(kTokPerBlock) void rowmap_single_kernel(
    const int32_t *__restrict__ topk_idx, int T, int k, int E, uint32_t kdiv, int kshift,
    int32_t *__restrict__ row_id_map, int32_t *__restrict__ expert_offsets,
    int32_t *__restrict__ dev_status) {
  extern __shared__ int s_cnt[];                         // [E] counts, then offsets
  __shared__ uint16_t s_idx[kSingleMaxEntries];          // experts, 0xFFFF = invalid
  __shared__ int s_pre[EPW];
  __shared__ int s_base[kWavesPerBlock][EPW];
  __shared__ unsigned long long s_mask[kWavesPerBlock][EPW];
  __shared__ int wave_tot[kTokPerBlock / kWave];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int e0 = blockIdx.y * EPW;
  const int ne = min(EPW, E - e0);
  const int n = T * k;
  const int t_blk = b * kTokPerBlock;

  // All 16-byte loads of a lane in flight at once (topk_idx is 16-byte
  // aligned on this path); the tail of n % 4 entries is read singly.
  constexpr int kLoads = (kSingleMaxEntries + 4 * kTokPerBlock - 1) / (4 * kTokPerBlock);
  const v4u *src4 = reinterpret_cast<const v4u *>(topk_idx);
  const int n4 = n / 4;
  v4u r[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; i++) {
    const int q = tid + i * kTokPerBlock;
    if (q < n4) r[i] = src4[q];
  }
  for (int e = tid; e < E; e += kTokPerBlock) s_cnt[e] = 0;
  if (tid < EPW) {
    s_pre[tid] = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; w++) s_mask[w][tid] = 0ull;
  }
  auto expert16 = [E](uint32_t e) -> uint16_t { return e < (uint32_t)E ? (uint16_t)e : 0xFFFF; };
#pragma unroll
  for (int i = 0; i < kLoads; i++) {
    const int q = tid + i * kTokPerBlock;
    if (q < n4) {
      s_idx[4 * q] = expert16(r[i].x);
      s_idx[4 * q + 1] = expert16(r[i].y);
      s_idx[4 * q + 2] = expert16(r[i].z);
      s_idx[4 * q + 3] = expert16(r[i].w);
    }
  }
  if (tid < n - 4 * n4) s_idx[4 * n4 + tid] = expert16((uint32_t)topk_idx[4 * n4 + tid]);
  __syncthreads();

  int bad = 0;
  for (int f = tid; f < n; f += kTokPerBlock) {
    const uint32_t e = s_idx[f];
    if (e == 0xFFFF) {
      bad |= MOE_DEV_BAD_EXPERT;
      continue;
    }
    atomicAdd(&s_cnt[e], 1);
    const int ge = (int)e - e0;
    if ((unsigned)ge < (unsigned)ne) {
      const int t = (int)(((uint64_t)__umulhi(kdiv, (uint32_t)f) + (uint32_t)f) >> kshift);
      if (t < t_blk) {
        atomicAdd(&s_pre[ge], 1);
      } else if (t < t_blk + kTokPerBlock) {
        const int tl = t - t_blk;
        const unsigned long long bit = 1ull << (tl & (kWave - 1));
        const unsigned long long old = atomicOr(&s_mask[tl / kWave][ge], bit);
        if (old & bit) bad |= MOE_DEV_DUP_EXPERT;
      }
    }
  }
  // every workgroup sees every index: the first one reports bad experts,
  // each reports the repeats it finds in its own block and experts
  if (b != 0 || blockIdx.y != 0) bad &= ~MOE_DEV_BAD_EXPERT;
  report(dev_status, bad);
  __syncthreads();
  const int total = block_scan_lds(s_cnt, E, wave_tot);
  if (b == 0 && blockIdx.y == 0) {
    for (int e = tid; e < E; e += kTokPerBlock) expert_offsets[e] = s_cnt[e];
    if (tid == 0) expert_offsets[E] = total;
  }
  if (tid < ne) {
    int run = s_cnt[e0 + tid] + s_pre[tid];
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; w++) {
      s_base[w][tid] = run;
      run += __popcll(s_mask[w][tid]);
    }
  }
  __syncthreads();
  write_block_rows<EPW>(s_mask, s_base, b, e0, ne, T, row_id_map);
}

// ----------------------------------------------------- mask-map (TE) form --
//
// d9d permute_with_probs.py (TransformerEngine mask-map permutation),
// make_row_id_map: a [T][E] routing mask instead of top-k indices, and a
// per-token map [T][2E+1]: the token's destination rows in descending
// order, then their experts, then their count.  The rows are the same
// counting sort as above; only the input and the final layout differ.  For a
// fixed token the rows grow with the expert (expert-major), so descending
// rows are simply the routed experts walked from E-1 down to 0.

// Masks from a [T][E] routing mask: lane l of wave w holds V experts and
// builds their 64-bit token masks over the wave's 64 tokens, one coalesced
// row segment per token.  MB: bytes per mask entry; V: experts per lane
// (one vector load of V entries).
template <int MB, int V>
__global__ __launch_bounds__(kTokPerBlock) void maskmap_count_kernel(
    const void *__restrict__ routing_map, int T, int E, unsigned long long *__restrict__ masks,
    int32_t *__restrict__ counts) {
  extern __shared__ int s_cnt[];  // [4][E]
  using Vec = typename std::conditional<
      MB * V == 16, v4u,
      typename std::conditional<MB * V == 4, uint32_t,
                                typename std::conditional<MB * V == 2, uint16_t,
                                                          uint8_t>::type>::type>::type;
  static_assert(sizeof(Vec) == MB * V, "one load per lane and token");
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int w = tid / kWave;
  const int lane = tid & (kWave - 1);
  const int tw = b * kTokPerBlock + w * kWave;   // first token of the wave tile
  const int ntw = max(0, min(kWave, T - tw));
  for (int e0 = lane * V; e0 < E; e0 += kWave * V) {
    unsigned long long bits[V];
#pragma unroll
    for (int c = 0; c < V; c++) bits[c] = 0ull;
    const char *base = static_cast<const char *>(routing_map) + ((int64_t)tw * E + e0) * MB;
#pragma unroll 8
    for (int i = 0; i < ntw; i++) {
      const Vec raw = *reinterpret_cast<const Vec *>(base + (int64_t)i * E * MB);
      const uint8_t *bytes = reinterpret_cast<const uint8_t *>(&raw);
#pragma unroll
      for (int c = 0; c < V; c++) {
        bool on;
        if constexpr (MB == 4)
          on = reinterpret_cast<const uint32_t *>(bytes)[c] != 0u;
        else
          on = bytes[c] != 0;
        bits[c] |= (unsigned long long)on << i;
      }
    }
#pragma unroll
    for (int c = 0; c < V; c++) {
      masks[((int64_t)b * kWavesPerBlock + w) * E + e0 + c] = bits[c];
      s_cnt[w * E + e0 + c] = __popcll(bits[c]);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kTokPerBlock)
    counts[(int64_t)b * E + e] =
        s_cnt[e] + s_cnt[E + e] + s_cnt[2 * E + e] + s_cnt[3 * E + e];
}

constexpr int kMaskChunk = kTokPerBlock;   // experts staged in LDS at a time

// Bit i of the result: entry i of a 16-byte vector of routing-mask entries
// (16 one-byte or 4 four-byte) is nonzero.
template <int MB>
__device__ __forceinline__ uint32_t nonzero_bits(v4u v) {
  uint32_t out = 0;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const uint32_t w = v[q];
    if constexpr (MB == 4) {
      out |= (uint32_t)(w != 0u) << q;
    } else {
      // high bit of each byte set iff the byte is nonzero, then the four high
      // bits gathered into a nibble by one multiply (no carries collide)
      const uint32_t h = (((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w) & 0x80808080u;
      out |= (((h >> 7) * 0x00204081u) >> 21 & 0xFu) << (4 * q);
    }
  }
  return out;
}

// Masks from a [T][E] routing mask by wave ballots, when every mask row is a
// whole number of 16-byte vectors on a 16-byte aligned base: lane = token of
// the wave tile; the lane reads its own row 64 experts at a time as a 64-bit
// set, and one ballot per expert is that expert's token mask for the tile.
// All of a lane's loads for a group of 64 experts are in flight together.
// (Used for up to 64 experts; the loop handles any count.)
template <int MB>
__global__ __launch_bounds__(kTokPerBlock) void maskmap_count_ballot_kernel(
    const void *__restrict__ routing_map, int T, int E, unsigned long long *__restrict__ masks,
    int32_t *__restrict__ counts) {
  extern __shared__ int s_cnt[];  // [4][E]
  constexpr int kPerVec = 16 / MB;         // mask entries per 16-byte vector
  constexpr int kVecs = kWave / kPerVec;   // vectors per 64 experts
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int w = tid / kWave;
  const int lane = tid & (kWave - 1);
  const int t = b * kTokPerBlock + tid;
  const bool live = t < T;
  const v4u *row = reinterpret_cast<const v4u *>(static_cast<const uint8_t *>(routing_map) +
                                                 (int64_t)(live ? t : 0) * E * MB);
  for (int g0 = 0; g0 < E; g0 += kWave) {
    const int nv = min(kVecs, (E - g0) / kPerVec);   // E * MB is a multiple of 16
    v4u v[kVecs];
#pragma unroll
    for (int q = 0; q < kVecs; q++)
      v[q] = (live && q < nv) ? row[g0 / kPerVec + q] : v4u{0u, 0u, 0u, 0u};
    unsigned long long bits = 0ull;
#pragma unroll
    for (int q = 0; q < kVecs; q++)
      bits |= (unsigned long long)nonzero_bits<MB>(v[q]) << (q * kPerVec);
    unsigned long long mine = 0ull;
    const int ng = min(kWave, E - g0);
    for (int i = 0; i < ng; i++) {
      const unsigned long long m = __ballot((bits >> i) & 1ull);
      mine = lane == i ? m : mine;
    }
    if (lane < ng) {
      masks[((int64_t)b * kWavesPerBlock + w) * E + g0 + lane] = mine;
      s_cnt[w * E + g0 + lane] = __popcll(mine);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kTokPerBlock)
    counts[(int64_t)b * E + e] =
        s_cnt[e] + s_cnt[E + e] + s_cnt[2 * E + e] + s_cnt[3 * E + e];
}

// Per-token map rows.  FUSED as for rowmap_write_kernel.  Each lane owns one
// token.  Chunk by chunk from the top expert down, the block stages each
// expert's wave-tile masks and row bases in LDS; the lane reads its own
// routing-mask row for the chunk (VEC: 16-byte vectors), turns it into a
// bitset and visits only its routed experts, highest first, appending the
// kept rows.  Entries past the token's count are not written.
template <bool FUSED, int MB, bool VEC>
__global__ __launch_bounds__(kTokPerBlock) void maskmap_write_kernel(
    const void *__restrict__ routing_map, const unsigned long long *__restrict__ masks,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ totals, int T, int E,
    int nb, int num_out, int32_t *__restrict__ map, int32_t *__restrict__ expert_offsets) {
  __shared__ int s_off[MOE_MAX_EXPERTS];
  __shared__ int s_pre[MOE_MAX_EXPERTS];   // rows of the earlier blocks (FUSED)
  __shared__ unsigned long long s_mask[kWavesPerBlock][kMaskChunk];
  __shared__ int s_base[kWavesPerBlock][kMaskChunk];
  __shared__ int wave_tot[kTokPerBlock / kWave];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  for (int e = tid; e < E; e += kTokPerBlock) {
    int tot = 0;
    if (FUSED) {
      int pre = 0;
#pragma unroll 16
      for (int b2 = 0; b2 < nb; b2++) {
        const int c = counts[(int64_t)b2 * E + e];
        tot += c;
        pre += (b2 < b) ? c : 0;
      }
      s_pre[e] = pre;
    } else {
      tot = totals[e];
    }
    s_off[e] = tot;
  }
  __syncthreads();
  const int total = block_scan_lds(s_off, E, wave_tot);
  const int kept = num_out >= 0 ? min(total, num_out) : total;
  if (b == 0 && expert_offsets != nullptr) {
    for (int e = tid; e < E; e += kTokPerBlock) expert_offsets[e] = min(s_off[e], kept);
    if (tid == 0) expert_offsets[E] = kept;
  }

  const int w = tid / kWave;
  const int t = b * kTokPerBlock + tid;
  const int64_t W = 2 * (int64_t)E + 1;
  int32_t *mrow = map + (int64_t)t * W;
  const uint8_t *rrow = static_cast<const uint8_t *>(routing_map) + (int64_t)t * E * MB;
  int n = 0;
  const int nchunks = (E + kMaskChunk - 1) / kMaskChunk;
  for (int ch = nchunks - 1; ch >= 0; ch--) {
    const int c0 = ch * kMaskChunk;
    const int nc = min(kMaskChunk, E - c0);
    // this lane's routed experts of the chunk, as a bitset (loads first)
    uint32_t bits[kMaskChunk / 32];
#pragma unroll
    for (int i = 0; i < kMaskChunk / 32; i++) bits[i] = 0u;
    if (t < T) {
      if constexpr (VEC) {
        constexpr int kPerVec = 16 / MB;
        const v4u *src = reinterpret_cast<const v4u *>(rrow + (int64_t)c0 * MB);
#pragma unroll
        for (int q = 0; q < kMaskChunk / kPerVec; q++) {
          if (q * kPerVec < nc) {
            const uint32_t nz = nonzero_bits<MB>(src[q]);
            bits[q * kPerVec / 32] |= nz << ((q * kPerVec) % 32);
          }
        }
      } else {
#pragma unroll
        for (int word = 0; word < kMaskChunk / 32; word++) {
          uint32_t x = 0u;
          for (int i2 = 0; i2 < 32 && word * 32 + i2 < nc; i2++) {
            const uint8_t *p = rrow + (int64_t)(c0 + word * 32 + i2) * MB;
            bool on;
            if constexpr (MB == 4)
              on = *reinterpret_cast<const uint32_t *>(p) != 0u;
            else
              on = *p != 0;
            x |= (uint32_t)on << i2;
          }
          bits[word] = x;
        }
      }
    }
    __syncthreads();   // the previous chunk's readers are done
    if (tid < nc) {
      const int e = c0 + tid;
      const int pre = FUSED ? s_pre[e] : counts[(int64_t)b * E + e];
      int run = s_off[e] + pre;
#pragma unroll
      for (int ww = 0; ww < kWavesPerBlock; ww++) {
        const unsigned long long m = masks[((int64_t)b * kWavesPerBlock + ww) * E + e];
        s_mask[ww][tid] = m;
        s_base[ww][tid] = run;
        run += __popcll(m);
      }
    }
    __syncthreads();
#pragma unroll
    for (int word = kMaskChunk / 32 - 1; word >= 0; word--) {
      uint32_t x = bits[word];
      while (x != 0u) {
        const int hb = 31 - __clz((int)x);
        x &= ~(1u << hb);
        const int i = word * 32 + hb;
        const unsigned long long m = s_mask[w][i];
        const int row = s_base[w][i] + (int)__builtin_amdgcn_mbcnt_hi(
                                           (unsigned)(m >> 32),
                                           __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
        if (row < kept) {
          mrow[n] = row;
          mrow[E + n] = c0 + i;
          n++;
        }
      }
    }
  }
  if (t < T) mrow[2 * E] = n;
}

__global__ void fill_kernel(int32_t *__restrict__ p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// floor(f / k) = (umulhi(m, f) + f) >> l for every f < 2^32, with
// l = ceil(log2 k) and m = floor(2^32 (2^l - k) / k) + 1 (Granlund and
// Montgomery, "Division by invariant integers using multiplication").
struct KDiv {
  uint32_t m;
  int l;
};

inline KDiv k_div(int k) {
  int l = 0;
  while ((1 << l) < k) l++;
  const uint64_t num = ((uint64_t)1 << 32) * (((uint64_t)1 << l) - (uint64_t)k);
  return KDiv{(uint32_t)(num / (uint64_t)k + 1), l};
}

struct Workspace {
  unsigned long long *masks;
  int32_t *counts;
  int32_t *totals;
};

Workspace carve(void *ws, int nb, int E) {
  char *p = reinterpret_cast<char *>(ws);
  Workspace w;
  w.masks = reinterpret_cast<unsigned long long *>(p);
  p += align256((size_t)nb * kWavesPerBlock * E * sizeof(unsigned long long));
  w.counts = reinterpret_cast<int32_t *>(p);
  p += align256((size_t)nb * E * sizeof(int32_t));
  w.totals = reinterpret_cast<int32_t *>(p);
  return w;
}

}  // namespace

size_t rowmap_workspace_bytes(int T, int k, int E) {
  (void)k;
  const size_t nb = (size_t)((T + kTokPerBlock - 1) / kTokPerBlock);
  return align256(nb * kWavesPerBlock * (size_t)E * sizeof(unsigned long long)) +
         align256(nb * (size_t)E * sizeof(int32_t)) + align256((size_t)E * sizeof(int32_t));
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
  const size_t lds_write = (size_t)E * sizeof(int);
  if ((int64_t)T * k <= kSingleMaxEntries && E <= kSingleMaxExperts &&
      reinterpret_cast<uintptr_t>(topk_idx) % 16 == 0) {
    constexpr int epw = MOE_SINGLE_EPW;
    const KDiv kd = k_div(k);
    hipLaunchKernelGGL((rowmap_single_kernel<epw>), dim3(nb, (E + epw - 1) / epw),
                       dim3(kTokPerBlock), lds_write, s, topk_idx, T, k, E, kd.m, kd.l,
                       row_id_map, expert_offsets, dev_status);
    return hipGetLastError();
  }
  const Workspace w = carve(ws, nb, E);
  const size_t lds_count = (size_t)kWavesPerBlock * E * sizeof(unsigned long long);
  const bool small = nb <= kSmallBlocks;
  const int epw = small ? 8 : kWriteEpwLarge;
  const dim3 wgrid(nb, (E + epw - 1) / epw);
  hipLaunchKernelGGL(rowmap_count_kernel, dim3(nb), dim3(kTokPerBlock), lds_count, s, topk_idx,
                     T, k, E, w.masks, w.counts, dev_status);
  if (nb <= kFusedMaxBlocks) {
    if (small)
      hipLaunchKernelGGL((rowmap_write_kernel<true, 8>), wgrid, dim3(kTokPerBlock), lds_write, s,
                         w.masks, w.counts, w.totals, T, E, nb, row_id_map, expert_offsets);
    else
      hipLaunchKernelGGL((rowmap_write_kernel<true, kWriteEpwLarge>), wgrid, dim3(kTokPerBlock),
                         lds_write, s, w.masks, w.counts, w.totals, T, E, nb, row_id_map,
                         expert_offsets);
  } else {
    hipLaunchKernelGGL(rowmap_colscan_kernel, dim3(E), dim3(kScanThreads), 0, s, w.counts, nb,
                       E, w.totals);
    hipLaunchKernelGGL((rowmap_write_kernel<false, kWriteEpwLarge>), wgrid, dim3(kTokPerBlock),
                       lds_write, s, w.masks, w.counts, w.totals, T, E, nb, row_id_map,
                       expert_offsets);
  }
  return hipGetLastError();
}

size_t maskmap_workspace_bytes(int T, int E) { return rowmap_workspace_bytes(T, 1, E); }

hipError_t launch_maskmap(const void *routing_map, int mask_bytes, int T, int E, int num_out,
                          int32_t *map, int32_t *expert_offsets, void *ws, hipStream_t s) {
  if (T == 0) {
    if (expert_offsets == nullptr) return hipSuccess;
    hipLaunchKernelGGL(fill_kernel, dim3((E + 1 + 255) / 256), dim3(256), 0, s, expert_offsets,
                       E + 1, 0);
    return hipGetLastError();
  }
  const int nb = (T + kTokPerBlock - 1) / kTokPerBlock;
  const Workspace w = carve(ws, nb, E);
  const size_t lds_count = (size_t)kWavesPerBlock * E * sizeof(int);
  // Vector loads of 4 entries when rows allow them.
  const uintptr_t a = reinterpret_cast<uintptr_t>(routing_map);
  const bool vec = E % 4 == 0 && a % (4 * (uintptr_t)mask_bytes) == 0;
  // Each lane's mask row is read in 16-byte vectors when every row starts
  // 16-byte aligned.
  const bool rvec = ((int64_t)E * mask_bytes) % 16 == 0 && a % 16 == 0;
#define MOE_MASK_COUNT(MB, V)                                                                 \
  hipLaunchKernelGGL((maskmap_count_kernel<MB, V>), dim3(nb), dim3(kTokPerBlock), lds_count, s, \
                     routing_map, T, E, w.masks, w.counts)
#define MOE_MASK_BALLOT(MB)                                                                   \
  hipLaunchKernelGGL((maskmap_count_ballot_kernel<MB>), dim3(nb), dim3(kTokPerBlock),         \
                     lds_count, s, routing_map, T, E, w.masks, w.counts)
  // Ballots for up to 64 experts (one ballot per expert; beyond that the
  // expert-per-lane walk over the tile's tokens was measured faster).
  const bool ballot = rvec && E <= kWave;
  if (mask_bytes == 4) {
    if (ballot) MOE_MASK_BALLOT(4); else if (vec) MOE_MASK_COUNT(4, 4); else MOE_MASK_COUNT(4, 1);
  } else {
    if (ballot) MOE_MASK_BALLOT(1); else if (vec) MOE_MASK_COUNT(1, 4); else MOE_MASK_COUNT(1, 1);
  }
#undef MOE_MASK_BALLOT
#undef MOE_MASK_COUNT
  const bool fused = nb <= kFusedMaxBlocks;
  if (!fused)
    hipLaunchKernelGGL(rowmap_colscan_kernel, dim3(E), dim3(kScanThreads), 0, s, w.counts, nb,
                       E, w.totals);
#define MOE_MASK_WRITE(F, MB, VC)                                                              \
  hipLaunchKernelGGL((maskmap_write_kernel<F, MB, VC>), dim3(nb), dim3(kTokPerBlock), 0, s,     \
                     routing_map, w.masks, w.counts, w.totals, T, E, nb, num_out, map,         \
                     expert_offsets)
  if (mask_bytes == 4) {
    if (fused) { if (rvec) MOE_MASK_WRITE(true, 4, true); else MOE_MASK_WRITE(true, 4, false); }
    else { if (rvec) MOE_MASK_WRITE(false, 4, true); else MOE_MASK_WRITE(false, 4, false); }
  } else {
    if (fused) { if (rvec) MOE_MASK_WRITE(true, 1, true); else MOE_MASK_WRITE(true, 1, false); }
    else { if (rvec) MOE_MASK_WRITE(false, 1, true); else MOE_MASK_WRITE(false, 1, false); }
  }
#undef MOE_MASK_WRITE
  return hipGetLastError();
}

}  // namespace moe
