// Fused chunk sort-and-pad and unpad-and-restore (TransformerEngine PR "Fuse
// MoE chunk sorting and padding", Description, Changes and Diagram): the
// sort-and-pad is one launch that builds the map and copies (padded buffers
// up to MOE_FUSED_MAX_BYTES), or a map kernel and a pad copy; the restore is
// one copy kernel.
//
// Map.  Wave 0 of every map workgroup rebuilds the small chunk tables in LDS
// from the device-resident split sizes and chunk order -- input-order source
// offsets, sorted-order prefixes, padded group starts -- with wave scans (DPP
// row shifts and lane reads) and no workgroup barrier: after the metadata
// loads, three LDS round trips and three scans, about 1.5 us with the row
// searches.  The workgroup then writes its slice of the padded destination ->
// source row map by two binary searches per row.
// Every workgroup validates the metadata the same way; on bad metadata the
// whole map is -1 (so the copies write zeros) and workgroup 0 reports it.
//
// Fused.  Every workgroup builds the tables the same way, resolves the source
// rows of its slice of destination rows, and copies the slice (see
// pad_fused_kernel).
//
// Copies.  Both walk a flat index over (row, unit) with 16-byte units where
// the row allows, consecutive lanes on consecutive units, each lane's units
// (one in the pad copy, four in the restore) loaded before any is stored.
// The pad copy writes every destination row (zeros where the map is -1).
// The restore scatters every mapped row
// back to its source and writes zeros to the rows past the token total,
// which it sums from the split sizes on the device.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

// Build-time tuning: units in flight per lane, and the streaming policy of
// calls larger than kStreamBytes (bit 0: non-temporal loads, bit 1:
// non-temporal stores); for the one-launch sort-and-pad, the largest padded
// buffer it takes (bytes; larger ones get the map + copy pair), its units
// per lane per stage, and the workgroup count its rows per workgroup aim at.
#ifndef MOE_PAD_ILP
#define MOE_PAD_ILP 1
#endif
#ifndef MOE_RESTORE_ILP
#define MOE_RESTORE_ILP 4
#endif
#ifndef MOE_PAD_STREAM
#define MOE_PAD_STREAM 2
#endif
// The pad copy's policy when the call streams but its padded buffer alone
// fits the Infinity Cache: the buffer is kept (plain stores) for the kernel
// that reads it next, and the source rows are streamed instead.
#ifndef MOE_PAD_STREAM_FIT
#define MOE_PAD_STREAM_FIT 1
#endif
#ifndef MOE_RESTORE_STREAM
#define MOE_RESTORE_STREAM 1
#endif
#ifndef MOE_FUSED_MAX_BYTES
#define MOE_FUSED_MAX_BYTES (128ll << 20)
#endif
#ifndef MOE_FUSED_ILP
#define MOE_FUSED_ILP 2
#endif
#ifndef MOE_FUSED_WGS
#define MOE_FUSED_WGS 2048
#endif
#ifndef MOE_COPY_THREADS
#define MOE_COPY_THREADS 256
#endif
constexpr int kCopyThreads = MOE_COPY_THREADS;
constexpr int kPadIlp = MOE_PAD_ILP;
constexpr int kRestoreIlp = MOE_RESTORE_ILP;
constexpr int kFusedIlp = MOE_FUSED_ILP;
constexpr int kMapRows = 256;         // row_map entries per map workgroup (one per lane)

// Row / unit split of a flat unit index u over rows of W units without a
// hardware divide: q = floor(u / W) = (umulhi(m, u) + u) >> l, with
// l = ceil(log2 W) and m = floor(2^32 (2^l - W) / W) + 1 (Granlund and
// Montgomery, "Division by invariant integers using multiplication", the
// unsigned N-bit case), exact for every u < 2^32.  The host computes (m, l)
// and falls back to 64-bit division when the flat index can reach 2^32.
struct RowDiv {
  uint32_t m;
  int l;
  int64_t W;
};

inline RowDiv row_div(int64_t W) {
  int l = 0;
  while (((int64_t)1 << l) < W) l++;
  const uint64_t num = ((uint64_t)1 << 32) * (((uint64_t)1 << l) - (uint64_t)W);
  return RowDiv{(uint32_t)(num / (uint64_t)W + 1), l, W};
}

template <bool IDX64>
__device__ __forceinline__ void split_unit(int64_t u, const RowDiv &dv, int64_t &d, int64_t &c) {
  if constexpr (IDX64) {
    d = u / dv.W;
  } else {
    const uint32_t x = (uint32_t)u;
    d = (int64_t)(((uint64_t)__umulhi(dv.m, x) + x) >> dv.l);
  }
  c = u - d * dv.W;
}

// ----------------------------------------------------------- chunk tables --

// Tables in LDS.  int32 entries are exact whenever the metadata is valid
// (every prefix is at most the token total <= n_cap); padded starts are
// int64 because a large alignment can push them past int32 before the
// capacity check rejects them.
struct ChunkTables {
  int64_t *g_pad;    // [G+1] padded start of each group; g_pad[G] = padded total
  int32_t *qoff;     // [C+1] sorted-order prefix of chunk sizes
  int32_t *qsrc;     // [C]   first source row of the chunk at each sorted position
  int32_t *src_off;  // [C]   first source row of each input chunk
  int32_t *size;     // [C]   chunk sizes (input order)
  int32_t *inv;      // [C]   sorted position of each input chunk (permutation check)
};

inline size_t chunk_tables_bytes(int C, int G) {
  return (size_t)(G + 1) * sizeof(int64_t) + (size_t)(5 * C + 1) * sizeof(int32_t);
}

__device__ inline ChunkTables carve_tables(void *lds, int C, int G) {
  ChunkTables t;
  t.g_pad = reinterpret_cast<int64_t *>(lds);
  t.qoff = reinterpret_cast<int32_t *>(t.g_pad + G + 1);
  t.qsrc = t.qoff + C + 1;
  t.src_off = t.qsrc + C;
  t.size = t.src_off + C;
  t.inv = t.size + C;
  return t;
}

// Chunks (and groups) per lane of the table build, a compile-time bound so
// that a lane's entries live in registers: 4 up to 256 chunks, 32 up to
// MOE_MAX_CHUNKS.
constexpr int kPerSmall = 4;
constexpr int kPerLarge = 32;
static_assert(kWave * kPerLarge >= MOE_MAX_CHUNKS, "table build covers every chunk count");
inline int table_per(int C) { return C <= kWave * kPerSmall ? kPerSmall : kPerLarge; }

// Lane l - S of the same 16-lane row (DPP row_shr:S), or 0 when that lane is
// in an earlier row.  Needs every lane of the wave active.
template <int S>
__device__ __forceinline__ int64_t row_shr64(int64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, 0x110 + S, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), 0x110 + S, 0xF, 0xF,
                                             false);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

__device__ __forceinline__ int64_t readlane64(int64_t v, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Exclusive scan across the 64 lanes of one wave (all active); *total gets
// the sum.  A scan inside each 16-lane row by DPP row shifts (1, 2, 4, 8),
// then the totals of the earlier rows (lanes 15, 31, 47) added: DPP moves
// and four lane reads instead of a chain of cross-lane permutes through LDS.
__device__ __forceinline__ int64_t wave_exclusive_scan(int64_t v, int64_t *total) {
  const int row = (threadIdx.x & (kWave - 1)) >> 4;
  int64_t incl = v;
  incl += row_shr64<1>(incl);
  incl += row_shr64<2>(incl);
  incl += row_shr64<4>(incl);
  incl += row_shr64<8>(incl);
  const int64_t r0 = readlane64(incl, 15), r1 = readlane64(incl, 31);
  const int64_t r2 = readlane64(incl, 47), r3 = readlane64(incl, 63);
  incl += (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
  *total = r0 + r1 + r2 + r3;
  return incl - v;
}

// OR of v over the wave (all lanes active).  Status bits are almost always
// zero, which one ballot shows; otherwise a butterfly of cross-lane permutes.
__device__ __forceinline__ int wave_or(int v) {
  if (__ballot(v != 0) == 0ull) return 0;
#pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) v |= __shfl_xor(v, d, kWave);
  return v;
}

// Built by ONE wave (call from all 64 lanes of wave 0): lane l owns the
// contiguous chunks [l * per, (l + 1) * per) (per <= PER), held in registers;
// scans run across lanes (DPP), and lanes exchange entries through LDS
// ordered by wave-level fences -- no workgroup barrier inside.  The order is
// checked to be a permutation by scattering each sorted position to its
// input chunk and reading it back: a repeated chunk leaves one of its
// positions overwritten.  Each step issues all its memory operations before
// using any, so the build is one global round trip and three LDS round
// trips.  Returns the device status bits (the same value in every lane);
// non-zero means the tables must not be used.
template <int PER>
__device__ int build_chunk_tables_wave(const int32_t *__restrict__ split_sizes,
                                       const int32_t *__restrict__ sorted_idx, int C, int R,
                                       int A, int n_cap, int out_cap, const ChunkTables &t) {
  const int G = C / R;
  const int lane = threadIdx.x & (kWave - 1);
  const int per = (C + kWave - 1) / kWave;
  const int c0 = min(C, lane * per), c1 = min(C, c0 + per);
  int sz[PER], od[PER];
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const int c = min(c0 + i, C - 1);
    sz[i] = split_sizes[c];
    od[i] = sorted_idx[c];
  }
  int bad = 0;
  int64_t seg = 0;
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const bool in = c0 + i < c1;
    const int s = in ? sz[i] : 0, o = in ? od[i] : 0;
    if (s < 0) bad |= MOE_DEV_BAD_CHUNKS;
    if (s > n_cap) bad |= MOE_DEV_OVERFLOW;
    if ((unsigned)o >= (unsigned)C) bad |= MOE_DEV_BAD_CHUNKS;
    sz[i] = max(s, 0);
    od[i] = (unsigned)o < (unsigned)C ? o : 0;
    seg += sz[i];
  }
  // Source offsets: exclusive scan of the sizes in input order.
  int64_t n_act;
  int64_t run = wave_exclusive_scan(seg, &n_act);
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const int c = c0 + i;  // as an input chunk, and as a sorted position
    if (c < c1) {
      t.size[c] = sz[i];
      t.src_off[c] = (int32_t)min(run, (int64_t)INT32_MAX);
      t.inv[od[i]] = c;
    }
    run += sz[i];
  }
  __syncwarp();
  // Per sorted position: its chunk's size and source start, and the check.
  int ssz[PER], qs[PER];
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const int q = c0 + i;
    const int back = t.inv[od[i]];
    ssz[i] = t.size[od[i]];
    qs[i] = t.src_off[od[i]];
    if (q < c1 && back != q) bad |= MOE_DEV_BAD_CHUNKS;
  }
  bad = wave_or(bad);
  if (n_act > n_cap) bad |= MOE_DEV_OVERFLOW;
  // Sorted-order prefix of the sizes (all zero when the metadata is bad).
  int64_t sseg = 0;
#pragma unroll
  for (int i = 0; i < PER; i++) {
    ssz[i] = (c0 + i < c1 && !bad) ? ssz[i] : 0;
    sseg += ssz[i];
  }
  int64_t stot;
  run = wave_exclusive_scan(sseg, &stot);
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const int q = c0 + i;
    if (q < c1) {
      t.qoff[q] = (int32_t)min(run, (int64_t)INT32_MAX);
      t.qsrc[q] = qs[i];
    }
    run += ssz[i];
  }
  if (lane == kWave - 1) t.qoff[C] = (int32_t)min(stot, (int64_t)INT32_MAX);
  __syncwarp();
  // Groups: padded lengths, then their exclusive scan (G <= C, so a lane
  // owns at most PER groups).
  const int perg = (G + kWave - 1) / kWave;
  const int g0 = min(G, lane * perg), g1 = min(G, g0 + perg);
  int64_t gp[PER];
  int64_t gseg = 0;
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const int g = min(g0 + i, G - 1);
    // n and A are non-negative int32 (qoff never decreases), so n + A - 1
    // fits 32 unsigned bits and the division needs no 64-bit routine
    const uint32_t n = (uint32_t)(t.qoff[(g + 1) * R] - t.qoff[g * R]);
    gp[i] = g0 + i < g1 ? (int64_t)((n + (uint32_t)A - 1u) / (uint32_t)A) * A : 0;
    gseg += gp[i];
  }
  int64_t pad_total;
  run = wave_exclusive_scan(gseg, &pad_total);
#pragma unroll
  for (int i = 0; i < PER; i++) {
    if (g0 + i < g1) t.g_pad[g0 + i] = run;
    run += gp[i];
  }
  if (lane == kWave - 1) t.g_pad[G] = pad_total;
  if (pad_total > out_cap) bad |= MOE_DEV_OVERFLOW;
  __syncwarp();
  return bad;
}

// Last index i in [lo, hi) with a[i] <= x, for non-decreasing a (a[lo] <= x).
template <typename T>
__device__ __forceinline__ int last_le(const T *a, int lo, int hi, int64_t x) {
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)a[mid] <= x)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// Source row of padded destination row d, or -1 for padding / tail rows.
__device__ __forceinline__ int32_t chunk_src_row(const ChunkTables &t, int G, int R, int64_t d) {
  if (d >= t.g_pad[G]) return -1;
  const int g = last_le(t.g_pad, 0, G, d);
  const int64_t local = d - t.g_pad[g];
  const int32_t gs = t.qoff[g * R];
  if (local >= (int64_t)t.qoff[(g + 1) * R] - gs) return -1;
  const int64_t u = gs + local;  // position in the sorted token order
  const int q = last_le(t.qoff, g * R, (g + 1) * R, u);
  return (int32_t)(t.qsrc[q] + (u - t.qoff[q]));
}

__device__ __forceinline__ void copy_prob(const uint8_t *src, int64_t si, uint8_t *dst,
                                          int64_t di, int prob_bytes) {
  if (prob_bytes == 4)
    reinterpret_cast<uint32_t *>(dst)[di] =
        si >= 0 ? reinterpret_cast<const uint32_t *>(src)[si] : 0u;
  else
    reinterpret_cast<uint16_t *>(dst)[di] =
        si >= 0 ? reinterpret_cast<const uint16_t *>(src)[si] : (uint16_t)0;
}

// --------------------------------------------------------------- the map --

// Grid ceil(out_cap / kMapRows): wave 0 of every workgroup builds the tables,
// then all lanes write the workgroup's slice of row_map.
template <int PER>
__global__ __launch_bounds__(kCopyThreads) void chunk_map_kernel(
    const int32_t *__restrict__ split_sizes, const int32_t *__restrict__ sorted_idx, int C, int R,
    int A, int n_cap, int out_cap, int32_t *__restrict__ row_map,
    int32_t *__restrict__ padded_offsets, int32_t *__restrict__ dev_status) {
  extern __shared__ int64_t lds[];
  __shared__ int bad_s;
  const int G = C / R;
  const ChunkTables t = carve_tables(lds, C, G);
  if (threadIdx.x < kWave) {
    const int bad =
        build_chunk_tables_wave<PER>(split_sizes, sorted_idx, C, R, A, n_cap, out_cap, t);
    if (threadIdx.x == 0) bad_s = bad;
  }
  __syncthreads();
  const int bad = bad_s;
  if (blockIdx.x == 0) {
    if (threadIdx.x == 0) report(dev_status, bad);
    for (int g = threadIdx.x; g <= G; g += kCopyThreads)
      padded_offsets[g] = bad ? 0 : (int32_t)t.g_pad[g];
  }
  const int64_t d0 = (int64_t)blockIdx.x * kMapRows;
  const int64_t d1 = min((int64_t)out_cap, d0 + kMapRows);
  for (int64_t d = d0 + threadIdx.x; d < d1; d += kCopyThreads)
    row_map[d] = bad ? -1 : chunk_src_row(t, G, R, d);
}

// Pad copy driven by the row map: out[d] = in[row_map[d]] or zeros.
// NTL / NTS: stream the source / the (dense, sequential) destination rows.
template <typename U, bool NTL, bool NTS, bool IDX64>
__global__ __launch_bounds__(kCopyThreads) void pad_copy_kernel(
    const U *__restrict__ in, const uint8_t *__restrict__ probs, int prob_bytes, RowDiv dv,
    int n_cap, const int32_t *__restrict__ row_map, int out_cap, U *__restrict__ out,
    uint8_t *__restrict__ out_probs, int32_t *__restrict__ dev_status) {
  const int64_t W = dv.W;
  const int64_t total = (int64_t)out_cap * W;
  const int64_t base0 = spill_block() * kCopyThreads * kPadIlp;
  if (base0 >= total) return;  // a workgroup past the end
  const int64_t base = base0 + threadIdx.x;
  U v[kPadIlp];
  int bad = 0;
#pragma unroll
  for (int i = 0; i < kPadIlp; i++) {
    const int64_t u = base + (int64_t)i * kCopyThreads;
    v[i] = zero_unit<U>();
    if (u < total) {
      int64_t d, c;
      split_unit<IDX64>(u, dv, d, c);
      int64_t s = row_map[d];
      if (s >= n_cap) {
        bad |= MOE_DEV_BAD_ROW;
        s = -1;
      }
      if (s >= 0) v[i] = ld_row<NTL>(in + s * W + c);
      if (c == 0 && out_probs != nullptr) copy_prob(probs, s, out_probs, d, prob_bytes);
    }
  }
#pragma unroll
  for (int i = 0; i < kPadIlp; i++) {
    const int64_t u = base + (int64_t)i * kCopyThreads;
    if (u < total) st_row<NTS>(v[i], out + u);
  }
  report(dev_status, bad);
}

// Buffer accesses: the descriptor holds a base and a length in bytes, and
// the hardware drops a store, and returns zero for a load, whose offset is
// past the length -- a tail lane or a padding row needs no branch and no
// select on loaded data.  Descriptor word 3 is the gfx9 data format field
// (32-bit data) that raw buffer accesses expect.
constexpr int kBufWord3 = 0x00020000;
constexpr uint32_t kNoRow = 0xFFFFFFF0u;  // an offset past every descriptor's length
constexpr int64_t kMaxBufBytes = kNoRow;  // lengths stay at or below it

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, kBufWord3);
}

template <bool NT, typename U>
__device__ __forceinline__ U buf_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  constexpr int aux = NT ? 2 : 0;
  if constexpr (sizeof(U) == 16)
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, aux);
  else if constexpr (sizeof(U) == 4)
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, aux);
  else
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, aux);
}

template <bool NT>
__device__ __forceinline__ void buf_store(v4u v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, NT ? 2 : 0);
}
template <bool NT>
__device__ __forceinline__ void buf_store(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, NT ? 2 : 0);
}
template <bool NT>
__device__ __forceinline__ void buf_store(uint16_t v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, NT ? 2 : 0);
}

// Map and pad copy in one launch, for calls small enough that the saved
// launch outweighs rebuilding the tables in every workgroup.  Workgroup b
// owns destination rows [b * rows_per, (b + 1) * rows_per), rows_per <=
// kWave: wave 0 builds the tables, resolves the slice's source rows into LDS
// (writing them to row_map and copying their probs), and after one barrier
// the whole workgroup copies the slice's units in stages of kFusedIlp units
// per lane.  The loads of stage j + 1 are issued before the stores of stage
// j, and every access is unconditional (a tail lane re-reads the slice's last
// unit and stores past the slice, a padding row loads zeros through an
// offset past the source), so the wait for a stage's loads never waits for
// the stores issued just before them.  Workgroup 0 also writes
// padded_offsets and reports bad metadata.  Needs a slice shorter than 2^31
// bytes and a source of at most kMaxBufBytes.
template <typename U, bool NTL, bool NTS, int PER>
__global__ __launch_bounds__(kCopyThreads) void pad_fused_kernel(
    const U *__restrict__ in, const uint8_t *__restrict__ probs, int prob_bytes, RowDiv dv,
    const int32_t *__restrict__ split_sizes, const int32_t *__restrict__ sorted_idx, int C, int R,
    int A, int n_cap, int out_cap, int rows_per, U *__restrict__ out,
    uint8_t *__restrict__ out_probs, int32_t *__restrict__ row_map,
    int32_t *__restrict__ padded_offsets, int32_t *__restrict__ dev_status) {
  extern __shared__ int64_t lds[];
  __shared__ int32_t s_src[kWave];
  const int G = C / R;
  const ChunkTables t = carve_tables(lds, C, G);
  const int64_t blk = spill_block();
  const int64_t d0 = blk * rows_per;
  const int n_rows = (int)max((int64_t)0, min((int64_t)rows_per, (int64_t)out_cap - d0));
  if (threadIdx.x < kWave) {
    const int bad =
        build_chunk_tables_wave<PER>(split_sizes, sorted_idx, C, R, A, n_cap, out_cap, t);
    if (blk == 0) {
      if (threadIdx.x == 0) report(dev_status, bad);
      for (int g = threadIdx.x; g <= G; g += kWave) padded_offsets[g] = bad ? 0 : (int32_t)t.g_pad[g];
    }
    if ((int)threadIdx.x < n_rows) {
      const int64_t d = d0 + threadIdx.x;
      const int32_t s = bad ? -1 : chunk_src_row(t, G, R, d);
      s_src[threadIdx.x] = s;
      row_map[d] = s;
      if (out_probs != nullptr) copy_prob(probs, s, out_probs, d, prob_bytes);
    }
  }
  __syncthreads();
  const int64_t W = dv.W;
  const int n_units = (int)(n_rows * W);
  if (n_units == 0) return;
  constexpr int kStep = kCopyThreads * kFusedIlp;
  const int n_stages = (n_units + kStep - 1) / kStep;
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t src = slice_rsrc(const_cast<U *>(in),
                                                (uint32_t)((int64_t)n_cap * W * sizeof(U)));
  const __amdgpu_buffer_rsrc_t dst = slice_rsrc(out + d0 * W, (uint32_t)n_units * sizeof(U));
  auto load_stage = [&](int j, U (&w)[kFusedIlp]) {
#pragma unroll
    for (int i = 0; i < kFusedIlp; i++) {
      const int u = min(j * kStep + i * kCopyThreads + tid, n_units - 1);
      int64_t r, c;
      split_unit<false>(u, dv, r, c);
      const int32_t s = s_src[r];
      const uint32_t off = s >= 0 ? (uint32_t)(((int64_t)s * W + c) * sizeof(U)) : kNoRow;
      w[i] = buf_load<NTL, U>(src, off);
    }
  };
  auto store_stage = [&](int j, const U (&w)[kFusedIlp]) {
#pragma unroll
    for (int i = 0; i < kFusedIlp; i++)
      buf_store<NTS>(w[i], dst, (uint32_t)(j * kStep + i * kCopyThreads + tid) * sizeof(U));
  };
  // Two register sets, two stages per trip: no copy between them, so no
  // wait on loads just issued.  A stage index past the last one stores
  // nothing (every offset is past the slice).
  U va[kFusedIlp], vb[kFusedIlp];
  load_stage(0, va);
  // Dropped stores, held after the first loads by the compiler fence, so
  // that entering the loop, as on every later trip, kFusedIlp stores sit
  // between one stage's loads and the next stage's: the wait at the loop
  // head then does not cover the stores issued just before the back edge.
  asm volatile("" ::: "memory");
  U zero[kFusedIlp];
#pragma unroll
  for (int i = 0; i < kFusedIlp; i++) zero[i] = zero_unit<U>();
  store_stage(n_stages + 1, zero);
  int j = 0;
  do {  // n_stages >= 1: no zero-trip branch for the first loads to sink past
    load_stage(min(j + 1, n_stages - 1), vb);
    store_stage(j, va);
    load_stage(min(j + 2, n_stages - 1), va);
    store_stage(j + 1, vb);
    j += 2;
  } while (j < n_stages);
}

// --------------------------------------------------------------- restore --

// Token total of the chunk metadata, summed by one wave (every lane gets it;
// all lanes of the wave active).
__device__ __forceinline__ int64_t wave_total(const int32_t *__restrict__ sizes, int C) {
  const int lane = threadIdx.x & (kWave - 1);
  int64_t s = 0;
  for (int i = lane; i < C; i += kWave) s += sizes[i];
  int64_t total;
  wave_exclusive_scan(s, &total);
  return total;
}

// Flat index over [0, max(out_cap, n_cap)) x W: unit (d, c) scatters padded
// row d (if mapped) and zero-fills restored row d (if past the token total).
// NTL / NTS: stream the (dense, sequential) padded source rows / the
// restored rows.
// A workgroup's units are one contiguous range, so the map entries, padded
// rows and probs it reads are slices, read through range-checked buffer
// descriptors: a lane loads all its map entries, then all its rows and
// probs (an unmapped unit's offset lies past the slice, and its load returns
// zero without touching memory), and stores only after that.  With the row
// loads under a branch on the map entry, each lane waited for one unit's
// row before the next unit's map entry arrived (the vector memory counter
// retires in issue order), one row in flight per lane.  PB: bytes per prob
// (2 or 4; a compile-time width keeps the prob loads branch-free too).
template <typename U, int PB, bool NTL, bool NTS, bool IDX64>
__global__ __launch_bounds__(kCopyThreads) void restore_copy_kernel(
    const U *__restrict__ in, const uint8_t *__restrict__ probs, RowDiv dv,
    const int32_t *__restrict__ row_map, const int32_t *__restrict__ split_sizes, int C,
    int out_cap, int n_cap, U *__restrict__ out, uint8_t *__restrict__ out_probs,
    int32_t *__restrict__ dev_status) {
  constexpr int kSpan = kCopyThreads * kRestoreIlp;
  const int64_t W = dv.W;
  const int64_t rows = max(out_cap, n_cap);
  const int64_t total = rows * W;
  const int64_t base0 = spill_block() * kSpan;
  if (base0 >= total) return;  // a workgroup past the end
  // Slices: padded rows [d_first, d_end) of row_map and probs, units
  // [base0, base0 + n_in) of in; each at most kSpan entries.
  int64_t d_first, d_last, c_unused;
  split_unit<IDX64>(base0, dv, d_first, c_unused);
  split_unit<IDX64>(min(total, base0 + kSpan) - 1, dv, d_last, c_unused);
  const int64_t d_end = min((int64_t)out_cap, d_last + 1);
  const int64_t n_map = max((int64_t)0, d_end - d_first);
  const int64_t n_in = max((int64_t)0, min((int64_t)out_cap * W, base0 + kSpan) - base0);
  const bool with_probs = out_probs != nullptr;
  // an empty slice (nothing of it is read) still gets a valid base address
  void *const any = const_cast<int32_t *>(split_sizes);
  const __amdgpu_buffer_rsrc_t map_r = slice_rsrc(
      n_map > 0 ? (void *)(const_cast<int32_t *>(row_map) + d_first) : any, (uint32_t)(n_map * 4));
  const __amdgpu_buffer_rsrc_t in_r = slice_rsrc(
      n_in > 0 ? (void *)(const_cast<U *>(in) + base0) : any, (uint32_t)(n_in * sizeof(U)));
  const bool prob_slice = with_probs && n_map > 0;
  const __amdgpu_buffer_rsrc_t prob_r =
      slice_rsrc(prob_slice ? (void *)(const_cast<uint8_t *>(probs) + d_first * PB) : any,
                 prob_slice ? (uint32_t)(n_map * PB) : 0u);
  const int tid = threadIdx.x;
  int64_t d[kRestoreIlp], c[kRestoreIlp];
  int32_t s[kRestoreIlp];
#pragma unroll
  for (int i = 0; i < kRestoreIlp; i++) {
    split_unit<IDX64>(base0 + tid + i * kCopyThreads, dv, d[i], c[i]);
    const uint32_t off = d[i] < d_end ? (uint32_t)((d[i] - d_first) * 4) : kNoRow;
    s[i] = (int32_t)buf_load<false, uint32_t>(map_r, off);
  }
  U v[kRestoreIlp];
  uint32_t pv[kRestoreIlp];
  int bad = 0;
#pragma unroll
  for (int i = 0; i < kRestoreIlp; i++) {
    const int32_t si = d[i] < d_end ? s[i] : -1;
    if (si >= n_cap) bad |= MOE_DEV_BAD_ROW;
    const bool mapped = si >= 0 && si < n_cap;
    s[i] = mapped ? si : -1;
    const uint32_t off = mapped ? (uint32_t)((tid + i * kCopyThreads) * sizeof(U)) : kNoRow;
    v[i] = buf_load<NTL, U>(in_r, off);
    const uint32_t poff = mapped && c[i] == 0 ? (uint32_t)((d[i] - d_first) * PB) : kNoRow;
    if constexpr (PB == 4)
      pv[i] = buf_load<false, uint32_t>(prob_r, poff);
    else
      pv[i] = buf_load<false, uint16_t>(prob_r, poff);
  }
  const int64_t n_act = wave_total(split_sizes, C);
  if (n_act > n_cap) bad |= MOE_DEV_OVERFLOW;
#pragma unroll
  for (int i = 0; i < kRestoreIlp; i++) {
    // An entry at or past the token total (a map saved for other split
    // sizes) would race the zero tail for its row: it is dropped and
    // reported.  The row's load above was harmless (the unit's own slice).
    if (s[i] >= n_act) {
      bad |= MOE_DEV_BAD_ROW;
      s[i] = -1;
    }
    if (s[i] >= 0) {
      st_row<NTS>(v[i], out + (int64_t)s[i] * W + c[i]);
      if (c[i] == 0 && with_probs) {
        if constexpr (PB == 4)
          reinterpret_cast<uint32_t *>(out_probs)[s[i]] = pv[i];
        else
          reinterpret_cast<uint16_t *>(out_probs)[s[i]] = (uint16_t)pv[i];
      }
    }
    if (d[i] >= n_act && d[i] < n_cap) {  // then the unit is below total
      st_row<NTS>(zero_unit<U>(), out + d[i] * W + c[i]);
      if (c[i] == 0 && with_probs) copy_prob(probs, -1, out_probs, d[i], PB);
    }
  }
  report(dev_status, bad);
}

inline int64_t copy_blocks(int64_t units, int ilp) {
  const int64_t per = (int64_t)kCopyThreads * ilp;
  return (units + per - 1) / per;
}

}  // namespace

hipError_t launch_chunk_map(const int32_t *split_sizes, const int32_t *sorted_idx, int C, int R,
                            int A, int n_cap, int out_cap, int32_t *row_map,
                            int32_t *padded_offsets, int32_t *dev_status, hipStream_t s) {
  const int G = C / R;
  const size_t lds = chunk_tables_bytes(C, G);
  const int blocks = out_cap > 0 ? (int)(((int64_t)out_cap + kMapRows - 1) / kMapRows) : 1;
  if (table_per(C) == kPerSmall)
    hipLaunchKernelGGL(chunk_map_kernel<kPerSmall>, dim3(blocks), dim3(kCopyThreads), lds, s,
                       split_sizes, sorted_idx, C, R, A, n_cap, out_cap, row_map, padded_offsets,
                       dev_status);
  else
    hipLaunchKernelGGL(chunk_map_kernel<kPerLarge>, dim3(blocks), dim3(kCopyThreads), lds, s,
                       split_sizes, sorted_idx, C, R, A, n_cap, out_cap, row_map, padded_offsets,
                       dev_status);
  return hipGetLastError();
}

hipError_t launch_pad_copy(const void *in, const void *probs, int prob_bytes, int unit_bytes,
                           int64_t row_units, int n_cap, const int32_t *row_map, int out_cap,
                           void *out, void *out_probs, int32_t *dev_status, hipStream_t s) {
  const int64_t units = (int64_t)out_cap * row_units;
  if (units == 0) return hipSuccess;
  const int64_t blocks = copy_blocks(units, kPadIlp);
  const dim3 grid = spill_grid(blocks), block(kCopyThreads);
  const auto *pp = static_cast<const uint8_t *>(probs);
  auto *op = static_cast<uint8_t *>(out_probs);
  // The call streams when its traffic (about twice the padded buffer) passes
  // the Infinity Cache.  Measured at 32768 tokens x 2048 (143 MB padded):
  // streaming the source reads and keeping the buffer cached gives the pad +
  // restore roundtrip 91.9 us warm and 92.3 cold, against 89.7 and 96.3 with
  // non-temporal stores; at 131072 tokens (570 MB padded) the stores stream
  // (366 / 336 against 373 / 350).
  const int64_t out_bytes = units * unit_bytes;
  const bool stream = out_bytes * 2 > kStreamBytes;
  const RowDiv dv = row_div(row_units);
  // flat indices of the last workgroup stay below 2^32 on the fast path
  const bool idx64 = blocks * kCopyThreads * kPadIlp >= ((int64_t)1 << 32);
#define MOE_PAD(UT, NTL, NTS)                                                                  \
  do {                                                                                         \
    if (idx64)                                                                                 \
      hipLaunchKernelGGL((pad_copy_kernel<UT, NTL, NTS, true>), grid, block, 0, s,             \
                         static_cast<const UT *>(in), pp, prob_bytes, dv, n_cap, row_map,      \
                         out_cap, static_cast<UT *>(out), op, dev_status);                     \
    else                                                                                       \
      hipLaunchKernelGGL((pad_copy_kernel<UT, NTL, NTS, false>), grid, block, 0, s,            \
                         static_cast<const UT *>(in), pp, prob_bytes, dv, n_cap, row_map,      \
                         out_cap, static_cast<UT *>(out), op, dev_status);                     \
  } while (0)
  switch (unit_bytes) {
    case 16:
      if (stream && out_bytes > kStreamBytes)
        MOE_PAD(v4u, (MOE_PAD_STREAM & 1) != 0, (MOE_PAD_STREAM & 2) != 0);
      else if (stream)
        MOE_PAD(v4u, (MOE_PAD_STREAM_FIT & 1) != 0, (MOE_PAD_STREAM_FIT & 2) != 0);
      else
        MOE_PAD(v4u, false, false);
      break;
    case 4: MOE_PAD(uint32_t, false, false); break;
    default: MOE_PAD(uint16_t, false, false); break;
  }
#undef MOE_PAD
  return hipGetLastError();
}

hipError_t launch_restore_copy(const void *in, const void *probs, int prob_bytes, int unit_bytes,
                               int64_t row_units, const int32_t *row_map,
                               const int32_t *split_sizes, int C, int out_cap, int n_cap,
                               void *out, void *out_probs, int32_t *dev_status, hipStream_t s) {
  const int64_t units = (int64_t)(out_cap > n_cap ? out_cap : n_cap) * row_units;
  if (units == 0) return hipSuccess;
  const int64_t blocks = copy_blocks(units, kRestoreIlp);
  const dim3 grid = spill_grid(blocks), block(kCopyThreads);
  const auto *pp = static_cast<const uint8_t *>(probs);
  auto *op = static_cast<uint8_t *>(out_probs);
  const bool stream = ((int64_t)out_cap + n_cap) * row_units * unit_bytes > kStreamBytes;
  const RowDiv dv = row_div(row_units);
  const bool idx64 = blocks * kCopyThreads * kRestoreIlp >= ((int64_t)1 << 32);
  // without probs nothing reads or writes them, whatever the width
  const bool half_probs = out_probs != nullptr && prob_bytes == 2;
#define MOE_RESTORE_PB(UT, PB, NTL, NTS)                                                       \
  do {                                                                                         \
    if (idx64)                                                                                 \
      hipLaunchKernelGGL((restore_copy_kernel<UT, PB, NTL, NTS, true>), grid, block, 0, s,     \
                         static_cast<const UT *>(in), pp, dv, row_map, split_sizes, C,         \
                         out_cap, n_cap, static_cast<UT *>(out), op, dev_status);              \
    else                                                                                       \
      hipLaunchKernelGGL((restore_copy_kernel<UT, PB, NTL, NTS, false>), grid, block, 0, s,    \
                         static_cast<const UT *>(in), pp, dv, row_map, split_sizes, C,         \
                         out_cap, n_cap, static_cast<UT *>(out), op, dev_status);              \
  } while (0)
#define MOE_RESTORE(UT, NTL, NTS)                                                              \
  do {                                                                                         \
    if (half_probs)                                                                            \
      MOE_RESTORE_PB(UT, 2, NTL, NTS);                                                         \
    else                                                                                       \
      MOE_RESTORE_PB(UT, 4, NTL, NTS);                                                         \
  } while (0)
  switch (unit_bytes) {
    case 16:
      if (stream)
        MOE_RESTORE(v4u, (MOE_RESTORE_STREAM & 1) != 0, (MOE_RESTORE_STREAM & 2) != 0);
      else
        MOE_RESTORE(v4u, false, false);
      break;
    case 4: MOE_RESTORE(uint32_t, false, false); break;
    default: MOE_RESTORE(uint16_t, false, false); break;
  }
#undef MOE_RESTORE_PB
#undef MOE_RESTORE
  return hipGetLastError();
}

hipError_t launch_sort_and_pad(const void *in, const void *probs, int prob_bytes, int unit_bytes,
                               int64_t row_units, const int32_t *split_sizes,
                               const int32_t *sorted_idx, int C, int R, int A, int n_cap,
                               int out_cap, void *out, void *out_probs, int32_t *row_map,
                               int32_t *padded_offsets, int32_t *dev_status, hipStream_t s) {
  const int G = C / R;
  // rows per workgroup: enough workgroups to fill the chip once, at most one
  // row per lane of wave 0
  const int64_t want = ((int64_t)out_cap + MOE_FUSED_WGS - 1) / MOE_FUSED_WGS;
  const int rows_per = (int)std::min<int64_t>(kWave, std::max<int64_t>(1, want));
  // fused only for a small destination, whose copy is short next to a
  // launch; the fused copy addresses the source and a workgroup's slice with
  // 32-bit byte offsets
  const int64_t out_bytes = (int64_t)out_cap * row_units * unit_bytes;
  const bool fits = (int64_t)n_cap * row_units * unit_bytes <= kMaxBufBytes &&
                    ((int64_t)rows_per + 2) * row_units * unit_bytes +
                            (int64_t)kCopyThreads * kFusedIlp * unit_bytes * 2 <
                        ((int64_t)1 << 31);
  if (out_bytes > (int64_t)MOE_FUSED_MAX_BYTES || !fits) {
    const hipError_t e = launch_chunk_map(split_sizes, sorted_idx, C, R, A, n_cap, out_cap,
                                          row_map, padded_offsets, dev_status, s);
    if (e != hipSuccess) return e;
    return launch_pad_copy(in, probs, prob_bytes, unit_bytes, row_units, n_cap, row_map, out_cap,
                           out, out_probs, dev_status, s);
  }
  const size_t lds = chunk_tables_bytes(C, G);
  const int64_t blocks = out_cap > 0 ? ((int64_t)out_cap + rows_per - 1) / rows_per : 1;
  const dim3 grid = spill_grid(blocks), block(kCopyThreads);
  const auto *pp = static_cast<const uint8_t *>(probs);
  auto *op = static_cast<uint8_t *>(out_probs);
  const bool stream = (int64_t)out_cap * row_units * unit_bytes * 2 > kStreamBytes;
  const RowDiv dv = row_div(row_units);
#define MOE_FUSED_P(UT, NTL, NTS, PER)                                                         \
  hipLaunchKernelGGL((pad_fused_kernel<UT, NTL, NTS, PER>), grid, block, lds, s,               \
                     static_cast<const UT *>(in), pp, prob_bytes, dv, split_sizes, sorted_idx, C, \
                     R, A, n_cap, out_cap, rows_per, static_cast<UT *>(out), op, row_map,      \
                     padded_offsets, dev_status)
#define MOE_FUSED(UT, NTL, NTS)                                                                \
  do {                                                                                         \
    if (table_per(C) == kPerSmall)                                                             \
      MOE_FUSED_P(UT, NTL, NTS, kPerSmall);                                                    \
    else                                                                                       \
      MOE_FUSED_P(UT, NTL, NTS, kPerLarge);                                                    \
  } while (0)
  switch (unit_bytes) {
    case 16:
      if (stream)
        MOE_FUSED(v4u, (MOE_PAD_STREAM & 1) != 0, (MOE_PAD_STREAM & 2) != 0);
      else
        MOE_FUSED(v4u, false, false);
      break;
    case 4: MOE_FUSED(uint32_t, false, false); break;
    default: MOE_FUSED(uint16_t, false, false); break;
  }
#undef MOE_FUSED
#undef MOE_FUSED_P
  return hipGetLastError();
}

}  // namespace moe
