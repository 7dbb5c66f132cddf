// Device helpers shared by the gfx950 kernels of the MoE permute library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"
#include "moe_perm.h"

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

// A dispatch packet counts its grid in work-items, 32 bits per dimension, so
// gridDim.x * blockDim.x must stay below 2^32 (beyond it the grid is silently
// cut short).  Launches of many workgroups therefore spill into gridDim.z:
// the workgroup index is x + gridDim.x * z, and the last z-slab may hold
// workgroups past the end, which return at once.
constexpr unsigned kMaxGridX = 1u << 20;

inline dim3 spill_grid(int64_t blocks, unsigned y = 1) {
  if (blocks < 1) blocks = 1;
  const unsigned x = (unsigned)(blocks < (int64_t)kMaxGridX ? blocks : (int64_t)kMaxGridX);
  return dim3(x, y, (unsigned)((blocks + x - 1) / x));
}

__device__ __forceinline__ int64_t spill_block() {
  return (int64_t)blockIdx.x + (int64_t)gridDim.x * blockIdx.z;
}

// 16 bytes as a native clang vector (the non-temporal builtins need one).
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Cache policy of a bulk row access: plain, or non-temporal (streamed past
// the caches).  Each row byte is read once or written once per call.
template <bool NT, typename U> __device__ __forceinline__ U ld_row(const U *p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT, typename U> __device__ __forceinline__ void st_row(U v, U *p) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// A call that moves more bytes than the MI355X Infinity Cache (256 MiB)
// holds streams its rows; a smaller call keeps plain accesses so the next
// call on the same buffers can still hit the cache.  Which accesses of a
// kernel stream (loads, stores or both) was measured per kernel and is set
// beside each kernel's launcher.
#ifndef MOE_STREAM_MIB
#define MOE_STREAM_MIB 256
#endif
constexpr int64_t kStreamBytes = (int64_t)MOE_STREAM_MIB << 20;

// Source-row prefetch of the streaming row scatters (the permutes).  When a
// call's rows do not fit the Infinity Cache, the row a workgroup copies comes
// from HBM while the rest of the chip streams its stores out, and every store
// of the workgroup waits for that read.  So each workgroup also reads one
// 16-byte piece of every 128-byte line of the row `ahead` tokens later; by
// the time that row's own workgroup starts, its lines are cached.  The
// distance is two dispatch rounds: twice the tokens the chip holds at once
// (256 CUs, 32 wave slots each, one token per workgroup), a multiple of 8, so
// under the round-robin dispatch over the 8 XCDs both workgroups run on the
// same XCD.  Measured on the 16384 x 7168 bf16 permute (7-wave workgroups,
// 2048 tokens ahead) with cold caches: 385 us against 420 (issued after the
// workgroup's stores), the same warm time; 1024 to 4096 ahead within 1%.
// The FP8 rows of the same size (4-wave workgroups) were slower with it at
// every distance, so the scaled permute goes without.  The lanes that issue
// the reads matter as well: the lanes whose own units start a line (8 per
// wave, in every wave) give the gain, while one read per lane on lanes
// 0..111 (64 lines per instruction) gave none.
constexpr int kNumCUs = 256;
constexpr int kWaveSlotsPerCU = 32;
inline int prefetch_ahead(int threads) {
  const int waves = (threads + kWave - 1) / kWave;
  const int per_cu = kWaveSlotsPerCU / waves > 0 ? kWaveSlotsPerCU / waves : 1;
  return 2 * kNumCUs * per_cu;
}

// All words of a unit folded into one.  (Keeping only one word of a 16-byte
// load would free its other three registers at once, and the compiler then
// waits for the load before reusing them.)
template <typename U> __device__ __forceinline__ uint32_t fold_words(const U &v) {
  if constexpr (sizeof(U) == 16) return v.x ^ v.y ^ v.z ^ v.w;
  else return (uint32_t)v;
}

// Issue the prefetch of units [begin, end) of `row`, a workgroup's slice of
// blockDim.x * VPT units (lane l's units: begin + l + i * blockDim.x): each
// lane reads those of its units that start a 128-byte stretch of the row.
// The other lanes (and all lanes when row == NULL) read `fallback`, an
// address the workgroup reads anyway, so the load is not under a branch.
// Returns the loaded words, to be passed to keep_loaded(): the wave waits
// for them at its end.
template <typename U, int VPT>
__device__ __forceinline__ uint32_t prefetch_lines(const U *__restrict__ row, int64_t begin,
                                                   int64_t end, const U *__restrict__ fallback) {
  constexpr int64_t kPerLine = 128 / (int64_t)sizeof(U);
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < VPT; i++) {
    const int64_t u = (int64_t)threadIdx.x + (int64_t)i * blockDim.x;
    const bool on = row != nullptr && begin + u < end && ((begin + u) % kPerLine) == 0;
    w ^= fold_words(*(on ? row + begin + u : fallback));
  }
  return w;
}
__device__ __forceinline__ void keep_loaded(uint32_t w) { asm volatile("" ::"v"(w)); }

// bf16 -> fp32 is exact: the bf16 pattern is the top half of the binary32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_one(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, IEEE round to nearest, ties to even, on the 16 discarded
// bits; a NaN keeps its sign and upper payload and gets the quiet bit.  On
// gfx950 the conversion is one instruction for two values
// (v_cvt_pk_bf16_f32, which the compiler emits for a float -> __bf16
// conversion); on MI355X it was checked equal, for all 2^32 fp32 inputs, to
// the integer form: (u + 0x7fff + ((u >> 16) & 1)) >> 16 for non-NaN u,
// (u >> 16) | 0x40 for NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t b = __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// fp64 -> bf16 RNE without double rounding: round to odd at fp32 precision
// (fp32 keeps 16 more bits than bf16 at every exponent, so the second
// rounding is then exact), then round that fp32 value to bf16 as above.
// Round to odd from the hardware's nearest conversion: when it was inexact,
// step one place toward zero if it rounded away (the truncated value; at
// overflow, infinity becomes the largest finite fp32) and set the last bit.
__device__ __forceinline__ float f64_to_f32_odd(double d) {
  const float f = (float)d;
  uint32_t u = __float_as_uint(f);
  const double back = (double)f;
  if (d == d && back != d) {
    if (__builtin_fabs(back) > __builtin_fabs(d)) u -= 1u;
    u |= 1u;
  }
  return __uint_as_float(u);
}
// Round an fp32 value to bf16 precision, keeping it as fp32.
__device__ __forceinline__ float round_to_bf16(float f) {
  return __uint_as_float(f32_to_bf16(f) << 16);
}

// A unit of a bf16 row: 8 elements in a 16-byte vector, or 1 element.
template <int EPV> struct Bf16Unit;

template <> struct Bf16Unit<8> {
  using T = v4u;
  __device__ __forceinline__ static void unpack(const v4u &v, float *f) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  }
  __device__ __forceinline__ static v4u pack(const float *f) {
    v4u r;
    r.x = pack_bf16x2(f[0], f[1]);
    r.y = pack_bf16x2(f[2], f[3]);
    r.z = pack_bf16x2(f[4], f[5]);
    r.w = pack_bf16x2(f[6], f[7]);
    return r;
  }
  __device__ __forceinline__ static v4u zero() { return v4u{0u, 0u, 0u, 0u}; }
};

template <> struct Bf16Unit<1> {
  using T = uint16_t;
  __device__ __forceinline__ static void unpack(const uint16_t &v, float *f) { f[0] = bf16_one(v); }
  __device__ __forceinline__ static uint16_t pack(const float *f) {
    return (uint16_t)f32_to_bf16(f[0]);
  }
  __device__ __forceinline__ static uint16_t zero() { return 0; }
};

template <typename U> __device__ __forceinline__ U zero_unit();
template <> __device__ __forceinline__ v4u zero_unit<v4u>() { return v4u{0u, 0u, 0u, 0u}; }
template <> __device__ __forceinline__ uint32_t zero_unit<uint32_t>() { return 0u; }
template <> __device__ __forceinline__ uint16_t zero_unit<uint16_t>() { return 0; }

// OR status bits into the caller's device status word (vector atomic).
__device__ __forceinline__ void report(int32_t *status, int bits) {
  if (status != nullptr && bits != 0) atomicOr(status, bits);
}

// A token's side row held in registers while it is stored to each of the
// token's destinations: lane l of the first wave keeps words 4l .. 4l+3, when
// the row is whole 4-byte words and has at most 256 of them (FP8 rows of 7168
// elements with fp32 scales per 128 have 56).  Reading the row inside the
// destination loop makes each read wait for the stores issued before it (the
// vector memory counter counts both in issue order), one destination's
// stores at a time.
constexpr int kSideRegs = 4;
constexpr int64_t kSideHeldWords = (int64_t)kSideRegs * kWave;
struct SideCache {
  uint32_t w[kSideRegs];
  bool held;
};

__device__ __forceinline__ SideCache load_side_row(const SideRows &s, int64_t from) {
  SideCache c;
  const int64_t n = s.bytes / 4;
  c.held = s.words && n <= kSideHeldWords;
  const uint32_t *a = reinterpret_cast<const uint32_t *>(s.src) + from * n;
  const int64_t idx0 = (int64_t)threadIdx.x * kSideRegs;
  if (s.words == 2 && c.held && idx0 < n) {
    // rows of whole 16-byte units on 16-byte aligned bases: one access
    const v4u q = *reinterpret_cast<const v4u *>(a + idx0);
    c.w[0] = q.x; c.w[1] = q.y; c.w[2] = q.z; c.w[3] = q.w;
    return c;
  }
#pragma unroll
  for (int i = 0; i < kSideRegs; i++) {
    const int64_t idx = idx0 + i;
    c.w[i] = (c.held && idx < n) ? a[idx] : 0u;
  }
  return c;
}

// Row `from` of a side tensor to row `to`, by the whole workgroup.
__device__ __forceinline__ void copy_side_row(const SideRows &s, int64_t from, int64_t to) {
  if (s.words) {
    const int64_t n = s.bytes / 4;
    const uint32_t *a = reinterpret_cast<const uint32_t *>(s.src) + from * n;
    uint32_t *b = reinterpret_cast<uint32_t *>(s.dst) + to * n;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) b[i] = a[i];
  } else {
    const uint8_t *a = s.src + from * s.bytes;
    uint8_t *b = s.dst + to * s.bytes;
    for (int64_t i = threadIdx.x; i < s.bytes; i += blockDim.x) b[i] = a[i];
  }
}

// The side row of load_side_row to row `to` (copied from row `from` when it
// was not held).
__device__ __forceinline__ void store_side_row(const SideRows &s, const SideCache &c, int64_t from,
                                               int64_t to) {
  if (!c.held) {
    copy_side_row(s, from, to);
    return;
  }
  const int64_t n = s.bytes / 4;
  uint32_t *b = reinterpret_cast<uint32_t *>(s.dst) + to * n;
  const int64_t idx0 = (int64_t)threadIdx.x * kSideRegs;
  if (s.words == 2) {
    if (idx0 < n) *reinterpret_cast<v4u *>(b + idx0) = v4u{c.w[0], c.w[1], c.w[2], c.w[3]};
    return;
  }
#pragma unroll
  for (int i = 0; i < kSideRegs; i++) {
    const int64_t idx = idx0 + i;
    if (idx < n) b[idx] = c.w[i];
  }
}

// Wave-wide fp32 sum (every lane of the wave active); every lane gets the
// total.  DPP row permutes (quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror) leave each lane of a 16-lane row holding the
// row's sum, then the four row sums are added in a fixed order: register
// moves and four lane reads instead of a chain of cross-lane permutes
// through LDS.  The pattern is fixed, so the result is reproducible.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
// Inclusive scan of an int across the wave (every lane active): DPP row
// shifts by 1, 2, 4, 8 inside each 16-lane row (a lane whose source is in an
// earlier row adds 0), then the totals of the earlier rows (lanes 15, 31, 47).
template <int S>
__device__ __forceinline__ int row_shr_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0x110 + S, 0xF, 0xF, false);
}
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int row = (threadIdx.x & (kWave - 1)) >> 4;
  v += row_shr_i32<1>(v);
  v += row_shr_i32<2>(v);
  v += row_shr_i32<4>(v);
  v += row_shr_i32<8>(v);
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}

}  // namespace moe
