// Fused top-k softmax router and its gradient (moe-ops README, "Fused Top-K
// Softmax": top-k selection and softmax in registers, fp32 routing weights,
// exact softmax gradients scattered back to the logits).
//
// gfx950 design.  A token is handled by a group of G lanes (G = 16, one DPP
// row, for E <= 256; G = 64, the whole wave, above).  Lane l of a group
// holds logits l, l + G, l + 2G, ... (PER of them) as order-preserving
// 32-bit keys, so a comparison of logits is one unsigned compare.  Each of
// the k rounds finds the group's largest key below the previous one with a
// subtract and a min per key and a DPP row reduction (plus two cross-row
// exchanges when G = 64).  bf16 keys carry the expert in their low half, so
// they are distinct and the tie-break is built in; fp32 keys fall back to an
// exact round-by-round selection (largest key, then lowest expert) in the
// rare wave whose top k holds equal logits.  The softmax over the k is an
// fp32 exp of each difference from the first and a fixed-order sum.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kRouterWaves = 4;   // waves per workgroup
constexpr int kMaxPerLane = MOE_MAX_EXPERTS / kWave;
static_assert(kMaxPerLane == 32, "E <= 2048 over a 64-lane group");

// Key of a logit: larger logit -> larger key.  -0 is folded into +0 (equal
// logits tie), every NaN maps to 1 (below -inf, whose key is 0x007FFFFF) and
// 0 is reserved for a taken or absent slot.
__device__ __forceinline__ uint32_t logit_key(float f) {
  if (f != f) return 1u;
  const uint32_t u = f == 0.0f ? 0u : __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_logit(uint32_t key) {
  if (key <= 1u) return __uint_as_float(0x7FC00000u);
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// DPP row permutes (gfx9 encodings): quad_perm [1,0,3,2], quad_perm
// [2,3,0,1], row_half_mirror, row_mirror.  Applied in this order they make
// every lane of a 16-lane row see the whole row.
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

// Lane `l`'s value (a 64-lane group combines its four row results this way).
__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

template <int G>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
  v = max(v, dpp<kDppQuadXor1>(v));
  v = max(v, dpp<kDppQuadXor2>(v));
  v = max(v, dpp<kDppHalfMirror>(v));
  v = max(v, dpp<kDppMirror>(v));
  if constexpr (G == 64) {
    v = max(max(lane_u32(v, 0), lane_u32(v, 16)), max(lane_u32(v, 32), lane_u32(v, 48)));
  }
  return v;
}

template <int G>
__device__ __forceinline__ uint32_t group_min(uint32_t v) {
  v = min(v, dpp<kDppQuadXor1>(v));
  v = min(v, dpp<kDppQuadXor2>(v));
  v = min(v, dpp<kDppHalfMirror>(v));
  v = min(v, dpp<kDppMirror>(v));
  if constexpr (G == 64) {
    v = min(min(lane_u32(v, 0), lane_u32(v, 16)), min(lane_u32(v, 32), lane_u32(v, 48)));
  }
  return v;
}

template <int G>
__device__ __forceinline__ float group_sum(float v) {
  v += __uint_as_float(dpp<kDppQuadXor1>(__float_as_uint(v)));
  v += __uint_as_float(dpp<kDppQuadXor2>(__float_as_uint(v)));
  v += __uint_as_float(dpp<kDppHalfMirror>(__float_as_uint(v)));
  v += __uint_as_float(dpp<kDppMirror>(__float_as_uint(v)));
  if constexpr (G == 64) {
    v = (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
  }
  return v;
}

template <int G>
__device__ __forceinline__ uint32_t group_sum_u32(uint32_t v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  if constexpr (G == 64) {
    v = (lane_u32(v, 0) + lane_u32(v, 16)) + (lane_u32(v, 32) + lane_u32(v, 48));
  }
  return v;
}

// bf16 logit -> 16-bit order-preserving key, as logit_key: -0 folded into +0,
// NaN -> 1, real keys >= 0x7F.
__device__ __forceinline__ uint32_t bf16_key(uint32_t b) {
  if ((b & 0x7F80u) == 0x7F80u && (b & 0x7Fu) != 0u) return 1u;
  if (b == 0x8000u) b = 0u;
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

__device__ __forceinline__ float bf16_key_logit(uint32_t key16) {
  if (key16 <= 1u) return __uint_as_float(0x7FC00000u);
  const uint32_t b = (key16 & 0x8000u) ? (key16 & 0x7FFFu) : (~key16 & 0xFFFFu);
  return __uint_as_float(b << 16);
}

// The k largest keys of the group by repeated "largest key below the last
// one": with lim = last - 1, lim - key is small for keys below the last and
// wraps to a large value for the others, so one min over (lim - key) per
// round finds the next key without clearing anything.  Returns whether the
// k keys came out strictly decreasing and real (> 1 never needed: real keys
// are >= 1); group lane 0 stores them in skey[0..k).
// FIND: the lane holding each selected key also stores its expert in
// sidx[j] (one holder per key when the keys are distinct; the caller
// discards sidx otherwise).
template <int G, int PER, bool FIND>
__device__ __forceinline__ bool select_below(const uint32_t (&key)[PER], int k, int gl,
                                             uint32_t *skey, int *sidx, uint32_t &last) {
  uint32_t below = 0xFFFFFFFFu;   // above every key
  bool strict = true;
  for (int j = 0; j < k; j++) {
    const uint32_t lim = below - 1u;
    uint32_t dmin = 0xFFFFFFFFu;
#pragma unroll
    for (int s = 0; s < PER; s++) dmin = min(dmin, lim - key[s]);
    const uint32_t m = lim - group_min<G>(dmin);
    strict = strict && m < below && m != 0u;
    if (gl == 0) skey[j] = m;
    if constexpr (FIND) {
      int fs = -1;
#pragma unroll
      for (int s = PER - 1; s >= 0; s--) fs = key[s] == m ? s : fs;
      if (fs >= 0) sidx[j] = fs * G + gl;
    }
    below = m;
  }
  last = below;
  return strict;
}

// Exact selection for keys that may repeat: per round the largest untaken
// key, then the lowest expert holding it; the winner is cleared.
template <int G, int PER>
__device__ __forceinline__ void select_exact(uint32_t (&key)[PER], int k, int gl, float *sval,
                                             int *sidx) {
  for (int j = 0; j < k; j++) {
    uint32_t bk = 0;
#pragma unroll
    for (int s = 0; s < PER; s++) bk = max(bk, key[s]);
    const uint32_t top_key = group_max<G>(bk);
    int fs = -1;
#pragma unroll
    for (int s = PER - 1; s >= 0; s--) fs = key[s] == top_key ? s : fs;
    const uint32_t mine = fs < 0 ? (uint32_t)INT32_MAX : (uint32_t)(fs * G + gl);
    const uint32_t we = group_min<G>(mine);
    int cs = we == mine ? fs : -1;
    asm volatile("" : "+v"(cs));   // one VGPR select, not a mask per slot
#pragma unroll
    for (int s = 0; s < PER; s++) key[s] = s == cs ? 0u : key[s];
    if (gl == 0) {
      sval[j] = key_logit(top_key);
      sidx[j] = (int)we;
    }
  }
}

// Every lane of the wave runs every step (tokens past T are clamped to the
// last one and store nothing), so the DPP and cross-lane exchanges always
// read active lanes.
//
// bf16 logits: the key is (16-bit logit key << 16) | (0xFFFF - expert), so
// keys are distinct, larger logits first and the lower expert first among
// equal logits; select_below alone is exact and the expert is in the key.
// fp32 logits: select_below on the 32-bit logit keys is exact when the k
// keys found are distinct and exactly k elements of the group reach the
// last of them (no ties in the top k); the lane holding each key stores its
// expert as the key is found.  Otherwise the wave takes the exact path.
template <int EB, int G, int PER>
__global__ __launch_bounds__(kRouterWaves * kWave) void topk_softmax_kernel(
    const void *__restrict__ logits, int T, int E, int k, int32_t *__restrict__ topk_idx,
    void *__restrict__ probs, int prob_bytes) {
  constexpr int kGroups = kRouterWaves * (kWave / G);
  __shared__ float sval[kGroups][MOE_MAX_TOPK];
  __shared__ int sidx[kGroups][MOE_MAX_TOPK];
  __shared__ uint32_t skey[kGroups][MOE_MAX_TOPK];
  const int grp = threadIdx.x / G;
  const int gl = threadIdx.x % G;
  const int64_t b = spill_block();
  if (b * kGroups >= T) return;  // a workgroup past the last token
  const int64_t t = b * kGroups + grp;
  const bool live = t < T;
  const int64_t row = (int64_t)(live ? t : T - 1) * E;

  uint32_t key[PER];
  uint32_t last;
  if constexpr (EB == 2) {
    const uint16_t *lr = static_cast<const uint16_t *>(logits) + row;
#pragma unroll
    for (int s = 0; s < PER; s++) {
      const int e = s * G + gl;
      key[s] = e < E ? (bf16_key(lr[e]) << 16) | (0xFFFFu - (uint32_t)e) : 0u;
    }
    select_below<G, PER, false>(key, k, gl, skey[grp], sidx[grp], last);
    __syncwarp();
    for (int j = gl; j < k; j += G) {
      const uint32_t m = skey[grp][j];
      sidx[grp][j] = (int)(0xFFFFu - (m & 0xFFFFu));
      sval[grp][j] = bf16_key_logit(m >> 16);
    }
  } else {
    const float *lr = static_cast<const float *>(logits) + row;
#pragma unroll
    for (int s = 0; s < PER; s++) {
      const int e = s * G + gl;
      key[s] = e < E ? logit_key(lr[e]) : 0u;
    }
    const bool strict = select_below<G, PER, true>(key, k, gl, skey[grp], sidx[grp], last);
    uint32_t cnt = 0;
#pragma unroll
    for (int s = 0; s < PER; s++) cnt += key[s] >= last ? 1u : 0u;
    cnt = group_sum_u32<G>(cnt);
    if (__all(strict && cnt == (uint32_t)k)) {
      __syncwarp();
      for (int j = gl; j < k; j += G) sval[grp][j] = key_logit(skey[grp][j]);
    } else {
      __syncwarp();   // the fast path's stores land before the exact path rewrites them
      select_exact<G, PER>(key, k, gl, sval[grp], sidx[grp]);
    }
  }
  __syncwarp();
  const float top = sval[grp][0];
  float ex = 0.0f;
  for (int j = gl; j < k; j += G) ex += expf(sval[grp][j] - top);
  const float sum = group_sum<G>(ex);
  if (!live) return;
  for (int j = gl; j < k; j += G) {
    topk_idx[(int64_t)t * k + j] = sidx[grp][j];
    const float w = expf(sval[grp][j] - top) / sum;
    if (prob_bytes == 4)
      static_cast<float *>(probs)[(int64_t)t * k + j] = w;
    else
      static_cast<uint16_t *>(probs)[(int64_t)t * k + j] = (uint16_t)f32_to_bf16(w);
  }
}

template <int B>
__device__ __forceinline__ float load_real(const void *p, int64_t i) {
  if constexpr (B == 2)
    return __uint_as_float((uint32_t)static_cast<const uint16_t *>(p)[i] << 16);
  else
    return static_cast<const float *>(p)[i];
}

// d_logits[t][e_j] = w_j (dp_j - sum_i w_i dp_i); other experts +0.  One
// wave per token: the k gradients are scattered into an LDS copy of the
// output row, which is then written out whole with coalesced stores.
// PB: bytes of the weights and their gradients (fp32 / bf16); OB: bytes of
// d_logits.  The arithmetic is fp32 either way.
template <int PB, int OB>
__global__ __launch_bounds__(kRouterWaves * kWave) void topk_softmax_bwd_kernel(
    const void *__restrict__ d_probs, const void *__restrict__ probs,
    const int32_t *__restrict__ topk_idx, int T, int E, int k, void *__restrict__ d_logits,
    int32_t *__restrict__ dev_status) {
  __shared__ float srow[kRouterWaves][MOE_MAX_EXPERTS];
  const int wv = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = spill_block() * kRouterWaves + wv;
  if (t >= T) return;   // whole wave leaves; only wave-level syncs below
  for (int e = lane; e < E; e += kWave) srow[wv][e] = 0.0f;
  // k <= 64: lane j owns slot j
  const bool has = lane < k;
  const float w = has ? load_real<PB>(probs, (int64_t)t * k + lane) : 0.0f;
  const float dp = has ? load_real<PB>(d_probs, (int64_t)t * k + lane) : 0.0f;
  const int e = has ? topk_idx[(int64_t)t * k + lane] : -1;
  const float dot = wave_sum(__builtin_fmaf(w, dp, 0.0f));
  __syncwarp();
  int bad = 0;
  if (has) {
    if ((unsigned)e < (unsigned)E)
      srow[wv][e] = w * (dp - dot);
    else
      bad = MOE_DEV_BAD_EXPERT;
  }
  report(dev_status, bad);
  __syncwarp();
  if constexpr (OB == 4) {
    float *dst = static_cast<float *>(d_logits) + (int64_t)t * E;
    for (int i = lane; i < E; i += kWave) dst[i] = srow[wv][i];
  } else {
    uint16_t *dst = static_cast<uint16_t *>(d_logits) + (int64_t)t * E;
    for (int i = lane; i < E; i += kWave) dst[i] = (uint16_t)f32_to_bf16(srow[wv][i]);
  }
}

template <int EB, int G>
void launch_router_g(const void *logits, int T, int E, int k, int32_t *topk_idx, void *probs,
                     int prob_bytes, hipStream_t s) {
  constexpr int kGroups = kRouterWaves * (kWave / G);
  const dim3 grid = spill_grid((T + kGroups - 1) / kGroups), block(kRouterWaves * kWave);
  const int per = (E + G - 1) / G;
#define MOE_ROUTER_CASE(P)                                                                 \
  if (per <= P) {                                                                          \
    hipLaunchKernelGGL((topk_softmax_kernel<EB, G, P>), grid, block, 0, s, logits, T, E,  \
                       k, topk_idx, probs, prob_bytes);                                    \
    return;                                                                                \
  }
  if constexpr (G == 16) {
    MOE_ROUTER_CASE(1)
    MOE_ROUTER_CASE(2)
    MOE_ROUTER_CASE(4)
    MOE_ROUTER_CASE(8)
    MOE_ROUTER_CASE(16)
  } else {
    MOE_ROUTER_CASE(8)
    MOE_ROUTER_CASE(16)
    MOE_ROUTER_CASE(32)
  }
#undef MOE_ROUTER_CASE
}

}  // namespace

hipError_t launch_topk_softmax(const void *logits, int logit_bytes, int T, int E, int k,
                               int32_t *topk_idx, void *probs, int prob_bytes, hipStream_t s) {
  if (E > kMaxPerLane * kWave || k > MOE_MAX_TOPK) return hipErrorInvalidValue;
  const bool row16 = E <= 16 * 16;
  if (logit_bytes == 2) {
    if (row16) launch_router_g<2, 16>(logits, T, E, k, topk_idx, probs, prob_bytes, s);
    else launch_router_g<2, 64>(logits, T, E, k, topk_idx, probs, prob_bytes, s);
  } else {
    if (row16) launch_router_g<4, 16>(logits, T, E, k, topk_idx, probs, prob_bytes, s);
    else launch_router_g<4, 64>(logits, T, E, k, topk_idx, probs, prob_bytes, s);
  }
  return hipGetLastError();
}

hipError_t launch_topk_softmax_bwd(const void *d_probs, const void *probs, int prob_bytes,
                                   const int32_t *topk_idx, int T, int E, int k, void *d_logits,
                                   int logit_bytes, int32_t *dev_status, hipStream_t s) {
  if (E > MOE_MAX_EXPERTS || k > kWave) return hipErrorInvalidValue;
  const dim3 grid = spill_grid((T + kRouterWaves - 1) / kRouterWaves),
             block(kRouterWaves * kWave);
#define MOE_ROUTER_BWD(PB, OB)                                                              \
  hipLaunchKernelGGL((topk_softmax_bwd_kernel<PB, OB>), grid, block, 0, s, d_probs, probs, \
                     topk_idx, T, E, k, d_logits, dev_status)
  if (prob_bytes == 4 && logit_bytes == 4) MOE_ROUTER_BWD(4, 4);
  else if (prob_bytes == 4) MOE_ROUTER_BWD(4, 2);
  else if (logit_bytes == 4) MOE_ROUTER_BWD(2, 4);
  else MOE_ROUTER_BWD(2, 2);
#undef MOE_ROUTER_BWD
  return hipGetLastError();
}

}  // namespace moe
