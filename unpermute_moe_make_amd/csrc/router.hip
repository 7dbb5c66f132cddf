// Fused top-k softmax router and its gradient (moe-ops README, "Fused Top-K
// Softmax": top-k selection and softmax in registers, fp32 routing weights,
// exact softmax gradients scattered back to the logits).
//
// gfx950 design.  A token is handled by a group of G lanes (G = 16, one DPP
// row, for E <= 256; G = 64, the whole wave, above).  Lane l of a group
// holds logits l, l + G, l + 2G, ... (PER of them) as order-preserving
// 32-bit keys, so a comparison of logits is one unsigned compare.  Each of
// the k rounds reduces the largest untaken key over the group, then the
// lowest expert holding that key (the tie-break), both with DPP row permutes
// (plus two cross-row exchanges when G = 64), and the lane that owned the
// winner clears it.  The group's k winners come out in
// descending order with deterministic tie-breaks; the softmax over them is
// an fp32 exp of each difference from the first and a fixed-order sum.
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

template <int EB>
__device__ __forceinline__ float load_logit(const void *p, int64_t i) {
  if constexpr (EB == 2)
    return __uint_as_float((uint32_t)static_cast<const uint16_t *>(p)[i] << 16);
  else
    return static_cast<const float *>(p)[i];
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

template <int G>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
  v = max(v, dpp<kDppQuadXor1>(v));
  v = max(v, dpp<kDppQuadXor2>(v));
  v = max(v, dpp<kDppHalfMirror>(v));
  v = max(v, dpp<kDppMirror>(v));
  if constexpr (G == 64) {
    v = max(v, (uint32_t)__shfl_xor((int)v, 16, kWave));
    v = max(v, (uint32_t)__shfl_xor((int)v, 32, kWave));
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
    v = min(v, (uint32_t)__shfl_xor((int)v, 16, kWave));
    v = min(v, (uint32_t)__shfl_xor((int)v, 32, kWave));
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
    v += __shfl_xor(v, 16, kWave);
    v += __shfl_xor(v, 32, kWave);
  }
  return v;
}

// Every lane of the wave runs every step (tokens past T are clamped to the
// last one and store nothing), so the DPP and cross-lane exchanges always
// read active lanes.
template <int EB, int G, int PER>
__global__ __launch_bounds__(kRouterWaves * kWave) void topk_softmax_kernel(
    const void *__restrict__ logits, int T, int E, int k, int32_t *__restrict__ topk_idx,
    void *__restrict__ probs, int prob_bytes) {
  constexpr int kGroups = kRouterWaves * (kWave / G);
  __shared__ float sval[kGroups][MOE_MAX_TOPK];
  __shared__ int sidx[kGroups][MOE_MAX_TOPK];
  const int grp = threadIdx.x / G;
  const int gl = threadIdx.x % G;
  const int t = blockIdx.x * kGroups + grp;
  const bool live = t < T;
  const int64_t row = (int64_t)(live ? t : T - 1) * E;

  uint32_t key[PER];
#pragma unroll
  for (int s = 0; s < PER; s++) {
    const int e = s * G + gl;
    key[s] = e < E ? logit_key(load_logit<EB>(logits, row + e)) : 0u;
  }
  for (int j = 0; j < k; j++) {
    // the group's largest untaken key ...
    uint32_t bk = 0;
#pragma unroll
    for (int s = 0; s < PER; s++) bk = max(bk, key[s]);
    const uint32_t top_key = group_max<G>(bk);
    // ... and the lowest expert holding it (k <= E: one always exists)
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
      sval[grp][j] = key_logit(top_key);
      sidx[grp][j] = (int)we;
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
  const int t = blockIdx.x * kRouterWaves + wv;
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
  const dim3 grid((T + kGroups - 1) / kGroups), block(kRouterWaves * kWave);
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
  const dim3 grid((T + kRouterWaves - 1) / kRouterWaves), block(kRouterWaves * kWave);
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
