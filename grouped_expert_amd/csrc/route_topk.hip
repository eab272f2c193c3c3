// Router top-k with renormalised softmax gates, one wavefront per token.
//
// "M6.2 - Expert Parallelism and DeepSeek MoE", 0x06L1 (Mixtral row): FP32
// softmax over all experts, keep the top k, renormalise the kept mass to one.
// "M6.6 - MoE Runtime Systems", 0x0AE: logits and the top-k comparison in
// FP32.  Softmax is monotone, so the k largest logits are selected directly;
// the full-softmax denominator cancels in the renormalised gates.
//
// Each lane holds up to V = ceil(E/64) logits (expert e = lane + 64*v).  A
// logit becomes an order-preserving 32-bit key (+0 and -0 share one key).
// Each of the k rounds takes the wavefront max of the keys, then the
// wavefront min of the expert indices holding that key (ties go to the lower
// expert), both as DPP / lane-swap butterflies without LDS; the winner's owner
// lane clears that key.
#include "common.h"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) == 0) u = 0;                // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
  return __uint_as_float(u);
}

// Wavefront-wide reductions without LDS traffic: inside each 16-lane row,
// DPP quad permutations pair lanes at distance 1 and 2 and the half-row /
// row mirrors pair the two quads of an 8-lane half and the two halves of a
// row (the compiler folds each into the VALU op as a DPP source); then
// v_permlane16_swap and v_permlane32_swap (gfx950) exchange whole rows and
// wave halves.  With both operands equal, a swap returns {rows 0,0,2,2 ;
// rows 1,1,3,3} (16) or {lo,lo ; hi,hi} (32), so combining the two results
// gives the pairwise result in every lane.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = umax(v, dpp<0xB1>(v));     // quad_perm [1,0,3,2]
  v = umax(v, dpp<0x4E>(v));     // quad_perm [2,3,0,1]
  v = umax(v, dpp<0x141>(v));    // row_half_mirror
  v = umax(v, dpp<0x140>(v));    // row_mirror
  const auto p16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = umax(p16[0], p16[1]);
  const auto p32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return umax(p32[0], p32[1]);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = umin(v, dpp<0xB1>(v));
  v = umin(v, dpp<0x4E>(v));
  v = umin(v, dpp<0x141>(v));
  v = umin(v, dpp<0x140>(v));
  const auto p16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = umin(p16[0], p16[1]);
  const auto p32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return umin(p32[0], p32[1]);
}

// The builtin works on int: go through uint32_t, never by sign extension.
__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
}

// Wavefront-wide fp32 sum with the same lane pairings.
template <int CTRL>
__device__ __forceinline__ float add_dpp(float v) {
  return v + __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  v = add_dpp<0xB1>(v);
  v = add_dpp<0x4E>(v);
  v = add_dpp<0x141>(v);
  v = add_dpp<0x140>(v);
  const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
  const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}

constexpr int kTokensPerBlock = 4;

template <int V>
__global__ __launch_bounds__(kTokensPerBlock * kWave) void route_topk_kernel(
    const float* __restrict__ logits, int64_t T, int32_t E, int32_t k, int32_t* __restrict__ ids,
    float* __restrict__ weights, uint32_t* flags) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokensPerBlock + threadIdx.x / kWave;
  if (t >= T) return;                                   // whole wavefront leaves together
  const float* row = logits + t * E;

  // key[v]: order key of expert lane + 64 v (0 = no expert; a finite or
  // infinite logit has a key >= 0x007FFFFF)
  uint32_t key[V];
  bool bad = false;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int e = lane + v * kWave;
    key[v] = 0;
    if (e < E) {
      const float z = row[e];
      bad |= !isfinite(z);
      key[v] = order_key(z);
    }
  }
  const bool token_bad = ballot(bad) != 0;

  // k selection rounds: the largest key, then the lowest expert holding it;
  // lane j keeps the j-th winner.  The winner's owner lane clears that key.
  uint32_t mine_key = 0, top_key = 0;
  int32_t mine_e = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t lmax = key[0];
#pragma unroll
    for (int v = 1; v < V; ++v) lmax = umax(lmax, key[v]);
    const uint32_t K = uniform(wave_max_u32(lmax));
    uint32_t lmin = 0xFFFFFFFFu;
#pragma unroll
    for (int v = V - 1; v >= 0; --v) lmin = key[v] == K ? static_cast<uint32_t>(lane + v * kWave) : lmin;
    const uint32_t ew = uniform(wave_min_u32(lmin));
    const int vw = static_cast<int>(ew / kWave), lw = static_cast<int>(ew % kWave);
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (v == vw && lane == lw) key[v] = 0;
    if (lane == j) {
      mine_key = K;
      mine_e = static_cast<int32_t>(ew);
    }
    if (j == 0) top_key = K;
  }

  const float z = key_value(mine_key);
  const float z0 = key_value(top_key);
  const float p = lane < k ? expf(z - z0) : 0.0f;
  const float s = wave_sum_f32(p);
  if (lane < k) {
    ids[t * k + lane] = token_bad ? -1 : mine_e;
    weights[t * k + lane] = token_bad ? 0.0f : p / s;
  }
  if (token_bad && lane == 0) flag_or(flags, MOE_FLAG_NONFINITE_LOGIT);
}

template <int V>
void launch(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids, float* w, uint32_t* flags,
            hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((T + kTokensPerBlock - 1) / kTokensPerBlock);
  hipLaunchKernelGGL(HIP_KERNEL_NAME(route_topk_kernel<V>), dim3(blocks), dim3(kTokensPerBlock * kWave), 0, s,
                     logits, T, E, k, ids, w, flags);
}

}  // namespace
}  // namespace moe

MOE_API int moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t gating,
                           int32_t* topk_ids, float* topk_w, uint32_t* dev_flags, hipStream_t stream) {
  using namespace moe;
  MOE_CHECK(T >= 0 && E >= 1 && E <= MOE_MAX_EXPERTS, MOE_EINVAL);
  MOE_CHECK(k >= 1 && k <= E && k <= MOE_MAX_TOPK, MOE_EINVAL);
  MOE_CHECK(gating == MOE_GATING_SOFTMAX_TOPK_RENORM, MOE_EUNSUPPORTED);
  MOE_CHECK(T <= INT32_MAX / k, MOE_EUNSUPPORTED);          // routes are int32-indexed
  if (T == 0) return MOE_OK;
  MOE_CHECK(logits && topk_ids && topk_w, MOE_EINVAL);
  MOE_CHECK(aligned4(logits) && aligned4(topk_ids) && aligned4(topk_w), MOE_EINVAL);
  const int V = (E + kWave - 1) / kWave;
  if (V <= 1) launch<1>(logits, T, E, k, topk_ids, topk_w, dev_flags, stream);
  else if (V <= 2) launch<2>(logits, T, E, k, topk_ids, topk_w, dev_flags, stream);
  else if (V <= 4) launch<4>(logits, T, E, k, topk_ids, topk_w, dev_flags, stream);
  else if (V <= 6) launch<6>(logits, T, E, k, topk_ids, topk_w, dev_flags, stream);
  else if (V <= 8) launch<8>(logits, T, E, k, topk_ids, topk_w, dev_flags, stream);
  else launch<16>(logits, T, E, k, topk_ids, topk_w, dev_flags, stream);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
