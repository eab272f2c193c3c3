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
#include <cmath>

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

// k selection rounds over the keys of one wavefront (expert lane + 64 v):
// the largest key, then the lowest expert holding it; the winner's owner lane
// clears that key.  Lane j keeps the j-th winner; top_key is the first one.
template <int V>
__device__ __forceinline__ void select_topk(uint32_t (&key)[V], int k, int lane, uint32_t& mine_key,
                                            int32_t& mine_e, uint32_t& top_key) {
  mine_key = 0;
  mine_e = 0;
  top_key = 0;
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
}

// full_mass = 0: gates renormalised over the k kept experts;
// full_mass = 1 (V1): gates are the kept full-softmax probabilities.
template <int V>
__global__ __launch_bounds__(kTokensPerBlock * kWave) void route_topk_kernel(
    const float* __restrict__ logits, int64_t T, int32_t E, int32_t k, int32_t full_mass, int32_t* __restrict__ ids,
    float* __restrict__ weights, uint32_t* flags) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokensPerBlock + threadIdx.x / kWave;
  if (t >= T) return;                                   // whole wavefront leaves together
  const float* row = logits + t * E;

  // key[v]: order key of expert lane + 64 v (0 = no expert; a finite or
  // infinite logit has a key >= 0x007FFFFF); zf[v] the logit itself
  uint32_t key[V];
  float zf[V];
  bool bad = false;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int e = lane + v * kWave;
    key[v] = 0;
    zf[v] = -INFINITY;
    if (e < E) {
      const float z = row[e];
      bad |= !isfinite(z);
      key[v] = order_key(z);
      zf[v] = z;
    }
  }
  const bool token_bad = ballot(bad) != 0;

  uint32_t mine_key, top_key;
  int32_t mine_e;
  select_topk<V>(key, k, lane, mine_key, mine_e, top_key);

  const float z = key_value(mine_key);
  const float z0 = key_value(top_key);
  const float p = lane < k ? expf(z - z0) : 0.0f;
  float mass = 0.0f;
  if (full_mass) {
#pragma unroll
    for (int v = 0; v < V; ++v) mass += expf(zf[v] - z0);
  } else {
    mass = p;
  }
  const float s = wave_sum_f32(mass);
  if (lane < k) {
    ids[t * k + lane] = token_bad ? -1 : mine_e;
    weights[t * k + lane] = token_bad ? 0.0f : p / s;
  }
  if (token_bad && lane == 0) flag_or(flags, MOE_FLAG_NONFINITE_LOGIT);
}

template <int V>
void launch(const float* logits, int64_t T, int32_t E, int32_t k, int32_t full_mass, int32_t* ids, float* w,
            uint32_t* flags, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((T + kTokensPerBlock - 1) / kTokensPerBlock);
  hipLaunchKernelGGL(HIP_KERNEL_NAME(route_topk_kernel<V>), dim3(blocks), dim3(kTokensPerBlock * kWave), 0, s,
                     logits, T, E, k, full_mass, ids, w, flags);
}

// Group-restricted router (V2 when sigmoid_bias = 0, V3 when 1).  One
// wavefront per token.  Each lane turns its logits into selection keys (V2:
// the logit; V3: the fp32-rounded fp64 sigmoid plus the bias in fp32) and stores them in the wavefront's
// LDS row; lane g < n_group then scans group g's G contiguous keys for the
// group score (V2: largest key; V3: fp32 sum of the two largest corrected
// scores).  topk_group rounds of max / lowest-index pick the groups, the
// experts outside them get key 0, and the usual k rounds pick the experts.
template <int V>
__global__ __launch_bounds__(kTokensPerBlock * kWave) void route_grouped_kernel(
    const float* __restrict__ logits, int64_t T, int32_t E, int32_t k, int32_t sigmoid_bias, int32_t n_group,
    int32_t topk_group, float route_scale, const float* __restrict__ bias, int32_t* __restrict__ ids,
    float* __restrict__ weights, uint32_t* flags) {
  extern __shared__ uint32_t keys_lds[];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokensPerBlock + wave;
  if (t >= T) return;                                   // whole wavefront leaves together
  const float* row = logits + t * E;
  uint32_t* lk = keys_lds + wave * E;                   // this wavefront's LDS row

  uint32_t key[V];
  float val[V];                                         // V2: logit; V3: sigmoid affinity
  bool bad = false;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int e = lane + v * kWave;
    key[v] = 0;
    val[v] = -INFINITY;
    if (e < E) {
      const float z = row[e];
      bad |= !isfinite(z);
      if (sigmoid_bias) {
        // the affinity as a decision key: the sigmoid evaluated in fp64 and
        // rounded once to fp32, so that it is the fp32 value nearest to the
        // sigmoid (any other fp32 evaluation depends on the exp used); the
        // corrected score is one fp32 addition
        const float sg = static_cast<float>(1.0 / (1.0 + exp(-static_cast<double>(z))));
        const float c = sg + (bias ? bias[e] : 0.0f);
        bad |= !isfinite(c);
        key[v] = order_key(c);
        val[v] = sg;
      } else {
        key[v] = order_key(z);
        val[v] = z;
      }
      lk[e] = key[v];
    }
  }
  const bool token_bad = ballot(bad) != 0;
  // the LDS row is written and read by this wavefront only: its LDS accesses
  // complete in order; the fence keeps the compiler from reordering them
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // group scores: lane g scans group g
  const int G = E / n_group;
  uint32_t gkey = 0;
  if (lane < n_group) {
    if (sigmoid_bias) {
      uint32_t k1 = 0, k2 = 0;                          // two largest keys, k1 >= k2
      for (int i = 0; i < G; ++i) {
        const uint32_t x = lk[lane * G + i];
        if (x > k1) {
          k2 = k1;
          k1 = x;
        } else if (x > k2) {
          k2 = x;
        }
      }
      gkey = order_key(key_value(k1) + key_value(k2));
    } else {
      for (int i = 0; i < G; ++i) gkey = umax(gkey, lk[lane * G + i]);
    }
  }
  // topk_group rounds over groups (one group per lane)
  uint64_t kept = 0;
  for (int r = 0; r < topk_group; ++r) {
    const uint32_t K = uniform(wave_max_u32(gkey));
    const uint32_t gw = uniform(wave_min_u32(gkey == K && lane < n_group ? static_cast<uint32_t>(lane) : 0xFFFFFFFFu));
    kept |= 1ull << (gw & 63u);
    if (lane == static_cast<int>(gw)) gkey = 0;
  }
  // experts outside the kept groups leave the selection
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int e = lane + v * kWave;
    if (e < E && !((kept >> (e / G)) & 1ull)) key[v] = 0;
  }

  uint32_t mine_key, top_key;
  int32_t mine_e;
  select_topk<V>(key, k, lane, mine_key, mine_e, top_key);
  (void)top_key;

  // the selected expert's value, fetched from its owner lane
  float mine_val = 0.0f;
  for (int j = 0; j < k; ++j) {
    const int ej = __builtin_amdgcn_readlane(mine_e, j);
    const int vw = ej / kWave, lw = ej % kWave;
    float vv = 0.0f;
#pragma unroll
    for (int v = 0; v < V; ++v) vv = v == vw ? val[v] : vv;
    const float got = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vv), lw));
    if (lane == j) mine_val = got;
  }

  float gate;
  if (sigmoid_bias) {
    const float ssum = wave_sum_f32(lane < k ? mine_val : 0.0f);
    gate = route_scale * mine_val / ssum;
  } else {
    // full softmax over all E experts: the largest logit of the token
    uint32_t lmax = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = lane + v * kWave;
      if (e < E) lmax = umax(lmax, order_key(val[v]));
    }
    const float zmax = key_value(uniform(wave_max_u32(lmax)));
    float mass = 0.0f;
#pragma unroll
    for (int v = 0; v < V; ++v) mass += expf(val[v] - zmax);
    const float denom = wave_sum_f32(mass);
    gate = route_scale * expf(mine_val - zmax) / denom;
  }
  if (lane < k) {
    ids[t * k + lane] = token_bad ? -1 : mine_e;
    weights[t * k + lane] = token_bad ? 0.0f : gate;
  }
  if (token_bad && lane == 0) flag_or(flags, MOE_FLAG_NONFINITE_LOGIT);
}

template <int V>
void launch_grouped(const float* logits, int64_t T, int32_t E, int32_t k, int32_t sigmoid_bias, int32_t n_group,
                    int32_t topk_group, float scale, const float* bias, int32_t* ids, float* w, uint32_t* flags,
                    hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((T + kTokensPerBlock - 1) / kTokensPerBlock);
  const size_t lds = static_cast<size_t>(kTokensPerBlock) * E * sizeof(uint32_t);
  hipLaunchKernelGGL(HIP_KERNEL_NAME(route_grouped_kernel<V>), dim3(blocks), dim3(kTokensPerBlock * kWave), lds, s,
                     logits, T, E, k, sigmoid_bias, n_group, topk_group, scale, bias, ids, w, flags);
}

}  // namespace
}  // namespace moe

MOE_API int moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t gating,
                           int32_t* topk_ids, float* topk_w, uint32_t* dev_flags, hipStream_t stream) {
  using namespace moe;
  MOE_CHECK(T >= 0 && E >= 1 && E <= MOE_MAX_EXPERTS, MOE_EINVAL);
  MOE_CHECK(k >= 1 && k <= E && k <= MOE_MAX_TOPK, MOE_EINVAL);
  MOE_CHECK(gating == MOE_GATING_SOFTMAX_TOPK_RENORM || gating == MOE_GATING_SOFTMAX_TOPK, MOE_EUNSUPPORTED);
  MOE_CHECK(T <= INT32_MAX / k, MOE_EUNSUPPORTED);          // routes are int32-indexed
  if (T == 0) return MOE_OK;
  MOE_CHECK(logits && topk_ids && topk_w, MOE_EINVAL);
  MOE_CHECK(aligned4(logits) && aligned4(topk_ids) && aligned4(topk_w), MOE_EINVAL);
  const int full = gating == MOE_GATING_SOFTMAX_TOPK ? 1 : 0;
  const int V = (E + kWave - 1) / kWave;
  if (V <= 1) launch<1>(logits, T, E, k, full, topk_ids, topk_w, dev_flags, stream);
  else if (V <= 2) launch<2>(logits, T, E, k, full, topk_ids, topk_w, dev_flags, stream);
  else if (V <= 4) launch<4>(logits, T, E, k, full, topk_ids, topk_w, dev_flags, stream);
  else if (V <= 6) launch<6>(logits, T, E, k, full, topk_ids, topk_w, dev_flags, stream);
  else if (V <= 8) launch<8>(logits, T, E, k, full, topk_ids, topk_w, dev_flags, stream);
  else launch<16>(logits, T, E, k, full, topk_ids, topk_w, dev_flags, stream);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

MOE_API int moe_route_topk_grouped(const float* logits, int64_t T, int32_t E, int32_t k, int32_t gating,
                                   int32_t n_group, int32_t topk_group, float route_scale, const float* bias,
                                   int32_t* topk_ids, float* topk_w, uint32_t* dev_flags, hipStream_t stream) {
  using namespace moe;
  MOE_CHECK(gating == MOE_GATING_SOFTMAX_GROUP_LIMITED || gating == MOE_GATING_SIGMOID_BIAS_GROUP_TOP2,
            MOE_EUNSUPPORTED);
  const int sig = gating == MOE_GATING_SIGMOID_BIAS_GROUP_TOP2 ? 1 : 0;
  MOE_CHECK(T >= 0 && E >= 1 && E <= MOE_MAX_EXPERTS, MOE_EINVAL);
  MOE_CHECK(n_group >= 1 && n_group <= kWave && E % n_group == 0, MOE_EINVAL);
  MOE_CHECK(topk_group >= 1 && topk_group <= n_group, MOE_EINVAL);
  MOE_CHECK(k >= 1 && k <= MOE_MAX_TOPK && k <= topk_group * (E / n_group), MOE_EINVAL);
  MOE_CHECK(!sig || E / n_group >= 2, MOE_EINVAL);
  MOE_CHECK(sig || bias == nullptr, MOE_EINVAL);
  MOE_CHECK(std::isfinite(route_scale), MOE_EINVAL);
  MOE_CHECK(T <= INT32_MAX / k, MOE_EUNSUPPORTED);
  if (T == 0) return MOE_OK;
  MOE_CHECK(logits && topk_ids && topk_w, MOE_EINVAL);
  MOE_CHECK(aligned4(logits) && aligned4(topk_ids) && aligned4(topk_w) && (!bias || aligned4(bias)), MOE_EINVAL);
  const int V = (E + kWave - 1) / kWave;
  if (V <= 1) launch_grouped<1>(logits, T, E, k, sig, n_group, topk_group, route_scale, bias, topk_ids, topk_w, dev_flags, stream);
  else if (V <= 2) launch_grouped<2>(logits, T, E, k, sig, n_group, topk_group, route_scale, bias, topk_ids, topk_w, dev_flags, stream);
  else if (V <= 4) launch_grouped<4>(logits, T, E, k, sig, n_group, topk_group, route_scale, bias, topk_ids, topk_w, dev_flags, stream);
  else if (V <= 8) launch_grouped<8>(logits, T, E, k, sig, n_group, topk_group, route_scale, bias, topk_ids, topk_w, dev_flags, stream);
  else launch_grouped<16>(logits, T, E, k, sig, n_group, topk_group, route_scale, bias, topk_ids, topk_w, dev_flags, stream);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
