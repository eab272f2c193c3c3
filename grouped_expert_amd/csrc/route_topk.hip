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

// ---------------------------------------------------------------------------
// moe_route_topk: L lanes per token (L = 1..16, a power of two), V logits per
// lane (expert e = 4 (l + L j) + q for value v = 4 j + q with 16-byte loads,
// or e = l + L v with 4-byte loads), KL = the power of two >= k.
//
// 1. Each lane keeps the KL largest of its values as a sorted list: inserting
//    x into a descending list a is a'_0 = max(a_0, x), a'_i = med3(a_{i-1},
//    a_i, x) -- one v_med3_f32 per list entry and value, no data-dependent
//    branch.
// 2. log2(L) butterfly steps merge the lists of a token's lanes (the partner's
//    list arrives through a DPP lane permutation): c_i = max(a_i,
//    b_{KL-1-i}) is a bitonic sequence holding the KL largest of both, and
//    log2(KL) half-cleaner stages sort it.  Every lane of the token then holds
//    the token's KL largest values t_0 >= ... >= t_{KL-1}, ties included.
// 3. With tau = t_{k-1}, every value >= tau is a candidate; each lane writes
//    its candidates (value, expert) to its LDS slots.  If the token has
//    exactly k candidates and t_0 > t_1 > ... > t_{k-1}, candidate x takes
//    slot #{i < k : t_i > x}, which is its rank (no two candidates are equal).
// 4. Otherwise (equal values among or at the boundary of the k largest) the
//    token takes k exact rounds over its lanes: the largest remaining value,
//    then the lowest expert holding it (ties to the lower expert).
// Values are compared as fp32 numbers (-0 == +0); a token with a NaN or
// infinite logit gets ids -1 and weights 0.
constexpr int kRouteThreads = 256;
// Padding past the last expert: finite (so x * 0 stays 0) and below every
// finite logit but -FLT_MAX itself, which it ties with; a tie puts the lower
// (real) expert first, and k <= E real experts always exist.
constexpr float kPad = -3.402823466e+38f;
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dppi(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// Butterfly partner patterns inside a 16-lane row: xor 1, xor 2, then the
// half-row mirror (i <-> 7 - i) and the row mirror (i <-> 15 - i), which pair
// the two merged halves of 8- and 16-lane groups.
template <int STEP>
struct Partner;
template <> struct Partner<0> { static constexpr int C = 0xB1; };
template <> struct Partner<1> { static constexpr int C = 0x4E; };
template <> struct Partner<2> { static constexpr int C = 0x141; };
template <> struct Partner<3> { static constexpr int C = 0x140; };

// max / min as one v_med3_f32 each (fmaxf / fminf would first quiet every
// operand; NaN tokens are detected separately and their selection discarded)
__device__ __forceinline__ float fmax1(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, INFINITY); }
__device__ __forceinline__ float fmin1(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, -INFINITY); }

template <int KL, int STEP>
__device__ __forceinline__ void merge_step(float (&a)[KL]) {
  constexpr int CT = Partner<STEP>::C;
  float c[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i) c[i] = fmax1(a[i], dppf<CT>(a[KL - 1 - i]));
#pragma unroll
  for (int st = KL / 2; st >= 1; st /= 2)
#pragma unroll
    for (int i = 0; i < KL; ++i)
      if ((i & st) == 0) {
        const float hi = fmax1(c[i], c[i + st]), lo = fmin1(c[i], c[i + st]);
        c[i] = hi;
        c[i + st] = lo;
      }
#pragma unroll
  for (int i = 0; i < KL; ++i) a[i] = c[i];
}

template <int STEP>
__device__ __forceinline__ float group_sum_step(float v) { return v + dppf<Partner<STEP>::C>(v); }
template <int STEP>
__device__ __forceinline__ int group_isum_step(int v) { return v + dppi<Partner<STEP>::C>(v); }
template <int STEP>
__device__ __forceinline__ float group_max_step(float v) { return fmax1(v, dppf<Partner<STEP>::C>(v)); }
template <int STEP>
__device__ __forceinline__ int group_imin_step(int v) {
  const int o = dppi<Partner<STEP>::C>(v);
  return o < v ? o : v;
}

// reductions over the L lanes of a token (L a power of two, 1..16)
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  if (L >= 2) v = group_sum_step<0>(v);
  if (L >= 4) v = group_sum_step<1>(v);
  if (L >= 8) v = group_sum_step<2>(v);
  if (L >= 16) v = group_sum_step<3>(v);
  return v;
}
template <int L>
__device__ __forceinline__ int group_isum(int v) {
  if (L >= 2) v = group_isum_step<0>(v);
  if (L >= 4) v = group_isum_step<1>(v);
  if (L >= 8) v = group_isum_step<2>(v);
  if (L >= 16) v = group_isum_step<3>(v);
  return v;
}
template <int L>
__device__ __forceinline__ float group_max(float v) {
  if (L >= 2) v = group_max_step<0>(v);
  if (L >= 4) v = group_max_step<1>(v);
  if (L >= 8) v = group_max_step<2>(v);
  if (L >= 16) v = group_max_step<3>(v);
  return v;
}
template <int L>
__device__ __forceinline__ int group_imin(int v) {
  if (L >= 2) v = group_imin_step<0>(v);
  if (L >= 4) v = group_imin_step<1>(v);
  if (L >= 8) v = group_imin_step<2>(v);
  if (L >= 16) v = group_imin_step<3>(v);
  return v;
}

// 48 values per lane (384 experts on 8 lanes): five workgroups per CU (at
// most 102 VGPRs, a few dwords spilled) hide the loads better than three
// (168 VGPRs): 23.4 against 24.3 us for 65,536 tokens
template <int L, int V, int KL, bool VEC>
__global__ __launch_bounds__(kRouteThreads, V == 48 ? 5 : 1) void route_list_kernel(
    const float* __restrict__ logits, int64_t T, int32_t E, int32_t k, int32_t full_mass,
    int32_t* __restrict__ ids, float* __restrict__ weights, uint32_t* flags) {
  __shared__ uint2 cand[kRouteThreads * KL];           // (value bits, expert) candidates, KL per lane
  const int lane = threadIdx.x % kWave;
  const int l = lane % L;                               // position inside the token's lanes
  const int64_t tpb = kRouteThreads / L;                // tokens per block
  const int64_t t = static_cast<int64_t>(blockIdx.x) * tpb + threadIdx.x / L;
  const bool live = t < T;                              // lanes of a missing token still join the DPP steps
  const float* row = logits + (live ? t : 0) * E;

  // values and their expert ids
  auto expert_of = [&](int v) { return VEC ? 4 * (l + L * (v / 4)) + v % 4 : l + L * v; };
  auto load_values = [&](float (&val)[V]) {
    if constexpr (VEC) {
#pragma unroll
      for (int j = 0; j < V / 4; ++j) {
        const int e0 = 4 * (l + L * j);
        f32x4 q = {kPad, kPad, kPad, kPad};
        if (live && e0 < E) q = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + e0));
        val[4 * j] = q[0];
        val[4 * j + 1] = q[1];
        val[4 * j + 2] = q[2];
        val[4 * j + 3] = q[3];
      }
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int e = l + L * v;
        val[v] = live && e < E ? __builtin_nontemporal_load(row + e) : kPad;
      }
    }
  };
  float val[V];
  load_values(val);

  // 1. per-lane sorted list of the KL largest; x * 0 is 0 for finite x and NaN otherwise
  float lst[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i) lst[i] = -INFINITY;
  float nf = 0.0f;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const float x = val[v];
    nf = fmaf(x, 0.0f, nf);
#pragma unroll
    for (int i = KL - 1; i >= 1; --i) lst[i] = __builtin_amdgcn_fmed3f(lst[i - 1], lst[i], x);
    lst[0] = fmax1(lst[0], x);
  }
  // 2. merge the token's lists
  if (L >= 2) merge_step<KL, 0>(lst);
  if (L >= 4) merge_step<KL, 1>(lst);
  if (L >= 8) merge_step<KL, 2>(lst);
  if (L >= 16) merge_step<KL, 3>(lst);
  const bool bad = group_sum<L>(nf != 0.0f ? 1.0f : 0.0f) != 0.0f;     // NaN != 0 as well
  float tau = lst[0];
#pragma unroll
  for (int i = 1; i < KL; ++i) tau = i == k - 1 ? lst[i] : tau;
  const float z0 = lst[0];

  // gate denominator: the k kept values, or (V1) every expert's logit
  float denom;
  if (full_mass) {
    float m = 0.0f;
#pragma unroll
    for (int v = 0; v < V; ++v) m += __expf(val[v] - z0);       // padding adds exp(-FLT_MAX - z0) = 0
    denom = group_sum<L>(m);
  } else {
    denom = 0.0f;
#pragma unroll
    for (int i = 0; i < KL; ++i)
      if (i < k) denom += __expf(lst[i] - z0);
  }

  const float rden = 1.0f / denom;

  // 3. candidates
  uint2* mine = cand + threadIdx.x * KL;
  int cnt = 0;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    if (val[v] >= tau) {
      // past KL candidates the last slot is overwritten: more than k
      // candidates send the token to the exact rounds anyway
      mine[cnt < KL ? cnt : KL - 1] = make_uint2(__float_as_uint(val[v]), static_cast<uint32_t>(expert_of(v)));
      ++cnt;
    }
  }
  const int n_cand = group_isum<L>(cnt);
  bool strict = true;
#pragma unroll
  for (int i = 0; i + 1 < KL; ++i)
    if (i + 1 < k) strict = strict && lst[i] > lst[i + 1];
  const bool fast = n_cand == k && strict;
  int32_t* out_ids = ids + (live ? t : 0) * k;
  float* out_w = weights + (live ? t : 0) * k;
  if (live && bad) {
    if (l == 0) flag_or(flags, MOE_FLAG_NONFINITE_LOGIT);
    for (int j = l; j < k; j += L) {
      out_ids[j] = -1;
      out_w[j] = 0.0f;
    }
  }
  if (live && !bad && fast) {
    for (int c = 0; c < cnt && c < KL; ++c) {
      const uint2 cv = mine[c];
      const float x = __uint_as_float(cv.x);
      int slot = 0;
#pragma unroll
      for (int i = 0; i < KL; ++i) slot += (i < k && lst[i] > x) ? 1 : 0;
      out_ids[slot] = static_cast<int32_t>(cv.y);
      out_w[slot] = __expf(x - z0) * rden;
    }
  }
  // 4. exact rounds for tokens with equal values (every lane of the wave
  // joins the reductions; only such tokens' lanes write)
  const bool slow = live && !bad && !fast;
  if (ballot(slow) != 0) {
    for (int r = 0; r < k; ++r) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        if (val[v] > bv) {                              // strict: the first (lowest) expert among equals
          bv = val[v];
          be = expert_of(v);
        }
      }
      const float gmax = group_max<L>(bv);
      const int emin = group_imin<L>(bv == gmax ? be : 0x7fffffff);
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (expert_of(v) == emin) val[v] = -INFINITY;   // taken (valid tokens hold finite values only)
      if (slow && l == 0) {
        out_ids[r] = emin;
        out_w[r] = __expf(gmax - z0) * rden;
      }
    }
  }
}

template <int L, int V, int KL, bool VEC>
void launch_list(const float* logits, int64_t T, int32_t E, int32_t k, int32_t full, int32_t* ids, float* w,
                 uint32_t* flags, hipStream_t s) {
  constexpr int64_t tpb = kRouteThreads / L;
  const unsigned blocks = static_cast<unsigned>((T + tpb - 1) / tpb);
  hipLaunchKernelGGL(HIP_KERNEL_NAME(route_list_kernel<L, V, KL, VEC>), dim3(blocks), dim3(kRouteThreads), 0, s,
                     logits, T, E, k, full, ids, w, flags);
}

template <int L, int KL>
void launch_list_v(int V, const float* logits, int64_t T, int32_t E, int32_t k, int32_t full, int32_t* ids,
                   float* w, uint32_t* flags, hipStream_t s) {
  if (V <= 8) launch_list<L, 8, KL, true>(logits, T, E, k, full, ids, w, flags, s);
  else if (V <= 16) launch_list<L, 16, KL, true>(logits, T, E, k, full, ids, w, flags, s);
  else if (V <= 24) launch_list<L, 24, KL, true>(logits, T, E, k, full, ids, w, flags, s);
  else if (V <= 32) launch_list<L, 32, KL, true>(logits, T, E, k, full, ids, w, flags, s);
  else if (V <= 48) launch_list<L, 48, KL, true>(logits, T, E, k, full, ids, w, flags, s);
  else launch_list<L, 64, KL, true>(logits, T, E, k, full, ids, w, flags, s);
}

template <int KL>
void launch_list_lv(int L, int V, const float* logits, int64_t T, int32_t E, int32_t k, int32_t full,
                    int32_t* ids, float* w, uint32_t* flags, hipStream_t s) {
  switch (L) {
    case 1: launch_list_v<1, KL>(V, logits, T, E, k, full, ids, w, flags, s); break;
    case 2: launch_list_v<2, KL>(V, logits, T, E, k, full, ids, w, flags, s); break;
    case 4: launch_list_v<4, KL>(V, logits, T, E, k, full, ids, w, flags, s); break;
    case 8: launch_list_v<8, KL>(V, logits, T, E, k, full, ids, w, flags, s); break;
    default: launch_list_v<16, KL>(V, logits, T, E, k, full, ids, w, flags, s); break;
  }
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

// The same router with 16 lanes per token (4 tokens per wavefront), for
// shapes where every lane holds the same groups: V = E / 16 values per lane
// (expert e = l + 16 v) and M = G / 16 values of each group per lane (value v
// in group v / M).  Every reduction runs over the token's 16 lanes (one DPP
// row) instead of the wavefront, which cuts the instructions per token.  The
// decisions are those of route_grouped_kernel: group scores from the same
// keys (V3: the fp32 sum of the two largest, a multiset of the group's keys;
// V2: the largest), topk_group rounds taking the largest score and the lowest
// group among equals, then k rounds taking the largest key and the lowest
// expert among equals, the winner's key cleared.
__device__ __forceinline__ uint32_t row16_umax(uint32_t v) {
  v = umax(v, dpp<0xB1>(v));
  v = umax(v, dpp<0x4E>(v));
  v = umax(v, dpp<0x141>(v));
  return umax(v, dpp<0x140>(v));
}
__device__ __forceinline__ uint32_t row16_umin(uint32_t v) {
  v = umin(v, dpp<0xB1>(v));
  v = umin(v, dpp<0x4E>(v));
  v = umin(v, dpp<0x141>(v));
  return umin(v, dpp<0x140>(v));
}
__device__ __forceinline__ uint32_t row16_or(uint32_t v) {
  v |= dpp<0xB1>(v);
  v |= dpp<0x4E>(v);
  v |= dpp<0x141>(v);
  return v | dpp<0x140>(v);
}
__device__ __forceinline__ float row16_sum(float v) {
  v += __uint_as_float(dpp<0xB1>(__float_as_uint(v)));
  v += __uint_as_float(dpp<0x4E>(__float_as_uint(v)));
  v += __uint_as_float(dpp<0x141>(__float_as_uint(v)));
  return v + __uint_as_float(dpp<0x140>(__float_as_uint(v)));
}

template <int V, int M>
__global__ __launch_bounds__(256) void route_grouped16_kernel(
    const float* __restrict__ logits, int64_t T, int32_t E, int32_t k, int32_t sigmoid_bias, int32_t topk_group,
    float route_scale, const float* __restrict__ bias, int32_t* __restrict__ ids, float* __restrict__ weights,
    uint32_t* flags) {
  constexpr int L = 16, NG = V / M;
  static_assert(V % M == 0 && NG <= 32, "whole groups per lane");
  const int l = threadIdx.x % L;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (256 / L) + threadIdx.x / L;
  const bool live = t < T;                              // a missing token's lanes compute on zeros
  const float* row = logits + (live ? t : 0) * E;

  uint32_t key[V];
  float val[V];
  bool bad = false;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int e = l + L * v;
    const float z = live ? __builtin_nontemporal_load(row + e) : 0.0f;
    bad |= !isfinite(z);
    if (sigmoid_bias) {
      // as in route_grouped_kernel: fp64 sigmoid rounded once to fp32, plus the bias in fp32
      const float sg = static_cast<float>(1.0 / (1.0 + exp(-static_cast<double>(z))));
      const float c = sg + (bias ? bias[e] : 0.0f);
      bad |= !isfinite(c);
      key[v] = order_key(c);
      val[v] = sg;
    } else {
      key[v] = order_key(z);
      val[v] = z;
    }
  }
  const bool token_bad = row16_or(bad ? 1u : 0u) != 0;

  // group scores (every lane of the token ends with all of them)
  uint32_t gkey[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    uint32_t k1 = 0, k2 = 0;                            // two largest keys, k1 >= k2
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const uint32_t x = key[g * M + i];
      k2 = umax(k2, umin(k1, x));
      k1 = umax(k1, x);
    }
    if (sigmoid_bias) {
#define MOE_TOP2_STEP(CT)                                              \
  {                                                                    \
    const uint32_t b1 = dpp<CT>(k1), b2 = dpp<CT>(k2);                 \
    k2 = umax(umin(k1, b1), umax(k2, b2));                             \
    k1 = umax(k1, b1);                                                 \
  }
      MOE_TOP2_STEP(0xB1)
      MOE_TOP2_STEP(0x4E)
      MOE_TOP2_STEP(0x141)
      MOE_TOP2_STEP(0x140)
#undef MOE_TOP2_STEP
      gkey[g] = order_key(key_value(k1) + key_value(k2));
    } else {
      gkey[g] = row16_umax(k1);
    }
  }
  // topk_group rounds: the largest score, the lowest group among equals
  uint32_t kept = 0;
  for (int r = 0; r < topk_group; ++r) {
    uint32_t best = 0;
    int bg = -1;
#pragma unroll
    for (int g = 0; g < NG; ++g)
      if (!((kept >> g) & 1u) && gkey[g] > best) {
        best = gkey[g];
        bg = g;
      }
    if (bg >= 0) kept |= 1u << bg;
  }
#pragma unroll
  for (int v = 0; v < V; ++v)
    if (!((kept >> (v / M)) & 1u)) key[v] = 0;

  // k rounds over the token's lanes
  int32_t mine_e = 0;
  float mine_val = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint32_t lmax = key[0];
#pragma unroll
    for (int v = 1; v < V; ++v) lmax = umax(lmax, key[v]);
    const uint32_t K = row16_umax(lmax);
    uint32_t lmin = 0xFFFFFFFFu;
#pragma unroll
    for (int v = V - 1; v >= 0; --v) lmin = key[v] == K ? static_cast<uint32_t>(l + L * v) : lmin;
    const uint32_t ew = row16_umin(lmin);
    const int vw = static_cast<int>(ew / L), lw = static_cast<int>(ew % L);
    uint32_t vb = 0;
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (v == vw && l == lw) {
        vb = __float_as_uint(val[v]);
        key[v] = 0;
      }
    const float wv = __uint_as_float(row16_or(vb));      // the winner's value (the other lanes give 0 bits)
    if (l == j) {
      mine_e = static_cast<int32_t>(ew);
      mine_val = wv;
    }
  }

  float gate;
  if (sigmoid_bias) {
    const float ssum = row16_sum(l < k ? mine_val : 0.0f);
    gate = route_scale * mine_val / ssum;
  } else {
    uint32_t lmax = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) lmax = umax(lmax, order_key(val[v]));
    const float zmax = key_value(row16_umax(lmax));
    float mass = 0.0f;
#pragma unroll
    for (int v = 0; v < V; ++v) mass += expf(val[v] - zmax);
    const float denom = row16_sum(mass);
    gate = route_scale * expf(mine_val - zmax) / denom;
  }
  if (live && l < k) {
    ids[t * k + l] = token_bad ? -1 : mine_e;
    weights[t * k + l] = token_bad ? 0.0f : gate;
  }
  if (live && token_bad && l == 0) flag_or(flags, MOE_FLAG_NONFINITE_LOGIT);
}

template <int V, int M>
void launch_grouped16(const float* logits, int64_t T, int32_t E, int32_t k, int32_t sigmoid_bias, int32_t topk_group,
                      float scale, const float* bias, int32_t* ids, float* w, uint32_t* flags, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((T + 15) / 16);
  hipLaunchKernelGGL(HIP_KERNEL_NAME(route_grouped16_kernel<V, M>), dim3(blocks), dim3(256), 0, s, logits, T, E, k,
                     sigmoid_bias, topk_group, scale, bias, ids, w, flags);
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
  // 16-byte loads when every row starts on a 16-byte boundary
  const int vec = (E % 4 == 0 && aligned16(logits)) ? 1 : 0;
  if (!vec) {
    // rows not on 16-byte boundaries: one general configuration with 4-byte
    // loads (16 lanes of up to 64 values, lists of 16)
    launch_list<16, 64, 16, false>(logits, T, E, k, full, topk_ids, topk_w, dev_flags, stream);
  } else {
    // lanes per token: the fewest (a power of two) that hold at most 64 values
    // each, then more while the grid would give fewer than 2048 wavefronts
    auto values_per_lane = [&](int L) { return 4 * ((E + 4 * L - 1) / (4 * L)); };
    int L = 1;
    while (L < 16 && values_per_lane(L) > 64) L *= 2;
    while (L < 16 && T * L < 2048 * static_cast<int64_t>(kWave) && values_per_lane(2 * L) >= 4) L *= 2;
    const int V = values_per_lane(L);
    const int KL = k <= 2 ? 2 : (k <= 4 ? 4 : (k <= 8 ? 8 : 16));
    if (KL == 2) launch_list_lv<2>(L, V, logits, T, E, k, full, topk_ids, topk_w, dev_flags, stream);
    else if (KL == 4) launch_list_lv<4>(L, V, logits, T, E, k, full, topk_ids, topk_w, dev_flags, stream);
    else if (KL == 8) launch_list_lv<8>(L, V, logits, T, E, k, full, topk_ids, topk_w, dev_flags, stream);
    else launch_list_lv<16>(L, V, logits, T, E, k, full, topk_ids, topk_w, dev_flags, stream);
  }
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
  // 16 lanes per token where the groups fall evenly on the lanes
  const int G = E / n_group;
  if (E % 16 == 0 && G % 16 == 0 && k <= 16) {
    const int V16 = E / 16, M16 = G / 16;
    bool done = true;
    if (V16 == 16 && M16 == 1) launch_grouped16<16, 1>(logits, T, E, k, sig, topk_group, route_scale, bias, topk_ids, topk_w, dev_flags, stream);
    else if (V16 == 16 && M16 == 2) launch_grouped16<16, 2>(logits, T, E, k, sig, topk_group, route_scale, bias, topk_ids, topk_w, dev_flags, stream);
    else if (V16 == 16 && M16 == 4) launch_grouped16<16, 4>(logits, T, E, k, sig, topk_group, route_scale, bias, topk_ids, topk_w, dev_flags, stream);
    else if (V16 == 8 && M16 == 1) launch_grouped16<8, 1>(logits, T, E, k, sig, topk_group, route_scale, bias, topk_ids, topk_w, dev_flags, stream);
    else if (V16 == 8 && M16 == 2) launch_grouped16<8, 2>(logits, T, E, k, sig, topk_group, route_scale, bias, topk_ids, topk_w, dev_flags, stream);
    else done = false;
    if (done) {
      MOE_LAUNCH_CHECK();
      return MOE_OK;
    }
  }
  const int V = (E + kWave - 1) / kWave;
  if (V <= 1) launch_grouped<1>(logits, T, E, k, sig, n_group, topk_group, route_scale, bias, topk_ids, topk_w, dev_flags, stream);
  else if (V <= 2) launch_grouped<2>(logits, T, E, k, sig, n_group, topk_group, route_scale, bias, topk_ids, topk_w, dev_flags, stream);
  else if (V <= 4) launch_grouped<4>(logits, T, E, k, sig, n_group, topk_group, route_scale, bias, topk_ids, topk_w, dev_flags, stream);
  else if (V <= 8) launch_grouped<8>(logits, T, E, k, sig, n_group, topk_group, route_scale, bias, topk_ids, topk_w, dev_flags, stream);
  else launch_grouped<16>(logits, T, E, k, sig, n_group, topk_group, route_scale, bias, topk_ids, topk_w, dev_flags, stream);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
