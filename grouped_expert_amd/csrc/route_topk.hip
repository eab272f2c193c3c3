// Router top-k with renormalised softmax gates, one wavefront per token.
//
// "M6.2 - Expert Parallelism and DeepSeek MoE", 0x06L1 (Mixtral row): FP32
// softmax over all experts, keep the top k, renormalise the kept mass to one.
// "M6.6 - MoE Runtime Systems", 0x0AE: logits and the top-k comparison in
// FP32.  Softmax is monotone, so the k largest logits are selected directly;
// the full-softmax denominator cancels in the renormalised gates.
//
// Each lane holds up to V = ceil(E/64) logits (expert e = lane + 64*v).  A
// logit becomes an order-preserving 32-bit key (+0 and -0 share one key) and
// is packed with the complement of its expert index into 64 bits, so one
// unsigned max picks the largest logit and, among equal logits, the lowest
// expert.  k rounds of a wavefront max (butterfly shuffles) pick the experts
// in order; the winner's owner lane clears that slot.
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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off, kWave);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off, kWave);
    const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
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

  uint64_t slot[V];
  bool bad = false;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int e = lane + v * kWave;
    slot[v] = 0;
    if (e < E) {
      const float z = row[e];
      bad |= !isfinite(z);
      slot[v] = (static_cast<uint64_t>(order_key(z)) << 32) | static_cast<uint32_t>(~e);
    }
  }
  const bool token_bad = ballot(bad) != 0;

  // k selection rounds; lane j keeps the j-th winner.
  uint64_t mine = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) best = slot[v] > best ? slot[v] : best;
    best = wave_max_u64(best);
    const int e = static_cast<int>(~static_cast<uint32_t>(best));
    if (lane == (e % kWave)) {
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (v == e / kWave) slot[v] = 0;
    }
    if (lane == j) mine = best;
  }

  const float z = key_value(static_cast<uint32_t>(mine >> 32));
  const float z0 = __shfl(z, 0, kWave);
  const float p = lane < k ? expf(z - z0) : 0.0f;
  const float s = wave_sum_f32(p);
  if (lane < k) {
    const int e = static_cast<int>(~static_cast<uint32_t>(mine));
    ids[t * k + lane] = token_bad ? -1 : e;
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
