// Deterministic stable bucket ranking, shared by the permute, the pooled-wave
// pack and the receiver compaction.
//
// Given n items in index order and a bucket id per item (or none), it
// produces, without any order-dependent atomics:
//   sel[b]      items in bucket b
//   counts[b]   min(sel[b], cap)              (cap < 0: no cap)
//   offsets     exclusive prefix of counts, offsets[B] = accepted total
//   pos_i       #{i' < i : bucket(i') = bucket(i)}   (handed to an emitter)
// This is the count / exclusive prefix / stable permutation of "M6.2 -
// Expert Parallelism and DeepSeek MoE", 0x03B, with the capacity of 0x01C.
//
// A Bucket functor has load(i) -> raw 32-bit value of item i (no side
// effects) and classify(raw, flags) -> bucket or -1 (may raise a flag), so
// that a wavefront can issue the loads of all its steps before using any.
//
// Three launches:
//   1. count: one wavefront walks one chunk of 64*steps items and builds the
//      chunk's bucket histogram in LDS (LDS atomics: counts do not depend on
//      order); the histogram is stored chunk-major, table[c*B + b].
//   2. scan: one workgroup turns the table into per-(chunk, bucket) exclusive
//      prefixes over chunks, and forms sel / counts / offsets / dropped.
//   3. emit: each wavefront walks its chunk again, 64 items per step; lanes
//      with equal bucket find each other with ceil(log2(B+1)) ballots, the
//      in-step rank is a popcount of the lower-lane peers, and the chunk's
//      running base per bucket lives in LDS.  pos is therefore exactly the
//      route-order rank.
#pragma once

#include "common.h"

namespace moe {
namespace {   // every translation unit gets its own copy of these kernels

constexpr int kRankWaves = 4;                 // wavefronts per workgroup in passes 1 and 3
constexpr int kRankThreads = kRankWaves * kWave;
constexpr int kRankMaxSteps = 32;             // steps per chunk (bounded by rank_geom)

struct RankGeom {
  int64_t n;       // items
  int32_t B;       // buckets (1..MOE_MAX_EXPERTS)
  int32_t steps;   // 64-item steps per chunk
  int64_t chunks;  // ceil(n / (64*steps))
  int32_t nbits;   // bits of a bucket code in [0, B]
};

inline RankGeom rank_geom(int64_t n, int32_t B) {
  RankGeom g;
  g.n = n;
  g.B = B;
  // at least 4 steps (256 items) per chunk and at most 32 (2048 items),
  // aiming at about 512 chunks: two wavefronts per CU in passes 1 and 3,
  // while the one-workgroup scan still reads only chunks * B table entries
  int64_t s = (n + 64 * 512 - 1) / (64 * 512);
  g.steps = static_cast<int32_t>(s < 4 ? 4 : (s > kRankMaxSteps ? kRankMaxSteps : s));
  const int64_t chunk = 64ll * g.steps;
  g.chunks = (n + chunk - 1) / chunk;
  int bits = 0;
  while ((1 << bits) <= B) ++bits;
  g.nbits = bits;
  return g;
}

inline size_t rank_table_bytes(const RankGeom& g) {
  return align_up(static_cast<size_t>(g.chunks > 0 ? g.chunks : 1) * g.B * sizeof(int32_t), 256);
}

// ---- pass 1 -----------------------------------------------------------------

template <class Bucket>
__global__ __launch_bounds__(kRankThreads) void rank_count_kernel(Bucket bucket, RankGeom g,
                                                                  int32_t* __restrict__ table,
                                                                  uint32_t* flags) {
  extern __shared__ int32_t lds[];
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  int32_t* h = lds + w * g.B;
  for (int b = lane; b < g.B; b += kWave) h[b] = 0;
  __syncthreads();
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kRankWaves + w;
  if (c < g.chunks) {
    const int64_t base = c * 64 * g.steps;
    uint32_t raw[kRankMaxSteps];
#pragma unroll
    for (int s = 0; s < kRankMaxSteps; ++s) {
      const int64_t i = base + s * 64 + lane;
      if (s < g.steps && i < g.n) raw[s] = bucket.load(i);
    }
#pragma unroll
    for (int s = 0; s < kRankMaxSteps; ++s) {
      const int64_t i = base + s * 64 + lane;
      if (s < g.steps && i < g.n) {
        const int b = bucket.classify(raw[s], flags);
        if (b >= 0) atomicAdd(&h[b], 1);
      }
    }
  }
  __syncthreads();
  if (c < g.chunks)
    for (int b = lane; b < g.B; b += kWave) table[c * g.B + b] = h[b];
}

// ---- pass 2 -----------------------------------------------------------------

struct RankScanOut {
  int32_t* sel;       // [B] or nullptr
  int32_t* counts;    // [B] or nullptr
  int32_t* offsets;   // [B+1] (required: pass 3 reads it)
  int32_t* dropped;   // [1] or nullptr
  int32_t drop_all_items;  // 1: dropped = n - accepted; 0: dropped = sum(sel) - accepted
};

__global__ __launch_bounds__(1024) void rank_scan_kernel(RankGeom g, int64_t cap,
                                                         int32_t* __restrict__ table, RankScanOut out) {
  __shared__ int32_t part[1024];
  __shared__ int32_t sh16[17];
  const int t = threadIdx.x;
  const int tpb = 1024 / g.B;                   // >= 1 since B <= 1024
  const int active = g.B * tpb;
  const int b = t % g.B, sub = t / g.B;
  const int64_t per = (g.chunks + tpb - 1) / tpb;
  const int64_t c0 = static_cast<int64_t>(sub) * per;
  const int64_t c1 = c0 + per < g.chunks ? c0 + per : g.chunks;
  int32_t sum = 0;
  if (t < active) {
#pragma unroll 8
    for (int64_t c = c0; c < c1; ++c) sum += table[c * g.B + b];
  }
  part[t] = t < active ? sum : 0;
  __syncthreads();
  if (t < active) {
    int32_t run = 0;
    for (int s = 0; s < sub; ++s) run += part[s * g.B + b];
#pragma unroll 8
    for (int64_t c = c0; c < c1; ++c) {
      const int32_t v = table[c * g.B + b];
      table[c * g.B + b] = run;
      run += v;
    }
  }
  int32_t sel = 0;
  if (t < g.B)
    for (int s = 0; s < tpb; ++s) sel += part[s * g.B + t];
  const int32_t cnt = t < g.B ? (cap < 0 ? sel : (sel < cap ? sel : static_cast<int32_t>(cap))) : 0;
  int32_t accepted = 0;
  const int32_t off = block_exclusive_scan_1024(cnt, sh16, &accepted);
  __syncthreads();
  int32_t sel_total = 0;
  (void)block_exclusive_scan_1024(t < g.B ? sel : 0, sh16, &sel_total);
  if (t < g.B) {
    if (out.sel) out.sel[t] = sel;
    if (out.counts) out.counts[t] = cnt;
    out.offsets[t] = off;
  }
  if (t == 0) {
    out.offsets[g.B] = accepted;
    if (out.dropped)
      out.dropped[0] = out.drop_all_items ? static_cast<int32_t>(g.n - accepted) : sel_total - accepted;
  }
}

// ---- pass 3 -----------------------------------------------------------------

// Emit is called for every item i < n as emit(i, b, pos); b = -1 (no bucket)
// comes with pos = -1.
template <class Bucket, class Emit>
__global__ __launch_bounds__(kRankThreads) void rank_emit_kernel(Bucket bucket, Emit emit, RankGeom g,
                                                                 const int32_t* __restrict__ table) {
  extern __shared__ int32_t lds[];
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  int32_t* h = lds + w * g.B;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kRankWaves + w;
  if (c < g.chunks)
    for (int b = lane; b < g.B; b += kWave) h[b] = table[c * g.B + b];
  __syncthreads();
  if (c >= g.chunks) return;
  const uint64_t lt = lanemask_lt();
  const int64_t base = c * 64 * g.steps;
  // batches of 8 steps: the 8 loads are issued before the first is used
  for (int s0 = 0; s0 < g.steps; s0 += 8) {
    uint32_t raw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = base + (s0 + u) * 64 + lane;
      if (s0 + u < g.steps && i < g.n) raw[u] = bucket.load(i);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (s0 + u < g.steps) {
        const int64_t i = base + (s0 + u) * 64 + lane;
        const bool in = i < g.n;
        const int b = in ? bucket.classify(raw[u], nullptr) : -1;
        const int code = b >= 0 ? b : g.B;
        uint64_t peers = ~0ull;
        for (int bit = 0; bit < g.nbits; ++bit) {
          const bool on = (code >> bit) & 1;
          const uint64_t m = ballot(on);
          peers &= on ? m : ~m;
        }
        if (b >= 0) {
          const int32_t rank = __popcll(peers & lt);
          const int32_t cnt = __popcll(peers);
          const int32_t start = h[b];
          emit(i, b, start + rank);
          if (rank == 0) h[b] = start + cnt;
        } else if (in) {
          emit(i, -1, -1);
        }
      }
    }
  }
}

// ---- host driver --------------------------------------------------------------

template <class Bucket, class Emit>
inline int bucket_rank(const RankGeom& g, Bucket bucket, Emit emit, int64_t cap, RankScanOut out,
                       int32_t* table, uint32_t* flags, hipStream_t stream) {
  if (g.n == 0) {
    // nothing to rank: zero the counters with the scan kernel on an empty table
    RankGeom z = g;
    z.chunks = 0;
    hipLaunchKernelGGL(rank_scan_kernel, dim3(1), dim3(1024), 0, stream, z, cap, table, out);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
  }
  const unsigned blocks = static_cast<unsigned>((g.chunks + kRankWaves - 1) / kRankWaves);
  const size_t lds = static_cast<size_t>(kRankWaves) * g.B * sizeof(int32_t);
  hipLaunchKernelGGL(HIP_KERNEL_NAME(rank_count_kernel<Bucket>), dim3(blocks), dim3(kRankThreads), lds,
                     stream, bucket, g, table, flags);
  MOE_LAUNCH_CHECK();
  hipLaunchKernelGGL(rank_scan_kernel, dim3(1), dim3(1024), 0, stream, g, cap, table, out);
  MOE_LAUNCH_CHECK();
  hipLaunchKernelGGL(HIP_KERNEL_NAME(rank_emit_kernel<Bucket, Emit>), dim3(blocks), dim3(kRankThreads),
                     lds, stream, bucket, emit, g, table);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace
}  // namespace moe
