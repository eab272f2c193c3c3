// Dispatch permutation: expert histogram, exclusive prefix, capacity and
// stable ranks (shared bucket-rank passes), then the row movement (token-major
// scatter: each token row is read once and written to its accepted slots).
//
// "M6.2 - Expert Parallelism and DeepSeek MoE", 0x03B: counts, exclusive
// prefix with the final sentinel, stable permutation by (expert, route id)
// and its inverse; 0x01C: capacity turns routing into bounded buffers and the
// overflow is dropped.  "M6.6 - MoE Runtime Systems", 0x03A: route rows are
// gathered from the hidden states (one copy per route); 0x0CD: accepted plus
// dropped routes equal T*k and the counts sum to the accepted total.
#include <atomic>

#include "bucket_rank.h"
#include "fp8.h"

namespace moe {
namespace {

struct ExpertBucket {
  const int32_t* ids;
  int32_t E;
  __device__ uint32_t load(int64_t r) const { return static_cast<uint32_t>(ids[r]); }
  __device__ int classify(uint32_t raw, uint32_t* flags) const {
    const int32_t e = static_cast<int32_t>(raw);
    if (e >= 0 && e < E) return e;
    if (e != -1) flag_or(flags, MOE_FLAG_BAD_EXPERT);
    return -1;
  }
};

struct PermuteEmit {
  int64_t cap, R;
  const int32_t* offsets;
  int32_t* inv;
  int32_t* src;
  __device__ void operator()(int64_t r, int e, int32_t pos) const {
    if (e >= 0 && (cap < 0 || pos < cap)) {
      const int32_t p = offsets[e] + pos;
      inv[r] = p;
      if (p >= 0 && p < R) src[p] = static_cast<int32_t>(r);
    } else {
      inv[r] = -1;
    }
  }
};

// One wavefront per token: the token row is read once into registers (up to
// kPiece x 16 B per lane at a time) and written to each of its accepted
// slots x_perm[inv[t*k + j]], so x is read once instead of k times.  Every
// thread also clears one entry of the tail src[A .. R) (the grid has 64T >= R
// threads), which the bucket-rank passes leave unwritten.
constexpr int kTokPerBlock = 4;
constexpr int kPiece = 8;

__global__ __launch_bounds__(kTokPerBlock * kWave) void scatter_rows_kernel(
    const vec16* __restrict__ x, int64_t T, int64_t row_vecs, int32_t k, const int32_t* __restrict__ accepted,
    const int32_t* __restrict__ inv, int32_t* __restrict__ src, vec16* __restrict__ x_perm) {
  const int64_t R = T * k;
  const int32_t A = *accepted;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (A + gid < R) src[A + gid] = -1;
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokPerBlock + threadIdx.x / kWave;
  if (t >= T || !x_perm) return;
  int32_t slot[MOE_MAX_TOPK];
  int live = 0;
  for (int j = 0; j < k; ++j) {
    const int32_t p = inv[t * k + j];
    if (p >= 0 && p < A) slot[live++] = p;
  }
  if (live == 0) return;
  const vec16* in = x + t * row_vecs;
  for (int64_t c0 = 0; c0 < row_vecs; c0 += kPiece * kWave) {
    vec16 v[kPiece];
#pragma unroll
    for (int u = 0; u < kPiece; ++u) {
      const int64_t c = c0 + u * kWave + lane;
      if (c < row_vecs) v[u] = ld_stream(in + c);
    }
    for (int j = 0; j < live; ++j) {
      vec16* out = x_perm + static_cast<int64_t>(slot[j]) * row_vecs;
#pragma unroll
      for (int u = 0; u < kPiece; ++u) {
        const int64_t c = c0 + u * kWave + lane;
        if (c < row_vecs) out[c] = v[u];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Fused rank and scatter for problems whose chunk table is small (T*k <=
// kFuseMaxRoutes): after the count pass (chunks of 64*steps routes, at most
// kFuseMaxChunks of them), one launch does the rest.  Every block takes
// kFuseTok tokens (routes r0 .. r0 + kFuseTok*k) and, redundantly and
// identically in every block:
//   sel[e] = sum over chunks of table[c][e], counts = min(sel, cap), offsets
//   = exclusive prefix of counts (one block also writes them out);
// then for its own routes the route-order rank pos_r = (routes of expert e in
// chunks before the chunk c0 holding r0) + (routes of e in [c0 * chunk, r0))
// + (rank among the block's own routes, ballots over the expert code); inv,
// src and the row copies follow as in the three-pass path.  The block's
// first term sums a column of the table, the second reads at most one
// chunk of ids.
constexpr int kFuseTok = 4;                       // tokens (wavefronts) per block (4 * k <= 64 routes)
static_assert(kFuseTok * MOE_MAX_TOPK <= kWave, "a block's routes fit one wavefront");
constexpr int kFuseThreads = kFuseTok * kWave;
constexpr int kFuseMaxChunks = 32;
constexpr int64_t kFuseMaxRoutes = 64ll * kRankMaxSteps * kFuseMaxChunks;

// Count-pass geometry of the fused path: as many steps per chunk as keep the
// table at kFuseMaxChunks rows (at least 4 steps).
inline RankGeom rank_geom_fused(int64_t n, int32_t B) {
  RankGeom g = rank_geom(n, B);
  const int64_t s = (n + 64ll * kFuseMaxChunks - 1) / (64ll * kFuseMaxChunks);
  g.steps = static_cast<int32_t>(s < 4 ? 4 : (s > kRankMaxSteps ? kRankMaxSteps : s));
  const int64_t chunk = 64ll * g.steps;
  g.chunks = (n + chunk - 1) / chunk;
  return g;
}

// Exclusive prefix of v[0 .. n) in LDS, in place, by all kFuseThreads
// threads (each scans a run of consecutive entries, then the runs' totals
// are scanned across the block); returns the grand total.
__device__ __forceinline__ int32_t block_scan_lds(int32_t* v, int n, int32_t* wave_tot) {
  const int t = threadIdx.x, lane = t % kWave, w = t / kWave;
  const int per = (n + kFuseThreads - 1) / kFuseThreads;
  const int b0 = t * per, b1 = b0 + per < n ? b0 + per : n;
  int32_t run = 0;
  for (int b = b0; b < b1; ++b) run += v[b];
  int32_t incl = run;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int32_t u = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += u;
  }
  if (lane == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  int32_t wbase = 0, total = 0;
  for (int i = 0; i < kFuseTok; ++i) {
    if (i < w) wbase += wave_tot[i];
    total += wave_tot[i];
  }
  int32_t acc = wbase + incl - run;
  for (int b = b0; b < b1; ++b) {
    const int32_t x = v[b];
    v[b] = acc;
    acc += x;
  }
  __syncthreads();
  return total;
}

// FULL (short route lists, R <= kFullScanMaxRoutes): no count pass and no
// table -- every block reads all R expert ids itself and counts, per expert,
// all routes and the routes before its first one (LDS atomics); block 0 also
// flags invalid ids, as the count pass does.  Decode-sized lists (512
// routes): 18.8 -> 11.6 us per call.  At the mid layer's 16,384 routes the
// per-block scan (64 KB, two atomics per route) costs more than the count
// pass it replaces (25.7 -> 26.7 us), hence the bound.
constexpr int64_t kFullScanMaxRoutes = 4096;

template <bool FULL>
__global__ __launch_bounds__(kFuseThreads) void permute_fused_kernel(
    const vec16* __restrict__ x, int64_t T, int64_t row_vecs, int32_t k, const int32_t* __restrict__ ids,
    int32_t E, int64_t cap, RankGeom g, const int32_t* __restrict__ table, int32_t* __restrict__ inv,
    int32_t* __restrict__ src, int32_t* __restrict__ sel_out, int32_t* __restrict__ counts_out,
    int32_t* __restrict__ offsets_out, int32_t* __restrict__ dropped_out, vec16* __restrict__ x_perm,
    uint32_t* flags) {
  extern __shared__ int32_t lds[];
  int32_t* sel = lds;                 // [E]   routes per expert
  int32_t* base = lds + E;            // [E]   running route-order rank base of the block
  int32_t* offs = lds + 2 * E;        // [E+1] offsets of the accepted counts
  __shared__ int32_t slot_of[kFuseTok * MOE_MAX_TOPK];
  __shared__ int32_t wave_tot[kFuseTok];
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  const int64_t R = T * k;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kFuseTok;
  const int64_t r0 = t0 * k;
  const int64_t r1 = r0 + kFuseTok * k < R ? r0 + kFuseTok * k : R;
  const int64_t chunk = 64ll * g.steps;
  const int64_t c0 = r0 / chunk;
  const int64_t t = t0 + w;                               // this wavefront's token
  const bool copy = t < T && x_perm != nullptr;
  // Every load that depends on no other result is issued first: the table
  // column pieces, the ids of chunk c0 before r0, the block's own ids and the
  // first piece of the token row (its latency hides behind the rank work).
  // table entries per thread and batch (one batch holds the whole table up to
  // 128 experts)
  constexpr int kTabPer = kFuseMaxChunks * 128 / kFuseThreads;
  const int64_t entries = FULL ? 0 : g.chunks * E;
  const int32_t q = kFuseThreads / E, rr = kFuseThreads % E;
  int32_t tv[kTabPer];
  constexpr int kPrePer = 64 * kRankMaxSteps / kFuseThreads;                 // chunk ids per thread, at most
  int32_t pv[kPrePer];
  if constexpr (!FULL) {
#pragma unroll
    for (int u = 0; u < kTabPer; ++u) {
      const int64_t idx = tid + static_cast<int64_t>(u) * kFuseThreads;
      tv[u] = idx < entries ? table[idx] : 0;
    }
#pragma unroll
    for (int u = 0; u < kPrePer; ++u) {
      const int64_t r = c0 * chunk + tid + u * kFuseThreads;
      pv[u] = r < r0 ? ids[r] : -1;
    }
  }
  const int64_t rme = r0 + lane;
  const int32_t my_id = (w == 0 && rme < r1) ? ids[rme] : -1;
  vec16 v[kPiece];
  const vec16* in = x + (copy ? t : 0) * row_vecs;
#pragma unroll
  for (int u = 0; u < kPiece; ++u) {
    const int64_t c = u * kWave + lane;
    if (copy && c < row_vecs) v[u] = ld_stream(in + c);
  }
  for (int b = tid; b < E; b += kFuseThreads) sel[b] = 0, base[b] = 0;
  __syncthreads();
  if constexpr (FULL) {
    // every route's expert: the totals, and the routes before this block's first
    constexpr int kScanUnroll = 8;
    for (int64_t r00 = 0; r00 < R; r00 += static_cast<int64_t>(kScanUnroll) * kFuseThreads) {
      int32_t e8[kScanUnroll];
#pragma unroll
      for (int u = 0; u < kScanUnroll; ++u) {
        const int64_t r = r00 + tid + u * kFuseThreads;
        e8[u] = r < R ? ids[r] : -1;
      }
#pragma unroll
      for (int u = 0; u < kScanUnroll; ++u) {
        const int64_t r = r00 + tid + u * kFuseThreads;
        const int32_t e = e8[u];
        if (e >= 0 && e < E) {
          atomicAdd(&sel[e], 1);
          if (r < r0) atomicAdd(&base[e], 1);
        } else if (e != -1 && r < R && blockIdx.x == 0) {
          flag_or(flags, MOE_FLAG_BAD_EXPERT);
        }
      }
    }
  }
  // expert totals and the routes of every expert in the chunks before c0
  for (int64_t b0 = 0; b0 < entries; b0 += static_cast<int64_t>(kTabPer) * kFuseThreads) {
    if (b0 > 0) {
#pragma unroll
      for (int u = 0; u < kTabPer; ++u) {
        const int64_t idx = b0 + tid + static_cast<int64_t>(u) * kFuseThreads;
        tv[u] = idx < entries ? table[idx] : 0;
      }
    }
    // entry idx is (chunk idx / E, expert idx % E); stepping idx by the block
    // size steps the chunk by q and the expert by rr (with one carry), so the
    // loop divides nothing.  Where E divides the block size every entry of a
    // thread is one expert's: sum in registers, two LDS atomics per thread.
    int64_t c = (b0 + tid) / E;
    int b = static_cast<int>((b0 + tid) - c * E);
    if (rr == 0) {
      int32_t all = 0, before = 0;
#pragma unroll
      for (int u = 0; u < kTabPer; ++u) {
        const int64_t idx = b0 + tid + static_cast<int64_t>(u) * kFuseThreads;
        const int32_t x = idx < entries ? tv[u] : 0;
        all += x;
        before += c + u * q < c0 ? x : 0;
      }
      if (all != 0) atomicAdd(&sel[b], all);
      if (before != 0) atomicAdd(&base[b], before);
    } else {
#pragma unroll
      for (int u = 0; u < kTabPer; ++u) {
        const int64_t idx = b0 + tid + static_cast<int64_t>(u) * kFuseThreads;
        if (idx < entries) {
          atomicAdd(&sel[b], tv[u]);
          if (c < c0) atomicAdd(&base[b], tv[u]);
        }
        c += q;
        b += rr;
        if (b >= E) b -= E, ++c;
      }
    }
  }
  // routes of chunk c0 before the block's first route
  if constexpr (!FULL) {
#pragma unroll
    for (int u = 0; u < kPrePer; ++u)
      if (pv[u] >= 0 && pv[u] < E) atomicAdd(&base[pv[u]], 1);
  }
  __syncthreads();
  for (int b = tid; b < E; b += kFuseThreads) offs[b] = cap < 0 ? sel[b] : (sel[b] < cap ? sel[b] : static_cast<int32_t>(cap));
  __syncthreads();
  const int32_t A = block_scan_lds(offs, E, wave_tot);
  if (tid == 0) offs[E] = A;
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int b = tid; b < E; b += kFuseThreads) {
      if (sel_out) sel_out[b] = sel[b];
      counts_out[b] = cap < 0 ? sel[b] : (sel[b] < cap ? sel[b] : static_cast<int32_t>(cap));
      offsets_out[b] = offs[b];
    }
    if (tid == 0) {
      offsets_out[E] = A;
      dropped_out[0] = static_cast<int32_t>(R - A);
    }
  }
  // src entries past the accepted total
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kFuseThreads + tid;
  if (A + gid < R) src[A + gid] = -1;
  // the block's routes (at most 64: wavefront 0): stable ranks by ballots over
  // the expert code
  if (w == 0) {
    int nbits = 0;
    while ((1 << nbits) <= E) ++nbits;
    const bool inb = rme < r1;
    const bool valid = my_id >= 0 && my_id < E;
    const int code = valid ? my_id : E;
    uint64_t peers = ~0ull;
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (code >> bit) & 1;
      const uint64_t m = ballot(on);
      peers &= on ? m : ~m;
    }
    int32_t slot = -1;
    if (valid) {
      const int32_t pos = base[my_id] + __popcll(peers & lanemask_lt());
      if (cap < 0 || pos < cap) slot = offs[my_id] + pos;
    }
    if (inb) {
      inv[rme] = slot;
      if (slot >= 0) src[slot] = static_cast<int32_t>(rme);
      slot_of[lane] = slot;
    }
  }
  __syncthreads();
  // row copies: one wavefront per token, the row read once
  if (!copy) return;
  int32_t slot[MOE_MAX_TOPK];
  int live = 0;
  for (int j = 0; j < k; ++j) {
    const int32_t p = slot_of[w * k + j];
    if (p >= 0) slot[live++] = p;
  }
  if (live == 0) return;
  for (int64_t cc = 0; cc < row_vecs; cc += kPiece * kWave) {
    if (cc > 0) {
#pragma unroll
      for (int u = 0; u < kPiece; ++u) {
        const int64_t c = cc + u * kWave + lane;
        if (c < row_vecs) v[u] = ld_stream(in + c);
      }
    }
    for (int j = 0; j < live; ++j) {
      vec16* out = x_perm + static_cast<int64_t>(slot[j]) * row_vecs;
#pragma unroll
      for (int u = 0; u < kPiece; ++u) {
        const int64_t c = cc + u * kWave + lane;
        if (c < row_vecs) out[c] = v[u];
      }
    }
  }
}

}  // namespace
}  // namespace moe

// The no-allocation entry point's rank table: a file-scope device array (one
// copy per GPU, alive until the process ends).  Host code never passes its
// name to a kernel: the host-side symbol is only a stand-in, so kernels get
// the device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[MOE_PERMUTE_NOALLOC_SCRATCH_BYTES];

namespace moe {
namespace {

// Device address of `scratch` on the device of `stream`, looked up once per
// device with that device current (a race between host threads only repeats
// the same lookup).
int scratch_address(hipStream_t stream, void** out) {
  static std::atomic<void*> addr[64];
  int dev = 0, cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return MOE_EHIP;
  dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return MOE_EHIP;
  if (dev < 0 || dev >= 64) return MOE_EUNSUPPORTED;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return MOE_EHIP;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return MOE_EHIP;
    if (e != hipSuccess || !p) return MOE_EHIP;
    addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return MOE_OK;
}

// Argument checks shared by both entry points (no HIP call).
int permute_check(const void* x, int32_t x_dtype, int64_t T, int32_t d, const int32_t* topk_ids, int32_t k,
                  int32_t E, int64_t capacity, const void* x_perm, const int32_t* src, const int32_t* inv,
                  const int32_t* counts, const int32_t* offsets, const int32_t* n_dropped) {
  MOE_CHECK(T >= 0 && k >= 1 && k <= MOE_MAX_TOPK && E >= 1 && E <= MOE_MAX_EXPERTS, MOE_EINVAL);
  MOE_CHECK(T <= INT32_MAX / k, MOE_EUNSUPPORTED);
  MOE_CHECK(capacity >= -1, MOE_EINVAL);
  MOE_CHECK(x_dtype == MOE_F32 || x_dtype == MOE_BF16 || is_fp8(x_dtype), MOE_EINVAL);
  // fp8 records move whole: codes and scales together (M6.2 0x0AC)
  const int64_t rb = row_bytes(x_dtype, d);
  MOE_CHECK(counts && offsets && n_dropped, MOE_EINVAL);
  MOE_CHECK(T == 0 || (topk_ids && src && inv), MOE_EINVAL);
  if (x_perm) {
    MOE_CHECK(x && d >= 1 && rb % 16 == 0 && (!is_fp8(x_dtype) || d % 8 == 0), MOE_EINVAL);
    MOE_CHECK(aligned16(x) && aligned16(x_perm), MOE_EINVAL);
  }
  return MOE_OK;
}

// The launches of one permute, with the rank table at `table`.
int permute_launch(const void* x, int32_t x_dtype, int64_t T, int32_t d, const int32_t* topk_ids, int32_t k,
                   int32_t E, int64_t capacity, void* x_perm, int32_t* src, int32_t* inv, int32_t* sel_counts,
                   int32_t* counts, int32_t* offsets, int32_t* n_dropped, int32_t* table, uint32_t* dev_flags,
                   hipStream_t stream) {
  const int64_t R = T * k;
  if (R > 0 && R <= kFullScanMaxRoutes) {
    // one launch: every block counts all routes, then ranks and scatters its own
    const RankGeom g = rank_geom_fused(R, E);
    const int64_t row_vecs = x_perm ? row_bytes(x_dtype, d) / 16 : 0;
    const unsigned blocks = static_cast<unsigned>((T + kFuseTok - 1) / kFuseTok);
    const size_t lds = static_cast<size_t>(3 * E + 1) * sizeof(int32_t);
    hipLaunchKernelGGL(HIP_KERNEL_NAME(permute_fused_kernel<true>), dim3(blocks), dim3(kFuseThreads), lds, stream,
                       static_cast<const vec16*>(x), T, row_vecs, k, topk_ids, E, capacity, g,
                       static_cast<const int32_t*>(nullptr), inv, src, sel_counts, counts, offsets, n_dropped,
                       static_cast<vec16*>(x_perm), dev_flags);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
  }
  if (R > 0 && R <= kFuseMaxRoutes) {
    // count pass, then the fused rank and scatter
    const RankGeom g = rank_geom_fused(R, E);
    const unsigned cblocks = static_cast<unsigned>((g.chunks + kRankWaves - 1) / kRankWaves);
    const size_t clds = static_cast<size_t>(kRankWaves) * g.B * sizeof(int32_t);
    hipLaunchKernelGGL(HIP_KERNEL_NAME(rank_count_kernel<ExpertBucket>), dim3(cblocks), dim3(kRankThreads), clds,
                       stream, ExpertBucket{topk_ids, E}, g, table, dev_flags);
    MOE_LAUNCH_CHECK();
    const int64_t row_vecs = x_perm ? row_bytes(x_dtype, d) / 16 : 0;
    const unsigned blocks = static_cast<unsigned>((T + kFuseTok - 1) / kFuseTok);
    const size_t lds = static_cast<size_t>(3 * E + 1) * sizeof(int32_t);
    hipLaunchKernelGGL(HIP_KERNEL_NAME(permute_fused_kernel<false>), dim3(blocks), dim3(kFuseThreads), lds, stream,
                       static_cast<const vec16*>(x), T, row_vecs, k, topk_ids, E, capacity, g, table, inv, src,
                       sel_counts, counts, offsets, n_dropped, static_cast<vec16*>(x_perm), dev_flags);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
  }
  const RankGeom g = rank_geom(T * k, E);
  RankScanOut out{sel_counts, counts, offsets, n_dropped, 1};
  int st = bucket_rank(g, ExpertBucket{topk_ids, E}, PermuteEmit{capacity, R, offsets, inv, src}, capacity, out,
                       table, dev_flags, stream);
  if (st != MOE_OK) return st;
  if (R > 0) {
    const int64_t row_vecs = x_perm ? row_bytes(x_dtype, d) / 16 : 0;
    const unsigned blocks = static_cast<unsigned>((T + kTokPerBlock - 1) / kTokPerBlock);
    hipLaunchKernelGGL(scatter_rows_kernel, dim3(blocks), dim3(kTokPerBlock * kWave), 0, stream,
                       static_cast<const vec16*>(x), T, row_vecs, k, offsets + E, inv, src,
                       static_cast<vec16*>(x_perm));
    MOE_LAUNCH_CHECK();
  }
  return MOE_OK;
}

}  // namespace
}  // namespace moe

MOE_API size_t moe_permute_workspace(int64_t T, int32_t k, int32_t E) {
  using namespace moe;
  if (T < 0 || k < 1 || E < 1 || E > MOE_MAX_EXPERTS) return 0;
  return rank_table_bytes(rank_geom(T * k, E));
}

MOE_API int moe_permute(const void* x, int32_t x_dtype, int64_t T, int32_t d, const int32_t* topk_ids,
                        int32_t k, int32_t E, int64_t capacity, void* x_perm, int32_t* src, int32_t* inv,
                        int32_t* sel_counts, int32_t* counts, int32_t* offsets, int32_t* n_dropped, void* ws,
                        size_t ws_bytes, uint32_t* dev_flags, hipStream_t stream) {
  using namespace moe;
  int st = permute_check(x, x_dtype, T, d, topk_ids, k, E, capacity, x_perm, src, inv, counts, offsets, n_dropped);
  if (st != MOE_OK) return st;
  MOE_CHECK(ws && ws_bytes >= rank_table_bytes(rank_geom(T * k, E)), MOE_EWORKSPACE);
  return permute_launch(x, x_dtype, T, d, topk_ids, k, E, capacity, x_perm, src, inv, sel_counts, counts, offsets,
                        n_dropped, static_cast<int32_t*>(ws), dev_flags, stream);
}

MOE_API int moe_permute_noalloc(const void* x, int32_t x_dtype, int64_t T, int32_t d, const int32_t* topk_ids,
                                int32_t k, int32_t E, int64_t capacity, void* x_perm, int32_t* src, int32_t* inv,
                                int32_t* sel_counts, int32_t* counts, int32_t* offsets, int32_t* n_dropped,
                                uint32_t* dev_flags, hipStream_t stream) {
  using namespace moe;
  int st = permute_check(x, x_dtype, T, d, topk_ids, k, E, capacity, x_perm, src, inv, counts, offsets, n_dropped);
  if (st != MOE_OK) return st;
  MOE_CHECK(rank_table_bytes(rank_geom(T * k, E)) <= MOE_PERMUTE_NOALLOC_SCRATCH_BYTES, MOE_ESCRATCH);
  void* table = nullptr;
  st = scratch_address(stream, &table);
  if (st != MOE_OK) return st;
  return permute_launch(x, x_dtype, T, d, topk_ids, k, E, capacity, x_perm, src, inv, sel_counts, counts, offsets,
                        n_dropped, static_cast<int32_t*>(table), dev_flags, stream);
}
