// Pooled-wave sender pack into fixed destination pools with a header row.
//
// "Fixed pooled-wave all-to-all for the 8-of-384 MoE", 02: the sender keeps
// one pool per destination GPU and wave; an expert id gives a destination and
// a local expert id; a route's ordinal among this sender's routes to its
// destination picks the wave (ordinal mod n_waves) and the pool row (ordinal
// div n_waves) -- the ordinal is the page's "rank" (the only reading that fits
// the pool shape [64, 3005, 3072] per wave and the per-destination, per-wave
// capacity of 04); extra rows are
// dropped; the first full-width row of a pool carries the packed local expert
// ids so that no count exchange is needed (reading: as many such rows as the
// 16-bit ids need, e.g. two for the two-wave profile of 05).  Rows are bf16
// or fp8 records ("M6.2 - Expert Parallelism and DeepSeek MoE", 0x0AB-0x0AC:
// the scales travel inside the row); the kernels move rows as 16-byte
// vectors and never look inside them.
// 03: every wave has the same static shape.
//
// Launches: the shared bucket-rank passes with bucket = destination (pass 3
// writes route_loc and the header id of every placed row), then one launch
// whose blocks either scatter token rows (each token row read once, written to
// its placed copies) or fill the unused rows (zero data, 0xFFFF header tail)
// so that the pools are fully defined.
#include "bucket_rank.h"
#include "fp8.h"

namespace moe {
namespace {

struct DestBucket {
  const int32_t* ids;
  int32_t E, epd;
  __device__ uint32_t load(int64_t r) const { return static_cast<uint32_t>(ids[r]); }
  __device__ int classify(uint32_t raw, uint32_t* flags) const {
    const int32_t e = static_cast<int32_t>(raw);
    if (e >= 0 && e < E) return e / epd;
    if (e != -1) flag_or(flags, MOE_FLAG_BAD_EXPERT);
    return -1;
  }
};

struct PackEmit {
  const int32_t* ids;
  int32_t epd, n_dest, n_waves, pool_rows, re, wave_sel, H;    // re: 16-bit elements per row
  int32_t* route_loc;
  bf16_t* pools;
  __device__ void operator()(int64_t r, int dest, int32_t o) const {
    if (dest < 0) {
      route_loc[r] = -1;
      return;
    }
    const int32_t w = o % n_waves, row = o / n_waves;
    if (row >= pool_rows) {
      route_loc[r] = -1;
      return;
    }
    const int64_t P1 = static_cast<int64_t>(pool_rows) + H;
    route_loc[r] = static_cast<int32_t>((static_cast<int64_t>(w) * n_dest + dest) * P1 + H + row);
    if (wave_sel < 0 || wave_sel == w) {
      const int64_t slab = wave_sel < 0 ? w : 0;
      pools[((slab * n_dest + dest) * P1) * re + row] = static_cast<bf16_t>(ids[r] % epd);
    }
  }
};

// One wavefront per token: the row is read once into registers (in pieces of
// up to 8 x 16 B per lane) and written to each of the token's placed slots.
// Plain (cached) loads and stores: measured faster here than the streaming
// forms.
constexpr int kTokPerBlock = 4;
constexpr int kPiece = 8;
constexpr int kPackThreads = kTokPerBlock * kWave;

__device__ __forceinline__ void pack_token_rows(const vec16* __restrict__ x, int64_t T, int64_t row_vecs, int32_t k,
                                                const int32_t* __restrict__ route_loc, int64_t slab_lo,
                                                int64_t slab_hi, vec16* __restrict__ pools, int64_t blk) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = blk * kTokPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  int32_t loc[MOE_MAX_TOPK];
  int live = 0;
  for (int j = 0; j < k; ++j) {
    const int32_t l = route_loc[t * k + j];
    if (l >= slab_lo && l < slab_hi) loc[live++] = static_cast<int32_t>(l - slab_lo);
  }
  if (live == 0) return;
  const vec16* in = x + t * row_vecs;
  for (int64_t c0 = 0; c0 < row_vecs; c0 += kPiece * kWave) {
    vec16 v[kPiece];
#pragma unroll
    for (int u = 0; u < kPiece; ++u) {
      const int64_t c = c0 + u * kWave + lane;
      if (c < row_vecs) v[u] = in[c];
    }
    for (int j = 0; j < live; ++j) {
      vec16* out = pools + static_cast<int64_t>(loc[j]) * row_vecs;
#pragma unroll
      for (int u = 0; u < kPiece; ++u) {
        const int64_t c = c0 + u * kWave + lane;
        if (c < row_vecs) out[c] = v[u];
      }
    }
  }
}

// Quantizing pack (bf16 rows in, fp8 records out; "M6.2 - Expert Parallelism
// and DeepSeek MoE", 0x0AB-0x0AC): one wavefront per token; the token row is
// quantized once, with the arithmetic of moe_quantize_fp8, and its record
// (codes, scales, zero padding) is written to each placed slot, so the
// records never make a round trip through memory.  Per-128 scales: 16 lanes
// hold a group; per-row scales: a first pass over the row finds the largest
// magnitude.
template <bool ROW>
__device__ __forceinline__ void pack_token_rows_fp8(const bf16_t* __restrict__ x, int64_t T, int32_t d, int64_t rb,
                                                    int32_t k, const int32_t* __restrict__ route_loc,
                                                    int64_t slab_lo, int64_t slab_hi, uint8_t* __restrict__ pools,
                                                    int64_t blk, uint32_t* flags) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = blk * kTokPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  int32_t loc[MOE_MAX_TOPK];
  int live = 0;
  for (int j = 0; j < k; ++j) {
    const int32_t l = route_loc[t * k + j];
    if (l >= slab_lo && l < slab_hi) loc[live++] = static_cast<int32_t>(l - slab_lo);
  }
  if (live == 0) return;
  const bf16_t* xr = x + t * d;
  const int32_t G = fp8_groups(ROW ? MOE_FP8_ROW : MOE_FP8_B128, d);
  bool bad_any = false;
  float row_scale = 0.0f, row_inv = 0.0f;
  bool row_zero = false;
  if (ROW) {
    float amax = 0.0f;
    bool bad = false;
    for (int32_t c = lane * 8; c < d; c += kWave * 8) {
      float v[8];
      load_row8<bf16_t>(xr + c, v);
      amax = fmaxf(amax, amax8(v, &bad));
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
    bad_any = __any(bad);
    row_zero = bad_any || amax == 0.0f;
    row_scale = row_zero ? 0.0f : amax / 448.0f;
    row_inv = row_zero ? 0.0f : 448.0f / amax;
  }
  // pieces of 16 values per lane (16 code bytes: one 16-byte store per slot),
  // kQPiece of them loaded before any is used; a 128-value group is 8 lanes
  constexpr int kQPiece = 4;
  for (int32_t c0 = 0; c0 < d; c0 += kQPiece * kWave * 16) {
    float v[kQPiece][2][8];
#pragma unroll
    for (int u = 0; u < kQPiece; ++u) {
      const int32_t c = c0 + (u * kWave + lane) * 16;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (c + 8 * h < d) {
          load_row8<bf16_t>(xr + c + 8 * h, v[u][h]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[u][h][i] = 0.0f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kQPiece; ++u) {
      const int32_t c = c0 + (u * kWave + lane) * 16;
      if (c0 + u * kWave * 16 >= d) break;                // wave-uniform: no piece of this step is in the row
      float scale = row_scale, inv = row_inv;
      bool zero = row_zero;
      if (!ROW) {
        bool bad = false;
        float amax = fmaxf(amax8(v[u][0], &bad), amax8(v[u][1], &bad));
        int badi = bad ? 1 : 0;
#pragma unroll
        for (int off = 4; off > 0; off >>= 1) {           // the 8 lanes of one 128-value group
          amax = fmaxf(amax, __shfl_xor(amax, off, 8));
          badi |= __shfl_xor(badi, off, 8);
        }
        zero = badi != 0 || amax == 0.0f;
        scale = zero ? 0.0f : amax / 448.0f;
        inv = zero ? 0.0f : 448.0f / amax;
        bad_any |= badi != 0;
      }
      const uint2 q0 = encode8(v[u][0], inv, zero), q1 = encode8(v[u][1], inv, zero);
      if (c < d) {
        const bool full = c + 16 <= d;                    // d % 16 == 8: the row's last piece has 8 values
        for (int j = 0; j < live; ++j) {
          uint8_t* out = pools + static_cast<int64_t>(loc[j]) * rb;
          if (full) {
            const vec16 q = {q0.x, q0.y, q1.x, q1.y};
            *reinterpret_cast<vec16*>(out + c) = q;
          } else {
            *reinterpret_cast<uint2*>(out + c) = q0;
          }
          if (!ROW && lane % 8 == 0) *reinterpret_cast<float*>(out + d + 4 * (c / 128)) = scale;
        }
      }
    }
  }
  // zero padding: fewer than 128 bytes from a 4-byte boundary, one word per lane
  const int32_t tail_words = (static_cast<int32_t>(rb) - d - 4 * G) / 4;
  for (int j = 0; j < live; ++j) {
    uint8_t* out = pools + static_cast<int64_t>(loc[j]) * rb;
    if (ROW && lane == 0) *reinterpret_cast<float*>(out + d) = row_scale;
    if (lane < tail_words) reinterpret_cast<uint32_t*>(out + d + 4 * G)[lane] = 0u;
  }
  if (bad_any && lane == 0) flag_or(flags, MOE_FLAG_NONFINITE_INPUT);
}

// Unused rows of one pool (row block rblk of pool `pool` = slab * n_dest +
// dest): zero data rows past the wave's fill and 0xFFFF header elements past
// it.  These rows are disjoint from every placed row.
constexpr int kFillRows = 16;

__device__ __forceinline__ void pack_fill_rows(const int32_t* __restrict__ dest_counts, int32_t n_dest,
                                               int32_t n_waves, int32_t pool_rows, int32_t re, int32_t H,
                                               int32_t wave_sel, bf16_t* __restrict__ pools, int64_t pool,
                                               int32_t rblk) {
  const int32_t dest = static_cast<int32_t>(pool % n_dest);
  const int32_t w = wave_sel < 0 ? static_cast<int32_t>(pool / n_dest) : wave_sel;
  const int64_t cap_all = static_cast<int64_t>(n_waves) * pool_rows;
  const int64_t n = dest_counts[dest];
  const int64_t m = n < cap_all ? n : cap_all;
  const int32_t filled = m > w ? static_cast<int32_t>((m - w + n_waves - 1) / n_waves) : 0;
  const int64_t P1 = static_cast<int64_t>(pool_rows) + H;
  bf16_t* base = pools + pool * P1 * re;
  if (rblk == 0) {
    const int64_t hdr = static_cast<int64_t>(H) * re;    // 16-bit header elements of the pool
    for (int64_t i = filled + threadIdx.x; i < hdr; i += blockDim.x) base[i] = 0xFFFF;
  }
  const int32_t r0 = rblk * kFillRows;
  if (r0 + kFillRows <= filled) return;
  const int64_t row_vecs = static_cast<int64_t>(re) / 8;
  const vec16 zero = {0u, 0u, 0u, 0u};
  for (int32_t rr = 0; rr < kFillRows; ++rr) {
    const int32_t row = r0 + rr;
    if (row < filled || row >= pool_rows) continue;
    vec16* out = reinterpret_cast<vec16*>(base + (H + static_cast<int64_t>(row)) * re);
    for (int64_t c = threadIdx.x; c < row_vecs; c += blockDim.x) st_stream(zero, out + c);
  }
}

// One launch for both: blocks [0, tok_blocks) scatter token rows, the rest
// fill unused rows (fill_blocks_per_pool row blocks per pool), so the fill's
// writes overlap the scatter instead of following it.  Q: 0 moves rows as
// they are, 1 / 2 quantizes bf16 rows into fp8 records with row / 128-value
// scales (d is the row width in values, row_vecs the record width / 16).
template <int Q>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(
    const vec16* __restrict__ x, int64_t T, int64_t row_vecs, int32_t k, const int32_t* __restrict__ route_loc,
    int64_t slab_lo, int64_t slab_hi, int64_t tok_blocks, const int32_t* __restrict__ dest_counts, int32_t n_dest,
    int32_t n_waves, int32_t pool_rows, int32_t re, int32_t H, int32_t wave_sel, int32_t fill_blocks_per_pool,
    bf16_t* __restrict__ pools, int32_t d, uint32_t* flags) {
  const int64_t b = blockIdx.x;
  if (b < tok_blocks) {
    if constexpr (Q == 0)
      pack_token_rows(x, T, row_vecs, k, route_loc, slab_lo, slab_hi, reinterpret_cast<vec16*>(pools), b);
    else
      pack_token_rows_fp8<Q == 1>(reinterpret_cast<const bf16_t*>(x), T, d, row_vecs * 16, k, route_loc, slab_lo,
                                  slab_hi, reinterpret_cast<uint8_t*>(pools), b, flags);
  } else {
    const int64_t f = b - tok_blocks;
    pack_fill_rows(dest_counts, n_dest, n_waves, pool_rows, re, H, wave_sel, pools, f / fill_blocks_per_pool,
                   static_cast<int32_t>(f % fill_blocks_per_pool));
  }
}

}  // namespace
}  // namespace moe

MOE_API size_t moe_pool_pack_workspace(int64_t T, int32_t k, int32_t n_dest) {
  using namespace moe;
  if (T < 0 || k < 1 || n_dest < 1 || n_dest > MOE_MAX_EXPERTS) return 0;
  return rank_table_bytes(rank_geom(T * k, n_dest)) + align_up((n_dest + 1) * sizeof(int32_t), 256);
}

MOE_API int moe_pool_pack(const void* x, int32_t x_dtype, int32_t pool_dtype, int64_t T, int32_t d,
                          const int32_t* topk_ids, int32_t k, int32_t E,
                          int32_t experts_per_dest, int32_t n_dest, int32_t n_waves, int32_t pool_rows,
                          int32_t wave, void* pools, int32_t* route_loc, int32_t* dest_counts,
                          int32_t* sender_dropped, void* ws, size_t ws_bytes, uint32_t* dev_flags,
                          hipStream_t stream) {
  using namespace moe;
  MOE_CHECK(T >= 0 && k >= 1 && k <= MOE_MAX_TOPK && E >= 1, MOE_EINVAL);
  MOE_CHECK(T <= INT32_MAX / k, MOE_EUNSUPPORTED);
  MOE_CHECK(experts_per_dest >= 1 && experts_per_dest < 0xFFFF, MOE_EINVAL);
  MOE_CHECK(n_dest >= 1 && n_dest <= MOE_MAX_EXPERTS && n_waves >= 1 && pool_rows >= 0, MOE_EINVAL);
  MOE_CHECK(E <= static_cast<int64_t>(n_dest) * experts_per_dest, MOE_EINVAL);
  MOE_CHECK(wave >= -1 && wave < n_waves, MOE_EINVAL);
  MOE_CHECK(d >= 8 && d % 8 == 0, MOE_EINVAL);
  MOE_CHECK(x_dtype == MOE_BF16 || is_fp8(x_dtype), MOE_EINVAL);
  // rows are moved as they are, or bf16 rows are quantized into fp8 records
  MOE_CHECK(pool_dtype == x_dtype || (x_dtype == MOE_BF16 && is_fp8(pool_dtype)), MOE_EINVAL);
  const int64_t rb = row_bytes(pool_dtype, d);                    // pool row bytes, a multiple of 16 (of 128 for records)
  MOE_CHECK(rb <= INT32_MAX, MOE_EUNSUPPORTED);
  const int32_t re = static_cast<int32_t>(rb / 2);                // 16-bit elements per row
  const int32_t H = static_cast<int32_t>(pool_header_rows(rb, pool_rows));   // one 16-bit id per data row
  const int64_t P1 = static_cast<int64_t>(pool_rows) + H;
  MOE_CHECK(static_cast<int64_t>(n_waves) * n_dest * P1 <= INT32_MAX, MOE_EUNSUPPORTED);
  MOE_CHECK(pools && dest_counts && sender_dropped, MOE_EINVAL);
  MOE_CHECK(T == 0 || (x && topk_ids && route_loc), MOE_EINVAL);
  MOE_CHECK(aligned16(pools) && (T == 0 || aligned16(x)), MOE_EINVAL);
  const RankGeom g = rank_geom(T * k, n_dest);
  const size_t tb = rank_table_bytes(g);
  MOE_CHECK(ws && ws_bytes >= moe_pool_pack_workspace(T, k, n_dest), MOE_EWORKSPACE);
  int32_t* table = static_cast<int32_t*>(ws);
  int32_t* offsets = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + tb);
  const int64_t cap_all = static_cast<int64_t>(n_waves) * pool_rows;
  RankScanOut out{dest_counts, nullptr, offsets, sender_dropped, 1};
  bf16_t* pb = static_cast<bf16_t*>(pools);
  int st = bucket_rank(g, DestBucket{topk_ids, E, experts_per_dest},
                       PackEmit{topk_ids, experts_per_dest, n_dest, n_waves, pool_rows, re, wave, H, route_loc, pb},
                       cap_all, out, table, dev_flags, stream);
  if (st != MOE_OK) return st;
  const int64_t row_vecs = rb / 16;
  const int64_t slab_rows = static_cast<int64_t>(n_dest) * P1;
  const int64_t lo = wave < 0 ? 0 : wave * slab_rows;
  const int64_t hi = wave < 0 ? n_waves * slab_rows : lo + slab_rows;
  const int64_t tok_blocks = (T + kTokPerBlock - 1) / kTokPerBlock;
  const int64_t n_pools = static_cast<int64_t>(wave < 0 ? n_waves : 1) * n_dest;
  const int32_t fill_blocks = (pool_rows + kFillRows - 1) / kFillRows;
  const int32_t fill_per_pool = fill_blocks > 0 ? fill_blocks : 1;
  const int64_t blocks = tok_blocks + n_pools * fill_per_pool;
  MOE_CHECK(blocks <= INT32_MAX, MOE_EUNSUPPORTED);
  if (pool_dtype == x_dtype)
    hipLaunchKernelGGL(HIP_KERNEL_NAME(pack_kernel<0>), dim3(static_cast<unsigned>(blocks)), dim3(kPackThreads), 0,
                       stream, static_cast<const vec16*>(x), T, row_vecs, k, route_loc, lo, hi, tok_blocks,
                       dest_counts, n_dest, n_waves, pool_rows, re, H, wave, fill_per_pool, pb, d, dev_flags);
  else if (pool_dtype == MOE_FP8_ROW)
    hipLaunchKernelGGL(HIP_KERNEL_NAME(pack_kernel<1>), dim3(static_cast<unsigned>(blocks)), dim3(kPackThreads), 0,
                       stream, static_cast<const vec16*>(x), T, row_vecs, k, route_loc, lo, hi, tok_blocks,
                       dest_counts, n_dest, n_waves, pool_rows, re, H, wave, fill_per_pool, pb, d, dev_flags);
  else
    hipLaunchKernelGGL(HIP_KERNEL_NAME(pack_kernel<2>), dim3(static_cast<unsigned>(blocks)), dim3(kPackThreads), 0,
                       stream, static_cast<const vec16*>(x), T, row_vecs, k, route_loc, lo, hi, tok_blocks,
                       dest_counts, n_dest, n_waves, pool_rows, re, H, wave, fill_per_pool, pb, d, dev_flags);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
