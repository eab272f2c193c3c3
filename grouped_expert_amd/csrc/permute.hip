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
  const RankGeom g = rank_geom(T * k, E);
  const int64_t R = T * k;
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
