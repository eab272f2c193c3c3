// Receiver compaction of one wave's incoming pools into static per-expert
// arrays.
//
// "Fixed pooled-wave all-to-all for the 8-of-384 MoE", 02/03: the receiver
// reads each row's local expert id from the header row of its pool and groups
// the rows into static [n_local, cap, d] expert arrays, dropping rows above
// the receiver capacity; 04: the capacity is per local expert per wave; 07:
// rows keep a fixed source order and overflow does not look at router scores;
// the rotation of that order per receiver (the fairness fix 07 proposes) is
// the src_rotation argument: sources are visited from src_rotation onwards,
// wrapping round.  A pool has H = max(1, ceil(pool_rows / d)) header rows.
// "M6.6 - MoE Runtime Systems", 0x03C2: this is the second, receive-side
// stable permutation into local-expert order.
//
// Launches: the shared bucket-rank passes over rows in (source, row) order
// with bucket = header id (pass 3 writes row_slot), then a row copy that
// moves every accepted row to its slot and marks the header rows -1; the
// same pass records each slot's pool row (slot_row) and clears the return
// rows of every row without a slot, for a receiver whose expert GEMM stores
// its results straight into pool-row order (pooled wave 03).  With
// fp8 records in the pools ("M6.2 - Expert Parallelism and DeepSeek MoE",
// 0x0AC) the copy dequantizes each accepted row with its own scales into the
// bf16 arrays, so the expert GEMM reads bf16 as before.
#include "bucket_rank.h"
#include "fp8.h"

namespace moe {
namespace {

// Rows are ranked in visiting order i = v * P + r, where v is the visit
// number of source s = (v + rot) mod S.
__device__ __forceinline__ int64_t visit_source(int64_t v, int64_t rot, int64_t S) {
  const int64_t s = v + rot;
  return s >= S ? s - S : s;
}

struct HeaderBucket {
  const bf16_t* pools;
  int64_t P, P1, re, rot, S;                              // re: 16-bit elements per pool row
  int32_t L;
  __device__ uint32_t load(int64_t i) const {
    const int64_t v = i / P, r = i - v * P;
    return pools[visit_source(v, rot, S) * P1 * re + r];  // id of data row r: element r of the header rows
  }
  __device__ int classify(uint32_t h, uint32_t* flags) const {
    if (h < static_cast<uint32_t>(L)) return static_cast<int>(h);
    if (h != 0xFFFFu) flag_or(flags, MOE_FLAG_BAD_HEADER);
    return -1;
  }
};

struct CompactEmit {
  int64_t P, P1, H, rot, S, cap;
  int32_t* row_slot;
  __device__ void operator()(int64_t i, int h, int32_t q) const {
    const int64_t v = i / P, r = i - v * P;
    const int32_t slot = (h >= 0 && q < cap) ? static_cast<int32_t>(h * cap + q) : -1;
    row_slot[visit_source(v, rot, S) * P1 + H + r] = slot;
  }
};

constexpr int kRowsPerBlock = 4;   // one wavefront per incoming row

// fp8 records: one wavefront per incoming row; every lane dequantizes 8
// values at a time (codes and the group's scale from the same record) and
// stores them as 16 bytes of bf16.
// Return-row side of the copy: rows without a slot get zero return rows
// (ret_vecs 16-byte pieces each), accepted rows record their pool row.
struct RowSide {
  int32_t* slot_row;
  vec16* ret;
  int64_t ret_vecs;
  __device__ void reject(int64_t row, int lane) const {
    if (!ret) return;
    const vec16 zero = {0u, 0u, 0u, 0u};
    vec16* out = ret + row * ret_vecs;
    for (int64_t c = lane; c < ret_vecs; c += kWave) st_stream(zero, out + c);
  }
  __device__ void accept(int64_t row, int32_t slot, int lane) const {
    if (slot_row && lane == 0) slot_row[slot] = static_cast<int32_t>(row);
  }
};

template <bool ROW>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void compact_fp8_rows_kernel(
    const uint8_t* __restrict__ pools, int64_t n_rows, int64_t P1, int64_t H, int64_t rb, int32_t d,
    int32_t* __restrict__ row_slot, bf16_t* __restrict__ compact, RowSide side) {
  const int lane = threadIdx.x % kWave;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + threadIdx.x / kWave;
  if (row >= n_rows) return;
  if (row % P1 < H) {
    if (lane == 0) row_slot[row] = -1;
    side.reject(row, lane);
    return;
  }
  const int32_t slot = row_slot[row];
  if (slot < 0) {
    side.reject(row, lane);
    return;
  }
  side.accept(row, slot, lane);
  const uint8_t* in = pools + row * rb;
  bf16_t* out = compact + static_cast<int64_t>(slot) * d;
  for (int32_t c = lane * 8; c < d; c += kWave * 8) {
    float v[8];
    fp8_dequant8<ROW>(in, c, d, v);
    st_stream(pack_bf16x8(v), reinterpret_cast<vec16*>(out + c));
  }
}

__global__ __launch_bounds__(kRowsPerBlock * kWave) void compact_rows_kernel(
    const vec16* __restrict__ pools, int64_t n_rows, int64_t P1, int64_t H, int64_t row_vecs,
    int32_t* __restrict__ row_slot, vec16* __restrict__ compact, RowSide side) {
  const int lane = threadIdx.x % kWave;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + threadIdx.x / kWave;
  if (row >= n_rows) return;
  if (row % P1 < H) {
    if (lane == 0) row_slot[row] = -1;
    side.reject(row, lane);
    return;
  }
  const int32_t slot = row_slot[row];
  if (slot < 0) {
    side.reject(row, lane);
    return;
  }
  side.accept(row, slot, lane);
  const vec16* in = pools + row * row_vecs;
  vec16* out = compact + static_cast<int64_t>(slot) * row_vecs;
  for (int64_t c = lane; c < row_vecs; c += kWave) st_stream(ld_stream(in + c), out + c);
}

}  // namespace
}  // namespace moe

MOE_API size_t moe_recv_compact_workspace(int32_t n_src, int32_t pool_rows, int32_t n_local) {
  using namespace moe;
  if (n_src < 0 || pool_rows < 0 || n_local < 1 || n_local > MOE_MAX_EXPERTS) return 0;
  const int64_t n = static_cast<int64_t>(n_src) * pool_rows;
  return rank_table_bytes(rank_geom(n, n_local)) + 2 * align_up((n_local + 1) * sizeof(int32_t), 256);
}

MOE_API int moe_recv_compact(const void* pools_in, int32_t pool_dtype, int32_t n_src, int32_t pool_rows, int32_t d,
                             int32_t n_local,
                             int32_t cap, int32_t src_rotation, void* compact, int32_t* counts, int32_t* arrived,
                             int32_t* row_slot, int32_t* recv_dropped, int32_t* slot_row, void* ret,
                             int32_t ret_dtype, void* ws, size_t ws_bytes, uint32_t* dev_flags,
                             hipStream_t stream) {
  using namespace moe;
  MOE_CHECK(n_src >= 0 && pool_rows >= 0 && n_local >= 1 && n_local <= MOE_MAX_EXPERTS && cap >= 0, MOE_EINVAL);
  MOE_CHECK(d >= 8 && d % 8 == 0, MOE_EINVAL);
  MOE_CHECK(src_rotation >= 0 && src_rotation < (n_src > 0 ? n_src : 1), MOE_EINVAL);
  MOE_CHECK(pool_dtype == MOE_BF16 || is_fp8(pool_dtype), MOE_EINVAL);
  const int64_t rb = row_bytes(pool_dtype, d);                      // bytes per pool row
  const int64_t re = rb / 2;                                        // 16-bit elements per pool row
  const int64_t H = pool_header_rows(rb, pool_rows);
  const int64_t P1 = static_cast<int64_t>(pool_rows) + H;
  const int64_t n_rows = static_cast<int64_t>(n_src) * P1;
  MOE_CHECK(n_rows <= INT32_MAX && static_cast<int64_t>(n_local) * cap <= INT32_MAX, MOE_EUNSUPPORTED);
  MOE_CHECK(counts && recv_dropped, MOE_EINVAL);
  MOE_CHECK(n_src == 0 || (pools_in && row_slot), MOE_EINVAL);
  MOE_CHECK(n_src == 0 || cap == 0 || compact, MOE_EINVAL);
  MOE_CHECK((pools_in == nullptr || aligned16(pools_in)) && (compact == nullptr || aligned16(compact)), MOE_EINVAL);
  MOE_CHECK(ret == nullptr || ((ret_dtype == MOE_F32 || ret_dtype == MOE_BF16) && aligned16(ret)), MOE_EINVAL);
  MOE_CHECK(slot_row == nullptr || aligned4(slot_row), MOE_EINVAL);
  const RowSide side{slot_row, static_cast<vec16*>(ret),
                     static_cast<int64_t>(d) * (ret_dtype == MOE_F32 ? 4 : 2) / 16};
  const int64_t n = static_cast<int64_t>(n_src) * pool_rows;
  const RankGeom g = rank_geom(n, n_local);
  const size_t tb = rank_table_bytes(g);
  MOE_CHECK(ws && ws_bytes >= moe_recv_compact_workspace(n_src, pool_rows, n_local), MOE_EWORKSPACE);
  int32_t* table = static_cast<int32_t*>(ws);
  int32_t* offsets = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + tb);
  int32_t* arrived_ws = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + tb +
                                                   align_up((n_local + 1) * sizeof(int32_t), 256));
  RankScanOut out{arrived ? arrived : arrived_ws, counts, offsets, recv_dropped, 0};
  const bf16_t* pb = static_cast<const bf16_t*>(pools_in);
  int st = bucket_rank(g, HeaderBucket{pb, pool_rows, P1, re, src_rotation, n_src, n_local},
                       CompactEmit{pool_rows, P1, H, src_rotation, n_src, cap, row_slot}, cap, out, table, dev_flags,
                       stream);
  if (st != MOE_OK) return st;
  if (n_rows > 0) {
    const unsigned blocks = static_cast<unsigned>((n_rows + kRowsPerBlock - 1) / kRowsPerBlock);
    if (pool_dtype == MOE_BF16)
      hipLaunchKernelGGL(compact_rows_kernel, dim3(blocks), dim3(kRowsPerBlock * kWave), 0, stream,
                         static_cast<const vec16*>(pools_in), n_rows, P1, H, static_cast<int64_t>(d) / 8, row_slot,
                         static_cast<vec16*>(compact), side);
    else if (pool_dtype == MOE_FP8_ROW)
      hipLaunchKernelGGL(HIP_KERNEL_NAME(compact_fp8_rows_kernel<true>), dim3(blocks), dim3(kRowsPerBlock * kWave),
                         0, stream, static_cast<const uint8_t*>(pools_in), n_rows, P1, H, rb, d, row_slot,
                         static_cast<bf16_t*>(compact), side);
    else
      hipLaunchKernelGGL(HIP_KERNEL_NAME(compact_fp8_rows_kernel<false>), dim3(blocks), dim3(kRowsPerBlock * kWave),
                         0, stream, static_cast<const uint8_t*>(pools_in), n_rows, P1, H, rb, d, row_slot,
                         static_cast<bf16_t*>(compact), side);
    MOE_LAUNCH_CHECK();
  }
  return MOE_OK;
}
