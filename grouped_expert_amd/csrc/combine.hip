// Un-permute and gate-weighted FP32 combine, its backward, and the
// receiver's row expansion.
//
// "M6.6 - MoE Runtime Systems", 0x03C3: the return path applies the inverse
// permutation and the combine is a weighted scatter-add over the semantic key
// (origin token); 0x0CD: gather by the inverse, multiply by the route's gate,
// add into the token row; 0x0AE: gate and token accumulation in FP32.
//
// The scatter-add is turned into a gather: one workgroup owns one token row
// slice, reads the k route rows through idx in ascending slot order and adds
// them in registers, so every output element is written once, with no
// atomics, in a fixed order (deterministic).
#include "common.h"

namespace moe {
namespace {

template <typename ZT>
struct Vec;

template <>
struct Vec<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* v) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
};

template <>
struct Vec<bf16_t> {
  static constexpr int N = 8;
  __device__ static void load(const bf16_t* p, float* v) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

template <typename ZT>
__global__ __launch_bounds__(256) void combine_kernel(const ZT* __restrict__ z, int32_t d,
                                                      const int32_t* __restrict__ idx, int64_t lo, int64_t hi,
                                                      const float* __restrict__ gates, int32_t k,
                                                      float* __restrict__ y, int32_t accumulate, uint32_t* flags) {
  constexpr int N = Vec<ZT>::N;
  const int64_t t = blockIdx.x;
  const int64_t col = (static_cast<int64_t>(blockIdx.y) * blockDim.x + threadIdx.x) * N;
  float acc[N];
  float* yrow = y + t * d + col;
  const bool live = col < d;
  if (live && accumulate) {
#pragma unroll
    for (int q = 0; q < N; q += 4) {
      const float4 a = *reinterpret_cast<const float4*>(yrow + q);
      acc[q] = a.x; acc[q + 1] = a.y; acc[q + 2] = a.z; acc[q + 3] = a.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < N; ++q) acc[q] = 0.0f;
  }
  for (int j = 0; j < k; ++j) {
    const int64_t r = t * k + j;
    const int32_t i = idx[r];
    if (i < -1) {
      if (threadIdx.x == 0 && blockIdx.y == 0) flag_or(flags, MOE_FLAG_BAD_INDEX);
      continue;
    }
    if (i < lo || i >= hi) continue;
    const float g = gates ? gates[r] : 1.0f;
    if (!live) continue;
    float v[N];
    Vec<ZT>::load(z + (i - lo) * d + col, v);
#pragma unroll
    for (int q = 0; q < N; ++q) acc[q] = fmaf(g, v[q], acc[q]);
  }
  if (live) {
#pragma unroll
    for (int q = 0; q < N; q += 4)
      *reinterpret_cast<float4*>(yrow + q) = make_float4(acc[q], acc[q + 1], acc[q + 2], acc[q + 3]);
  }
}

template <typename ZT>
void launch(const void* z, int32_t d, const int32_t* idx, int64_t lo, int64_t hi, const float* gates, int64_t T,
            int32_t k, float* y, int32_t acc, uint32_t* flags, hipStream_t s) {
  constexpr int N = Vec<ZT>::N;
  const int64_t lanes = (d + N - 1) / N;
  const int threads = static_cast<int>(lanes >= 256 ? 256 : ((lanes + 63) / 64) * 64);
  const unsigned gy = static_cast<unsigned>((lanes + threads - 1) / threads);
  hipLaunchKernelGGL(HIP_KERNEL_NAME(combine_kernel<ZT>), dim3(static_cast<unsigned>(T), gy), dim3(threads), 0, s,
                     static_cast<const ZT*>(z), d, idx, lo, hi, gates, k, y, acc, flags);
}

// Backward of the combine ("M6.2 - Expert Parallelism and DeepSeek MoE",
// 0x03D): one wavefront per token; for every accepted route the token's
// upstream gradient row, scaled by the gate, is written to the route's row of
// dz, and a wavefront sum of the products with the route's forward row z
// gives the gate gradient.
constexpr int kBwdTok = 4;

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float (&v)[8]) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&v)[8]);

template <>
__device__ __forceinline__ void store8<float>(float* p, const float (&v)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

template <>
__device__ __forceinline__ void store8<bf16_t>(bf16_t* p, const float (&v)[8]) {
  uint4 q;
  q.x = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
  q.y = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
  q.z = f32_to_bf16(v[4]) | (static_cast<uint32_t>(f32_to_bf16(v[5])) << 16);
  q.w = f32_to_bf16(v[6]) | (static_cast<uint32_t>(f32_to_bf16(v[7])) << 16);
  *reinterpret_cast<uint4*>(p) = q;
}

template <typename ZT, typename DT>
__global__ __launch_bounds__(kBwdTok * kWave) void combine_backward_kernel(
    const float* __restrict__ dy, int64_t T, int32_t d, const ZT* __restrict__ z, int64_t rows,
    const int32_t* __restrict__ idx, const float* __restrict__ gates, int32_t k, DT* __restrict__ dz,
    float* __restrict__ dgates, uint32_t* flags) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kBwdTok + threadIdx.x / kWave;
  if (t >= T) return;
  const float* dyrow = dy + t * d;
  for (int j = 0; j < k; ++j) {             // the dY row is re-read per route from cache, not HBM
    const int64_t r = t * k + j;
    const int32_t i = idx[r];
    if (i < 0 || i >= rows) {
      if (lane == 0) {
        if (i != -1) flag_or(flags, MOE_FLAG_BAD_INDEX);
        dgates[r] = 0.0f;
      }
      continue;
    }
    const float gj = gates[r];
    const ZT* zrow = z + static_cast<int64_t>(i) * d;
    DT* dzrow = dz + static_cast<int64_t>(i) * d;
    float acc = 0.0f;
    for (int c = lane * 8; c < d; c += kWave * 8) {
      float v[8], zv[8], o[8];
      load8<float>(dyrow + c, v);
      load8<ZT>(zrow + c, zv);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        acc = fmaf(v[q], zv[q], acc);
        o[q] = gj * v[q];
      }
      store8<DT>(dzrow + c, o);
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kWave);
    if (lane == 0) dgates[r] = acc;
  }
}

template <typename ZT, typename DT>
void launch_combine_bwd(const float* dy, int64_t T, int32_t d, const void* z, int64_t rows, const int32_t* idx,
                        const float* gates, int32_t k, void* dz, float* dgates, uint32_t* flags, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((T + kBwdTok - 1) / kBwdTok);
  hipLaunchKernelGGL(HIP_KERNEL_NAME(combine_backward_kernel<ZT, DT>), dim3(blocks), dim3(kBwdTok * kWave), 0, s,
                     dy, T, d, static_cast<const ZT*>(z), rows, idx, gates, k, static_cast<DT*>(dz), dgates, flags);
}

// Row expansion: one wavefront per output row, each lane moving 16-byte
// output pieces (8 bf16 or 4 fp32 values) read from the slot's row.
constexpr int kExpandRows = 4;

template <typename ZT, typename RT>
__device__ __forceinline__ vec16 expand_piece(const ZT* zrow, int64_t c);

template <>
__device__ __forceinline__ vec16 expand_piece<bf16_t, bf16_t>(const bf16_t* zrow, int64_t c) {
  return reinterpret_cast<const vec16*>(zrow)[c];
}

template <>
__device__ __forceinline__ vec16 expand_piece<float, float>(const float* zrow, int64_t c) {
  return reinterpret_cast<const vec16*>(zrow)[c];
}

template <>
__device__ __forceinline__ vec16 expand_piece<float, bf16_t>(const float* zrow, int64_t c) {
  const float4 a = reinterpret_cast<const float4*>(zrow)[2 * c];
  const float4 b = reinterpret_cast<const float4*>(zrow)[2 * c + 1];
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  vec16 o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
  return o;
}

template <>
__device__ __forceinline__ vec16 expand_piece<bf16_t, float>(const bf16_t* zrow, int64_t c) {
  const uint2 q = reinterpret_cast<const uint2*>(zrow)[c];
  vec16 o;
  o[0] = q.x << 16;
  o[1] = q.x & 0xffff0000u;
  o[2] = q.y << 16;
  o[3] = q.y & 0xffff0000u;
  return o;
}

template <typename ZT, typename RT>
__global__ __launch_bounds__(kExpandRows * kWave) void expand_rows_kernel(
    const ZT* __restrict__ z, int64_t d, const int32_t* __restrict__ row_slot, int64_t n_rows, int64_t n_slots,
    RT* __restrict__ ret, uint32_t* flags) {
  const int lane = threadIdx.x % kWave;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kExpandRows + threadIdx.x / kWave;
  if (row >= n_rows) return;
  const int32_t s = row_slot[row];
  const bool live = s >= 0 && s < n_slots;
  if (!live && s != -1 && lane == 0) flag_or(flags, MOE_FLAG_BAD_INDEX);
  const int64_t pieces = d * static_cast<int64_t>(sizeof(RT)) / 16;
  vec16* out = reinterpret_cast<vec16*>(ret + row * d);
  if (!live) {
    const vec16 zero = {0u, 0u, 0u, 0u};
    for (int64_t c = lane; c < pieces; c += kWave) st_stream(zero, out + c);
    return;
  }
  const ZT* zrow = z + static_cast<int64_t>(s) * d;
  for (int64_t c = lane; c < pieces; c += kWave) st_stream(expand_piece<ZT, RT>(zrow, c), out + c);
}

template <typename ZT, typename RT>
void launch_expand(const void* z, int32_t d, const int32_t* row_slot, int64_t n_rows, int64_t n_slots, void* ret,
                   uint32_t* flags, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((n_rows + kExpandRows - 1) / kExpandRows);
  hipLaunchKernelGGL(HIP_KERNEL_NAME(expand_rows_kernel<ZT, RT>), dim3(blocks), dim3(kExpandRows * kWave), 0, s,
                     static_cast<const ZT*>(z), static_cast<int64_t>(d), row_slot, n_rows, n_slots,
                     static_cast<RT*>(ret), flags);
}

}  // namespace
}  // namespace moe

MOE_API int moe_expand_rows(const void* z, int32_t z_dtype, int32_t d, const int32_t* row_slot, int64_t n_rows,
                            int64_t n_slots, void* ret, int32_t ret_dtype, uint32_t* dev_flags,
                            hipStream_t stream) {
  using namespace moe;
  MOE_CHECK((z_dtype == MOE_F32 || z_dtype == MOE_BF16) && (ret_dtype == MOE_F32 || ret_dtype == MOE_BF16),
            MOE_EINVAL);
  MOE_CHECK(d >= 8 && d % 8 == 0 && n_rows >= 0 && n_slots >= 0, MOE_EINVAL);
  // the launch's total work-item count must fit 32 bits
  MOE_CHECK(n_rows <= 0xFFFFFFFFLL / kWave && n_slots <= 0x80000000LL, MOE_EUNSUPPORTED);
  if (n_rows == 0) return MOE_OK;
  MOE_CHECK(row_slot && ret && (z || n_slots == 0), MOE_EINVAL);
  MOE_CHECK(aligned16(ret) && (z == nullptr || aligned16(z)) && aligned4(row_slot), MOE_EINVAL);
  if (z_dtype == MOE_BF16 && ret_dtype == MOE_BF16)
    launch_expand<bf16_t, bf16_t>(z, d, row_slot, n_rows, n_slots, ret, dev_flags, stream);
  else if (z_dtype == MOE_F32 && ret_dtype == MOE_F32)
    launch_expand<float, float>(z, d, row_slot, n_rows, n_slots, ret, dev_flags, stream);
  else if (z_dtype == MOE_F32)
    launch_expand<float, bf16_t>(z, d, row_slot, n_rows, n_slots, ret, dev_flags, stream);
  else
    launch_expand<bf16_t, float>(z, d, row_slot, n_rows, n_slots, ret, dev_flags, stream);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

MOE_API int moe_combine_backward(const float* dy, int64_t T, int32_t d, const void* z, int32_t z_dtype,
                                 int64_t rows, const int32_t* idx, const float* gates, int32_t k, void* dz,
                                 int32_t dz_dtype, float* dgates, uint32_t* dev_flags, hipStream_t stream) {
  using namespace moe;
  MOE_CHECK((z_dtype == MOE_F32 || z_dtype == MOE_BF16) && (dz_dtype == MOE_F32 || dz_dtype == MOE_BF16),
            MOE_EINVAL);
  MOE_CHECK(T >= 0 && k >= 1 && k <= MOE_MAX_TOPK && d >= 8 && d % 8 == 0 && rows >= 0, MOE_EINVAL);
  MOE_CHECK(T <= INT32_MAX / k && T <= 0xFFFFFFFFLL / kWave && rows <= INT32_MAX, MOE_EUNSUPPORTED);
  if (T == 0) return MOE_OK;
  MOE_CHECK(dy && idx && gates && dgates && (rows == 0 || (z && dz)), MOE_EINVAL);
  MOE_CHECK(aligned16(dy) && (z == nullptr || aligned16(z)) && (dz == nullptr || aligned16(dz)), MOE_EINVAL);
  MOE_CHECK(aligned4(idx) && aligned4(gates) && aligned4(dgates), MOE_EINVAL);
  if (z_dtype == MOE_BF16 && dz_dtype == MOE_BF16)
    launch_combine_bwd<bf16_t, bf16_t>(dy, T, d, z, rows, idx, gates, k, dz, dgates, dev_flags, stream);
  else if (z_dtype == MOE_BF16)
    launch_combine_bwd<bf16_t, float>(dy, T, d, z, rows, idx, gates, k, dz, dgates, dev_flags, stream);
  else if (dz_dtype == MOE_BF16)
    launch_combine_bwd<float, bf16_t>(dy, T, d, z, rows, idx, gates, k, dz, dgates, dev_flags, stream);
  else
    launch_combine_bwd<float, float>(dy, T, d, z, rows, idx, gates, k, dz, dgates, dev_flags, stream);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

MOE_API int moe_unpermute_combine(const void* z, int32_t z_dtype, int32_t d, const int32_t* idx, int64_t lo,
                                  int64_t hi, const float* gates, int64_t T, int32_t k, float* y,
                                  int32_t accumulate, uint32_t* dev_flags, hipStream_t stream) {
  using namespace moe;
  MOE_CHECK(z_dtype == MOE_F32 || z_dtype == MOE_BF16, MOE_EINVAL);
  MOE_CHECK(T >= 0 && k >= 1 && d >= 1 && lo >= 0 && hi >= lo, MOE_EINVAL);
  MOE_CHECK(T <= INT32_MAX / k && T <= 0x7fffffffLL, MOE_EUNSUPPORTED);
  MOE_CHECK(d % (z_dtype == MOE_F32 ? 4 : 8) == 0, MOE_EINVAL);
  if (T == 0) return MOE_OK;
  MOE_CHECK(idx && y && (z || hi == lo), MOE_EINVAL);
  MOE_CHECK((z == nullptr || aligned16(z)) && aligned16(y) && aligned4(idx), MOE_EINVAL);
  MOE_CHECK(gates == nullptr || aligned4(gates), MOE_EINVAL);
  if (z_dtype == MOE_F32)
    launch<float>(z, d, idx, lo, hi, gates, T, k, y, accumulate, dev_flags, stream);
  else
    launch<bf16_t>(z, d, idx, lo, hi, gates, T, k, y, accumulate, dev_flags, stream);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
