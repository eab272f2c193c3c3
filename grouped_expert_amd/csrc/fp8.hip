// fp8 dispatch records: quantization of rows and dequantization back.
//
// "M6.2 - Expert Parallelism and DeepSeek MoE", 0x0AB-0x0AC: the dispatched
// activation may be fp8 data plus fp32 scales (one per row or per 128
// values); quantization produces the pair, the scales stay with their row
// through every permutation, and dequantization uses the scale at the same
// row.  The scale rule (largest magnitude maps to 448) is the library's.
//
// One wavefront per row.  Per-row scales take two passes over the row (the
// largest magnitude first, the second pass re-reads the row from cache);
// per-128 scales take one: 16 lanes hold a group's 128 values, so a 16-lane
// reduction gives the group's scale before its codes are written.
#include "fp8.h"

namespace moe {
namespace {

constexpr int kQRows = 4;              // rows (wavefronts) per workgroup

template <typename XT, bool ROW>
__global__ __launch_bounds__(kQRows * kWave) void quantize_kernel(const XT* __restrict__ x, int64_t n, int32_t d,
                                                                  uint8_t* __restrict__ rec, int64_t W,
                                                                  uint32_t* flags) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kQRows + threadIdx.x / kWave;
  if (t >= n) return;
  const XT* xr = x + t * d;
  uint8_t* rr = rec + t * W;
  const int32_t G = fp8_groups(ROW ? MOE_FP8_ROW : MOE_FP8_B128, d);
  if (ROW) {
    float amax = 0.0f;
    bool bad = false;
    for (int32_t c = lane * 8; c < d; c += kWave * 8) {
      float v[8];
      load_row8<XT>(xr + c, v);
      amax = fmaxf(amax, amax8(v, &bad));
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
    bad = __any(bad);
    const bool zero = bad || amax == 0.0f;
    // each a correctly rounded fp32 division (the HIP default for '/')
    const float scale = zero ? 0.0f : amax / 448.0f;
    const float inv = zero ? 0.0f : 448.0f / amax;
    for (int32_t c = lane * 8; c < d; c += kWave * 8) {
      float v[8];
      load_row8<XT>(xr + c, v);
      *reinterpret_cast<uint2*>(rr + c) = encode8(v, inv, zero);
    }
    if (lane == 0) {
      *reinterpret_cast<float*>(rr + d) = scale;
      if (bad) flag_or(flags, MOE_FLAG_NONFINITE_INPUT);
    }
  } else {
    for (int32_t c0 = 0; c0 < d; c0 += kWave * 8) {
      const int32_t c = c0 + lane * 8;
      const bool live = c < d;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (live) load_row8<XT>(xr + c, v);
      bool bad = false;
      float amax = amax8(v, &bad);
      int badi = bad ? 1 : 0;
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) {             // the 16 lanes of one 128-value group
        amax = fmaxf(amax, __shfl_xor(amax, off, 16));
        badi |= __shfl_xor(badi, off, 16);
      }
      const bool zero = badi != 0 || amax == 0.0f;
      const float scale = zero ? 0.0f : amax / 448.0f;
      const float inv = zero ? 0.0f : 448.0f / amax;
      if (live) {
        *reinterpret_cast<uint2*>(rr + c) = encode8(v, inv, zero);
        if (lane % 16 == 0) {
          *reinterpret_cast<float*>(rr + d + 4 * (c / 128)) = scale;
          if (badi) flag_or(flags, MOE_FLAG_NONFINITE_INPUT);
        }
      }
    }
  }
  // zero padding: fewer than 128 bytes from a 4-byte boundary (d % 8 == 0),
  // one word per lane
  const int32_t tail_words = (static_cast<int32_t>(W) - d - 4 * G) / 4;
  if (lane < tail_words) reinterpret_cast<uint32_t*>(rr + d + 4 * G)[lane] = 0u;
}

template <typename OT, bool ROW>
__global__ __launch_bounds__(kQRows * kWave) void dequantize_kernel(const uint8_t* __restrict__ rec, int64_t n,
                                                                    int32_t d, int64_t W, OT* __restrict__ out) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kQRows + threadIdx.x / kWave;
  if (t >= n) return;
  const uint8_t* rr = rec + t * W;
  OT* orow = out + t * d;
  for (int32_t c = lane * 8; c < d; c += kWave * 8) {
    float v[8];
    fp8_dequant8<ROW>(rr, c, d, v);
    if constexpr (sizeof(OT) == 2) {
      *reinterpret_cast<vec16*>(orow + c) = pack_bf16x8(v);
    } else {
      reinterpret_cast<float4*>(orow + c)[0] = make_float4(v[0], v[1], v[2], v[3]);
      reinterpret_cast<float4*>(orow + c)[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

}  // namespace
}  // namespace moe

MOE_API size_t moe_row_bytes(int32_t dtype, int32_t d) {
  return static_cast<size_t>(moe::row_bytes(dtype, d));
}

MOE_API int moe_pool_geometry(int32_t row_dtype, int32_t d, int64_t pool_rows, int64_t* header_rows,
                              int64_t* pool_height) {
  using namespace moe;
  const int64_t rb = row_bytes(row_dtype, d);
  MOE_CHECK(rb > 0 && d % 8 == 0 && pool_rows >= 0 && header_rows && pool_height, MOE_EINVAL);
  const int64_t H = pool_header_rows(rb, pool_rows);
  *header_rows = H;
  *pool_height = pool_rows + H;
  return MOE_OK;
}

MOE_API int moe_pool_rows_of_height(int32_t row_dtype, int32_t d, int64_t pool_height, int64_t* pool_rows) {
  using namespace moe;
  const int64_t rb = row_bytes(row_dtype, d);
  MOE_CHECK(rb > 0 && d % 8 == 0 && pool_height >= 1 && pool_rows, MOE_EINVAL);
  // the header grows by one row per rb / 2 data rows, so at most one data-row
  // count fits a height; search the few header counts that can
  const int64_t per_row = rb / 2;
  for (int64_t h = 1; h <= pool_height && h <= pool_height / per_row + 2; ++h) {
    const int64_t p = pool_height - h;
    if (pool_header_rows(rb, p) == h) {
      *pool_rows = p;
      return MOE_OK;
    }
  }
  return MOE_EINVAL;
}

MOE_API int moe_quantize_fp8(const void* x, int32_t x_dtype, int64_t n, int32_t d, int32_t rec_dtype, void* rec,
                             uint32_t* dev_flags, hipStream_t stream) {
  using namespace moe;
  MOE_CHECK((x_dtype == MOE_BF16 || x_dtype == MOE_F32) && is_fp8(rec_dtype), MOE_EINVAL);
  MOE_CHECK(n >= 0 && d >= 8 && d % 8 == 0, MOE_EINVAL);
  MOE_CHECK(n <= 0xFFFFFFFFLL / kWave, MOE_EUNSUPPORTED);
  if (n == 0) return MOE_OK;
  MOE_CHECK(x && rec && aligned16(x) && aligned16(rec), MOE_EINVAL);
  const int64_t W = row_bytes(rec_dtype, d);
  const unsigned blocks = static_cast<unsigned>((n + kQRows - 1) / kQRows);
  const bool row = rec_dtype == MOE_FP8_ROW;
  uint8_t* r = static_cast<uint8_t*>(rec);
  if (x_dtype == MOE_BF16) {
    const bf16_t* xp = static_cast<const bf16_t*>(x);
    if (row)
      hipLaunchKernelGGL(HIP_KERNEL_NAME(quantize_kernel<bf16_t, true>), dim3(blocks), dim3(kQRows * kWave), 0,
                         stream, xp, n, d, r, W, dev_flags);
    else
      hipLaunchKernelGGL(HIP_KERNEL_NAME(quantize_kernel<bf16_t, false>), dim3(blocks), dim3(kQRows * kWave), 0,
                         stream, xp, n, d, r, W, dev_flags);
  } else {
    const float* xp = static_cast<const float*>(x);
    if (row)
      hipLaunchKernelGGL(HIP_KERNEL_NAME(quantize_kernel<float, true>), dim3(blocks), dim3(kQRows * kWave), 0,
                         stream, xp, n, d, r, W, dev_flags);
    else
      hipLaunchKernelGGL(HIP_KERNEL_NAME(quantize_kernel<float, false>), dim3(blocks), dim3(kQRows * kWave), 0,
                         stream, xp, n, d, r, W, dev_flags);
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

MOE_API int moe_dequantize_fp8(const void* rec, int32_t rec_dtype, int64_t n, int32_t d, void* out,
                               int32_t out_dtype, uint32_t* dev_flags, hipStream_t stream) {
  using namespace moe;
  (void)dev_flags;
  MOE_CHECK(is_fp8(rec_dtype) && (out_dtype == MOE_BF16 || out_dtype == MOE_F32), MOE_EINVAL);
  MOE_CHECK(n >= 0 && d >= 8 && d % 8 == 0, MOE_EINVAL);
  MOE_CHECK(n <= 0xFFFFFFFFLL / kWave, MOE_EUNSUPPORTED);
  if (n == 0) return MOE_OK;
  MOE_CHECK(rec && out && aligned16(rec) && aligned16(out), MOE_EINVAL);
  const int64_t W = row_bytes(rec_dtype, d);
  const unsigned blocks = static_cast<unsigned>((n + kQRows - 1) / kQRows);
  const uint8_t* r = static_cast<const uint8_t*>(rec);
  const bool row = rec_dtype == MOE_FP8_ROW;
  if (out_dtype == MOE_BF16) {
    bf16_t* o = static_cast<bf16_t*>(out);
    if (row)
      hipLaunchKernelGGL(HIP_KERNEL_NAME(dequantize_kernel<bf16_t, true>), dim3(blocks), dim3(kQRows * kWave), 0,
                         stream, r, n, d, W, o);
    else
      hipLaunchKernelGGL(HIP_KERNEL_NAME(dequantize_kernel<bf16_t, false>), dim3(blocks), dim3(kQRows * kWave), 0,
                         stream, r, n, d, W, o);
  } else {
    float* o = static_cast<float*>(out);
    if (row)
      hipLaunchKernelGGL(HIP_KERNEL_NAME(dequantize_kernel<float, true>), dim3(blocks), dim3(kQRows * kWave), 0,
                         stream, r, n, d, W, o);
    else
      hipLaunchKernelGGL(HIP_KERNEL_NAME(dequantize_kernel<float, false>), dim3(blocks), dim3(kQRows * kWave), 0,
                         stream, r, n, d, W, o);
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
