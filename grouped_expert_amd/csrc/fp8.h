// fp8 dispatch records: row widths and the OCP E4M3 codec.
//
// "M6.2 - Expert Parallelism and DeepSeek MoE", 0x0AB-0x0AC: an fp8 payload
// is data plus fp32 scales, one per row or one per 128 values, and the
// scales belong to the row.  A record is the row's d codes, its G scales and
// zero bytes up to a multiple of 16, so every row-moving kernel moves codes
// and scales together.
#pragma once

#include "common.h"

namespace moe {

inline bool is_fp8(int32_t dtype) { return dtype == MOE_FP8_ROW || dtype == MOE_FP8_B128; }

// values per scale group
__host__ __device__ inline int32_t fp8_group_width(int32_t dtype, int32_t d) { return dtype == MOE_FP8_ROW ? d : 128; }

__host__ __device__ inline int32_t fp8_groups(int32_t dtype, int32_t d) {
  return dtype == MOE_FP8_ROW ? 1 : (d + 127) / 128;
}

// Bytes of one stored row; 0 for an unknown dtype.
inline int64_t row_bytes(int32_t dtype, int64_t d) {
  if (d < 1) return 0;
  switch (dtype) {
    case MOE_F32: return 4 * d;
    case MOE_BF16: return 2 * d;
    case MOE_FP8_ROW:
    case MOE_FP8_B128: return (d + 4 * fp8_groups(dtype, static_cast<int32_t>(d)) + 15) / 16 * 16;
    default: return 0;
  }
}

// float -> E4M3 (bias 7, 3 mantissa bits, largest finite 448, 0x7F NaN, no
// infinity): nearest, ties to even, saturating at +-448, sign bit kept.
// Normal results: round the fp32 pattern at bit 20 (half to even), which
// carries into the exponent when needed, and rebias (127 -> 7).  Results
// below 2^-6 are counts of 2^-9: |x| * 512 is exact and rintf rounds half to
// even.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;               // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;              // |x| >= 448 (infinity included)
  if (a >= 0x3c800000u) {                                 // |x| >= 2^-6
    const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
    return sign | (r - (120u << 3));
  }
  return sign | static_cast<uint32_t>(rintf(__uint_as_float(a) * 512.0f));
}

// E4M3 -> float (exact).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t mag = c & 0x7fu;
  float v;
  if (mag == 0x7fu)
    v = __uint_as_float(0x7fc00000u);
  else if (mag < 8u)
    v = static_cast<float>(mag) * (1.0f / 512.0f);        // subnormal: mag units of 2^-9
  else
    v = __uint_as_float(((mag >> 3) + 120u) << 23 | (mag & 7u) << 20);
  return (c & 0x80u) ? -v : v;
}

// The 8 values of record row `rec` at columns [c, c + 8) (c % 8 == 0, so all
// in one scale group): decode(code) * scale, each one fp32 product.
template <bool ROW>
__device__ __forceinline__ void fp8_dequant8(const uint8_t* __restrict__ rec, int32_t c, int32_t d, float (&v)[8]) {
  const uint2 q = *reinterpret_cast<const uint2*>(rec + c);
  const float s = *reinterpret_cast<const float*>(rec + d + 4 * (ROW ? 0 : c / 128));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = e4m3_decode((q.x >> (8 * i)) & 0xffu) * s;
    v[4 + i] = e4m3_decode((q.y >> (8 * i)) & 0xffu) * s;
  }
}

__device__ __forceinline__ vec16 pack_bf16x8(const float (&v)[8]) {
  vec16 o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
  return o;
}

}  // namespace moe
