// fp8 dispatch records: row widths and the OCP E4M3 codec.
//
// "M6.2 - Expert Parallelism and DeepSeek MoE", 0x0AB-0x0AC: an fp8 payload
// is data plus fp32 scales, one per row or one per 128 values, and the
// scales belong to the row.  A record is the row's d codes, its G scales and
// zero bytes up to a multiple of 128, so every row-moving kernel moves codes
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

// Bytes of one stored row; 0 for an unknown dtype.  fp8 records are padded to
// whole 128-byte cache lines, so no line holds the end of one record and the
// start of the next (rows written by different waves at different times):
// with 16-byte padding the quantizing pack ran about 10 % slower.
inline int64_t row_bytes(int32_t dtype, int64_t d) {
  if (d < 1) return 0;
  switch (dtype) {
    case MOE_F32: return 4 * d;
    case MOE_BF16: return 2 * d;
    case MOE_FP8_ROW:
    case MOE_FP8_B128: return (d + 4 * fp8_groups(dtype, static_cast<int32_t>(d)) + 127) / 128 * 128;
    default: return 0;
  }
}

// Header rows of a pool whose rows are rb bytes and which holds pool_rows
// data rows: one 16-bit local id per data row, rb / 2 ids per header row, at
// least one row ("Fixed pooled-wave all-to-all for the 8-of-384 MoE", 02 and
// 05: one packed full-width row at the page's sizes).  0 for rb < 2 or a
// negative row count.
inline int64_t pool_header_rows(int64_t rb, int64_t pool_rows) {
  if (rb < 2 || pool_rows < 0) return 0;
  const int64_t per_row = rb / 2;
  return pool_rows > per_row ? (pool_rows + per_row - 1) / per_row : 1;
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

// Quantization helpers shared by moe_quantize_fp8 and the quantizing pack:
// 8 values of a row, their largest magnitude, their codes.
template <typename XT>
__device__ __forceinline__ void load_row8(const XT* p, float (&v)[8]);

template <>
__device__ __forceinline__ void load_row8<bf16_t>(const bf16_t* p, float (&v)[8]) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void load_row8<float>(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Largest magnitude of 8 values; *bad set when one is NaN or infinite.
__device__ __forceinline__ float amax8(const float (&v)[8], bool* bad) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = fabsf(v[i]);
    if (!(a <= 3.402823466e38f)) *bad = true;
    m = fmaxf(m, a);
  }
  return m;
}

// The 8 codes of one piece, as two words.  With amax = 0 or a bad group every
// code is 0.  x * inv is one fp32 product.
__device__ __forceinline__ uint2 encode8(const float (&v)[8], float inv, bool zero) {
  uint2 q = {0u, 0u};
  if (zero) return q;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    q.x |= e4m3_encode(v[i] * inv) << (8 * i);
    q.y |= e4m3_encode(v[4 + i] * inv) << (8 * i);
  }
  return q;
}

}  // namespace moe
