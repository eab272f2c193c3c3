// Shared device helpers for the gfx950 kernels of the routed-expert layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace moe {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kXcds = 8;           // MI355X: 8 accelerator complex dies, one L2 each

using bf16_t = uint16_t;

// 16-byte vector used by the row-movement kernels (a native clang vector so
// that the nontemporal builtins accept it).
typedef uint32_t vec16 __attribute__((ext_vector_type(4)));

// --- host-side argument checks ----------------------------------------------

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

#define MOE_CHECK(cond, status) \
  do {                          \
    if (!(cond)) return (status); \
  } while (0)

#define MOE_LAUNCH_CHECK()                                     \
  do {                                                         \
    if (hipGetLastError() != hipSuccess) return MOE_EHIP;      \
  } while (0)

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// --- device helpers -----------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even; NaN stays NaN (quiet bit forced).  Written
// without branches (a select) so that it vectorises in GEMM epilogues.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet = (u >> 16) | 0x40u;
  return static_cast<bf16_t>((u & 0x7fffffffu) > 0x7f800000u ? quiet : rounded);
}

__device__ __forceinline__ void flag_or(uint32_t* flags, uint32_t bit) {
  if (flags) atomicOr(flags, bit);
}

// Bijective block-id remap so that consecutive logical tiles run on the same
// XCD (the hardware deals workgroups round-robin over the 8 XCDs).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t id, uint32_t total) {
  const uint32_t q = total / kXcds, r = total % kXcds;
  const uint32_t xcd = id % kXcds, local = id / kXcds;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// Streaming (nontemporal) 16-byte load / store for data touched once.
__device__ __forceinline__ vec16 ld_stream(const vec16* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_stream(vec16 v, vec16* p) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const uint32_t l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Exclusive scan over a 1024-thread block (16 wavefronts); returns the prefix
// and writes the block total to *total.
__device__ __forceinline__ int32_t block_exclusive_scan_1024(int32_t v, int32_t* sh16, int32_t* total) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  int32_t incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int32_t t = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += t;
  }
  if (lane == kWave - 1) sh16[w] = incl;
  __syncthreads();
  if (w == 0) {
    int32_t x = lane < 16 ? sh16[lane] : 0;
    int32_t xi = x;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int32_t t = __shfl_up(xi, off, kWave);
      if (lane >= off) xi += t;
    }
    if (lane < 16) sh16[lane] = xi - x;       // exclusive wave bases
    if (lane == 15) sh16[16] = xi;            // grand total
  }
  __syncthreads();
  const int32_t r = sh16[w] + incl - v;
  *total = sh16[16];
  return r;
}

}  // namespace moe
