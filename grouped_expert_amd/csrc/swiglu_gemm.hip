// Grouped SwiGLU expert GEMM over ragged row segments.
//
// "M6.6 - MoE Runtime Systems", 0x04A: every expert is bias-free SwiGLU,
// G = X W_g^T, U = X W_u^T, E(X) = (SiLU(G) * U) W_2^T, with 6 n d d_ff
// matmul FLOPs for n rows; 0x04C: a grouped runner keeps the exact row count
// of every active expert and shares one launch, with per-problem state built
// for every non-empty segment (a zero-row expert must not shift the weights of
// later experts, 0x04G).  "Fixed pooled-wave all-to-all for the 8-of-384
// MoE", 03: one batched SwiGLU serves all local experts of a wave.
//
// Launch sequence (no host synchronisation; the grid is sized from the
// host-known row bound and idle workgroups leave at once):
//   1. tile table: one workgroup turns seg_start / seg_count into a list of
//      (expert, first row, segment end) M-tiles.
//   2. gate/up: per (M-tile, N-tile) workgroup, G and U tiles on bf16 MFMA
//      with fp32 accumulation; epilogue H = SiLU(G) * U rounded to bf16.
//   3. down: Z = H W_d^T on bf16 MFMA, fp32 accumulation, stored bf16 or fp32.
//
// Data layout (all row-major, K contiguous for both operands):
//   x [rows, d], W_g / W_u [E, d_ff, d], W_d [E, d, d_ff], H [rows, d_ff]
//   (workspace), z [rows, d].  Both products are "A times B^T" with the K
//   dimension contiguous in A and in B, which is the native operand order of
//   the MFMA (each lane reads 8 consecutive K values of one row).
//
// The fp32 variant (dtype MOE_F32) runs the same three steps with an LDS-tiled
// FMA kernel in fp32.
#include "common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct TileEntry {
  int32_t expert, row0, row_end, pad;
};

// ---------------------------------------------------------------------------
// 1. tile table
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ seg_start,
                                                           const int32_t* __restrict__ seg_count, int32_t E,
                                                           int64_t rows, int32_t BM, int32_t max_tiles,
                                                           TileEntry* __restrict__ tiles,
                                                           int32_t* __restrict__ n_tiles, uint32_t* flags) {
  __shared__ int32_t sh16[17];
  const int t = threadIdx.x;
  int32_t s = 0, c = 0;
  if (t < E) {
    s = seg_start[t];
    c = seg_count[t];
    const bool ok = s >= 0 && c >= 0 && static_cast<int64_t>(s) + c <= rows;
    if (!ok) {
      flag_or(flags, MOE_FLAG_BAD_SEGMENT);
      c = 0;
    }
  }
  const int32_t cnt = (c + BM - 1) / BM;
  int32_t total = 0;
  const int32_t pre = block_exclusive_scan_1024(cnt, sh16, &total);
  for (int32_t i = 0; i < cnt; ++i) {
    const int32_t idx = pre + i;
    if (idx < max_tiles) tiles[idx] = TileEntry{t, s + i * BM, s + c, 0};
  }
  if (t == 0) {
    n_tiles[0] = total < max_tiles ? total : max_tiles;
    if (total > max_tiles) flag_or(flags, MOE_FLAG_BAD_SEGMENT);   // overlapping segments
  }
}

// ---------------------------------------------------------------------------
// 2./3. bf16 MFMA GEMM:  C[m, n] = sum_k A[m, k] * B[n, k]
// ---------------------------------------------------------------------------
constexpr int kThreads = 256;   // 4 wavefronts

// LDS tile of R rows x BK bf16 (BK = 64: 8 chunks of 16 B per row).  The chunk
// index is XOR-swizzled with (row / 2) so that the 16 lanes of one 256-byte
// LDS access phase hit 16 different bank groups for both the fragment reads
// (lanes walk rows) and the tile writes (lanes walk chunks of two rows).
__device__ __forceinline__ int lds_off(int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 7)) << 3); }

template <int BM, int BNB, int WM, int WN, bool GATEUP, bool OUT_F32>
struct GemmCfg {
  static constexpr int BK = 64;
  static constexpr int WTM = BM / WM;                     // rows per wave
  static constexpr int TM = WTM / 32;                     // 32-row MFMA tiles per wave
  // GATEUP: the B tile holds BNB/2 gate rows then BNB/2 up rows; the output
  // tile has BNB/2 columns of H.  Otherwise BNB output columns.
  static constexpr int BN_OUT = GATEUP ? BNB / 2 : BNB;
  static constexpr int WTN = BN_OUT / WN;                 // output columns per wave
  static constexpr int TN = WTN / 32;
  static constexpr int NB = GATEUP ? 2 : 1;               // B halves per output tile
  static constexpr int A_VECS = BM * BK / 8 / kThreads;   // 16-byte loads per thread per K tile
  static constexpr int B_VECS = BNB * BK / 8 / kThreads;
  static_assert(WM * WN == 4, "four wavefronts");
  static_assert(TM >= 1 && TN >= 1, "wave tile too small");
  static_assert(A_VECS >= 1 && B_VECS >= 1, "tile too small");
};

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

template <int BM, int BNB, int WM, int WN, bool GATEUP, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void grouped_gemm_bf16_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1,
    void* __restrict__ C, int32_t K, int32_t N, const TileEntry* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles_ptr, int32_t n_tiles_n) {
  using Cfg = GemmCfg<BM, BNB, WM, WN, GATEUP, OUT_F32>;
  constexpr int BK = Cfg::BK;
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BNB * BK];

  const uint32_t total = static_cast<uint32_t>(*n_tiles_ptr) * n_tiles_n;
  if (blockIdx.x >= total) return;
  const uint32_t logical = xcd_remap(blockIdx.x, total);
  const int mt = static_cast<int>(logical / n_tiles_n);
  const int nt = static_cast<int>(logical % n_tiles_n);
  const TileEntry te = tiles[mt];
  const int64_t e = te.expert;
  const int32_t row0 = te.row0, row_end = te.row_end;
  const int32_t n0 = nt * Cfg::BN_OUT;

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;

  // global -> register staging coordinates
  const bf16_t* a_src[Cfg::A_VECS];
  bool a_ok[Cfg::A_VECS];
  int a_lds[Cfg::A_VECS];
#pragma unroll
  for (int v = 0; v < Cfg::A_VECS; ++v) {
    const int idx = tid + v * kThreads;
    const int r = idx / 8, c = idx % 8;
    const int32_t row = row0 + r;
    a_ok[v] = row < row_end;
    a_src[v] = A + static_cast<int64_t>(a_ok[v] ? row : row0) * K + c * 8;
    a_lds[v] = lds_off(r, c);
  }
  const bf16_t* b_src[Cfg::B_VECS];
  int b_lds[Cfg::B_VECS];
#pragma unroll
  for (int v = 0; v < Cfg::B_VECS; ++v) {
    const int idx = tid + v * kThreads;
    const int r = idx / 8, c = idx % 8;
    const bf16_t* base;
    int n;
    if (GATEUP) {
      const bool up = r >= BNB / 2;
      base = up ? B1 : B0;
      n = n0 + (up ? r - BNB / 2 : r);
    } else {
      base = B0;
      n = n0 + r;
    }
    b_src[v] = base + (e * N + n) * static_cast<int64_t>(K) + c * 8;
    b_lds[v] = lds_off(r, c);
  }

  f32x16 acc[Cfg::NB][Cfg::TM][Cfg::TN];
#pragma unroll
  for (int h = 0; h < Cfg::NB; ++h)
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[h][i][j][q] = 0.0f;

  uint4 ra[Cfg::A_VECS], rb[Cfg::B_VECS];
  auto gload = [&](int kt) {
    const int64_t ko = static_cast<int64_t>(kt) * BK;
#pragma unroll
    for (int v = 0; v < Cfg::A_VECS; ++v)
      ra[v] = a_ok[v] ? *reinterpret_cast<const uint4*>(a_src[v] + ko) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < Cfg::B_VECS; ++v) rb[v] = *reinterpret_cast<const uint4*>(b_src[v] + ko);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int v = 0; v < Cfg::A_VECS; ++v) *reinterpret_cast<uint4*>(&As[buf][a_lds[v]]) = ra[v];
#pragma unroll
    for (int v = 0; v < Cfg::B_VECS; ++v) *reinterpret_cast<uint4*>(&Bs[buf][b_lds[v]]) = rb[v];
  };

  const int KT = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();

  const int lr = lane % 32, lk = lane / 32;
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int chunk = kk * 2 + lk;
      bf16x8 af[Cfg::TM];
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(&As[buf][lds_off(wm * Cfg::WTM + i * 32 + lr, chunk)]);
#pragma unroll
      for (int h = 0; h < Cfg::NB; ++h) {
#pragma unroll
        for (int j = 0; j < Cfg::TN; ++j) {
          const int brow = h * (BNB / 2) + wn * Cfg::WTN + j * 32 + lr;
          const bf16x8 bfr = *reinterpret_cast<const bf16x8*>(&Bs[buf][lds_off(brow, chunk)]);
#pragma unroll
          for (int i = 0; i < Cfg::TM; ++i)
            acc[h][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr, acc[h][i][j], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < KT) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: acc[q] holds C[m = 8*(q/4) + 4*(lane/32) + q%4][n = lane%32]
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i) {
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) {
      const int col = n0 + wn * Cfg::WTN + j * 32 + lr;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int32_t row = row0 + wm * Cfg::WTM + i * 32 + 8 * (q / 4) + 4 * lk + (q % 4);
        if (row >= row_end) continue;
        const int64_t o = static_cast<int64_t>(row) * N + col;
        if (GATEUP) {
          const float h = silu_f32(acc[0][i][j][q]) * acc[Cfg::NB - 1][i][j][q];
          static_cast<bf16_t*>(C)[o] = f32_to_bf16(h);
        } else if (OUT_F32) {
          static_cast<float*>(C)[o] = acc[0][i][j][q];
        } else {
          static_cast<bf16_t*>(C)[o] = f32_to_bf16(acc[0][i][j][q]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 path: LDS-tiled FMA GEMM, 64 x 64 output tile, 4 x 4 per thread
// ---------------------------------------------------------------------------
constexpr int kF32BM = 64, kF32BN = 64, kF32BK = 16;

template <bool GATEUP>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(const float* __restrict__ A,
                                                               const float* __restrict__ B0,
                                                               const float* __restrict__ B1, float* __restrict__ C,
                                                               int32_t K, int32_t N,
                                                               const TileEntry* __restrict__ tiles,
                                                               const int32_t* __restrict__ n_tiles_ptr,
                                                               int32_t n_tiles_n) {
  constexpr int NB = GATEUP ? 2 : 1;
  __shared__ float As[kF32BK][kF32BM + 4];
  __shared__ float Bs[NB][kF32BK][kF32BN + 4];
  const uint32_t total = static_cast<uint32_t>(*n_tiles_ptr) * n_tiles_n;
  if (blockIdx.x >= total) return;
  const uint32_t logical = xcd_remap(blockIdx.x, total);
  const int mt = static_cast<int>(logical / n_tiles_n), nt = static_cast<int>(logical % n_tiles_n);
  const TileEntry te = tiles[mt];
  const int64_t e = te.expert;
  const int32_t row0 = te.row0, row_end = te.row_end, n0 = nt * kF32BN;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[NB][4][4] = {};
  for (int k0 = 0; k0 < K; k0 += kF32BK) {
    for (int idx = threadIdx.x; idx < kF32BM * kF32BK; idx += 256) {
      const int r = idx / kF32BK, c = idx % kF32BK;
      const int32_t row = row0 + r;
      As[c][r] = row < row_end ? A[static_cast<int64_t>(row) * K + k0 + c] : 0.0f;
    }
    for (int h = 0; h < NB; ++h) {
      const float* Bh = h ? B1 : B0;
      for (int idx = threadIdx.x; idx < kF32BN * kF32BK; idx += 256) {
        const int r = idx / kF32BK, c = idx % kF32BK;
        Bs[h][c][r] = Bh[(e * N + n0 + r) * static_cast<int64_t>(K) + k0 + c];
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kF32BK; ++kk) {
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int h = 0; h < NB; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float b = Bs[h][kk][tx * 4 + j];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[h][i][j] = fmaf(a[i], b, acc[h][i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t row = row0 + ty * 4 + i;
    if (row >= row_end) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      const float v = GATEUP ? silu_f32(acc[0][i][j]) * acc[NB - 1][i][j] : acc[0][i][j];
      C[static_cast<int64_t>(row) * N + col] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
constexpr int kBM = 128;                  // rows per M-tile, bf16 path
constexpr int kGU_BNB = 128;              // gate/up B rows per tile (64 gate + 64 up) -> 64 H columns
constexpr int kDN_BNB = 128;              // down output columns per tile

struct WsLayout {
  size_t h_off, h_bytes, tiles_off, ntiles_off, total;
  int32_t max_tiles, bm;
};

inline WsLayout ws_layout(int64_t rows, int32_t E, int32_t d_ff, int32_t dtype) {
  WsLayout w;
  w.bm = dtype == MOE_F32 ? kF32BM : kBM;
  const size_t elt = dtype == MOE_F32 ? 4 : 2;
  w.max_tiles = static_cast<int32_t>((rows + w.bm - 1) / w.bm + E);
  w.h_off = 0;
  w.h_bytes = align_up(static_cast<size_t>(rows) * d_ff * elt, 256);
  w.tiles_off = w.h_bytes;
  w.ntiles_off = w.tiles_off + align_up(static_cast<size_t>(w.max_tiles) * sizeof(TileEntry), 256);
  w.total = w.ntiles_off + 256;
  return w;
}

}  // namespace
}  // namespace moe

MOE_API size_t moe_grouped_swiglu_workspace(int64_t rows, int32_t E, int32_t d_ff, int32_t dtype) {
  using namespace moe;
  if (rows < 0 || E < 1 || E > MOE_MAX_EXPERTS || d_ff < 1 || (dtype != MOE_F32 && dtype != MOE_BF16)) return 0;
  return ws_layout(rows, E, d_ff, dtype).total;
}

MOE_API int moe_grouped_swiglu(const void* x, int32_t dtype, int32_t d, int32_t d_ff, int32_t E,
                               const int32_t* seg_start, const int32_t* seg_count, int64_t rows,
                               const void* w_gate, const void* w_up, const void* w_down, void* z, int32_t z_dtype,
                               void* ws, size_t ws_bytes, uint32_t* dev_flags, hipStream_t stream) {
  using namespace moe;
  MOE_CHECK(dtype == MOE_F32 || dtype == MOE_BF16, MOE_EINVAL);
  MOE_CHECK(z_dtype == MOE_F32 || z_dtype == MOE_BF16, MOE_EINVAL);
  MOE_CHECK(dtype == MOE_BF16 || z_dtype == MOE_F32, MOE_EUNSUPPORTED);
  MOE_CHECK(E >= 1 && E <= MOE_MAX_EXPERTS && d >= 1 && d_ff >= 1 && rows >= 0, MOE_EINVAL);
  MOE_CHECK(d % 64 == 0 && d_ff % 64 == 0, MOE_EUNSUPPORTED);
  if (dtype == MOE_BF16) MOE_CHECK(d % kDN_BNB == 0 && d_ff % (kGU_BNB / 2) == 0, MOE_EUNSUPPORTED);
  MOE_CHECK(rows <= INT32_MAX - kBM, MOE_EUNSUPPORTED);
  MOE_CHECK(seg_start && seg_count && w_gate && w_up && w_down, MOE_EINVAL);
  MOE_CHECK(rows == 0 || (x && z), MOE_EINVAL);
  MOE_CHECK((x == nullptr || aligned16(x)) && (z == nullptr || aligned16(z)), MOE_EINVAL);
  MOE_CHECK(aligned16(w_gate) && aligned16(w_up) && aligned16(w_down), MOE_EINVAL);
  const WsLayout L = ws_layout(rows, E, d_ff, dtype);
  MOE_CHECK(ws && ws_bytes >= L.total && aligned16(ws), MOE_EWORKSPACE);
  char* wsb = static_cast<char*>(ws);
  void* H = wsb + L.h_off;
  TileEntry* tiles = reinterpret_cast<TileEntry*>(wsb + L.tiles_off);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(wsb + L.ntiles_off);

  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, stream, seg_start, seg_count, E, rows, L.bm,
                     L.max_tiles, tiles, n_tiles, dev_flags);
  MOE_LAUNCH_CHECK();
  if (rows == 0) return MOE_OK;

  if (dtype == MOE_F32) {
    const int nt1 = d_ff / kF32BN, nt2 = d / kF32BN;
    hipLaunchKernelGGL(HIP_KERNEL_NAME(grouped_gemm_f32_kernel<true>), dim3(L.max_tiles * nt1), dim3(256), 0,
                       stream, static_cast<const float*>(x), static_cast<const float*>(w_gate),
                       static_cast<const float*>(w_up), static_cast<float*>(H), d, d_ff, tiles, n_tiles, nt1);
    MOE_LAUNCH_CHECK();
    hipLaunchKernelGGL(HIP_KERNEL_NAME(grouped_gemm_f32_kernel<false>), dim3(L.max_tiles * nt2), dim3(256), 0,
                       stream, static_cast<const float*>(H), static_cast<const float*>(w_down),
                       static_cast<const float*>(nullptr), static_cast<float*>(z), d_ff, d, tiles, n_tiles, nt2);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
  }

  const int nt1 = d_ff / (kGU_BNB / 2), nt2 = d / kDN_BNB;
  MOE_CHECK(static_cast<int64_t>(L.max_tiles) * (nt1 > nt2 ? nt1 : nt2) <= INT32_MAX, MOE_EUNSUPPORTED);
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  hipLaunchKernelGGL(HIP_KERNEL_NAME(grouped_gemm_bf16_kernel<kBM, kGU_BNB, 2, 2, true, false>),
                     dim3(L.max_tiles * nt1), dim3(kThreads), 0, stream, xb, static_cast<const bf16_t*>(w_gate),
                     static_cast<const bf16_t*>(w_up), H, d, d_ff, tiles, n_tiles, nt1);
  MOE_LAUNCH_CHECK();
  if (z_dtype == MOE_F32)
    hipLaunchKernelGGL(HIP_KERNEL_NAME(grouped_gemm_bf16_kernel<kBM, kDN_BNB, 2, 2, false, true>),
                       dim3(L.max_tiles * nt2), dim3(kThreads), 0, stream, static_cast<const bf16_t*>(H),
                       static_cast<const bf16_t*>(w_down), static_cast<const bf16_t*>(nullptr), z, d_ff, d, tiles,
                       n_tiles, nt2);
  else
    hipLaunchKernelGGL(HIP_KERNEL_NAME(grouped_gemm_bf16_kernel<kBM, kDN_BNB, 2, 2, false, false>),
                       dim3(L.max_tiles * nt2), dim3(kThreads), 0, stream, static_cast<const bf16_t*>(H),
                       static_cast<const bf16_t*>(w_down), static_cast<const bf16_t*>(nullptr), z, d_ff, d, tiles,
                       n_tiles, nt2);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}
