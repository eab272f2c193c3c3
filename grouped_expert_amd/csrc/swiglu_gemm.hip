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
//   3. down: Z = H W_d^T on bf16 MFMA, fp32 accumulation, stored bf16 or fp32;
//      with a row map, row i of Z is stored as row z_rows[i] of the output
//      (the receiver writes expert results straight into pool-row order, so
//      no separate expansion pass reads them back: "Fixed pooled-wave
//      all-to-all for the 8-of-384 MoE", 03).
//
// Data layout (all row-major, K contiguous for both operands):
//   x [rows, d], W_g / W_u [E, d_ff, d], W_d [E, d, d_ff], H [rows, d_ff]
//   (workspace), z [rows, d].  Both products are "A times B^T" with the K
//   dimension contiguous in A and in B, which is the native operand order of
//   the MFMA (each lane reads 8 consecutive K values of one row).
//
// The fp32 variant (dtype MOE_F32) runs the same three steps with an LDS-tiled
// FMA kernel in fp32.
#include "gemm_core.h"

namespace moe {
namespace {

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
                                                               int32_t n_tiles_n,
                                                               const int32_t* __restrict__ out_rows,
                                                               int32_t out_n) {
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
    const int32_t orow = dest_row(out_rows, out_n, row);
    if (orow < 0) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      const float v = GATEUP ? silu_f32(acc[0][i][j]) * acc[NB - 1][i][j] : acc[0][i][j];
      C[static_cast<int64_t>(orow) * N + col] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
inline int32_t tile_bm(int32_t dtype, TileKind t) {
  if (dtype == MOE_F32) return kF32BM;
  return t == kLarge ? CfgLgGU::BM : (t == kMedium ? CfgMdGU::BM : CfgSmGU::BM);
}
static_assert(CfgLgGU::BM == CfgLgDF::BM && CfgLgGU::BM == CfgLgDB::BM, "one M tiling per kind");
static_assert(CfgMdGU::BM == CfgMdDF::BM && CfgMdGU::BM == CfgMdDB::BM, "one M tiling per kind");
static_assert(CfgMdGUr::BM == CfgMdGU::BM && CfgMdDFr::BM == CfgMdGU::BM && CfgMdDBr::BM == CfgMdGU::BM,
              "one M tiling per kind");
static_assert(CfgSmGU::BM == CfgSmDF::BM && CfgSmGU::BM == CfgSmDB::BM, "one M tiling per kind");

struct WsLayout {
  size_t h_off, h_bytes, tiles_off, ntiles_off, total;
  int32_t max_tiles, bm;
};

inline WsLayout ws_layout(int64_t rows, int32_t E, int32_t d_ff, int32_t dtype) {
  WsLayout w;
  w.bm = tile_bm(dtype, pick_tiles(rows, E));
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
                               const int32_t* z_rows, int64_t z_n_rows, void* act, void* ws, size_t ws_bytes,
                               uint32_t* dev_flags, hipStream_t stream) {
  using namespace moe;
  MOE_CHECK(dtype == MOE_F32 || dtype == MOE_BF16, MOE_EINVAL);
  MOE_CHECK(z_dtype == MOE_F32 || z_dtype == MOE_BF16, MOE_EINVAL);
  MOE_CHECK(dtype == MOE_BF16 || z_dtype == MOE_F32, MOE_EUNSUPPORTED);
  MOE_CHECK(E >= 1 && E <= MOE_MAX_EXPERTS && d >= 1 && d_ff >= 1 && rows >= 0, MOE_EINVAL);
  MOE_CHECK(d % 64 == 0 && d_ff % 64 == 0, MOE_EUNSUPPORTED);
  MOE_CHECK(rows <= INT32_MAX - 256, MOE_EUNSUPPORTED);
  // element offsets inside x / H and inside one expert's matrices are 32-bit
  MOE_CHECK(rows * (d > d_ff ? d : d_ff) < (int64_t(1) << 32) &&
                static_cast<int64_t>(d) * d_ff * 2 < (int64_t(1) << 32), MOE_EUNSUPPORTED);
  MOE_CHECK(seg_start && seg_count && w_gate && w_up && w_down, MOE_EINVAL);
  MOE_CHECK(rows == 0 || (x && z), MOE_EINVAL);
  // without a map z has `rows` rows; with one, z_n_rows rows (int32 row indexes)
  MOE_CHECK(z_rows == nullptr || (z_n_rows >= 0 && aligned4(z_rows)), MOE_EINVAL);
  MOE_CHECK(z_n_rows <= INT32_MAX, MOE_EUNSUPPORTED);
  const int32_t z_n = z_rows ? static_cast<int32_t>(z_n_rows) : 0;
  MOE_CHECK((x == nullptr || aligned16(x)) && (z == nullptr || aligned16(z)), MOE_EINVAL);
  MOE_CHECK(aligned16(w_gate) && aligned16(w_up) && aligned16(w_down), MOE_EINVAL);
  // saved activations: bf16 path only
  MOE_CHECK(act == nullptr || dtype == MOE_BF16, MOE_EUNSUPPORTED);
  MOE_CHECK(act == nullptr || aligned16(act), MOE_EINVAL);
  const WsLayout L = ws_layout(rows, E, d_ff, dtype);
  MOE_CHECK(ws && ws_bytes >= L.total && aligned16(ws), MOE_EWORKSPACE);
  char* wsb = static_cast<char*>(ws);
  // H in the workspace, or in the H plane of the saved activations
  void* H = act ? static_cast<char*>(act) + static_cast<size_t>(rows) * 2 * d_ff * 2 : wsb + L.h_off;
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
                       static_cast<const float*>(w_up), static_cast<float*>(H), d, d_ff, tiles, n_tiles, nt1,
                       static_cast<const int32_t*>(nullptr), 0);
    MOE_LAUNCH_CHECK();
    hipLaunchKernelGGL(HIP_KERNEL_NAME(grouped_gemm_f32_kernel<false>), dim3(L.max_tiles * nt2), dim3(256), 0,
                       stream, static_cast<const float*>(H), static_cast<const float*>(w_down),
                       static_cast<const float*>(nullptr), static_cast<float*>(z), d_ff, d, tiles, n_tiles, nt2,
                       z_rows, z_n);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
  }
  switch (pick_tiles(rows, E)) {
    case kLarge:
      return launch_bf16<CfgLgGU, CfgLgGUS, CfgLgDF, CfgLgDB, kPersistLg>(x, rows, d, d_ff, w_gate, w_up, w_down, H, z, z_dtype, z_rows,
                                                                z_n, tiles, n_tiles, L.max_tiles, act, stream);
    case kMedium:
      // (both products must also fit the persistent form's 32-bit output
      // offsets; it has no one-tile fallback at this staging depth)
      if (rs_slices_ok<CfgMdGUr>(d / 64) && rs_slices_ok<CfgMdDFr>(d_ff / 64) &&
          rows * d_ff * 2 < 0xFFFFF000ll &&
          (z_rows ? z_n_rows : rows) > 0 && (z_rows ? z_n_rows : rows) * d * (z_dtype == MOE_F32 ? 4 : 2) < 0xFFFFF000ll)
        return launch_bf16<CfgMdGUr, CfgMdGUS, CfgMdDFr, CfgMdDBr, kPersistMd>(x, rows, d, d_ff, w_gate, w_up, w_down, H,
                                                                              z, z_dtype, z_rows, z_n, tiles, n_tiles,
                                                                              L.max_tiles, act, stream);
      return launch_bf16<CfgMdGU, CfgMdGUS, CfgMdDF, CfgMdDB, kPersistMd>(x, rows, d, d_ff, w_gate, w_up, w_down, H, z, z_dtype, z_rows,
                                                                z_n, tiles, n_tiles, L.max_tiles, act, stream);
    default:
      return launch_bf16<CfgSmGU, CfgSmGUS, CfgSmDF, CfgSmDB, kPersistSm>(x, rows, d, d_ff, w_gate, w_up, w_down, H, z, z_dtype, z_rows,
                                                                z_n, tiles, n_tiles, L.max_tiles, act, stream);
  }
}
