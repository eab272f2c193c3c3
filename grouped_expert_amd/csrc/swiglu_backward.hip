// Backward of the grouped SwiGLU experts over ragged row segments.
//
// "M6.2 - Expert Parallelism and DeepSeek MoE", 0x03D: the expert backward
// turns the route gradients into route-input gradients and expert-parameter
// gradients, and the segmentation is backward state.  The chain rule through
// the bias-free SwiGLU of "M6.6 - MoE Runtime Systems", 0x04A
// (G = X W_g^T, U = X W_u^T, H = SiLU(G) U, Z = H W_d^T):
//   dH = dZ W_d,  dW_d = dZ^T H,
//   dG = dH U SiLU'(G),  dU = dH SiLU(G),
//   dX = dG W_g + dU W_u,  dW_g = dG^T X,  dW_u = dU^T X.
//
// Launch sequence (no host synchronisation):
//   1. tile table: the M-tiles of the GEMM tiling, and each expert's first
//      row and row count as validated there (for step 5).
//   2. dH = dZ W_d: GEMM with K = d, N = d_ff, bf16 out.  W_d [d, d_ff] is
//      K-major here, so its tiles are read with the transposing LDS read (no
//      transposed copy of the weights).
//   3. the gate/up GEMM recomputed from X with the SwiGLU backward epilogue:
//      dGU = [dG | dU] [rows, 2 d_ff] and H [rows, d_ff], bf16; or, with the
//      forward's saved activations (G | U and H), a row pass over the M-tiles
//      that forms dGU from dH and the saved G | U, so that W_g and W_u are
//      read once (by step 4) instead of twice.
//   4. dX = dGU [W_g; W_u]: GEMM with K = 2 d_ff, N = d; K-major B, k < d_ff
//      from W_g and the rest from W_u.
//   5. weight gradients (fp32): dW_d[e] = dZ_e^T H_e and
//      [dW_g; dW_u][e] = dGU_e^T X_e, reduced over the expert's rows straight
//      from the row-major activations (no transposed copies).
#include "gemm_core.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// weight gradients: per expert e, C_e[m, n] = sum over the expert's rows r of
// A[r, m] * B[r, n], fp32 out; rows m < M0 go to C0[e], the rest to C1[e]
// ---------------------------------------------------------------------------
// A [rows, M] and B [rows, N] are the row-major activations themselves (dZ and
// H for dW_d; dG | dU and X for dW_g | dW_u), so the reduction runs down their
// columns: a K slice is 64 consecutive rows of the expert, held in LDS as 64
// k-rows of the tile's BM (A) and BN (B) columns, and both MFMA operands are
// read with the gfx950 transposing LDS read (in each 16-lane group, lane j
// receives value i of the 8-byte row addressed by lane 4i + j/4, element
// j%4).  Rows past the expert's end are loaded from its last row (in bounds)
// and their A values are zeroed in registers, so they add nothing.
template <int BM_, int BN_, int WM_, int WN_, int STAGES_, int OCC_>
struct WgCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = STAGES_, BK = 64;
  static constexpr int OCC = OCC_;                              // workgroups per CU (LDS and registers allow)
  static constexpr int NW = WM * WN, THREADS = NW * kWave;
  static constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
  static constexpr int ARB = BM * 2, BRB = BN * 2;              // bytes per k-row of each region
  static constexpr int ACPR = BM / 8, BCPR = BN / 8;            // 16-byte chunks per k-row
  static constexpr int ARPI = 1024 / ARB, BRPI = 1024 / BRB;    // k-rows one wave-wide DMA load fills
  static constexpr int ALOADS = BK / ARPI, BLOADS = BK / BRPI;  // DMA loads per slice and region
  static constexpr int LOADS = (ALOADS + BLOADS) / NW;          // per wavefront and slice
  static constexpr int A_BYTES = BK * ARB, SLICE_BYTES = BK * (ARB + BRB);
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wavefront tile");
  static_assert(ARB <= 1024 && BRB <= 1024 && (ALOADS + BLOADS) % NW == 0, "slice vs DMA loads");
  static_assert(STAGES >= 2 && (STAGES - 2) * LOADS < 64, "pipeline depth");
  static_assert(OCC * STAGES * SLICE_BYTES <= 160 * 1024 && BM * BN * 4 <= STAGES * SLICE_BYTES, "LDS per CU");
  // logical chunk c of k-row r sits at c ^ sw(r): the 4 k-rows x 4 chunks
  // that the 32 lanes of a transposing read's half address (two 16-lane
  // groups, 32 columns) land in 16 distinct 16-byte bank positions
  template <int CPR>
  static __device__ __forceinline__ int sw(int r) { return ((r % 4) * 4) % CPR; }
};

// MFMA fragment (k = 8 (lane / 32) + 0..7 of the 16-row step kk, column
// col0 + lane % 32) from a region of k-rows RB bytes long.
template <class W, int RB, int CPR>
__device__ __forceinline__ bf16x8 wg_frag(const char* region, int kk, int col0, int lane) {
  const int g = lane / 16, r = lane % 16;
  const int n = col0 + 16 * (g % 2) + 4 * (r % 4);
  v4s part[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int kr = kk * 16 + 8 * (g / 2) + 4 * q + r / 4;
    const int byte = kr * RB + (((n / 8) ^ W::template sw<CPR>(kr)) * 16) + (n % 8) * 2;
    part[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(const_cast<char*>(region) + byte));
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// One slice: 4 k-steps of 16 rows.  MASK: only the slice's first kvalid rows
// count (the expert's last slice).
template <class W, bool MASK>
__device__ __forceinline__ void wg_compute(const char* stage, f32x16 (&acc)[W::TM][W::TN], int wm, int wn, int lane,
                                           int kvalid) {
  const char* areg = stage;
  const char* breg = stage + W::A_BYTES;
#pragma unroll
  for (int kk = 0; kk < W::BK / 16; ++kk) {
    bf16x8 a[W::TM], b[W::TN];
#pragma unroll
    for (int i = 0; i < W::TM; ++i) {
      a[i] = wg_frag<W, W::ARB, W::ACPR>(areg, kk, wm * W::WTM + i * 32, lane);
      if constexpr (MASK) {
        // element e holds k = k0 + e: keep the first nv (branch-free selects)
        const int nv = kvalid - (kk * 16 + 8 * (lane / 32));
        vec16 u = __builtin_bit_cast(vec16, a[i]);
#pragma unroll
        for (int w = 0; w < 4; ++w)
          u[w] &= (2 * w < nv ? 0x0000ffffu : 0u) | (2 * w + 1 < nv ? 0xffff0000u : 0u);
        a[i] = __builtin_bit_cast(bf16x8, u);
      }
    }
#pragma unroll
    for (int j = 0; j < W::TN; ++j) b[j] = wg_frag<W, W::BRB, W::BCPR>(breg, kk, wn * W::WTN + j * 32, lane);
#pragma unroll
    for (int i = 0; i < W::TM; ++i)
#pragma unroll
      for (int j = 0; j < W::TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// One workgroup per (expert, M-tile, N-tile), N-tiles of one M-tile adjacent;
// the expert's rows (first row, count) come from the tile-table pass, which
// validated the segments; an expert without rows writes zeros.  The tile
// leaves through LDS as whole fp32 row pieces.  Several workgroups share a
// CU, so one's loads and stores overlap another's matrix-core work.
template <class W>
__global__ __launch_bounds__(W::THREADS, W::OCC) void grouped_wgrad_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, int32_t M, int32_t N, int32_t M0,
    float* __restrict__ C0, float* __restrict__ C1, const int32_t* __restrict__ exp_rows, int32_t n_mt,
    int32_t n_nt) {
  __shared__ __attribute__((aligned(16))) char ring[W::STAGES * W::SLICE_BYTES];
  const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x);
  const int per_e = n_mt * n_nt;
  const int e = static_cast<int>(logical) / per_e;
  const int rem = static_cast<int>(logical) - e * per_e;
  const int mt = rem / n_nt, nt = rem - mt * n_nt;
  const int m0 = mt * W::BM, n0 = nt * W::BN;
  const int2 er = reinterpret_cast<const int2*>(exp_rows)[e];
  const int32_t row0 = er.x, nrows = er.y;
  const int KT = (nrows + W::BK - 1) / W::BK;

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / W::WN, wn = wave % W::WN;
  // per load: the source matrix, its row stride, the k-row in the slice and
  // the element column (clamped into the matrix; such columns are not stored)
  const bf16_t* src[W::LOADS];
  int32_t ld[W::LOADS], kr[W::LOADS], col[W::LOADS];
#pragma unroll
  for (int i = 0; i < W::LOADS; ++i) {
    const int blk = wave * W::LOADS + i;
    if (blk < W::ALOADS) {
      kr[i] = blk * W::ARPI + lane / W::ACPR;
      const int c = (lane % W::ACPR) ^ W::template sw<W::ACPR>(kr[i]);
      col[i] = m0 + 8 * c < M ? m0 + 8 * c : M - 8;
      src[i] = A;
      ld[i] = M;
    } else {
      kr[i] = (blk - W::ALOADS) * W::BRPI + lane / W::BCPR;
      const int c = (lane % W::BCPR) ^ W::template sw<W::BCPR>(kr[i]);
      col[i] = n0 + 8 * c < N ? n0 + 8 * c : N - 8;
      src[i] = B;
      ld[i] = N;
    }
  }
  // The slices' LDS DMA is issued as inline asm and waited for explicitly
  // (vmcnt, then a barrier): seen as LDS writes, the compiler would wait for
  // every DMA in flight, the prefetched slices included, before each slice's
  // first LDS read.
  auto issue = [&](int kt) {
    char* stage = ring + (kt % W::STAGES) * W::SLICE_BYTES;
#pragma unroll
    for (int i = 0; i < W::LOADS; ++i) {
      const int r = kt * W::BK + kr[i] < nrows ? kt * W::BK + kr[i] : nrows - 1;
      const bf16_t* p = src[i] + (static_cast<uint32_t>(row0 + r) * static_cast<uint32_t>(ld[i]) + col[i]);
      dma_b128_asm(lds_addr(stage + (wave * W::LOADS + i) * 1024), p);
    }
  };
  f32x16 acc[W::TM][W::TN];
#pragma unroll
  for (int i = 0; i < W::TM; ++i)
#pragma unroll
    for (int j = 0; j < W::TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
#pragma unroll
  for (int s = 0; s < W::STAGES - 1; ++s)
    if (s < KT) issue(s);
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + W::STAGES - 2 < KT)
      wait_vmcnt_asm<(W::STAGES - 2) * W::LOADS>();
    else
      wait_vmcnt_asm<0>();
    barrier_nofence();
    if (kt + W::STAGES - 1 < KT) issue(kt + W::STAGES - 1);
    const char* stage = ring + (kt % W::STAGES) * W::SLICE_BYTES;
    const int kvalid = nrows - kt * W::BK;
    if (kvalid < W::BK)
      wg_compute<W, true>(stage, acc, wm, wn, lane, kvalid);
    else
      wg_compute<W, false>(stage, acc, wm, wn, lane, W::BK);
  }

  const int lr = lane % 32, lk = lane / 32;
  constexpr int OUT_ROW = W::BN * 4;
  static_assert(W::BM * OUT_ROW <= static_cast<int>(sizeof(ring)), "fp32 tile fits the ring");
  char* tile = ring;
  barrier_nofence();
#pragma unroll
  for (int i = 0; i < W::TM; ++i)
#pragma unroll
    for (int j = 0; j < W::TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = wm * W::WTM + i * 32 + 8 * (q / 4) + 4 * lk + (q % 4);
        const int cc = wn * W::WTN + j * 32 + lr;
        *reinterpret_cast<float*>(tile + r * OUT_ROW + cc * 4) = acc[i][j][q];
      }
  __syncthreads();
  constexpr int VPR = OUT_ROW / 16;
  const int rows_here = M - m0 < W::BM ? M - m0 : W::BM;
  const int vec_cols = (N - n0 < W::BN ? N - n0 : W::BN) / 4;
  for (int v = threadIdx.x; v < W::BM * VPR; v += W::THREADS) {
    const int r = v / VPR, cv = v % VPR;
    if (r >= rows_here || cv >= vec_cols) continue;
    const int m = m0 + r;
    float* dst = m < M0 ? C0 + (static_cast<int64_t>(e) * M0 + m) * N
                        : C1 + (static_cast<int64_t>(e) * (M - M0) + (m - M0)) * N;
    *reinterpret_cast<vec16*>(dst + n0 + cv * 4) = *reinterpret_cast<const vec16*>(tile + r * OUT_ROW + cv * 16);
  }
}

// SwiGLU backward from saved pre-activations, over the rows of the M-tiles:
//   s = 1 / (1 + exp(-g)),  dG = dH u s (1 + g (1 - s)),  dU = dH g s
// with g, u the saved bf16 G, U and dH the bf16 H gradient (fp32 arithmetic
// as in the recomputing GEMM's epilogue, results rounded to bf16).  One
// workgroup per M-tile; 16-byte pieces (d_ff % 64 == 0).
constexpr int kRowThreads = 256;

__global__ __launch_bounds__(kRowThreads) void swiglu_bwd_rows_kernel(const bf16_t* __restrict__ dH,
                                                                      const bf16_t* __restrict__ gu,
                                                                      bf16_t* __restrict__ dgu, int32_t d_ff,
                                                                      const TileEntry* __restrict__ tiles,
                                                                      const int32_t* __restrict__ n_tiles, int32_t bm) {
  const int t = blockIdx.x;
  if (t >= *n_tiles) return;
  const TileEntry te = tiles[t];
  const int rows_here = te.row_end - te.row0 < bm ? te.row_end - te.row0 : bm;
  const int vpr = d_ff / 8;
  for (int v = threadIdx.x; v < rows_here * vpr; v += kRowThreads) {
    const int r = v / vpr, c = (v - r * vpr) * 8;
    const int64_t row = static_cast<int64_t>(te.row0) + r;
    const vec16 hv = *reinterpret_cast<const vec16*>(dH + row * d_ff + c);
    const vec16 gv = *reinterpret_cast<const vec16*>(gu + row * 2 * d_ff + c);
    const vec16 uv = *reinterpret_cast<const vec16*>(gu + row * 2 * d_ff + d_ff + c);
    vec16 dg, du;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float dgp[2], dup[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float dh = bf16_to_f32(static_cast<bf16_t>(hv[w] >> (16 * h)));
        const float g = bf16_to_f32(static_cast<bf16_t>(gv[w] >> (16 * h)));
        const float u = bf16_to_f32(static_cast<bf16_t>(uv[w] >> (16 * h)));
        const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
        dgp[h] = dh * u * (sg * (1.0f + g * (1.0f - sg)));
        dup[h] = dh * (g * sg);
      }
      dg[w] = bf16x2_hw(dgp[0], dgp[1]);
      du[w] = bf16x2_hw(dup[0], dup[1]);
    }
    *reinterpret_cast<vec16*>(dgu + row * 2 * d_ff + c) = dg;
    *reinterpret_cast<vec16*>(dgu + row * 2 * d_ff + d_ff + c) = du;
  }
}

// Backward tile configurations, with the forward's M tilings: K-major-B tiles
// for the two data gradients (step 2 with bf16 out, step 4 with the caller's
// dtype; DMA ring, one tile per workgroup) and the gate/up tiling with the
// SwiGLU backward epilogue (step 3, never persistent).
template <bool F>
using CfgLgBT = Cfg<256, 128, 4, 2, 3, false, F, false, 64, 1, 4, 8, false, kEpiStore, true>;
template <bool F>
using CfgMdBT = Cfg<128, 256, 2, 4, 3, false, F, false, 64, 1, 2, 8, false, kEpiStore, true>;
template <bool F>
using CfgSmBT = Cfg<32, 256, 1, 4, 4, false, F, false, 64, 1, 1, 4, false, kEpiStore, true>;
using CfgLgGB = Cfg<256, 256, 4, 2, 2, true, false, false, 64, 1, 4, 8, true, kEpiSwigluBwd>;
using CfgMdGB = Cfg<128, 256, 2, 4, 3, true, false, false, 64, 1, 2, 8, false, kEpiSwigluBwd>;
using CfgSmGB = Cfg<32, 256, 1, 4, 4, true, false, false, 64, 1, 1, 4, false, kEpiSwigluBwd>;
static_assert(CfgLgGB::BM == CfgLgGU::BM && CfgMdGB::BM == CfgMdGU::BM && CfgSmGB::BM == CfgSmGU::BM &&
                  CfgLgBT<true>::BM == CfgLgGU::BM && CfgMdBT<true>::BM == CfgMdGU::BM &&
                  CfgSmBT<true>::BM == CfgSmGU::BM,
              "one M tiling per kind");
// weight gradients: 128 x 256 fp32 tiles, 8 wavefronts, 3-slice ring (144 KB)
using CfgWg = WgCfg<128, 256, 2, 4, 3, 1>;

struct BwdLayout {
  size_t tiles, ntiles, erows, dH, dGU, H, total;
  int32_t max_tiles, bm;
};

inline BwdLayout bwd_layout(int64_t rows, int32_t E, int32_t d, int32_t d_ff) {
  BwdLayout w;
  w.bm = pick_tiles(rows, E) == kLarge ? CfgLgGU::BM : (pick_tiles(rows, E) == kMedium ? CfgMdGU::BM : CfgSmGU::BM);
  w.max_tiles = static_cast<int32_t>((rows + w.bm - 1) / w.bm + E);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes, 256);
    return at;
  };
  const size_t r = static_cast<size_t>(rows), e = static_cast<size_t>(E), F = d_ff;
  (void)d;
  w.tiles = take(static_cast<size_t>(w.max_tiles) * sizeof(TileEntry));
  w.ntiles = take(4);
  w.erows = take(e * 8);
  w.dH = take(r * F * 2);
  w.dGU = take(r * 2 * F * 2);
  w.H = take(r * F * 2);
  w.total = o;
  return w;
}

template <class GB, class DB, class DF>
int launch_bwd_gemms(const void* x, const void* dz, int32_t d, int32_t d_ff, const void* wg, const void* wu,
                     const void* wd, void* dH, void* dGU, void* H, const void* gu_saved, void* dx, int32_t dx_dtype,
                     const TileEntry* tiles, const int32_t* n_tiles, int32_t max_tiles, hipStream_t stream) {
  const int nt_f = (d_ff + DB::BN_OUT - 1) / DB::BN_OUT;
  const int nt_g = (d_ff + GB::BN_OUT - 1) / GB::BN_OUT;
  const int nt_d = (d + DF::BN_OUT - 1) / DF::BN_OUT;
  const int nmax = nt_f > nt_g ? (nt_f > nt_d ? nt_f : nt_d) : (nt_g > nt_d ? nt_g : nt_d);
  MOE_CHECK(static_cast<int64_t>(max_tiles) * nmax <= INT32_MAX, MOE_EUNSUPPORTED);
  // dH = dZ W_d: W_d[e] is [d (K)][d_ff (N)]
  launch_one<DB>(false, dz, wd, nullptr, dH, d, d_ff, tiles, n_tiles, max_tiles, nt_f, stream);
  MOE_LAUNCH_CHECK();
  if (gu_saved)
    hipLaunchKernelGGL(swiglu_bwd_rows_kernel, dim3(static_cast<unsigned>(max_tiles)), dim3(kRowThreads), 0, stream,
                       static_cast<const bf16_t*>(dH), static_cast<const bf16_t*>(gu_saved),
                       static_cast<bf16_t*>(dGU), d_ff, tiles, n_tiles, GB::BM);
  else
    launch_one<GB>(false, x, wg, wu, dGU, d, d_ff, tiles, n_tiles, max_tiles, nt_g, stream, dH, H);
  MOE_LAUNCH_CHECK();
  // dX = [dG | dU] [W_g; W_u]: W_g[e], W_u[e] are [d_ff (K)][d (N)], split at K = d_ff
  if (dx_dtype == MOE_F32)
    launch_one<DF>(false, dGU, wg, wu, dx, 2 * d_ff, d, tiles, n_tiles, max_tiles, nt_d, stream, nullptr, nullptr,
                   d_ff);
  else
    launch_one<DB>(false, dGU, wg, wu, dx, 2 * d_ff, d, tiles, n_tiles, max_tiles, nt_d, stream, nullptr, nullptr,
                   d_ff);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace
}  // namespace moe

MOE_API size_t moe_grouped_swiglu_backward_workspace(int64_t rows, int32_t E, int32_t d, int32_t d_ff) {
  using namespace moe;
  if (rows < 0 || E < 1 || E > MOE_MAX_EXPERTS || d < 1 || d_ff < 1) return 0;
  return bwd_layout(rows, E, d, d_ff).total;
}

MOE_API int moe_grouped_swiglu_backward(const void* x, int32_t d, int32_t d_ff, int32_t E, const int32_t* seg_start,
                                        const int32_t* seg_count, int64_t rows, const void* w_gate,
                                        const void* w_up, const void* w_down, const void* dz, const void* act,
                                        void* dx, int32_t dx_dtype, float* dw_gate, float* dw_up, float* dw_down, void* ws,
                                        size_t ws_bytes, uint32_t* dev_flags, hipStream_t stream) {
  using namespace moe;
  MOE_CHECK(dx_dtype == MOE_F32 || dx_dtype == MOE_BF16, MOE_EINVAL);
  MOE_CHECK(E >= 1 && E <= MOE_MAX_EXPERTS && d >= 1 && d_ff >= 1 && rows >= 0, MOE_EINVAL);
  MOE_CHECK(d % 64 == 0 && d_ff % 64 == 0, MOE_EUNSUPPORTED);
  MOE_CHECK(rows <= INT32_MAX - 256, MOE_EUNSUPPORTED);
  MOE_CHECK(seg_start && seg_count && w_gate && w_up && w_down && dw_gate && dw_up && dw_down, MOE_EINVAL);
  MOE_CHECK(rows == 0 || (x && dz && dx), MOE_EINVAL);
  MOE_CHECK((x == nullptr || aligned16(x)) && (dz == nullptr || aligned16(dz)) && (dx == nullptr || aligned16(dx)),
            MOE_EINVAL);
  MOE_CHECK(aligned16(w_gate) && aligned16(w_up) && aligned16(w_down), MOE_EINVAL);
  MOE_CHECK(aligned16(dw_gate) && aligned16(dw_up) && aligned16(dw_down), MOE_EINVAL);
  MOE_CHECK(act == nullptr || aligned16(act), MOE_EINVAL);
  const BwdLayout L = bwd_layout(rows, E, d, d_ff);
  // 32-bit element offsets: rows x 2 d_ff and rows x d inside the row-major
  // operands, and one expert's matrices
  const int64_t wmax = d > 2 * d_ff ? d : 2 * static_cast<int64_t>(d_ff);
  MOE_CHECK(rows * wmax < (int64_t(1) << 32) && static_cast<int64_t>(d) * d_ff * 4 < (int64_t(1) << 32),
            MOE_EUNSUPPORTED);
  MOE_CHECK(ws && ws_bytes >= L.total && aligned16(ws), MOE_EWORKSPACE);
  char* w = static_cast<char*>(ws);
  TileEntry* tiles = reinterpret_cast<TileEntry*>(w + L.tiles);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(w + L.ntiles);
  int32_t* erows = reinterpret_cast<int32_t*>(w + L.erows);
  bf16_t* dH = reinterpret_cast<bf16_t*>(w + L.dH);
  bf16_t* dGU = reinterpret_cast<bf16_t*>(w + L.dGU);
  // H: recomputed into the workspace, or the forward's saved plane
  const bf16_t* gu_saved = static_cast<const bf16_t*>(act);
  bf16_t* H = act ? const_cast<bf16_t*>(gu_saved) + static_cast<size_t>(rows) * 2 * d_ff
                  : reinterpret_cast<bf16_t*>(w + L.H);

  // 1. tile table, with each expert's rows
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, stream, seg_start, seg_count, E, rows, L.bm,
                     L.max_tiles, tiles, n_tiles, dev_flags, erows);
  MOE_LAUNCH_CHECK();
  if (rows > 0) {
    // 2.-4. data gradients
    int st;
    switch (pick_tiles(rows, E)) {
      case kLarge:
        st = launch_bwd_gemms<CfgLgGB, CfgLgBT<false>, CfgLgBT<true>>(x, dz, d, d_ff, w_gate, w_up, w_down, dH,
                                                                      dGU, H, gu_saved, dx, dx_dtype, tiles, n_tiles,
                                                                      L.max_tiles, stream);
        break;
      case kMedium:
        st = launch_bwd_gemms<CfgMdGB, CfgMdBT<false>, CfgMdBT<true>>(x, dz, d, d_ff, w_gate, w_up, w_down, dH,
                                                                      dGU, H, gu_saved, dx, dx_dtype, tiles, n_tiles,
                                                                      L.max_tiles, stream);
        break;
      default:
        st = launch_bwd_gemms<CfgSmGB, CfgSmBT<false>, CfgSmBT<true>>(x, dz, d, d_ff, w_gate, w_up, w_down, dH,
                                                                      dGU, H, gu_saved, dx, dx_dtype, tiles, n_tiles,
                                                                      L.max_tiles, stream);
    }
    if (st != MOE_OK) return st;
  }
  // 5. weight gradients from the row-major activations (every expert: zero
  // where it has no rows; without rows no operand is read)
  using C = CfgWg;
  const bf16_t* zsrc = static_cast<const bf16_t*>(dz);
  const bf16_t* xsrc = static_cast<const bf16_t*>(x);
  {
    const int n_mt = (d + C::BM - 1) / C::BM, n_nt = (d_ff + C::BN - 1) / C::BN;
    hipLaunchKernelGGL(HIP_KERNEL_NAME(grouped_wgrad_kernel<C>), dim3(static_cast<unsigned>(E * n_mt * n_nt)),
                       dim3(C::THREADS), 0, stream, zsrc, H, d, d_ff, d, dw_down, dw_down, erows, n_mt, n_nt);
    MOE_LAUNCH_CHECK();
  }
  {
    const int n_mt = (2 * d_ff + C::BM - 1) / C::BM, n_nt = (d + C::BN - 1) / C::BN;
    hipLaunchKernelGGL(HIP_KERNEL_NAME(grouped_wgrad_kernel<C>), dim3(static_cast<unsigned>(E * n_mt * n_nt)),
                       dim3(C::THREADS), 0, stream, dGU, xsrc, 2 * d_ff, d, d_ff, dw_gate, dw_up, erows, n_mt,
                       n_nt);
    MOE_LAUNCH_CHECK();
  }
  return MOE_OK;
}
