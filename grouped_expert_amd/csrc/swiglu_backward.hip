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
//   1. tile tables: the M-tiles of the GEMM tiling, and 64-row K-tiles with
//      each expert's run of them (the padded K layout of step 6).
//   2. dH = dZ W_d: GEMM with K = d, N = d_ff, bf16 out.  W_d [d, d_ff] is
//      K-major here, so its tiles are read with the transposing LDS read (no
//      transposed copy of the weights).
//   3. the gate/up GEMM recomputed from X with the SwiGLU backward epilogue:
//      dGU = [dG | dU] [rows, 2 d_ff] and H [rows, d_ff], bf16.
//   4. dX = dGU [W_g; W_u]: GEMM with K = 2 d_ff, N = d; K-major B, k < d_ff
//      from W_g and the rest from W_u.
//   5. segment-padded transposes of dZ, H, dGU and X to [C, Kp]: expert e's
//      rows become columns starting at 64 * (its first K-tile), zero padded.
//   6. weight gradients (fp32): dW_d[e] = dZ_e^T H_e and
//      [dW_g; dW_u][e] = dGU_e^T X_e, with K = the expert's padded rows.
#include "gemm_core.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// 64 x 64 bf16 tile transposes through LDS
// ---------------------------------------------------------------------------
// Load: 256 threads read the tile's 64 rows as 16-byte pieces (8 per row) and
// scatter the 8 values into the transposed LDS tile; store: each output row
// (64 values = 128 bytes) leaves as 8 16-byte pieces.  The LDS row pitch of
// 72 elements keeps every output piece 16-byte aligned.
constexpr int kTp = 64, kTpPitch = 72, kTpThreads = 256;

__device__ __forceinline__ void transpose_tile(const bf16_t* __restrict__ src, int64_t src_ld, int valid_rows,
                                               bf16_t* __restrict__ dst, int64_t dst_ld, bf16_t* tile) {
  const int t = threadIdx.x, ch = t % 8;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = t / 8 + 32 * h;
    vec16 v = {0u, 0u, 0u, 0u};
    if (r < valid_rows) v = *reinterpret_cast<const vec16*>(src + r * src_ld + ch * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[(ch * 8 + 2 * i) * kTpPitch + r] = static_cast<bf16_t>(v[i] & 0xffffu);
      tile[(ch * 8 + 2 * i + 1) * kTpPitch + r] = static_cast<bf16_t>(v[i] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = t / 8 + 32 * h;
    *reinterpret_cast<vec16*>(dst + c * dst_ld + ch * 8) =
        *reinterpret_cast<const vec16*>(tile + c * kTpPitch + ch * 8);
  }
}

// Segment-padded transpose of row-major src [rows, C]: K-tile t (64 rows of
// one expert, zero past the segment end) becomes columns [64 t, 64 t + 64) of
// dst [C, Kp].  Grid (max K-tiles, C/64); tiles past the table leave.
__global__ __launch_bounds__(kTpThreads) void transpose_rows_kernel(const bf16_t* __restrict__ src, int32_t Cc,
                                                                    const TileEntry* __restrict__ ktiles,
                                                                    const int32_t* __restrict__ n_ktiles,
                                                                    bf16_t* __restrict__ dst, int64_t Kp) {
  __shared__ __attribute__((aligned(16))) bf16_t tile[kTp * kTpPitch];
  const int t = blockIdx.x;
  if (t >= *n_ktiles) return;
  const TileEntry te = ktiles[t];
  const int64_t c0 = static_cast<int64_t>(blockIdx.y) * kTp;
  const int valid = te.row_end - te.row0 < kTp ? te.row_end - te.row0 : kTp;
  transpose_tile(src + static_cast<int64_t>(te.row0) * Cc + c0, Cc, valid, dst + c0 * Kp + static_cast<int64_t>(t) * kTp,
                 Kp, tile);
}

// ---------------------------------------------------------------------------
// weight gradients: per expert e, C_e[m, n] = sum over the expert's padded K
// of AT[m, k] * BT[n, k], fp32 out; rows m < M0 go to C0[e], the rest to C1[e]
// ---------------------------------------------------------------------------
// One workgroup per (expert, M-tile, N-tile), the LDS-ring K loop of the
// grouped GEMM over the expert's run of 64-wide K-tiles; an expert without
// rows writes zeros.  The tile leaves through LDS as whole fp32 row pieces.
template <class C>
__global__ __launch_bounds__(C::THREADS, C::OCC) void grouped_wgrad_kernel(
    const bf16_t* __restrict__ AT, const bf16_t* __restrict__ BT, int64_t Kp, int32_t M, int32_t N, int32_t M0,
    float* __restrict__ C0, float* __restrict__ C1, const int32_t* __restrict__ exp_first,
    const int32_t* __restrict__ exp_ntile, int32_t n_mt, int32_t n_nt) {
  static_assert(!C::GATEUP && !C::RS && C::OUT_F32, "plain fp32 tiles with the DMA ring");
  __shared__ __attribute__((aligned(16))) bf16_t ring[C::STAGES * C::SLICE];
  const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x);
  const int per_e = n_mt * n_nt;
  const int e = static_cast<int>(logical) / per_e;
  const int rem = static_cast<int>(logical) - e * per_e;
  const int mt = rem / n_nt, nt = rem - mt * n_nt;         // N-tiles of one M-tile are adjacent
  const int m0 = mt * C::BM, n0 = nt * C::BN_OUT;
  const int KT = exp_ntile[e];
  const uint32_t kbase = static_cast<uint32_t>(exp_first[e]) * C::BK;

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const bf16_t* base[C::LOADS];
  uint32_t off[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int blk = C::block(wave, i);
    const int rr = blk * C::RPI + lane / C::CPR;
    const int c = (lane % C::CPR) ^ ((rr / (256 / C::RB)) % C::CPR);
    if (blk * C::RPI < C::BM) {
      const int m = m0 + rr < M ? m0 + rr : M - 1;
      base[i] = AT;
      off[i] = static_cast<uint32_t>(m) * static_cast<uint32_t>(Kp) + kbase + c * 8;
    } else {
      const int n = n0 + rr - C::BM < N ? n0 + rr - C::BM : N - 1;
      base[i] = BT;
      off[i] = static_cast<uint32_t>(n) * static_cast<uint32_t>(Kp) + kbase + c * 8;
    }
  }
  f32x16 acc[1][C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[0][i][j][q] = 0.0f;
#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s)
    if (s < KT) issue_slice<C>(ring + s * C::SLICE, base, off, static_cast<uint32_t>(s * C::BK), wave);
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + C::STAGES - 2 < KT)
      wait_vmcnt<(C::STAGES - 2) * C::LOADS>();
    else
      wait_vmcnt<0>();
    barrier_nofence();
    const int nk = kt + C::STAGES - 1;
    if (nk < KT)
      issue_slice<C>(ring + (nk % C::STAGES) * C::SLICE, base, off, static_cast<uint32_t>(nk * C::BK), wave);
    compute_slice<C>(ring + (kt % C::STAGES) * C::SLICE, ring + (kt % C::STAGES) * C::SLICE + C::BM * C::BK, acc,
                     wm, wn, lane);
  }

  constexpr int OUT_ROW = C::BN_OUT * 4;
  static_assert(C::BM * OUT_ROW <= static_cast<int>(sizeof(ring)), "fp32 tile fits the ring");
  char* tile = reinterpret_cast<char*>(ring);
  const int lr = lane % 32, lk = lane / 32;
  barrier_nofence();
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = wm * C::WTM + i * 32 + 8 * (q / 4) + 4 * lk + (q % 4);
        const int cc = wn * C::WTN + j * 32 + lr;
        *reinterpret_cast<float*>(tile + r * OUT_ROW + cc * 4) = acc[0][i][j][q];
      }
  __syncthreads();
  constexpr int VPR = OUT_ROW / 16;
  const int rows_here = M - m0 < C::BM ? M - m0 : C::BM;
  const int vec_cols = (N - n0 < C::BN_OUT ? N - n0 : C::BN_OUT) / 4;
  for (int v = threadIdx.x; v < C::BM * VPR; v += C::THREADS) {
    const int r = v / VPR, cv = v % VPR;
    if (r >= rows_here || cv >= vec_cols) continue;
    const int m = m0 + r;
    float* dst = m < M0 ? C0 + (static_cast<int64_t>(e) * M0 + m) * N
                        : C1 + (static_cast<int64_t>(e) * (M - M0) + (m - M0)) * N;
    *reinterpret_cast<vec16*>(dst + n0 + cv * 4) = *reinterpret_cast<const vec16*>(tile + r * OUT_ROW + cv * 16);
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
// weight gradients: 128 x 256 fp32 tiles, 8 wavefronts, 3-slice ring
using CfgWg = Cfg<128, 256, 2, 4, 3, false, true, false, 64, 1, 1, 8>;

struct BwdLayout {
  size_t tiles, ntiles, ktiles, nktiles, efirst, entile, dH, dGU, H, dZT, HT, GUT, XT, total;
  int32_t max_tiles, max_ktiles, bm;
  int64_t Kp;
};

inline BwdLayout bwd_layout(int64_t rows, int32_t E, int32_t d, int32_t d_ff) {
  BwdLayout w;
  w.bm = pick_tiles(rows, E) == kLarge ? CfgLgGU::BM : (pick_tiles(rows, E) == kMedium ? CfgMdGU::BM : CfgSmGU::BM);
  w.max_tiles = static_cast<int32_t>((rows + w.bm - 1) / w.bm + E);
  w.max_ktiles = static_cast<int32_t>((rows + kTp - 1) / kTp + E);
  w.Kp = static_cast<int64_t>(w.max_ktiles) * kTp;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes, 256);
    return at;
  };
  const size_t r = static_cast<size_t>(rows), e = static_cast<size_t>(E), D = d, F = d_ff;
  const size_t kp = static_cast<size_t>(w.Kp);
  w.tiles = take(static_cast<size_t>(w.max_tiles) * sizeof(TileEntry));
  w.ntiles = take(4);
  w.ktiles = take(static_cast<size_t>(w.max_ktiles) * sizeof(TileEntry));
  w.nktiles = take(4);
  w.efirst = take(e * 4);
  w.entile = take(e * 4);
  w.dH = take(r * F * 2);
  w.dGU = take(r * 2 * F * 2);
  w.H = take(r * F * 2);
  w.dZT = take(D * kp * 2);
  w.HT = take(F * kp * 2);
  w.GUT = take(2 * F * kp * 2);
  w.XT = take(D * kp * 2);
  w.total = o;
  return w;
}

template <class GB, class DB, class DF>
int launch_bwd_gemms(const void* x, const void* dz, int32_t d, int32_t d_ff, const void* wg, const void* wu,
                     const void* wd, void* dH, void* dGU, void* H, void* dx, int32_t dx_dtype,
                     const TileEntry* tiles, const int32_t* n_tiles, int32_t max_tiles, hipStream_t stream) {
  const int nt_f = (d_ff + DB::BN_OUT - 1) / DB::BN_OUT;
  const int nt_g = (d_ff + GB::BN_OUT - 1) / GB::BN_OUT;
  const int nt_d = (d + DF::BN_OUT - 1) / DF::BN_OUT;
  const int nmax = nt_f > nt_g ? (nt_f > nt_d ? nt_f : nt_d) : (nt_g > nt_d ? nt_g : nt_d);
  MOE_CHECK(static_cast<int64_t>(max_tiles) * nmax <= INT32_MAX, MOE_EUNSUPPORTED);
  // dH = dZ W_d: W_d[e] is [d (K)][d_ff (N)]
  launch_one<DB>(false, dz, wd, nullptr, dH, d, d_ff, tiles, n_tiles, max_tiles, nt_f, stream);
  MOE_LAUNCH_CHECK();
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
                                        const void* w_up, const void* w_down, const void* dz, void* dx,
                                        int32_t dx_dtype, float* dw_gate, float* dw_up, float* dw_down, void* ws,
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
  const BwdLayout L = bwd_layout(rows, E, d, d_ff);
  // 32-bit element offsets: rows x 2 d_ff and rows x d inside the row-major
  // operands, one expert's matrices, and the padded transposes
  const int64_t wmax = d > 2 * d_ff ? d : 2 * static_cast<int64_t>(d_ff);
  MOE_CHECK(rows * wmax < (int64_t(1) << 32) && static_cast<int64_t>(d) * d_ff * 4 < (int64_t(1) << 32) &&
                wmax * L.Kp < (int64_t(1) << 32), MOE_EUNSUPPORTED);
  MOE_CHECK(ws && ws_bytes >= L.total && aligned16(ws), MOE_EWORKSPACE);
  char* w = static_cast<char*>(ws);
  TileEntry* tiles = reinterpret_cast<TileEntry*>(w + L.tiles);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(w + L.ntiles);
  TileEntry* ktiles = reinterpret_cast<TileEntry*>(w + L.ktiles);
  int32_t* n_ktiles = reinterpret_cast<int32_t*>(w + L.nktiles);
  int32_t* efirst = reinterpret_cast<int32_t*>(w + L.efirst);
  int32_t* entile = reinterpret_cast<int32_t*>(w + L.entile);
  bf16_t* dH = reinterpret_cast<bf16_t*>(w + L.dH);
  bf16_t* dGU = reinterpret_cast<bf16_t*>(w + L.dGU);
  bf16_t* H = reinterpret_cast<bf16_t*>(w + L.H);
  bf16_t* dZT = reinterpret_cast<bf16_t*>(w + L.dZT);
  bf16_t* HT = reinterpret_cast<bf16_t*>(w + L.HT);
  bf16_t* GUT = reinterpret_cast<bf16_t*>(w + L.GUT);
  bf16_t* XT = reinterpret_cast<bf16_t*>(w + L.XT);

  // 1. tile tables
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, stream, seg_start, seg_count, E, rows, L.bm,
                     L.max_tiles, tiles, n_tiles, dev_flags, nullptr, nullptr);
  MOE_LAUNCH_CHECK();
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, stream, seg_start, seg_count, E, rows, kTp,
                     L.max_ktiles, ktiles, n_ktiles, nullptr, efirst, entile);
  MOE_LAUNCH_CHECK();
  if (rows > 0) {
    // 2.-4. data gradients
    int st;
    switch (pick_tiles(rows, E)) {
      case kLarge:
        st = launch_bwd_gemms<CfgLgGB, CfgLgBT<false>, CfgLgBT<true>>(x, dz, d, d_ff, w_gate, w_up, w_down, dH,
                                                                      dGU, H, dx, dx_dtype, tiles, n_tiles,
                                                                      L.max_tiles, stream);
        break;
      case kMedium:
        st = launch_bwd_gemms<CfgMdGB, CfgMdBT<false>, CfgMdBT<true>>(x, dz, d, d_ff, w_gate, w_up, w_down, dH,
                                                                      dGU, H, dx, dx_dtype, tiles, n_tiles,
                                                                      L.max_tiles, stream);
        break;
      default:
        st = launch_bwd_gemms<CfgSmGB, CfgSmBT<false>, CfgSmBT<true>>(x, dz, d, d_ff, w_gate, w_up, w_down, dH,
                                                                      dGU, H, dx, dx_dtype, tiles, n_tiles,
                                                                      L.max_tiles, stream);
    }
    if (st != MOE_OK) return st;
    // 5. segment-padded transposes
    const bf16_t* zsrc = static_cast<const bf16_t*>(dz);
    const bf16_t* xsrc = static_cast<const bf16_t*>(x);
    const unsigned kt = static_cast<unsigned>(L.max_ktiles);
    hipLaunchKernelGGL(transpose_rows_kernel, dim3(kt, d / kTp), dim3(kTpThreads), 0, stream, zsrc, d, ktiles,
                       n_ktiles, dZT, L.Kp);
    MOE_LAUNCH_CHECK();
    hipLaunchKernelGGL(transpose_rows_kernel, dim3(kt, d_ff / kTp), dim3(kTpThreads), 0, stream, H, d_ff, ktiles,
                       n_ktiles, HT, L.Kp);
    MOE_LAUNCH_CHECK();
    hipLaunchKernelGGL(transpose_rows_kernel, dim3(kt, 2 * d_ff / kTp), dim3(kTpThreads), 0, stream, dGU, 2 * d_ff,
                       ktiles, n_ktiles, GUT, L.Kp);
    MOE_LAUNCH_CHECK();
    hipLaunchKernelGGL(transpose_rows_kernel, dim3(kt, d / kTp), dim3(kTpThreads), 0, stream, xsrc, d, ktiles,
                       n_ktiles, XT, L.Kp);
    MOE_LAUNCH_CHECK();
  }
  // 6. weight gradients (every expert: zero where it has no rows)
  using C = CfgWg;
  {
    const int n_mt = (d + C::BM - 1) / C::BM, n_nt = (d_ff + C::BN_OUT - 1) / C::BN_OUT;
    hipLaunchKernelGGL(HIP_KERNEL_NAME(grouped_wgrad_kernel<C>), dim3(static_cast<unsigned>(E * n_mt * n_nt)),
                       dim3(C::THREADS), 0, stream, dZT, HT, L.Kp, d, d_ff, d, dw_down, dw_down, efirst, entile,
                       n_mt, n_nt);
    MOE_LAUNCH_CHECK();
  }
  {
    const int n_mt = (2 * d_ff + C::BM - 1) / C::BM, n_nt = (d + C::BN_OUT - 1) / C::BN_OUT;
    hipLaunchKernelGGL(HIP_KERNEL_NAME(grouped_wgrad_kernel<C>), dim3(static_cast<unsigned>(E * n_mt * n_nt)),
                       dim3(C::THREADS), 0, stream, GUT, XT, L.Kp, 2 * d_ff, d, d_ff, dw_gate, dw_up, efirst, entile,
                       n_mt, n_nt);
    MOE_LAUNCH_CHECK();
  }
  return MOE_OK;
}
