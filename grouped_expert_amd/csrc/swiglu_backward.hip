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

// Byte offset, inside a region of k-rows RB bytes long, of the 8-byte row
// the lane addresses in the first transposing read of a fragment whose 32
// columns start at col0 (k-step 0).  The swizzle of k-row kr depends on kr % 4
// only, which is the lane's (lane % 16) / 4 at every k-step and read, so the
// read for k-step kk and half q is this offset plus (16 kk + 4 q) RB.
template <class W, int RB, int CPR>
__device__ __forceinline__ int wg_frag_off(int col0, int lane) {
  const int g = lane / 16, r = lane % 16;
  const int n = col0 + 16 * (g % 2) + 4 * (r % 4);
  const int kr = 8 * (g / 2) + r / 4;
  return kr * RB + (((n / 8) ^ W::template sw<CPR>(kr)) * 16) + (n % 8) * 2;
}

// MFMA fragment: k = 8 (lane / 32) + 0..7 of k-step kk, column col0 + lane % 32
// (two transposing reads: in each 16-lane group, lane j receives value i of
// the 8-byte row addressed by lane 4i + j/4, element j % 4).
template <int RB>
__device__ __forceinline__ bf16x8 wg_frag(const char* region, int off, int kk) {
  v4s part[2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
    part[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4s_ptr)(const_cast<char*>(region) + off + (16 * kk + 4 * q) * RB));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// One slice: 4 k-steps of 16 rows, with the lane offsets of wg_frag_off.
// MASK: only the slice's first kvalid rows count (the expert's last slice).
template <class W, bool MASK>
__device__ __forceinline__ void wg_compute(const char* stage, f32x16 (&acc)[W::TM][W::TN], const int (&aoff)[W::TM],
                                           const int (&boff)[W::TN], int lane, int kvalid) {
  const char* areg = stage;
  const char* breg = stage + W::A_BYTES;
#pragma unroll
  for (int kk = 0; kk < W::BK / 16; ++kk) {
    bf16x8 a[W::TM], b[W::TN];
#pragma unroll
    for (int i = 0; i < W::TM; ++i) {
      a[i] = wg_frag<W::ARB>(areg, aoff[i], kk);
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
    for (int j = 0; j < W::TN; ++j) b[j] = wg_frag<W::BRB>(breg, boff[j], kk);
#pragma unroll
    for (int i = 0; i < W::TM; ++i)
#pragma unroll
      for (int j = 0; j < W::TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// Persistent: G workgroups (one per CU) walk the tiles slot, slot + G, ...
// (tile = (expert, M-tile, N-tile), N-tiles of one M-tile adjacent; the
// expert's first row and row count come from the tile-table pass, which
// validated the segments; an expert without rows writes zeros).  Slice k of
// a tile sits in ring stage k % 3.  After a tile's K loop the next tile's
// slice 0 is loaded into stage 0 while the fp32 result is staged through
// stages 1-2 (two passes of BM/2 rows) and stored as whole 16-byte row
// pieces; its slice 1 follows into stage 1 once the staging area is read, so
// the next tile's loads overlap this tile's epilogue.  Each thread issues the
// same number of stores per tile (pieces outside the output go to a junk
// line of its own), so the wait for the prefetched slice counts exactly.
template <class W>
__global__ __launch_bounds__(W::THREADS, 1) void grouped_wgrad_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, int32_t M, int32_t N, int32_t M0,
    float* __restrict__ C0, float* __restrict__ C1, const int32_t* __restrict__ exp_rows, int32_t n_mt,
    int32_t n_nt, int32_t total, vec16* __restrict__ junk) {
  static_assert(W::STAGES == 3 && W::WM == 2 && W::WTM * 2 == W::BM, "three stages, two row halves");
  constexpr int OUT_ROW = W::BN * 4, VPR = OUT_ROW / 16;
  constexpr int HALF = W::BM / 2;
  static_assert(HALF * OUT_ROW <= 2 * W::SLICE_BYTES, "half a tile fits stages 1-2");
  static_assert((HALF * VPR) % W::THREADS == 0, "equal stores per thread");
  constexpr int PST = HALF * VPR / W::THREADS;          // stores per thread and pass
  constexpr int NST = 2 * PST;                          // store instructions per wavefront and tile
  static_assert(NST + W::LOADS < 64, "vmcnt range");
  __shared__ __attribute__((aligned(16))) char ring[W::STAGES * W::SLICE_BYTES];
  const uint32_t G = gridDim.x;
  uint32_t tile = xcd_remap(blockIdx.x, G);
  if (tile >= static_cast<uint32_t>(total)) return;

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / W::WN, wn = wave % W::WN;
  struct Tile { int32_t e, m0, n0, row0, nrows, KT; };
  const int per_e = n_mt * n_nt;
  auto info = [&](uint32_t t) {
    Tile r;
    r.e = static_cast<int>(t) / per_e;
    const int rem = static_cast<int>(t) - r.e * per_e;
    r.m0 = (rem / n_nt) * W::BM;
    r.n0 = (rem % n_nt) * W::BN;
    const int2 er = reinterpret_cast<const int2*>(exp_rows)[r.e];
    r.row0 = er.x;
    r.nrows = er.y;
    r.KT = (er.y + W::BK - 1) / W::BK;
    return r;
  };
  // The slices' LDS DMA is issued as inline asm and waited for explicitly
  // (vmcnt, then a barrier): seen as LDS writes, the compiler would wait for
  // every DMA in flight, the prefetched slices included, before each slice's
  // first LDS read.
  // load i of the wavefront fills k-rows of A (blocks < ALOADS) or of B; a
  // lane's LDS position holds the swizzled chunk of its k-row (recomputed
  // per slice from the lane: arrays of them would cost registers)
  auto issue = [&](const Tile& t, int k) {
    char* stage = ring + (k % W::STAGES) * W::SLICE_BYTES;
    int ln = lane;
    asm volatile("" : "+v"(ln));                        // keeps the address math here (not hoisted, no spills)
#pragma unroll
    for (int i = 0; i < W::LOADS; ++i) {
      const int blk = wave * W::LOADS + i;              // wave-uniform
      const bool a = blk < W::ALOADS;
      const int kr = a ? blk * W::ARPI + ln / W::ACPR : (blk - W::ALOADS) * W::BRPI + ln / W::BCPR;
      const int cc = a ? 8 * ((ln % W::ACPR) ^ W::template sw<W::ACPR>(kr))
                       : 8 * ((ln % W::BCPR) ^ W::template sw<W::BCPR>(kr));
      const int r = k * W::BK + kr < t.nrows ? k * W::BK + kr : t.nrows - 1;
      const int lim = a ? M : N;
      int col = (a ? t.m0 : t.n0) + cc;
      col = col < lim ? col : lim - 8;
      const bf16_t* p = (a ? A : B) + (static_cast<uint32_t>(t.row0 + r) * static_cast<uint32_t>(lim) + col);
      dma_b128_asm(lds_addr(stage + blk * 1024), p);
    }
  };
  auto lds_barrier = [&]() {                           // LDS accesses done; DMA may stay in flight
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier_nofence();
  };

  int aoff[W::TM], boff[W::TN];
#pragma unroll
  for (int i = 0; i < W::TM; ++i) aoff[i] = wg_frag_off<W, W::ARB, W::ACPR>(wm * W::WTM + i * 32, lane);
#pragma unroll
  for (int j = 0; j < W::TN; ++j) boff[j] = wg_frag_off<W, W::BRB, W::BCPR>(wn * W::WTN + j * 32, lane);

  Tile cur = info(tile);
  if (cur.KT > 0) issue(cur, 0);
  if (cur.KT > 1) issue(cur, 1);
  bool stores_after_s0 = false;          // the previous tile's stores were issued after slice 0
  const int lr = lane % 32, lk = lane / 32;
  for (;;) {
    const uint32_t next_t = tile + G;
    const bool has_next = next_t < static_cast<uint32_t>(total);
    const Tile nxt = has_next ? info(next_t) : Tile{0, 0, 0, 0, 0, 0};
    f32x16 acc[W::TM][W::TN];
#pragma unroll
    for (int i = 0; i < W::TM; ++i)
#pragma unroll
      for (int j = 0; j < W::TN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
    for (int k = 0; k < cur.KT; ++k) {
      // memory instructions issued after slice k: at k = 0 the previous
      // tile's stores (when slice 0 was loaded before them), then slice 1;
      // later, slice k + 1
      if (k == 0) {
        if (stores_after_s0) {
          if (cur.KT > 1) wait_vmcnt_asm<NST + W::LOADS>();
          else wait_vmcnt_asm<NST>();
        } else {
          if (cur.KT > 1) wait_vmcnt_asm<W::LOADS>();
          else wait_vmcnt_asm<0>();
        }
      } else {
        if (k + 1 < cur.KT) wait_vmcnt_asm<W::LOADS>();
        else wait_vmcnt_asm<0>();
      }
      barrier_nofence();
      if (k + 2 < cur.KT) issue(cur, k + 2);
      const char* stage = ring + (k % W::STAGES) * W::SLICE_BYTES;
      const int kvalid = cur.nrows - k * W::BK;
      if (kvalid < W::BK)
        wg_compute<W, true>(stage, acc, aoff, boff, lane, kvalid);
      else
        wg_compute<W, false>(stage, acc, aoff, boff, lane, W::BK);
    }
    lds_barrier();                                      // every wave is done with the ring
    if (nxt.KT > 0) issue(nxt, 0);
    // epilogue: rows [pass * BM/2, + BM/2) through stages 1-2
    char* tile_lds = ring + W::SLICE_BYTES;
    const int vec_cols = (N - cur.n0 < W::BN ? N - cur.n0 : W::BN) / 4;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      if (wm == pass) {
#pragma unroll
        for (int i = 0; i < W::TM; ++i)
#pragma unroll
          for (int j = 0; j < W::TN; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
              const int r = i * 32 + 8 * (q / 4) + 4 * lk + (q % 4);
              const int c = wn * W::WTN + j * 32 + lr;
              *reinterpret_cast<float*>(tile_lds + r * OUT_ROW + c * 4) = acc[i][j][q];
            }
      }
      lds_barrier();
#pragma unroll
      for (int it = 0; it < PST; ++it) {
        const int v = tid + it * W::THREADS;
        const int r = v / VPR, cv = v % VPR;
        const int m = cur.m0 + pass * HALF + r;
        const vec16 val = *reinterpret_cast<const vec16*>(tile_lds + r * OUT_ROW + cv * 16);
        vec16* dst = junk + tid;
        if (m < M && cv < vec_cols) {
          float* row = m < M0 ? C0 + (static_cast<int64_t>(cur.e) * M0 + m) * N
                              : C1 + (static_cast<int64_t>(cur.e) * (M - M0) + (m - M0)) * N;
          dst = reinterpret_cast<vec16*>(row + cur.n0 + cv * 4);
        }
        *dst = val;
      }
      lds_barrier();                                    // the staging area is read
    }
    if (nxt.KT > 1) issue(nxt, 1);
    if (!has_next) break;
    stores_after_s0 = nxt.KT > 0;
    tile = next_t;
    cur = nxt;
  }
  wait_vmcnt_asm<0>();
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
  size_t tiles, ntiles, erows, junk, dH, dGU, H, total;
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
  w.junk = take(static_cast<size_t>(CfgWg::THREADS) * 16);
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
  vec16* junk = reinterpret_cast<vec16*>(w + L.junk);
  const int cus = device_cus();
  {
    const int n_mt = (d + C::BM - 1) / C::BM, n_nt = (d_ff + C::BN - 1) / C::BN;
    const int total = E * n_mt * n_nt;
    hipLaunchKernelGGL(HIP_KERNEL_NAME(grouped_wgrad_kernel<C>), dim3(static_cast<unsigned>(total < cus ? total : cus)),
                       dim3(C::THREADS), 0, stream, zsrc, H, d, d_ff, d, dw_down, dw_down, erows, n_mt, n_nt, total,
                       junk);
    MOE_LAUNCH_CHECK();
  }
  {
    const int n_mt = (2 * d_ff + C::BM - 1) / C::BM, n_nt = (d + C::BN - 1) / C::BN;
    const int total = E * n_mt * n_nt;
    hipLaunchKernelGGL(HIP_KERNEL_NAME(grouped_wgrad_kernel<C>), dim3(static_cast<unsigned>(total < cus ? total : cus)),
                       dim3(C::THREADS), 0, stream, dGU, xsrc, 2 * d_ff, d, d_ff, dw_gate, dw_up, erows, n_mt, n_nt,
                       total, junk);
    MOE_LAUNCH_CHECK();
  }
  return MOE_OK;
}
