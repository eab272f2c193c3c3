// Grouped bf16 MFMA GEMM core shared by the forward and backward expert
// calls: tile table, the LDS-ring GEMM kernels (one tile per workgroup, and
// persistent), the persistent register-staged kernel, the tile
// configurations and their launch helpers.
//
// C[m, n] = sum_k A[m, k] * B[n, k], both operands K-contiguous (each MFMA
// lane reads 8 consecutive K values of one row), A rows taken from ragged
// expert segments, B rows from the segment's expert matrices.
#pragma once

#include <atomic>
#include <type_traits>

#include "common.h"

namespace moe {
namespace {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// One M-tile of one expert segment.  first / ntile locate the expert's run of
// tiles in the table (used by the expert-blocked workgroup order).
struct TileEntry {
  int32_t expert, row0, row_end, first, ntile, pad0, pad1, pad2;
};

// ---------------------------------------------------------------------------
// 1. tile table
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ seg_start,
                                                           const int32_t* __restrict__ seg_count, int32_t E,
                                                           int64_t rows, int32_t BM, int32_t max_tiles,
                                                           TileEntry* __restrict__ tiles,
                                                           int32_t* __restrict__ n_tiles, uint32_t* flags,
                                                           int32_t* __restrict__ exp_rows = nullptr) {
  __shared__ int32_t sh16[17];
  __shared__ int32_t first_sh[1024], keep_sh[1024], start_sh[1024], end_sh[1024];
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
  // an expert whose tiles would run past the table (only with overlapping
  // segments) keeps the tiles that fit, so its run stays self-consistent
  const int32_t keep = pre >= max_tiles ? 0 : (cnt < max_tiles - pre ? cnt : max_tiles - pre);
  first_sh[t] = pre;
  keep_sh[t] = keep;
  start_sh[t] = s;
  end_sh[t] = s + c;
  __syncthreads();
  // every thread writes tiles v = t, t + 1024, ...: the expert of tile v is
  // the last expert whose first tile is <= v (binary search over the
  // nondecreasing first-tile table: an expert without tiles shares its first
  // tile with the next expert, which the search prefers)
  const int32_t n_out = total < max_tiles ? total : max_tiles;
  for (int32_t v = t; v < n_out; v += 1024) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (first_sh[mid] <= v) lo = mid;
      else hi = mid - 1;
    }
    const int32_t f = first_sh[lo], kp = keep_sh[lo];
    if (v - f < kp) tiles[v] = TileEntry{lo, start_sh[lo] + (v - f) * BM, end_sh[lo], f, kp, 0, 0, 0};
  }
  if (exp_rows && t < E) {               // per expert: first row and the rows its tiles cover
    exp_rows[2 * t] = s;
    exp_rows[2 * t + 1] = c < keep * BM ? c : keep * BM;
  }
  if (t == 0) {
    n_tiles[0] = total < max_tiles ? total : max_tiles;
    if (total > max_tiles) flag_or(flags, MOE_FLAG_BAD_SEGMENT);   // overlapping segments
  }
}

// ---------------------------------------------------------------------------
// 2./3. bf16 MFMA GEMM:  C[m, n] = sum_k A[m, k] * B[n, k]
// ---------------------------------------------------------------------------
// One workgroup (4 wavefronts) owns a BM x BN_OUT output tile.  The K loop
// runs over BK = 64 slices held in an LDS ring of STAGES slices; each slice
// holds the BM rows of A followed by the BNB rows of B, 128 bytes per row.
// Slices are filled by direct global -> LDS loads (global_load_lds_dwordx4:
// 16 bytes per lane, no staging registers), so STAGES - 1 slices are in
// flight while one is consumed.  Each load instruction of a wavefront fills
// 1 KB = 8 consecutive LDS rows; a lane picks the global 16-byte chunk that
// must land at its LDS position, which realises the XOR swizzle below.
//
// LDS row r, 16-byte chunk c is stored at r * 128 + ((c ^ ((r >> 1) & 7)) * 16):
// the 16 lanes of one 256-byte LDS phase (16 rows, one chunk, two rows per
// bank line) then hit 16 different bank groups on fragment reads.

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

// Byte offset of logical 16-byte chunk c of LDS row r in a slice whose rows
// are RB bytes long (RB = 2 * BK): rows sharing a 256-byte bank line are
// told apart by their position in the line, the XOR separates rows that
// share a position.
template <int RB>
__device__ __forceinline__ int swz_off(int r, int c) {
  constexpr int RPL = 256 / RB, CPR = RB / 16;
  return r * RB + ((c ^ ((r / RPL) % CPR)) << 4);
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without a memory fence: a fence would wait for every
// outstanding LDS DMA, including the slices still meant to be in flight.
// The empty asm statements keep the compiler from moving LDS accesses across.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}

// 16-byte LDS store the compiler does not see as an LDS access (so it adds no
// wait for LDS DMA in flight before it); the caller orders it with lgkmcnt
// waits and barriers.  LDS operations complete in order, so the compiler's
// own lgkmcnt waits for its LDS reads stay correct (at worst conservative).
__device__ __forceinline__ void ds_write_b128_asm(uint32_t addr, vec16 v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(v));
}

// Loads the compiler does not track.  With an LDS DMA in flight the compiler
// waits for every outstanding load (vmcnt(0)) before any LDS store, its own
// or inline, since it cannot tell LDS regions apart; a K loop that keeps DMA
// in flight across LDS stores therefore issues its loads itself and orders
// them with explicit vmcnt waits.  buffer_load_b128_asm's result register is
// written when the load returns: only a later inline LDS store, behind an
// explicit wait, may read it.
__device__ __forceinline__ void dma_b128_asm(uint32_t lds_dst, const void* src) {
  // LDS DMA: 16 bytes per lane from src to LDS at M0 + 16 * lane (M0 is
  // wave-uniform); one wait state between the M0 write and its use
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_dst), "v"(src) : "memory");
}

// Lane index formed by instructions the compiler cannot merge with an
// earlier copy: per-lane constants derived from it are recomputed where
// used instead of being kept live (or spilled) across a long loop.
__device__ __forceinline__ int lane_fresh() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// LDS DMA through a buffer resource: 16 bytes per lane from the buffer at
// voff + soff to LDS at M0 + 16 * lane (a 32-bit per-lane offset instead of a
// 64-bit address).
__device__ __forceinline__ void dma_buf_b128_asm(uint32_t lds_dst, __amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                                 uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds_dst), "v"(voff),
               "s"(rsrc), "s"(soff)
               : "memory");
}

__device__ __forceinline__ void buffer_load_b128_asm(vec16& r, __amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                                     uint32_t soff) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen" : "=v"(r) : "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}

// vmcnt wait as inline asm: ordered with the inline loads and stores above and,
// through the memory clobber, with every memory access of the compiler (a
// builtin wait may be scheduled past unrelated instructions).
template <int N>
__device__ __forceinline__ void wait_vmcnt_asm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>());
  }
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

// fp32 -> bf16, round to nearest even, with the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32, two values per instruction when the compiler pairs them).
__device__ __forceinline__ bf16_t bf16_hw(float f) { return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f)); }

// Two values in one v_cvt_pk_bf16_f32: a in the low half, b in the high half.
__device__ __forceinline__ uint32_t bf16x2_hw(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b16x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b16x2));
}

// SiLU with the hardware reciprocal (about 1 ulp), for the GEMM epilogue.
__device__ __forceinline__ float silu_fast(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// Epilogues: kEpiStore writes C (SiLU(G) * U for gate/up tiles); kEpiSwigluBwd
// (gate/up tiles only) reads the H gradient and writes the G and U gradients
// and H (the SwiGLU backward at the recomputed G, U).
constexpr int kEpiStore = 0, kEpiSwigluBwd = 1;

template <int BM_, int BNB_, int WM_, int WN_, int STAGES_, bool GATEUP_, bool OUT_F32_, bool EB_ = false,
          int BK_ = 64, int OCC_ = 1, int GM_ = 1, int NW_ = 4, bool RS_ = false, int EPI_ = kEpiStore,
          bool BT_ = false, int AST_ = 2, int PB_ = 1, int PA_ = 1, bool SW_ = false, bool SV_ = false, int NR_ = 2>
struct Cfg {
  static constexpr int EPI = EPI_;
  // NR (register staging): register stages of B rows; B slices are loaded
  // NR + 1 steps ahead of their use (the one-tile form: NR = 2 only)
  static constexpr int NR = NR_;
  // BT: B is stored K-major, [K][N] per expert with N contiguous (a weight
  // used transposed, as in the data-gradient products of the backward).  The
  // slice's B region then holds BK rows of BNB values, filled by LDS DMA, and
  // MFMA B fragments are read with the gfx950 transposing LDS read: in each
  // 16-lane group, lane j receives value i of the 8-byte row addressed by
  // lane 4i + j/4, element j%4, so 16 lanes that address 4 k-rows x 16
  // consecutive n get 4 consecutive k of one n each.
  static constexpr bool BT = BT_;
  static constexpr int NW = NW_;                          // wavefronts per workgroup
  // RS: the weight (B) rows of a slice travel HBM -> registers -> LDS through
  // two register stages, so two B slices are in flight with a two-stage LDS
  // ring; the A rows keep the direct LDS DMA (else: everything by DMA)
  static constexpr bool RS = RS_;
  // AST (register staging only): LDS stages of A rows; the A DMA runs
  // AST - 1 slices ahead of the slice being consumed
  static constexpr int AST = AST_;
  // MFMA fragment prefetch distances in MFMA groups (B fragment, A fragments)
  static constexpr int PB = PB_, PA = PA_;
  // SW: the MFMA takes the weight fragment as its first operand, so a lane's
  // accumulator holds 4 consecutive output columns of one row (instead of 4
  // consecutive rows of one column) and the epilogue moves 8- or 16-byte
  // pieces; plain-store tiles staged through LDS only
  static constexpr bool SW = SW_;
  // SV (gate/up tiles): the epilogue also stores the pre-activations G and U
  // (bf16) into a [rows, 2 N] buffer (G in columns [0, N), U in [N, 2 N)),
  // for a backward that takes them instead of recomputing them
  static constexpr bool SV = SV_;
  static constexpr int THREADS = NW * 64;
  static constexpr int GROUP_M = GM_;                     // M-tiles per band of the grouped order (1 = off)
  static constexpr int BM = BM_, BNB = BNB_, WM = WM_, WN = WN_, STAGES = STAGES_, BK = BK_;
  static constexpr int OCC = OCC_;                        // workgroups per CU the registers must allow
  static constexpr int RB = BK * 2;                       // bytes per LDS row
  static constexpr int CPR = BK / 8;                      // 16-byte chunks per row
  static constexpr int RPI = 1024 / RB;                   // rows filled by one wave-wide DMA load
  static constexpr bool GATEUP = GATEUP_, OUT_F32 = OUT_F32_, EXPERT_BLOCKED = EB_;
  static constexpr int WTM = BM / WM;                     // rows per wavefront
  static constexpr int TM = WTM / 32;                     // 32-row MFMA tiles per wavefront
  // GATEUP: B holds BNB/2 gate rows then BNB/2 up rows and the output tile has
  // BNB/2 columns of H.  Otherwise BNB output columns.
  static constexpr int BN_OUT = GATEUP ? BNB / 2 : BNB;
  static constexpr int WTN = BN_OUT / WN;                 // output columns per wavefront
  static constexpr int TN = WTN / 32;
  static constexpr int NB = GATEUP ? 2 : 1;
  static constexpr int ROWS = BM + BNB;                   // LDS rows per slice
  static constexpr int SLICE = ROWS * BK;                 // bf16 elements per slice
  // bf16 elements of the LDS ring: STAGES slices, or with register staging
  // AST stages of A rows followed by two stages of B rows
  static constexpr int RING = RS ? AST * BM * BK + 2 * BNB * BK : STAGES * SLICE;
  static constexpr int LOADS = ROWS / RPI / NW;           // load instructions per wavefront per slice
  static_assert(BK == 32 || BK == 64, "slice depth");
  static_assert(ROWS % (RPI * NW) == 0 && BM % RPI == 0 && (BNB / 2) % RPI == 0, "slice rows vs DMA blocks");
  static_assert(WM * WN == NW, "wavefront grid");
  static_assert(TM >= 1 && TN >= 1, "wavefront tile too small");
  static_assert(ROWS % 32 == 0 && BM % 16 == 0, "slice rows");
  static_assert(STAGES >= 2 && (STAGES - 2) * LOADS < 64, "pipeline depth");
  static_assert(!RS || STAGES == 2, "register staging uses a two-stage ring");
  static_assert(AST == 2 || (RS && (AST == 3 || AST == 4)), "three or four A stages only with register-staged B rows");
  static_assert(NR == 2 || (RS && NR >= 2 && NR <= 4), "register stages of B rows");
  static_assert(!SV || (GATEUP && !SW), "saved pre-activations: gate/up tiles in the unswapped layout");
  static_assert(EPI == kEpiStore || GATEUP, "the SwiGLU backward epilogue needs gate/up tiles");
  static_assert(!BT || (!GATEUP && !RS_ && BK == 64 && (BNB == 128 || BNB == 256)), "K-major B tiles");
  static constexpr int BRB = BNB * 2;                     // BT: bytes per k-row of the B region
  static constexpr int BCPR = BNB / 8;                    // BT: 16-byte chunks per k-row
  static constexpr int BRPI = 1024 / BRB;                 // BT: k-rows filled by one wave-wide DMA load
  // BT swizzle: logical chunk c of k-row r sits at c ^ bt_sw(r), so the 4
  // k-rows x 2 chunks of one transposing read land in 8 distinct positions
  static __device__ __forceinline__ int bt_sw(int r) { return ((r % 8) * 2) % BCPR; }
  // with RS every wavefront issues LA loads of A blocks and LB of B blocks
  static constexpr int LA = RS ? BM / RPI / NW : LOADS;
  static constexpr int LB = RS ? BNB / RPI / NW : 0;
  static_assert(!RS || (BM % (RPI * NW) == 0 && BNB % (RPI * NW) == 0 && LA + LB == LOADS && LB > 0),
                "register staging splits every wavefront's loads between A and B");
  static_assert(!RS || !GATEUP || (BNB / 2) % (LB * RPI) == 0,
                "with register staging all B rows of a wavefront come from one matrix");
  // 8-row block of the slice filled by load i of wavefront w
  static __device__ __forceinline__ int block(int w, int i) {
    return !RS ? w * LOADS + i : (i < LA ? w * LA + i : BM / RPI + w * LB + (i - LA));
  }
};

// Issue the loads of one K slice into an LDS stage.  Load i of a wavefront
// reads from a wave-uniform base (A, or the expert's gate / up / down
// matrix) plus a per-lane 32-bit element offset; ko is the slice's K offset.
// With K-major B (BT) the B loads read from bsel, the slice's first k-row of
// the right matrix, plus their offset.
template <class C>
__device__ __forceinline__ void issue_slice(bf16_t* stage, const bf16_t* const* base, const uint32_t* off,
                                            uint32_t ko, int wave, const bf16_t* bsel = nullptr) {
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const bool b_row = C::BT && C::block(wave, i) >= C::BM / C::RPI;
    const bf16_t* src = b_row ? bsel + off[i] : base[i] + (off[i] + ko);
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)(stage + C::block(wave, i) * 512), 16, 0, 0);
  }
}

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;

// Consume one K slice.  Fragments are software-pipelined: the LDS read of the
// next B fragment (and, at the last group of a k-step, of the next k-step's A
// fragments) is issued before the MFMA group that uses the current one, so
// LDS latency hides behind matrix-core work.  sched_barrier keeps the
// compiler from regrouping the reads behind the MFMAs.
// A rows of the slice sit at a_stage (row r at r * RB bytes), B rows at
// b_stage (B row r likewise); the swizzle repeats every 16 rows and BM is a
// multiple of 16, so both halves use their local row index.
// No memory work between MFMA groups.
struct NoMem {
  __device__ __forceinline__ void operator()(int) const {}
};

// mem(g) runs after the g-th group of MFMAs (g = kk * NF + f, one group per
// B fragment): it lets a caller spread its loads and LDS writes for later
// slices over the slice's matrix-core work instead of issuing them all at once.
template <class C, class Mem = NoMem>
__device__ __forceinline__ void compute_slice(const bf16_t* a_stage, const bf16_t* b_stage,
                                              f32x16 (&acc)[C::NB][C::TM][C::TN], int wm, int wn, int lane,
                                              Mem mem = Mem()) {
  constexpr int KS = C::BK / 16;               // MFMA k-steps per slice
  constexpr int NF = C::NB * C::TN;            // B fragments per k-step
  const int lr = lane % 32, lk = lane / 32;
  const char* abase = reinterpret_cast<const char*>(a_stage);
  const char* bbase = reinterpret_cast<const char*>(b_stage);
  auto a_frag = [&](int kk, int i) {
    return *reinterpret_cast<const bf16x8*>(abase + swz_off<C::RB>(wm * C::WTM + i * 32 + lr, kk * 2 + lk));
  };
  auto b_frag = [&](int kk, int f) {
    const int h = f / C::TN, j = f % C::TN;
    if constexpr (C::BT) {
      // two transposing reads give k = 8*(lane/32) + 0..3 and + 4..7 of
      // n = lane%32 of the fragment's 32 columns
      const int g = lane / 16, r = lane % 16;
      const int n = wn * C::WTN + j * 32 + 16 * (g % 2) + 4 * (r % 4);
      v4s part[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int kr = kk * 16 + 8 * (g / 2) + 4 * q + r / 4;
        const int byte = kr * C::BRB + (((n / 8) ^ C::bt_sw(kr)) * 16) + (n % 8) * 2;
        part[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(const_cast<char*>(bbase) + byte));
      }
      const v8s both = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
      return __builtin_bit_cast(bf16x8, both);
    } else {
      const int brow = h * (C::BNB / 2) + wn * C::WTN + j * 32 + lr;
      return *reinterpret_cast<const bf16x8*>(bbase + swz_off<C::RB>(brow, kk * 2 + lk));
    }
  };
  // Fragment schedule over the slice's KS * NF groups (group g = k-step g / NF,
  // B fragment g % NF): the B fragment of group g is read PB groups ahead, the
  // A fragments of a k-step PA groups before the k-step starts.
  constexpr int G = KS * NF;
  constexpr int PB = C::PB, PA = C::PA;
  static_assert(PB >= 1 && PB <= 3 && PA >= 1 && PA <= NF, "fragment prefetch distances");
  bf16x8 bq[G], aq[KS][C::TM];
#pragma unroll
  for (int i = 0; i < C::TM; ++i) aq[0][i] = a_frag(0, i);
#pragma unroll
  for (int g = 0; g < PB && g < G; ++g) bq[g] = b_frag(g / NF, g % NF);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int kk = g / NF, f = g % NF;
    if (g + PB < G) bq[g + PB] = b_frag((g + PB) / NF, (g + PB) % NF);
    if (kk + 1 < KS && f == NF - PA) {
#pragma unroll
      for (int i = 0; i < C::TM; ++i) aq[kk + 1][i] = a_frag(kk + 1, i);
    }
    const int h = f / C::TN, j = f % C::TN;
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
      acc[h][i][j] = C::SW ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(bq[g], aq[kk][i], acc[h][i][j], 0, 0, 0)
                           : __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[kk][i], bq[g], acc[h][i][j], 0, 0, 0);
    mem(g);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Even rounds for a grid of gridDim.x = G0 workgroups that walks `total`
// tiles with a static stride: of the launched workgroups, as many stay (the
// same number on every XCD) as make the rounds even, so the last round is
// not a handful of tiles run while the rest of the chip waits (mid layer
// gate/up: 1032 tiles run as 208 x 5 instead of 256 x 4 + 8).  Returns false
// for a workgroup with no tile; else its first tile `slot` and the stride G.
// Consecutive slots share an XCD (the hardware deals workgroups round-robin
// over the XCDs).
__device__ __forceinline__ bool even_rounds(uint32_t total, uint32_t* slot, uint32_t* G) {
  const uint32_t G0 = gridDim.x;
  const uint32_t rounds = (total + G0 - 1) / G0;
  uint32_t g = rounds > 0 ? (total + rounds - 1) / rounds : G0;
  uint32_t s;
  if (G0 % kXcds == 0) {
    const uint32_t per = (g + kXcds - 1) / kXcds;      // <= G0 / kXcds
    g = per * kXcds;
    const uint32_t x = blockIdx.x % kXcds, l = blockIdx.x / kXcds;
    if (l >= per) return false;
    s = x * per + l;
  } else {
    g = G0;
    s = xcd_remap(blockIdx.x, G0);
  }
  *slot = s;
  *G = g;
  return s < total;
}

// Output row of A row `row`: the row itself, or out_rows[row] when a row map
// is given (then -1 when the mapped row is outside [0, out_n): not stored).
__device__ __forceinline__ int32_t dest_row(const int32_t* __restrict__ out_rows, int32_t out_n, int32_t row) {
  if (!out_rows) return row;
  const int32_t o = out_rows[row];
  return o >= 0 && o < out_n ? o : -1;
}

// Row-map entry of the wave's tile row wm*WTM + lane (lanes past WTM repeat
// the wave's rows; rows past the segment give -1).  Fetched when the tile
// starts, so the load's latency hides under the K loop and the epilogue
// takes every row's entry from this register with a lane shuffle.
template <class C, bool MAP>
__device__ __forceinline__ int32_t lane_dest_row(const int32_t* __restrict__ out_rows, int32_t out_n, int32_t row0,
                                                 int32_t row_end, int wm, int lane) {
  static_assert(!MAP || C::WTM <= kWave, "one row-map entry per lane covers the wave's rows");
  if (!MAP) return 0;
  const int32_t row = row0 + wm * C::WTM + lane % C::WTM;
  return row < row_end ? dest_row(out_rows, out_n, row) : -1;
}

// Direct-store epilogue: every lane writes its fragments' values (value(i, j,
// q) is C[m][n] at m = 8*(q/4) + 4*(lane/32) + q%4, n = lane%32 of the 32x32
// block (i, j) of the wave's tile) to row m of Cout, or with a row map to the
// row held by lane_dst of the lane that owns m (lane_dest_row).
template <class C, bool MAP, class OutT, class Value>
__device__ __forceinline__ void store_direct_at(void* __restrict__ Cout, int32_t ld, int32_t col_off, int32_t N,
                                                int32_t row0, int32_t row_end, int32_t n0, int wm, int wn, int lane,
                                                int32_t lane_dst, Value value);

// Direct-store epilogue into a row-major [*, N] matrix.
template <class C, bool MAP, class OutT, class Value>
__device__ __forceinline__ void store_direct(void* __restrict__ Cout, int32_t N, int32_t row0, int32_t row_end,
                                             int32_t n0, int wm, int wn, int lane, int32_t lane_dst, Value value) {
  store_direct_at<C, MAP, OutT>(Cout, N, 0, N, row0, row_end, n0, wm, wn, lane, lane_dst, value);
}

// The same into columns [col_off, col_off + N) of a matrix with row stride ld
// (columns of the tile at or past N are not stored).
template <class C, bool MAP, class OutT, class Value>
__device__ __forceinline__ void store_direct_at(void* __restrict__ Cout, int32_t ld, int32_t col_off, int32_t N,
                                                int32_t row0, int32_t row_end, int32_t n0, int wm, int wn, int lane,
                                                int32_t lane_dst, Value value) {
  const int lr = lane % 32, lk = lane / 32;
  const bool full_rows = row0 + C::BM <= row_end;
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    int32_t dst[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int local = i * 32 + 8 * (q / 4) + 4 * lk + (q % 4);
      const int32_t row = row0 + wm * C::WTM + local;
      dst[q] = (!full_rows && row >= row_end) ? -1 : row;
    }
    if constexpr (MAP) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int32_t m = __shfl(lane_dst, i * 32 + 8 * (q / 4) + 4 * lk + (q % 4));   // every lane takes part
        dst[q] = dst[q] < 0 ? -1 : m;
      }
    }
    // one row address per destination row; the wave's TN column blocks are
    // immediate offsets from it (N is a multiple of 64, so a 32-column block
    // is either inside the matrix or wholly past its end)
    const int col0 = n0 + wn * C::WTN + lr;
    const bool all_cols = n0 + wn * C::WTN + C::TN * 32 <= N;          // wave-uniform
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (dst[q] < 0) continue;
      OutT* rowp = static_cast<OutT*>(Cout) +
                   static_cast<uint64_t>(static_cast<uint32_t>(dst[q])) * static_cast<uint32_t>(ld) + col_off + col0;
      if (all_cols) {
#pragma unroll
        for (int j = 0; j < C::TN; ++j) rowp[j * 32] = value(i, j, q);
      } else {
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
          if (col0 - lr + j * 32 < N) rowp[j * 32] = value(i, j, q);
      }
    }
  }
}

// M-tile (entry of the tile table) and N-tile of logical tile `logical` of
// `total`, in the workgroup order of configuration C.
template <class C>
__device__ __forceinline__ void tile_mn(const TileEntry* __restrict__ tiles, uint32_t logical, uint32_t total,
                                        int32_t n_tiles_n, int* mt_out, int* nt_out) {
  int mt, nt;
  if (C::EXPERT_BLOCKED) {
    // all N-tiles of one expert form a block; inside it the M-tiles of one
    // N-tile are adjacent, so they run together and share that weight slice
    const TileEntry tq = tiles[logical / n_tiles_n];
    const int local = static_cast<int>(logical) - tq.first * n_tiles_n;
    nt = local / tq.ntile;
    mt = tq.first + local % tq.ntile;
  } else if (C::GROUP_M > 1) {
    // bands of GROUP_M M-tiles: inside a band the M-tiles of one N-tile are
    // adjacent, so the workgroups running together on an XCD share both the
    // A rows of the band and the weight slices of a few N-tiles
    const int n_mt = static_cast<int>(total / n_tiles_n);
    const int band = static_cast<int>(logical) / (C::GROUP_M * n_tiles_n);
    const int idx = static_cast<int>(logical) - band * C::GROUP_M * n_tiles_n;
    const int gm = n_mt - band * C::GROUP_M < C::GROUP_M ? n_mt - band * C::GROUP_M : C::GROUP_M;
    nt = idx / gm;
    mt = band * C::GROUP_M + idx % gm;
  } else {
    mt = static_cast<int>(logical / n_tiles_n);
    nt = static_cast<int>(logical % n_tiles_n);
  }
  *mt_out = mt;
  *nt_out = nt;
}

// One output tile (logical tile index `logical` of `total`).  MAP: results
// are stored through the row map out_rows (dest_row).
template <class C, bool MAP>
__device__ __forceinline__ void gemm_tile(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1,
    void* __restrict__ Cout, int32_t K, int32_t N, const TileEntry* __restrict__ tiles, uint32_t total,
    int32_t n_tiles_n, const bf16_t* __restrict__ aux_in, bf16_t* __restrict__ aux_out, int32_t kb1,
    const int32_t* __restrict__ out_rows, int32_t out_n, bf16_t (&ring)[C::RING], uint32_t logical) {
  int mt, nt;
  tile_mn<C>(tiles, logical, total, n_tiles_n, &mt, &nt);
  const TileEntry te = tiles[mt];
  const int64_t e = te.expert;
  const int32_t row0 = te.row0, row_end = te.row_end;
  const int32_t n0 = nt * C::BN_OUT;

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int32_t lane_dst = lane_dest_row<C, MAP>(out_rows, out_n, row0, row_end, wm, lane);

  // Source of every load instruction: LDS row rr of the slice; the lane's
  // physical chunk p = lane % CPR holds logical chunk p ^ swizzle(rr).  Rows
  // past the segment (A) or past N (B) read a valid row instead; their
  // results are never stored.  All offsets fit 32 bits (checked on the host).
  const bf16_t* base[C::LOADS];
  uint32_t off[C::LOADS];
  // K-major B (BT): the expert's matrix is [K1][N], or, with a split K, k < K1
  // from B0 and k >= K1 from B1 (both [K1][N] per expert)
  const int32_t K1 = kb1 > 0 ? kb1 : K;
  const bf16_t* Bexp0 = B0 + e * N * static_cast<int64_t>(C::BT ? K1 : K);
  const bf16_t* Bexp1 = C::GATEUP ? B1 + e * N * static_cast<int64_t>(K)
                                  : (C::BT && B1 ? B1 + e * N * static_cast<int64_t>(K1) : Bexp0);
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int blk = C::block(wave, i);                     // 8-row block (wave-uniform)
    const int rr = blk * C::RPI + lane / C::CPR;
    const int c = (lane % C::CPR) ^ ((rr / (256 / C::RB)) % C::CPR);
    if (C::BT && blk * C::RPI >= C::BM) {
      // k-row kr of the B region, logical chunk cb; columns past N read a
      // valid chunk instead (never stored)
      const int kr = (blk - C::BM / C::RPI) * C::BRPI + lane / C::BCPR;
      const int cb = (lane % C::BCPR) ^ C::bt_sw(kr);
      int n = n0 + cb * 8;
      n = n <= N - 8 ? n : N - 8;
      base[i] = Bexp0;
      off[i] = static_cast<uint32_t>(kr) * static_cast<uint32_t>(N) + static_cast<uint32_t>(n);
    } else if (blk * C::RPI < C::BM) {
      int32_t row = row0 + rr;
      row = row < row_end ? row : row_end - 1;
      base[i] = A;
      off[i] = static_cast<uint32_t>(row) * static_cast<uint32_t>(K) + c * 8;
    } else {
      const int r = rr - C::BM;
      const bool up = C::GATEUP && r >= C::BNB / 2;
      int n = n0 + (up ? r - C::BNB / 2 : r);
      n = n < N ? n : N - 1;
      base[i] = up ? Bexp1 : Bexp0;
      off[i] = static_cast<uint32_t>(n) * static_cast<uint32_t>(K) + c * 8;
    }
  }

  f32x16 acc[C::NB][C::TM][C::TN];
#pragma unroll
  for (int h = 0; h < C::NB; ++h)
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[h][i][j][q] = 0.0f;

  auto issue_group = [&](int slice) {
    const int ko = slice * C::BK;
    const bf16_t* bsel = nullptr;
    if constexpr (C::BT)
      bsel = ko < K1 ? Bexp0 + static_cast<int64_t>(ko) * N : Bexp1 + static_cast<int64_t>(ko - K1) * N;
    issue_slice<C>(ring + (slice % C::STAGES) * C::SLICE, base, off, static_cast<uint32_t>(ko), wave, bsel);
  };

  // K loop over an LDS ring of STAGES slices: wait for slice kt (the loads of
  // the STAGES - 2 younger slices may stay in flight), barrier (every wave's
  // part of slice kt has landed and everyone is done with slice kt - 1),
  // refill the freed stage with slice kt + STAGES - 1, consume slice kt.
  const int KT = K / C::BK;
  if constexpr (C::RS) {
    // A rows by LDS DMA into a ring of AST stages, AD = AST - 1 slices ahead;
    // B rows through register stages rb0 / rb1 into a two-stage B ring: B of
    // slice s is loaded at step s - 3 (or in the prologue), written to LDS at
    // step s - 1 and consumed at step s.  Step j issues, spread over its MFMA
    // groups: the LDS write of B(j + 1) into the free B stage, the DMA of
    // A(j + AD) into the A stage consumed at step j - 1, and the loads of
    // B(j + 3) into the registers just written out.  At step kt the DMA of
    // A(kt) (issued at step kt - AD) must have landed: exactly LB + (AD - 1)
    // (LA + LB) younger loads of this wave may stay in flight.  Loads past the
    // last slice re-read the last slice into stages that are free at that
    // step (never consumed), so every step issues the same instructions and
    // the vmcnt counts stay exact.  The B writes are issued as inline
    // ds_write_b128: as compiler-visible LDS stores they would wait for every
    // LDS DMA in flight (the compiler cannot tell the stages apart), which
    // would pull the A DMA back to one slice ahead.  The compiler still waits
    // for their source registers, and the step barrier waits for them
    // (lgkmcnt(0)).
    constexpr int AS = C::AST, AD = AS - 1;
    constexpr int ASTEP = C::BM * C::BK, BSTEP = C::BNB * C::BK;     // elements per A / B stage
    vec16 rb0[C::LB], rb1[C::LB];
    auto clamp = [&](int slice) { return slice < KT ? slice : KT - 1; };
    // A rows: LDS DMA of 16 bytes per lane to the wave's 1 KB block of the stage
    auto dma_a1 = [&](int stage, int slice, int i) {
      dma_b128_asm(lds_addr(ring + stage * ASTEP + C::block(wave, i) * 512),
                   base[i] + (off[i] + static_cast<uint32_t>(slice * C::BK)));
    };
    // B loads are buffer loads over the wave's weight matrix (all B rows of a
    // wavefront come from one of gate / up): a per-lane byte offset fixed for
    // the tile plus the slice's K offset in a scalar register, so no address
    // arithmetic or 64-bit address registers per slice.  The matrix is
    // N * K * 2 bytes (< 2^32, checked on the host).
    const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(base[C::LA]), 0, static_cast<int>(static_cast<uint32_t>(N) * static_cast<uint32_t>(K) * 2u),
        0x00020000);
    uint32_t boff[C::LB];
#pragma unroll
    for (int i = 0; i < C::LB; ++i) boff[i] = off[C::LA + i] * 2u;
    auto gload_b1 = [&](vec16 (&r)[C::LB], int slice, int i) {
      buffer_load_b128_asm(r[i], rsrc_b, boff[i], static_cast<uint32_t>(slice * C::BK * 2));
    };
    // LDS byte address of this lane's 16 bytes of B piece 0 in B stage 0;
    // piece i of a stage lies a wave-uniform number of 1 KB blocks further
    bf16_t* const ring_b = ring + AS * ASTEP;
    const uint32_t b_lds = lds_addr(ring_b) + static_cast<uint32_t>(lane) * 16u;
    auto lstore_b1 = [&](int stage, const vec16 (&r)[C::LB], int i) {
      ds_write_b128_asm(b_lds + static_cast<uint32_t>((stage * BSTEP + (C::block(wave, C::LA + i) - C::BM / C::RPI) * 512) * 2),
                        r[i]);
    };
    // In a step the B registers written out were loaded two steps before:
    // the DMA of A(j + AD - 1) and the loads of B(j + 2) of the step before
    // may stay in flight.
    auto step_mem = [&](int a_stage, int b_stage, vec16 (&r)[C::LB], int a_slice, int b_slice) {
      return [&, a_stage, b_stage, a_slice, b_slice](int g) {
        if (g == 0) wait_vmcnt_asm<C::LA + C::LB>();
        if (g < C::LB) lstore_b1(b_stage, r, g);
        else if (g < C::LB + C::LA) dma_a1(a_stage, a_slice, g - C::LB);
        else if (g < 2 * C::LB + C::LA) gload_b1(r, b_slice, g - C::LB - C::LA);
      };
    };
    static_assert(2 * C::LB + C::LA <= (C::BK / 16) * C::NB * C::TN, "one memory instruction per MFMA group");
    auto step_sync = [&]() {
      wait_vmcnt_asm<C::LB + (AD - 1) * (C::LA + C::LB)>();
      __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): this wave's LDS writes have landed
      barrier_nofence();
    };
    // prologue: the issue order of steps -3 .. -1 (B(0); A(0), B(1) with AD = 2;
    // the write of B(0), A(AD - 1), B(2))
#pragma unroll
    for (int i = 0; i < C::LB; ++i) gload_b1(rb0, 0, i);
    if constexpr (AD == 2) {
#pragma unroll
      for (int i = 0; i < C::LA; ++i) dma_a1(0, 0, i);
    }
#pragma unroll
    for (int i = 0; i < C::LB; ++i) gload_b1(rb1, clamp(1), i);
    wait_vmcnt_asm<(AD - 1) * C::LA + C::LB>();  // B(0) has landed
#pragma unroll
    for (int i = 0; i < C::LB; ++i) lstore_b1(0, rb0, i);
#pragma unroll
    for (int i = 0; i < C::LA; ++i) dma_a1(AD - 1, clamp(AD - 1), i);
#pragma unroll
    for (int i = 0; i < C::LB; ++i) gload_b1(rb0, clamp(2), i);
    // steps in groups of U (stage indices repeat every U steps); a group's
    // steps past the last slice are skipped
    constexpr int U = AS == 2 ? 2 : 6;
    for (int kt = 0; kt < KT; kt += U) {
      static_for<U>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        if (u == 0 || kt + u < KT) {
          const int s = kt + u;
          step_sync();
          compute_slice<C>(ring + (u % AS) * ASTEP, ring_b + (u % 2) * BSTEP, acc, wm, wn, lane,
                           step_mem((u + AD) % AS, (u + 1) % 2, (u % 2) ? rb0 : rb1, clamp(s + AD), clamp(s + 3)));
        }
      });
    }
    // no DMA may still land in the ring and no load in a staging register:
    // the registers of the last (never stored) B loads stay allocated until
    // this wait, which no instruction of the epilogue may pass
    static_assert(C::LB == 4, "staging registers tied to the final wait");
    asm volatile("s_waitcnt vmcnt(0)"
                 : "+v"(rb0[0]), "+v"(rb0[1]), "+v"(rb0[2]), "+v"(rb0[3]), "+v"(rb1[0]), "+v"(rb1[1]),
                   "+v"(rb1[2]), "+v"(rb1[3])
                 :
                 : "memory");
  } else {
#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s)
    if (s < KT) issue_group(s);
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + C::STAGES - 2 < KT)
      wait_vmcnt<(C::STAGES - 2) * C::LOADS>();
    else
      wait_vmcnt<0>();
    barrier_nofence();
    const int nk = kt + C::STAGES - 1;
    if (nk < KT) issue_group(nk);
    compute_slice<C>(ring + (kt % C::STAGES) * C::SLICE, ring + (kt % C::STAGES) * C::SLICE + C::BM * C::BK, acc, wm, wn,
                     lane);
  }
  }

  // epilogue: acc[q] holds C[m = 8*(q/4) + 4*(lane/32) + q%4][n = lane%32]
  const int lr = lane % 32, lk = lane / 32;
  if constexpr (C::EPI == kEpiSwigluBwd) {
    // SwiGLU backward at the recomputed G (acc[0]) and U (acc[1]):
    //   s = sigmoid(G), SiLU = G s, SiLU' = s (1 + G (1 - s)),
    //   dG = dH U SiLU',  dU = dH SiLU,  H = SiLU U  (as the forward rounds it).
    // The dH tile is staged in LDS (t0) with 16-byte loads; each output goes
    // through t1 and leaves as whole 16-byte row pieces.  Cout is [rows, 2N]
    // (dG in columns [0, N), dU in [N, 2N)); aux_out is H [rows, N].
    constexpr int TROW = C::BN_OUT * 2;
    static_assert(2 * C::BM * TROW <= static_cast<int>(sizeof(ring)), "dH and one output tile fit the ring");
    constexpr int VPR = TROW / 16;
    char* t0 = reinterpret_cast<char*>(ring);
    char* t1 = t0 + C::BM * TROW;
    const int rows_here = row_end - row0 < C::BM ? row_end - row0 : C::BM;
    const int cols_here = N - n0 < C::BN_OUT ? N - n0 : C::BN_OUT;
    const int vec_cols = cols_here * 2 / 16;
    barrier_nofence();                                   // every wave is done reading the ring
    for (int v = threadIdx.x; v < C::BM * VPR; v += C::THREADS) {
      const int r = v / VPR, cv = v % VPR;
      if (r >= rows_here || cv >= vec_cols) continue;
      *reinterpret_cast<vec16*>(t0 + r * TROW + cv * 16) =
          *reinterpret_cast<const vec16*>(aux_in + static_cast<int64_t>(row0 + r) * N + n0 + cv * 8);
    }
    __syncthreads();
#pragma unroll
    for (int o = 0; o < 3; ++o) {
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int r = wm * C::WTM + i * 32 + 8 * (q / 4) + 4 * lk + (q % 4);
            const int cc = wn * C::WTN + j * 32 + lr;
            const float g = acc[0][i][j][q], u = acc[1][i][j][q];
            float val;
            if (o == 2) {
              val = silu_fast(g) * u;
            } else {
              const float dh = bf16_to_f32(*reinterpret_cast<const bf16_t*>(t0 + r * TROW + cc * 2));
              const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
              val = o == 0 ? dh * u * (sg * (1.0f + g * (1.0f - sg))) : dh * (g * sg);
            }
            *reinterpret_cast<bf16_t*>(t1 + r * TROW + cc * 2) = bf16_hw(val);
          }
      __syncthreads();
      for (int v = threadIdx.x; v < C::BM * VPR; v += C::THREADS) {
        const int r = v / VPR, cv = v % VPR;
        if (r >= rows_here || cv >= vec_cols) continue;
        bf16_t* dst = o == 2 ? aux_out + static_cast<int64_t>(row0 + r) * N + n0
                             : static_cast<bf16_t*>(Cout) + static_cast<int64_t>(row0 + r) * (2 * N) + o * N + n0;
        *reinterpret_cast<vec16*>(dst + cv * 8) = *reinterpret_cast<const vec16*>(t1 + r * TROW + cv * 16);
      }
      __syncthreads();
    }
    return;
  }
  using OutT = typename std::conditional<C::OUT_F32 && !C::GATEUP, float, bf16_t>::type;
  constexpr int OUT_ROW = C::BN_OUT * static_cast<int>(sizeof(OutT));          // bytes per tile row
  constexpr bool STAGED = C::BM * OUT_ROW <= static_cast<int>(sizeof(ring));  // tile fits the ring
  auto value = [&](int i, int j, int q) -> OutT {
    if constexpr (C::GATEUP) {
      return bf16_hw(silu_fast(acc[0][i][j][q]) * acc[C::NB - 1][i][j][q]);
    } else if constexpr (C::OUT_F32) {
      return acc[0][i][j][q];
    } else {
      return bf16_hw(acc[0][i][j][q]);
    }
  };
  if constexpr (C::SW) {
    // Acc value q of 32 x 32 block (i, j) is C[m][n] at m = i*32 + lane%32 of
    // the wave's rows and n = j*32 + 8*(q/4) + 4*(lane/32) + q%4 of its
    // columns: each lane writes groups of 4 consecutive columns into a
    // row-major LDS tile whose rows are padded by 16 bytes (the 16 lanes of
    // one LDS cycle write 16 different rows, which the padding puts in
    // different banks), PASS_ROWS rows at a time; then all threads store
    // whole rows with 16-byte writes (with a row map their destination rows
    // are fetched first, all at once).
    static_assert(C::EPI == kEpiStore, "plain store epilogue");
    constexpr int ROWP = OUT_ROW + 16;
    constexpr int PROWS = C::BM * ROWP <= static_cast<int>(sizeof(ring))
                              ? C::BM
                              : static_cast<int>(sizeof(ring)) / ROWP / C::WTM * C::WTM;
    static_assert(PROWS >= C::WTM && C::BM % PROWS == 0, "whole waves per pass");
    constexpr int PASSES = C::BM / PROWS;
    constexpr int VPR = OUT_ROW / 16;
    constexpr int ITERS = (PROWS * VPR + C::THREADS - 1) / C::THREADS;
    const int rows_here = row_end - row0 < C::BM ? row_end - row0 : C::BM;
    const int cols_here = N - n0 < C::BN_OUT ? N - n0 : C::BN_OUT;
    const int vec_cols = cols_here * static_cast<int>(sizeof(OutT)) / 16;   // N is a multiple of 64
    auto fval = [&](int i, int j, int q) -> float {
      if constexpr (C::GATEUP) return silu_fast(acc[0][i][j][q]) * acc[C::NB - 1][i][j][q];
      else return acc[0][i][j][q];
    };
    char* tile = reinterpret_cast<char*>(ring);
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      const int pr0 = pass * PROWS;
      int32_t orow[MAP ? ITERS : 1];
      if constexpr (MAP) {
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
          const int r = pr0 + (static_cast<int>(threadIdx.x) + it * C::THREADS) / VPR;
          orow[it] = r < rows_here ? dest_row(out_rows, out_n, row0 + r) : -1;
        }
      }
      barrier_nofence();                                 // the ring (or the previous pass) is free
      if (wm * C::WTM / PROWS == pass) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const int r = wm * C::WTM - pr0 + i * 32 + lr;
              const int c0 = wn * C::WTN + j * 32 + 8 * g4 + 4 * lk;
              char* dst = tile + r * ROWP + c0 * static_cast<int>(sizeof(OutT));
              if constexpr (sizeof(OutT) == 4) {
                vec16 v;
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = __float_as_uint(fval(i, j, 4 * g4 + t));
                *reinterpret_cast<vec16*>(dst) = v;
              } else {
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                u32x2 v;
                v[0] = bf16x2_hw(fval(i, j, 4 * g4), fval(i, j, 4 * g4 + 1));
                v[1] = bf16x2_hw(fval(i, j, 4 * g4 + 2), fval(i, j, 4 * g4 + 3));
                *reinterpret_cast<u32x2*>(dst) = v;
              }
            }
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        const int v = static_cast<int>(threadIdx.x) + it * C::THREADS;
        const int r = v / VPR, cv = v % VPR;
        if (r >= PROWS || cv >= vec_cols) continue;
        int64_t drow;
        if constexpr (MAP) {
          if (orow[it] < 0) continue;
          drow = orow[it];
        } else {
          if (pr0 + r >= rows_here) continue;
          drow = row0 + pr0 + r;
        }
        const vec16 val = *reinterpret_cast<const vec16*>(tile + r * ROWP + cv * 16);
        *reinterpret_cast<vec16*>(static_cast<char*>(Cout) + (drow * N + n0) * static_cast<int64_t>(sizeof(OutT)) +
                                  cv * 16) = val;
      }
    }
  } else if constexpr (STAGED) {
    // Transpose through LDS: every wave writes its fragments into a row-major
    // BM x BN_OUT tile, then all threads store whole rows with 16-byte writes
    // (thread tid stores pieces v = tid + it*THREADS, row v / VPR; with a row
    // map their destination rows are fetched first, all at once).
    constexpr int VPR = OUT_ROW / 16;                    // 16-byte vectors per tile row
    constexpr int ITERS = (C::BM * VPR + C::THREADS - 1) / C::THREADS;
    const int rows_here = row_end - row0 < C::BM ? row_end - row0 : C::BM;
    int32_t orow[MAP ? ITERS : 1];
    if constexpr (MAP) {
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        const int r = (static_cast<int>(threadIdx.x) + it * C::THREADS) / VPR;
        orow[it] = r < rows_here ? dest_row(out_rows, out_n, row0 + r) : -1;
      }
    }
    char* tile = reinterpret_cast<char*>(ring);
    barrier_nofence();                                   // every wave is done reading the ring
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = wm * C::WTM + i * 32 + 8 * (q / 4) + 4 * lk + (q % 4);
          const int cc = wn * C::WTN + j * 32 + lr;
          *reinterpret_cast<OutT*>(tile + r * OUT_ROW + cc * sizeof(OutT)) = value(i, j, q);
        }
    __syncthreads();
    const int cols_here = N - n0 < C::BN_OUT ? N - n0 : C::BN_OUT;
    const int vec_cols = cols_here * static_cast<int>(sizeof(OutT)) / 16;   // N is a multiple of 64
    if constexpr (MAP) {
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        const int v = static_cast<int>(threadIdx.x) + it * C::THREADS;
        const int r = v / VPR, cv = v % VPR;
        if (orow[it] < 0 || cv >= vec_cols) continue;
        const vec16 val = *reinterpret_cast<const vec16*>(tile + r * OUT_ROW + cv * 16);
        char* dst = static_cast<char*>(Cout) + (static_cast<int64_t>(orow[it]) * N + n0) * sizeof(OutT) + cv * 16;
        *reinterpret_cast<vec16*>(dst) = val;
      }
    } else {
      for (int v = threadIdx.x; v < C::BM * VPR; v += C::THREADS) {
        const int r = v / VPR, cv = v % VPR;
        if (r >= rows_here || cv >= vec_cols) continue;
        const vec16 val = *reinterpret_cast<const vec16*>(tile + r * OUT_ROW + cv * 16);
        char* dst = static_cast<char*>(Cout) + (static_cast<int64_t>(row0 + r) * N + n0) * sizeof(OutT) + cv * 16;
        *reinterpret_cast<vec16*>(dst) = val;
      }
    }
  } else {
    store_direct<C, MAP, OutT>(Cout, N, row0, row_end, n0, wm, wn, lane, lane_dst, value);
  }
  if constexpr (C::SV) {
    // the pre-activations G | U of the tile's rows into aux_out [rows, 2 N]
    store_direct_at<C, false, bf16_t>(aux_out, 2 * N, 0, N, row0, row_end, n0, wm, wn, lane, 0,
                                      [&](int i, int j, int q) { return bf16_hw(acc[0][i][j][q]); });
    store_direct_at<C, false, bf16_t>(aux_out, 2 * N, N, N, row0, row_end, n0, wm, wn, lane, 0,
                                      [&](int i, int j, int q) { return bf16_hw(acc[1][i][j][q]); });
  }
}

// Workgroups walk the tile list with even rounds (one tile at a time: the
// ring drains at the end of each tile, whose epilogue may stage through it;
// backward data-gradient GEMMs about 5 % faster than one tile per
// workgroup).  Register-staged tiles here keep one tile per workgroup (the
// loop costs this form spilled registers); they normally run in the
// persistent register-staged kernel, and come here only when their slice
// count does not fit its stage cycle.
template <class C, bool MAP>
__global__ __launch_bounds__(C::THREADS, C::OCC) void grouped_gemm_bf16_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1,
    void* __restrict__ Cout, int32_t K, int32_t N, const TileEntry* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles_ptr, int32_t n_tiles_n, const bf16_t* __restrict__ aux_in,
    bf16_t* __restrict__ aux_out, int32_t kb1, const int32_t* __restrict__ out_rows, int32_t out_n) {
  // The K-slice ring.  With register staging the A rows of the two stages
  // come first and the B rows of the two stages follow.  (One LDS array only:
  // with several, the compiler tracks the LDS DMA per array and waits for it
  // before every LDS read of that array.)
  __shared__ __attribute__((aligned(16))) bf16_t ring[C::RING];
  const uint32_t total = static_cast<uint32_t>(*n_tiles_ptr) * n_tiles_n;
  if constexpr (C::RS) {
    if (blockIdx.x < total)
      gemm_tile<C, MAP>(A, B0, B1, Cout, K, N, tiles, total, n_tiles_n, aux_in, aux_out, kb1, out_rows, out_n,
                        ring, xcd_remap(blockIdx.x, total));
    return;
  }
  uint32_t slot, G;
  if (!even_rounds(total, &slot, &G)) return;
  for (uint32_t logical = slot; logical < total; logical += G) {
    gemm_tile<C, MAP>(A, B0, B1, Cout, K, N, tiles, total, n_tiles_n, aux_in, aux_out, kb1, out_rows, out_n, ring,
                      logical);
    barrier_nofence();                       // every wave is done with the ring before the next tile's loads
  }
}

// Dynamic wait for the oldest in-flight slice: `after` younger slices (0 ..
// STAGES-2) may stay in flight.
template <class C, int N = C::STAGES - 2>
__device__ __forceinline__ void wait_slice(int after) {
  if constexpr (N <= 0) {
    wait_vmcnt<0>();
  } else {
    if (after >= N)
      wait_vmcnt<N * C::LOADS>();
    else
      wait_slice<C, N - 1>(after);
  }
}

// Persistent form: G workgroups walk the tile list with a static stride
// (round r takes tiles r*G + slot), and the K-slice ring runs on across tile
// boundaries: the first slices of the next tile are already in flight while
// the current tile finishes and writes its outputs (direct stores), so
// neither the pipeline fill nor the epilogue leaves the CU idle.  The rounds
// are even (even_rounds).
template <class C, bool MAP>
__global__ __launch_bounds__(C::THREADS, C::OCC) void grouped_gemm_bf16_persistent(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1,
    void* __restrict__ Cout, int32_t K, int32_t N, const TileEntry* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles_ptr, int32_t n_tiles_n, const int32_t* __restrict__ out_rows,
    int32_t out_n, bf16_t* __restrict__ aux_out) {
  __shared__ __attribute__((aligned(16))) bf16_t ring[C::RING];
  using OutT = typename std::conditional<C::OUT_F32 && !C::GATEUP, float, bf16_t>::type;
  static_assert(!C::SW, "the persistent form stores directly in the unswapped layout");

  const uint32_t total = static_cast<uint32_t>(*n_tiles_ptr) * n_tiles_n;
  uint32_t slot, G;
  if (!even_rounds(total, &slot, &G)) return;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int KT = K / C::BK;

  struct Coords { int64_t e; int32_t row0, row_end, n0; };
  auto coords = [&](uint32_t logical) {
    const int mt = static_cast<int>(logical / n_tiles_n), nt = static_cast<int>(logical % n_tiles_n);
    const TileEntry te = tiles[mt];
    return Coords{te.expert, te.row0, te.row_end, nt * C::BN_OUT};
  };

  // loader state: tile being loaded and its per-lane sources
  const bf16_t* base[C::LOADS];
  uint32_t off[C::LOADS];
  auto set_sources = [&](const Coords& t) {
    const bf16_t* Bexp0 = B0 + t.e * N * static_cast<int64_t>(K);
    const bf16_t* Bexp1 = C::GATEUP ? B1 + t.e * N * static_cast<int64_t>(K) : Bexp0;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int blk = C::block(wave, i);
      const int rr = blk * C::RPI + lane / C::CPR;
      const int c = (lane % C::CPR) ^ ((rr / (256 / C::RB)) % C::CPR);
      if (blk * C::RPI < C::BM) {
        int32_t row = t.row0 + rr;
        row = row < t.row_end ? row : t.row_end - 1;
        base[i] = A;
        off[i] = static_cast<uint32_t>(row) * static_cast<uint32_t>(K) + c * 8;
      } else {
        const int r = rr - C::BM;
        const bool up = C::GATEUP && r >= C::BNB / 2;
        int n = t.n0 + (up ? r - C::BNB / 2 : r);
        n = n < N ? n : N - 1;
        base[i] = up ? Bexp1 : Bexp0;
        off[i] = static_cast<uint32_t>(n) * static_cast<uint32_t>(K) + c * 8;
      }
    }
  };
  uint32_t ld_tile = slot;
  int ld_k = 0;
  bool ld_live = true;
  set_sources(coords(ld_tile));
  int issued = 0, consumed = 0;
  auto issue_next = [&]() {
    if (!ld_live) return;
    issue_slice<C>(ring + (issued % C::STAGES) * C::SLICE, base, off, static_cast<uint32_t>(ld_k * C::BK), wave);
    ++issued;
    if (++ld_k == KT) {
      ld_k = 0;
      ld_tile += G;
      ld_live = ld_tile < total;
      if (ld_live) set_sources(coords(ld_tile));
    }
  };
#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s) issue_next();

  f32x16 acc[C::NB][C::TM][C::TN];
  for (uint32_t tile = slot; tile < total; tile += G) {
    const Coords t = coords(tile);
    const int32_t lane_dst = lane_dest_row<C, MAP>(out_rows, out_n, t.row0, t.row_end, wm, lane);
#pragma unroll
    for (int h = 0; h < C::NB; ++h)
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[h][i][j][q] = 0.0f;
    for (int kt = 0; kt < KT; ++kt) {
      wait_slice<C>(issued - consumed - 1);
      barrier_nofence();
      issue_next();
      compute_slice<C>(ring + (consumed % C::STAGES) * C::SLICE, ring + (consumed % C::STAGES) * C::SLICE + C::BM * C::BK,
                         acc, wm, wn, lane);
      ++consumed;
    }
    store_direct<C, MAP, OutT>(Cout, N, t.row0, t.row_end, t.n0, wm, wn, lane, lane_dst,
                          [&](int i, int j, int q) -> OutT {
                            if constexpr (C::GATEUP)
                              return bf16_hw(silu_fast(acc[0][i][j][q]) * acc[C::NB - 1][i][j][q]);
                            else if constexpr (C::OUT_F32)
                              return acc[0][i][j][q];
                            else
                              return bf16_hw(acc[0][i][j][q]);
                          });
    if constexpr (C::SV) {
      // the pre-activations G | U of the tile's rows into aux_out [rows, 2 N]
      store_direct_at<C, false, bf16_t>(aux_out, 2 * N, 0, N, t.row0, t.row_end, t.n0, wm, wn, lane, 0,
                                        [&](int i, int j, int q) { return bf16_hw(acc[0][i][j][q]); });
      store_direct_at<C, false, bf16_t>(aux_out, 2 * N, N, N, t.row0, t.row_end, t.n0, wm, wn, lane, 0,
                                        [&](int i, int j, int q) { return bf16_hw(acc[1][i][j][q]); });
    }
  }
}

// Smallest slice count K / 64 of a tile for the persistent register-staged
// pipeline: a multiple of its stage cycle, and at least the B loader's lead
// (NR + 2 slices), so that no loader runs more than one tile ahead.
template <class C>
constexpr int rs_min_slices();

// Stage cycle of the persistent register-staged pipeline: the A ring, the
// two B stages in LDS and the NR register stages all repeat after U slices.
template <class C>
constexpr int rs_cycle() {
  auto gcd = [](int a, int b) {
    while (b) {
      const int t = a % b;
      a = b;
      b = t;
    }
    return a;
  };
  const int u = C::AST * 2 / gcd(C::AST, 2);
  return u * C::NR / gcd(u, C::NR);
}

template <class C>
constexpr int rs_min_slices() {
  const int u = rs_cycle<C>();
  return u >= C::NR + 2 ? u : u * ((C::NR + 2 + u - 1) / u);
}

// K / 64 runs the persistent register-staged pipeline of C
template <class C>
constexpr bool rs_slices_ok(int32_t kt) {
  return kt >= rs_min_slices<C>() && kt % rs_cycle<C>() == 0;
}

// Persistent form of the register-staged tiles (direct-store epilogue, or
// for swapped gate/up tiles one staged through the two ring stages the last
// slice freed).  G workgroups walk their tiles with a static stride (even
// rounds), and a workgroup's tiles form one sequence of K slices: the A DMA
// (AD slices ahead) and the B register loads (NR + 1 slices ahead, through
// NR register stages) run on across tile boundaries, so the first slices of the next tile are
// already loading while the current tile's last slices are consumed and its
// epilogue stores run -- neither the pipeline fill nor a new workgroup's
// start-up leaves the CU idle between tiles.  The stage indices repeat every
// U slices (rs_cycle) and K / BK is a multiple of U and at least the B
// loader's lead (rs_min_slices, checked on the host), so every tile starts
// at a group boundary and the loaders run at most one tile ahead.
template <class C, bool MAP>
__global__ __launch_bounds__(C::THREADS, C::OCC) void grouped_gemm_rs_persistent(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ B0, const bf16_t* __restrict__ B1,
    void* __restrict__ Cout, int32_t K, int32_t N, const TileEntry* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles_ptr, int32_t n_tiles_n, const int32_t* out_rows,
    int32_t out_n, uint32_t out_bytes) {
  static_assert(C::RS && C::AST >= 3 && C::EPI == kEpiStore && !C::SV && !C::BT && (!C::SW || C::GATEUP),
                "register-staged tiles with three or four A stages and the plain store epilogue");
  static_assert(C::LB == 4, "staging registers tied to the final wait");
  __shared__ __attribute__((aligned(16))) bf16_t ring[C::RING];
  using OutT = typename std::conditional<C::OUT_F32 && !C::GATEUP, float, bf16_t>::type;
  constexpr int AS = C::AST, AD = AS - 1, NR = C::NR, U = rs_cycle<C>();
  constexpr int ASTEP = C::BM * C::BK, BSTEP = C::BNB * C::BK;     // elements per A / B stage

  const uint32_t total = static_cast<uint32_t>(*n_tiles_ptr) * n_tiles_n;
  uint32_t slot, G;
  if (!even_rounds(total, &slot, &G)) return;
  const int mine = static_cast<int>((total - slot + G - 1) / G);    // tiles of this workgroup (>= 1)
  const int KT = K / C::BK;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / C::WN, wn = wave % C::WN;

  struct Coord {
    int64_t e;
    int32_t row0, row_end, n0;
  };
  auto coord = [&](int j) {
    int mt, nt;
    tile_mn<C>(tiles, slot + static_cast<uint32_t>(j) * G, total, n_tiles_n, &mt, &nt);
    const TileEntry te = tiles[mt];
    return Coord{te.expert, te.row0, te.row_end, nt * C::BN_OUT};
  };

  // A loader: the j-th tile's rows by LDS DMA through a buffer resource
  // based at the tile's first row, per-lane byte offsets (rows past the
  // segment read its last row; their results are never stored)
  __amdgpu_buffer_rsrc_t rsrc_a;
  uint32_t aoff[C::LA];
  int a_j = 0, a_k = 0;
  auto set_a = [&](const Coord& t) {
    const int32_t last = t.row_end - 1 - t.row0;
    const int ln = lane_fresh();
#pragma unroll
    for (int i = 0; i < C::LA; ++i) {
      const int rr = C::block(wave, i) * C::RPI + ln / C::CPR;
      const int c = (ln % C::CPR) ^ ((rr / (256 / C::RB)) % C::CPR);
      const int32_t row = rr < last ? rr : last;
      aoff[i] = (static_cast<uint32_t>(row) * static_cast<uint32_t>(K) + c * 8) * 2u;
    }
    rsrc_a = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(A + static_cast<int64_t>(t.row0) * K), 0,
                                               static_cast<int>(static_cast<uint32_t>(C::BM) * static_cast<uint32_t>(K) * 2u),
                                               0x00020000);
  };
  // B loader: buffer loads over the wave's weight matrix (all B rows of a
  // wavefront come from one of gate / up), per-lane byte offsets
  __amdgpu_buffer_rsrc_t rsrc_b;
  uint32_t boff[C::LB];
  int b_j = 0, b_k = 0;
  auto set_b = [&](const Coord& t) {
    // every B row of the wavefront lies in the gate half, or every one in the up half
    const bool up = C::GATEUP && C::block(wave, C::LA) * C::RPI - C::BM >= C::BNB / 2;
    const int ln = lane_fresh();
#pragma unroll
    for (int i = 0; i < C::LB; ++i) {
      const int rr = C::block(wave, C::LA + i) * C::RPI + ln / C::CPR;
      const int c = (ln % C::CPR) ^ ((rr / (256 / C::RB)) % C::CPR);
      const int r = rr - C::BM;
      int n = t.n0 + (up ? r - C::BNB / 2 : r);
      n = n < N ? n : N - 1;
      boff[i] = (static_cast<uint32_t>(n) * static_cast<uint32_t>(K) + c * 8) * 2u;
    }
    const bf16_t* bm = (up ? B1 : B0) + t.e * N * static_cast<int64_t>(K);
    rsrc_b = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(bm), 0,
                                               static_cast<int>(static_cast<uint32_t>(N) * static_cast<uint32_t>(K) * 2u),
                                               0x00020000);
  };
  // one slice further.  After step s the A loader is at slice s + AD + 1
  // and the B loader at s + NR + 2, so with K / BK a multiple of the stage
  // cycle U each can only leave its tile after one fixed step of a group
  // (WRAP: A after step UA, B after step UB, B first); past the last slice
  // of the workgroup's last tile they re-read that slice into stages that
  // are never consumed.
  // The B loader enters a new tile first (group step 2) and keeps its
  // coordinates in nx for the A loader (step 3) and the epilogue.
  Coord nx = coord(0);
  auto adv_a = [&](auto wrap) {
    ++a_k;
    if constexpr (decltype(wrap)::value) {
      if (a_k == KT) {
        if (a_j + 1 < mine) {
          a_k = 0;
          ++a_j;
          set_a(nx);
        } else {
          a_k = KT - 1;
        }
      }
    }
  };
  auto adv_b = [&](auto wrap) {
    ++b_k;
    if constexpr (decltype(wrap)::value) {
      if (b_k == KT) {
        if (b_j + 1 < mine) {
          b_k = 0;
          nx = coord(++b_j);
          set_b(nx);
        } else {
          b_k = KT - 1;
        }
      }
    }
  };
  using NoWrap = std::false_type;
  constexpr int UA = (U - (AD + 1) % U) % U, UB = (U - (NR + 2) % U) % U;
  static_assert(UA != UB && NR + 2 > AD + 1, "the loaders change tiles at different steps (B first)");
  vec16 rb[NR][C::LB];
  auto dma_a1 = [&](int stage, int i) {
    dma_buf_b128_asm(lds_addr(ring + stage * ASTEP + C::block(wave, i) * 512), rsrc_a, aoff[i],
                     static_cast<uint32_t>(a_k * C::BK * 2));
  };
  auto gload_b1 = [&](vec16 (&r)[C::LB], int i) {
    buffer_load_b128_asm(r[i], rsrc_b, boff[i], static_cast<uint32_t>(b_k * C::BK * 2));
  };
  bf16_t* const ring_b = ring + AS * ASTEP;
  const uint32_t b_lds = lds_addr(ring_b) + static_cast<uint32_t>(lane) * 16u;
  auto lstore_b1 = [&](int stage, const vec16 (&r)[C::LB], int i) {
    ds_write_b128_asm(b_lds + static_cast<uint32_t>((stage * BSTEP + (C::block(wave, C::LA + i) - C::BM / C::RPI) * 512) * 2),
                      r[i]);
  };
  // step memory work, spread over the step's MFMA groups (operation o of
  // the M after group o, or after group o * NG / M when there are more
  // operations than groups): the LDS write of B(s + 1) from the
  // registers loaded NR steps before, the DMA of A(s + AD), the loads of
  // B(s + NR + 1) into the registers just written out.  Before them, the
  // loads of those registers must have landed: (NR - 1) (LA + LB) younger
  // loads of the wave may stay in flight.
  constexpr int NG = (C::BK / 16) * C::NB * C::TN, M = 2 * C::LB + C::LA;
  auto step_mem = [&](int a_stage, int b_stage, vec16 (&r)[C::LB]) {
    return [&, a_stage, b_stage](int g) {
      if (g == 0) wait_vmcnt_asm<(NR - 1) * (C::LA + C::LB)>();
#pragma unroll
      for (int o = 0; o < M; ++o) {
        if ((M <= NG ? o : o * NG / M) != g) continue;
        if (o < C::LB) lstore_b1(b_stage, r, o);
        else if (o < C::LB + C::LA) dma_a1(a_stage, o - C::LB);
        else gload_b1(r, o - C::LB - C::LA);
      }
    };
  };
  static_assert((NR - 1) * (C::LA + C::LB) < 64 && C::LB + (AD - 1) * (C::LA + C::LB) < 64, "vmcnt range");
  auto step_sync = [&]() {
    wait_vmcnt_asm<C::LB + (AD - 1) * (C::LA + C::LB)>();
    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): this wave's LDS writes have landed
    barrier_nofence();
  };

  Coord ct = nx;
  // Row map: the raw entry of the wave's row wm*WTM + lane of a tile is
  // loaded one epilogue ahead -- before the previous tile's stores -- and
  // checked (row inside the segment, entry inside [0, out_n)) only when its
  // own epilogue starts, so the wait for it never stalls a K loop.
  auto map_raw = [&](const Coord& t) -> int32_t {
    if constexpr (!MAP) return 0;
    const int32_t row = t.row0 + wm * C::WTM + lane_fresh() % C::WTM;
    // (out_rows is not declared restrict here: the load then stays ahead of
    // the memory barrier that follows it instead of sinking behind the stores)
    return out_rows[row < t.row_end ? row : t.row_end - 1];   // rows past the segment: checked at use
  };
  int32_t raw_cur = map_raw(ct);
  if constexpr (MAP) asm volatile("" ::"v"(raw_cur));   // the first entry is waited for here, before any slice load
  // prologue: B(0) through the registers of stage 0 into LDS B stage 0,
  // B(1) .. B(NR) into register stages 1 .. NR (B(NR) reusing stage 0 once
  // B(0) is written out), A(0) .. A(AD - 1) by DMA; then the wave waits for
  // all of them, so every count-based wait of the steps holds from step 0
  // on (each later slice has exactly the younger loads the counts assume)
  set_a(nx);
  set_b(nx);
  static_assert(AD <= NR + 1, "prologue order");
#pragma unroll
  for (int i = 0; i < C::LB; ++i) gload_b1(rb[0], i);
  adv_b(NoWrap());
  static_for<NR + 1>([&](auto jc) {
    constexpr int j = decltype(jc)::value;             // 0 .. NR
    if constexpr (j < AD) {
#pragma unroll
      for (int i = 0; i < C::LA; ++i) dma_a1(j, i);
      adv_a(NoWrap());
    }
    if constexpr (j >= 1 && j < NR) {
#pragma unroll
      for (int i = 0; i < C::LB; ++i) gload_b1(rb[j], i);
      adv_b(NoWrap());
    }
    if constexpr (j == NR) {
      wait_vmcnt_asm<0>();
#pragma unroll
      for (int i = 0; i < C::LB; ++i) lstore_b1(0, rb[0], i);
#pragma unroll
      for (int i = 0; i < C::LB; ++i) gload_b1(rb[0], i);
      adv_b(NoWrap());
      wait_vmcnt_asm<0>();
    }
  });

  f32x16 acc[C::NB][C::TM][C::TN];
  auto zero_acc = [&]() {
#pragma unroll
    for (int h = 0; h < C::NB; ++h)
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[h][i][j][q] = 0.0f;
  };
  zero_acc();
  int c_j = 0, c_k = 0;
  for (;;) {
    static_for<U>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      step_sync();
      compute_slice<C>(ring + (u % AS) * ASTEP, ring_b + (u % 2) * BSTEP, acc, wm, wn, lane,
                       step_mem((u + AD) % AS, (u + 1) % 2, rb[(u + 1) % NR]));
      adv_b(std::integral_constant<bool, u == UB>());
      adv_a(std::integral_constant<bool, u == UA>());
    });
    c_k += U;
    if (c_k < KT) continue;
    const int32_t lane_dst =
        ct.row0 + wm * C::WTM + lane_fresh() % C::WTM < ct.row_end && raw_cur >= 0 && raw_cur < out_n ? raw_cur : -1;
    // nx: the next tile (the B loader's), or this one after the last tile
    if constexpr (MAP) {
      raw_cur = map_raw(nx);
      asm volatile("" ::: "memory");     // issued before the stores below
    }
    if constexpr (C::SW) {
      // Swapped layout (gate/up tiles): value q of block (i, j) is H[m][n] at
      // m = i*32 + lane%32 of the wave's rows, n = j*32 + 8*(q/4) +
      // 4*(lane/32) + q%4 of its columns.  The tile is staged in the two
      // ring stages the last slice used (A stage 2, B stage 1: the next
      // tile's first slices sit in the others), rows [0, BM/2) in one and
      // [BM/2, BM) in the other; chunk c of row r at position c ^ (r % 16)
      // (the lanes writing one chunk of 16 rows, and the threads reading 16
      // chunks of a row, hit 16 different positions).  Then every thread
      // stores whole 16-byte row pieces through a buffer resource (rows past
      // the segment, and columns past N, get an offset past its end).
      constexpr int TROW = C::BN_OUT * static_cast<int>(sizeof(OutT));
      constexpr int HALF = C::BM / 2;
      constexpr int CH = TROW / 16;                                   // 16-byte chunks per row
      static_assert(CH == 16 && HALF * TROW <= ASTEP * 2 && HALF * TROW <= BSTEP * 2 && C::WTM <= HALF,
                    "each half of the tile fits a free stage");
      char* const reg0 = reinterpret_cast<char*>(ring + 2 * ASTEP);
      char* const reg1 = reinterpret_cast<char*>(ring_b + BSTEP);
      const int lf = lane_fresh(), lr = lf % 32, lk = lf / 32;
      barrier_nofence();                 // every wave is done reading the last slice's stages
      {
        char* const reg = wm * C::WTM < HALF ? reg0 : reg1;
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
          const int r = (wm * C::WTM) % HALF + i * 32 + lr;
#pragma unroll
          for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const int chunk = (wn * C::WTN + j * 32 + 8 * g4) / 8;
              typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
              u32x2 v;
              auto f = [&](int q) { return silu_fast(acc[0][i][j][q]) * acc[C::NB - 1][i][j][q]; };
              v[0] = bf16x2_hw(f(4 * g4), f(4 * g4 + 1));
              v[1] = bf16x2_hw(f(4 * g4 + 2), f(4 * g4 + 3));
              *reinterpret_cast<u32x2*>(reg + r * TROW + ((chunk ^ (r % 16)) << 4) + lk * 8) = v;
            }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0)
      barrier_nofence();
      const __amdgpu_buffer_rsrc_t rsrc_o = __builtin_amdgcn_make_buffer_rsrc(
          static_cast<OutT*>(Cout) + ct.n0, 0, static_cast<int>(out_bytes - static_cast<uint32_t>(ct.n0) * sizeof(OutT)),
          0x00020000);
      const int rows_here = ct.row_end - ct.row0;
      const int chunks_here = (N - ct.n0) * static_cast<int>(sizeof(OutT)) / 16;
      constexpr int ITERS = C::BM * CH / C::THREADS;
      static_assert(ITERS * C::THREADS == C::BM * CH, "whole pieces per thread");
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        const int v = threadIdx.x + it * C::THREADS;
        const int r = v / CH, cv = v % CH;
        const int rr = r % HALF;
        const char* src = (r < HALF ? reg0 : reg1) + rr * TROW + ((cv ^ (rr % 16)) << 4);
        const vec16 val = *reinterpret_cast<const vec16*>(src);
        const uint32_t o = (r < rows_here && cv < chunks_here)
                               ? static_cast<uint32_t>(ct.row0 + r) * static_cast<uint32_t>(N * sizeof(OutT)) + cv * 16u
                               : 0xFFFFF000u;
        __builtin_amdgcn_raw_buffer_store_b128(val, rsrc_o, static_cast<int>(o), 0, 0);
      }
    } else {
      // epilogue: value q of 32 x 32 block (i, j) is C[m][n] at m = 8*(q/4) +
      // 4*(lane/32) + q%4, n = lane%32 of the block.  Stores go through a
      // buffer resource over the output from column n0 on: rows outside the
      // segment (or mapped to no row) get an offset past its end, which the
      // hardware drops, so the stores need no branches.  The destination row
      // of the lane's value q is the row-map entry held by lane m % 64 (read
      // with readlane: both halves of the wave take one of two known lanes).
      {
        const int lk = lane / 32;
        const __amdgpu_buffer_rsrc_t rsrc_o = __builtin_amdgcn_make_buffer_rsrc(
            static_cast<OutT*>(Cout) + ct.n0, 0, static_cast<int>(out_bytes - static_cast<uint32_t>(ct.n0) * sizeof(OutT)),
            0x00020000);
        const uint32_t col_b = static_cast<uint32_t>(wn * C::WTN + lane % 32) * sizeof(OutT);
        const uint32_t row_b = static_cast<uint32_t>(N) * sizeof(OutT);
        const int32_t rel_end = ct.row_end - ct.row0 - wm * C::WTM;      // wave rows < rel_end are valid
  #pragma unroll
        for (int i = 0; i < C::TM; ++i)
  #pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int m0 = i * 32 + 8 * (q / 4) + (q % 4);               // the lower half's row
            const int local = m0 + 4 * lk;
            int32_t d;
            if constexpr (MAP) {
              const int32_t d0 = __builtin_amdgcn_readlane(lane_dst, m0), d1 = __builtin_amdgcn_readlane(lane_dst, m0 + 4);
              d = lk ? d1 : d0;
            } else {
              d = ct.row0 + wm * C::WTM + local;
            }
            // 32-bit product as one instruction of our own: the compiler's
            // 64-bit multiply-add form would take an arbitrary register as
            // the unused high half of its addend -- possibly the row-map
            // entry still loading -- and wait for it
            uint32_t prod;
            asm("v_mul_lo_u32 %0, %1, %2" : "=v"(prod) : "v"(d), "s"(row_b));
            const uint32_t voff = (local < rel_end && d >= 0) ? prod + col_b : 0xFFFFF000u;
  #pragma unroll
            for (int j = 0; j < C::TN; ++j) {
              // a 32-column block at or past N (N is a multiple of 64) is not stored
              const uint32_t o = ct.n0 + wn * C::WTN + j * 32 < N ? voff + j * 32 * sizeof(OutT) : 0xFFFFF000u;
              const float v = acc[0][i][j][q];
              if constexpr (C::GATEUP) {
                __builtin_amdgcn_raw_buffer_store_b16(
                    __builtin_bit_cast(uint16_t, bf16_hw(silu_fast(v) * acc[C::NB - 1][i][j][q])), rsrc_o,
                    static_cast<int>(o), 0, 0);
              } else if constexpr (C::OUT_F32) {
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rsrc_o, static_cast<int>(o), 0, 0);
              } else {
                __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, bf16_hw(v)), rsrc_o,
                                                      static_cast<int>(o), 0, 0);
              }
            }
          }
      }
    }
    if (++c_j == mine) break;
    // next tile.  The epilogue's stores need no wait here: vector memory
    // operations complete in issue order, so the next step's count-based
    // wait (at most so many operations in flight, stores included) still
    // proves that the slices it needs have landed.
    ct = nx;
    zero_acc();
    c_k = 0;
    // the loaders' per-lane offsets are formed again here rather than kept
    // live across the epilogue (registers); both loaders are in tile c_j
    set_a(ct);
    set_b(ct);
  }
  // no DMA may still land in the ring and no load in a staging register
#pragma unroll
  for (int j = 0; j < NR; ++j)
    asm volatile("s_waitcnt vmcnt(0)" : "+v"(rb[j][0]), "+v"(rb[j][1]), "+v"(rb[j][2]), "+v"(rb[j][3])::"memory");
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// Three tile shapes, chosen from the mean rows per expert (rows / E), which the
// host knows without reading the device counts:
//   large  (mean >= 768 rows): 256 x 256 tiles, 8 wavefronts (two per SIMD, so
//          one wave's MFMAs cover the other's waits), LDS for three A and two
//          B slices (160 KB) with the weight rows register-staged three
//          slices ahead, persistent where K / 64 is a multiple of 6 (the
//          slice pipeline runs on across tiles), bands of 8 M-tiles for L2
//          reuse (the fp32 / gate-up tiles; 2, 4, 12, 16 measured slower) --
//          long MFMA-bound segments (static receiver arrays);
//   medium (mean >= 48 rows):  128 x 256 tiles, 8 wavefronts, 3-slice ring
//          (144 KB), persistent (the ring runs on across tiles; measured
//          3.5 % faster than one tile per workgroup on the mid layer) --
//          prefill-like weight streaming;
//   small  (otherwise):        32 x 256 tiles, 4 wavefronts, 4-slice ring
//          (144 KB), persistent -- decode-like segments of a few rows.
// Gate/up tiles hold 128 gate + 128 up rows of B (128 H columns); down tiles
// hold 256 output columns.
using CfgLgGU = Cfg<256, 256, 4, 2, 2, true, false, false, 64, 1, 8, 8, true, kEpiStore, false, 3, 1, 1, true>;
using CfgLgDF = Cfg<256, 256, 4, 2, 2, false, true, false, 64, 1, 8, 8, true, kEpiStore, false, 3>;
using CfgLgDB = Cfg<256, 256, 4, 2, 2, false, false, false, 64, 1, 4, 8, true, kEpiStore, false, 3>;
using CfgMdGU = Cfg<128, 256, 2, 4, 3, true, false, false, 64, 1, 2, 8>;
using CfgMdDF = Cfg<128, 256, 2, 4, 3, false, true, false, 64, 1, 2, 8>;
using CfgMdDB = Cfg<128, 256, 2, 4, 3, false, false, false, 64, 1, 2, 8>;
// medium tiles with the weight rows through four register stages (five
// slices ahead) and four A stages (three slices ahead), persistent: where
// K / 64 is a multiple of 4 for both products
using CfgMdGUr = Cfg<128, 256, 2, 4, 2, true, false, false, 64, 1, 2, 8, true, kEpiStore, false, 4, 1, 1, false, false, 4>;
using CfgMdDFr = Cfg<128, 256, 2, 4, 2, false, true, false, 64, 1, 2, 8, true, kEpiStore, false, 4, 1, 1, false, false, 4>;
using CfgMdDBr = Cfg<128, 256, 2, 4, 2, false, false, false, 64, 1, 2, 8, true, kEpiStore, false, 4, 1, 1, false, false, 4>;
using CfgSmGU = Cfg<32, 256, 1, 4, 4, true, false>;
// gate/up tiles that also save the pre-activations G | U (training forward):
// the same tilings in the unswapped layout
using CfgLgGUS = Cfg<256, 256, 4, 2, 2, true, false, false, 64, 1, 4, 8, true, kEpiStore, false, 3, 1, 1, false, true>;
using CfgMdGUS = Cfg<128, 256, 2, 4, 3, true, false, false, 64, 1, 2, 8, false, kEpiStore, false, 2, 1, 1, false, true>;
using CfgSmGUS = Cfg<32, 256, 1, 4, 4, true, false, false, 64, 1, 1, 4, false, kEpiStore, false, 2, 1, 1, false, true>;
using CfgSmDF = Cfg<32, 256, 1, 4, 4, false, true>;
using CfgSmDB = Cfg<32, 256, 1, 4, 4, false, false>;

constexpr bool kPersistLg = false, kPersistMd = true, kPersistSm = true;

enum TileKind { kLarge = 0, kMedium = 1, kSmall = 2 };

inline TileKind pick_tiles(int64_t rows, int32_t E) {
  const int64_t mean = rows / E;
  return mean >= 768 ? kLarge : (mean >= 48 ? kMedium : kSmall);
}

// Compute units of the current device (cached per device; the library keeps
// no other state).
inline int device_cus() {
  static std::atomic<int> cached[64];       // zero-initialised; a race only repeats the query
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Register-staged tiles run in the persistent register-staged form when the
// slice count K / BK is a multiple of its 6-slice stage cycle: tiles whose
// one-tile form stores directly from registers (the tile does not fit the
// LDS ring), and swapped gate/up tiles (staged through two free stages).
template <class C>
constexpr bool rs_persistent_ok() {
  using OutT = typename std::conditional<C::OUT_F32 && !C::GATEUP, float, bf16_t>::type;
  return C::RS && C::AST >= 3 && C::EPI == kEpiStore && !C::SV && !C::BT &&
         (C::SW ? C::GATEUP && C::BN_OUT * static_cast<int>(sizeof(OutT)) == 256
                : C::NR > 2 || C::BM * C::BN_OUT * static_cast<int>(sizeof(OutT)) > C::RING * 2);
}

template <class C, bool MAP>
int launch_kernel(bool persistent, const void* a, const void* b0, const void* b1, void* out, int32_t K, int32_t N,
                   const TileEntry* tiles, const int32_t* n_tiles, int32_t max_tiles, int32_t ntn,
                   hipStream_t stream, const void* aux_in, void* aux_out, int32_t kb1, const int32_t* out_rows,
                   int32_t out_n, int64_t c_rows) {
  const int64_t upper = static_cast<int64_t>(max_tiles) * ntn;
  if constexpr (rs_persistent_ok<C>()) {
    // the output is addressed through a buffer resource with 32-bit offsets
    // (an offset of 0xFFFFF000 and above marks a row that is not stored)
    using OutT = typename std::conditional<C::OUT_F32 && !C::GATEUP, float, bf16_t>::type;
    const int64_t out_bytes = c_rows * N * static_cast<int64_t>(sizeof(OutT));
    const int32_t kt = K / C::BK;
    if (rs_slices_ok<C>(kt) && c_rows > 0 && out_bytes < 0xFFFFF000ll) {
      const int64_t slots = static_cast<int64_t>(device_cus()) * C::OCC;
      const int64_t g = upper < slots ? upper : slots;
      hipLaunchKernelGGL(HIP_KERNEL_NAME(grouped_gemm_rs_persistent<C, MAP>), dim3(static_cast<unsigned>(g)),
                         dim3(C::THREADS), 0, stream, static_cast<const bf16_t*>(a), static_cast<const bf16_t*>(b0),
                         static_cast<const bf16_t*>(b1), out, K, N, tiles, n_tiles, ntn, out_rows, out_n,
                         static_cast<uint32_t>(out_bytes));
      return MOE_OK;
    }
  }
  if constexpr (C::NR > 2) {
    return MOE_EUNSUPPORTED;        // deeper register staging exists in the persistent form only
  } else {
    // the persistent form has the plain store epilogue only
    if (C::EPI == kEpiStore && !C::BT && !C::SW && persistent) {
      const int64_t slots = static_cast<int64_t>(device_cus()) * C::OCC;  // C::OCC workgroups per CU
      const int64_t g = upper < slots ? upper : slots;
      if constexpr (C::EPI == kEpiStore && !C::BT && !C::SW)
        hipLaunchKernelGGL(HIP_KERNEL_NAME(grouped_gemm_bf16_persistent<C, MAP>), dim3(static_cast<unsigned>(g)),
                           dim3(C::THREADS), 0, stream, static_cast<const bf16_t*>(a), static_cast<const bf16_t*>(b0),
                           static_cast<const bf16_t*>(b1), out, K, N, tiles, n_tiles, ntn, out_rows, out_n,
                           static_cast<bf16_t*>(aux_out));
    } else {
      // at most one workgroup per CU slot; each walks its tiles (even rounds);
      // register-staged tiles: one workgroup per tile
      const int64_t slots = static_cast<int64_t>(device_cus()) * C::OCC;
      const int64_t g = C::RS || upper < slots ? upper : slots;
      hipLaunchKernelGGL(HIP_KERNEL_NAME(grouped_gemm_bf16_kernel<C, MAP>), dim3(static_cast<unsigned>(g)),
                         dim3(C::THREADS), 0, stream, static_cast<const bf16_t*>(a), static_cast<const bf16_t*>(b0),
                         static_cast<const bf16_t*>(b1), out, K, N, tiles, n_tiles, ntn,
                         static_cast<const bf16_t*>(aux_in), static_cast<bf16_t*>(aux_out), kb1, out_rows, out_n);
    }
    return MOE_OK;
  }
}

// One GEMM launch; a row map (out_rows) selects the kernels built with it,
// which exist for plain-store tiles that are not gate/up tiles.
template <class C>
int launch_one(bool persistent, const void* a, const void* b0, const void* b1, void* out, int32_t K, int32_t N,
                const TileEntry* tiles, const int32_t* n_tiles, int32_t max_tiles, int32_t ntn, hipStream_t stream,
                const void* aux_in = nullptr, void* aux_out = nullptr, int32_t kb1 = 0,
                const int32_t* out_rows = nullptr, int32_t out_n = 0, int64_t c_rows = -1) {
  if constexpr (C::EPI == kEpiStore && !C::GATEUP) {
    if (out_rows)
      return launch_kernel<C, true>(persistent, a, b0, b1, out, K, N, tiles, n_tiles, max_tiles, ntn, stream, aux_in,
                                    aux_out, kb1, out_rows, out_n, out_n);
  }
  return launch_kernel<C, false>(persistent, a, b0, b1, out, K, N, tiles, n_tiles, max_tiles, ntn, stream, aux_in,
                                 aux_out, kb1, nullptr, 0, c_rows);
}

// Gate/up then down projection.  With gu_save the gate/up tiles GUS also
// store the pre-activations G | U there ([rows, 2 d_ff], bf16).
template <class GU, class GUS, class DF, class DB, bool PERSIST>
int launch_bf16(const void* x, int64_t rows, int32_t d, int32_t d_ff, const void* wg, const void* wu,
                const void* wdn, void* H, void* z, int32_t z_dtype, const int32_t* z_rows, int32_t z_n,
                const TileEntry* tiles, const int32_t* n_tiles, int32_t max_tiles, void* gu_save,
                hipStream_t stream) {
  static_assert(GU::BM == GUS::BM && GU::BN_OUT == GUS::BN_OUT, "one tiling with and without the saved G | U");
  const int nt1 = (d_ff + GU::BN_OUT - 1) / GU::BN_OUT;
  const int nt2 = (d + DF::BN_OUT - 1) / DF::BN_OUT;
  MOE_CHECK(static_cast<int64_t>(max_tiles) * (nt1 > nt2 ? nt1 : nt2) <= INT32_MAX, MOE_EUNSUPPORTED);
  int st;
  if (gu_save)
    st = launch_one<GUS>(PERSIST, x, wg, wu, H, d, d_ff, tiles, n_tiles, max_tiles, nt1, stream, nullptr, gu_save);
  else
    st = launch_one<GU>(PERSIST, x, wg, wu, H, d, d_ff, tiles, n_tiles, max_tiles, nt1, stream, nullptr, nullptr, 0,
                        nullptr, 0, rows);
  if (st != MOE_OK) return st;
  MOE_LAUNCH_CHECK();
  if (z_dtype == MOE_F32)
    st = launch_one<DF>(PERSIST, H, wdn, nullptr, z, d_ff, d, tiles, n_tiles, max_tiles, nt2, stream, nullptr, nullptr,
                        0, z_rows, z_n, rows);
  else
    st = launch_one<DB>(PERSIST, H, wdn, nullptr, z, d_ff, d, tiles, n_tiles, max_tiles, nt2, stream, nullptr, nullptr,
                        0, z_rows, z_n, rows);
  if (st != MOE_OK) return st;
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace
}  // namespace moe
