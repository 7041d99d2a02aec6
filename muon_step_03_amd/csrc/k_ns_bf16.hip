// Newton-Schulz products on bf16 matrix cores (gfx950 MFMA 32x32x16 bf16,
// float32 accumulation, float32 epilogues, one round-to-nearest-even per
// stored operand).
//
// One iteration, on X (p x q, short side first):
//   A = X X^T                 symmetric: only lower-triangle block tiles are
//                             computed, each written to both triangles
//   B = a*I + b*A + c*A A^T   A is symmetric, so A A = A A^T: the same
//                             symmetric form with K = p; b*A and a*I are
//                             added in fp32 before the one rounding
//   X' = B X                  full p x q output, a plain product
// which is X_k = aX + b(XX^T)X + c(XX^T)^2 X = (aI + bA + cA^2) X of "[논문
// AI 리뷰] MUON IS SCALABLE FOR LLM TRAINING TECHNICAL REPORT", section 2.
// Holding a*I in the stored polynomial (one more term on its diagonal tiles)
// spares the update an epilogue pass that would read its X tile a second
// time: the largest source of the update's re-read traffic.
//
// The first iteration receives the unnormalised U (the head cannot know
// ||U|| while it writes X0): its Gram is scaled by inv^2 and its update by
// inv, inv = 1/(||U||_F + 1e-7), which is the iteration applied to U*inv.
//
// Kernel structure (one template, three configurations per product):
//  * Block tiles are compile-time: symmetric products 128x128 (4 waves of
//    64x64, two blocks per CU), update 128x256 (4 waves of 64x128, two
//    blocks per CU), and for large matrices 256x256 for both (8 waves of
//    128x64, one block per CU).  A CU moves at most about 64 bytes per clock
//    from L2 into LDS, which is what a 128x128 tile needs to keep its matrix
//    cores busy; the larger tiles need half as much per flop.
//  * K steps of 64 (128-wide symmetric products) or 32 (update, 256x256
//    tiles), staged through LDS by 16-byte direct-to-LDS loads
//    (global_load_lds): STAGES buffers, loads for up to STAGES-1 later steps
//    in flight while step k is multiplied; one barrier per K step, and the
//    MFMA fragments double-buffered in registers.  Every load instruction
//    reads whole 128-byte lines (a CU loads rows of 64 bytes at half the
//    rate): operand rows of 128 bytes, the update's X rows of 512 bytes, and
//    the polynomial's output B stored in panels of 32 columns
//    ([p/32][p][32]), so that one K step of the update's B operand is a
//    contiguous block.  The loads address memory
//    as a scalar base (advanced once per K step) plus a per-lane offset
//    fixed for the tile, and the K loop is unrolled by STAGES so that every
//    LDS address is a lane's base plus an immediate: the loop body issues
//    MFMAs, LDS reads and loads with almost no vector address arithmetic.
//  * Epilogue: the fp32 tile is staged through LDS in 64-row passes and
//    stored as 16-byte rows of 8 bf16 (the plain updates of the 8-wave tiles
//    through one private window per wave instead, with no barrier between
//    waves).  The polynomial's linear term b*A: the 128x128 tiles pick it
//    from the K step whose columns are the tile's own (8-byte LDS reads at
//    the accumulator positions, added before staging); the 256x256 tiles
//    read it in the epilogue as 16-byte rows of A.
//  * K-contiguous operand tiles: rows of BK bf16 (4 or 8 chunks of 16 B),
//    chunk c of row m stored at c ^ f(m), f(m) = (m>>2) & 3 for 4 chunks,
//    (m>>1) & 7 for 8, so the fragment reads (32 consecutive rows, one
//    chunk) do not collide in gfx950's 64-bank LDS.  The swizzle is applied
//    by choosing which global chunk each lane fetches (a direct-to-LDS load
//    writes lane L's 16 bytes at base + 16 L).
//  * The update's X operand is N-contiguous: its tile is kept as 32 K-rows
//    of BN bf16 (chunk c of row k stored at c ^ g(k), g = {0,6,12,10}[k&3])
//    and MFMA B fragments are read with the transposing LDS read
//    ds_read_b64_tr_b16: within a 16-lane group, output lane i element j
//    comes from source lane 4j + i/4, element i%4, so lane s addresses
//    X[k0 + s/4][n0 + 4 (s%4)] and two reads give 8 consecutive k.
//  * Persistent blocks walk a static tile list: XCD x (the
//    hardware dispatches block b to XCD b % 8) takes one contiguous eighth of
//    every group's tiles, so its blocks work on consecutive tiles of one
//    matrix at a time and share its operands in that XCD's L2; a block's
//    next tile loads while its previous tile's stores drain.
#include <type_traits>

#include "muon_internal.h"

namespace muon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int WAVE_BYTES = 1024;    // bytes one direct-to-LDS instruction moves
constexpr int kPanel = 32;          // column panel width of the stored B

enum { MODE_GRAM = 0, MODE_POLY = 1, MODE_UPDATE = 2 };

template <int MODE>
struct Cfg;
// Symmetric products: K step of 64 (operand rows of 128 bytes, whole cache
// lines: a CU's load path moves rows of 64 bytes at half the rate, 31 vs 60
// bytes per clock measured), two stages of 32 KiB.
#ifndef MUON_SYRK_BK
#define MUON_SYRK_BK 64
#endif
#ifndef MUON_SYRK_STAGES
#define MUON_SYRK_STAGES (MUON_SYRK_BK == 64 ? 2 : 4)
#endif
#ifndef MUON_UPD_STAGES
#define MUON_UPD_STAGES 3
#endif
// Wave grid of the update block: WGM rows of waves.
#ifndef MUON_TAIL_GS
#define MUON_TAIL_GS 4
#endif
#ifndef MUON_UPD_WGM
#define MUON_UPD_WGM 2
#endif
// NW waves in a WGM x WGN grid; each wave holds WM x WN accumulators of
// 32x32; OCC blocks per CU (the register and LDS budget).
template <>
struct Cfg<MODE_GRAM> {
  static constexpr int BM = kSyrkTile, BN = kSyrkTile, NW = 4, WGM = 2, WGN = 2;
  static constexpr int WM = BM / (32 * WGM), WN = BN / (32 * WGN);
  static constexpr int BK = MUON_SYRK_BK;
  static constexpr int STAGES = MUON_SYRK_STAGES;
  static constexpr int OCC = kSyrkBlocksPerCU;
};
template <>
struct Cfg<MODE_POLY> : Cfg<MODE_GRAM> {};
// Symmetric products of large matrices: 256x256 tiles, 8 waves of 128x64,
// one block per CU (four stages of 32 KiB).  Every operand byte brought into
// a CU feeds twice the MFMA work of a 128x128 tile, which halves the L2 and
// fabric traffic of the long-K Gram products of wide matrices.
#ifndef MUON_SYRK_BIG_BK
#define MUON_SYRK_BIG_BK 32
#endif
struct CfgSyrkBig {
  static constexpr int BM = kSyrkBigTile, BN = kSyrkBigTile, NW = 8, WGM = 2, WGN = 4;
  static constexpr int WM = BM / (32 * WGM), WN = BN / (32 * WGN);
  static constexpr int BK = MUON_SYRK_BIG_BK;
  static constexpr int STAGES = BK == 64 ? 2 : 4;
  static constexpr int OCC = 1;
};
// Update of large matrices: 256x256 tiles, 8 waves of 128x64, one block
// per CU (four stages of 32 KiB).
struct CfgUpdBig {
  static constexpr int BM = kUpdBigTile, BN = kUpdBigTile, NW = 8, WGM = 2, WGN = 4;
  static constexpr int WM = BM / (32 * WGM), WN = BN / (32 * WGN);
  static constexpr int BK = 32;
  static constexpr int STAGES = 4;
  static constexpr int OCC = 1;
};
// Update of matrices whose padded short side is 512 (MoE experts): 512x128
// tiles, 8 waves of 128x64 (the wave tile of the 256x256 update), one block
// per CU, three stages of 40 KiB.  A tile spans the whole short side, so the
// long side is padded to a multiple of 128 only: 1408 stays 1408 (the
// 256-wide tiles pad it to 1536, 9 % more work and X traffic), and a
// matrix's 512x512 B, read by each of its long-side tiles, stays in L2.
struct CfgUpd512 {
  static constexpr int BM = 512, BN = 128, NW = 8, WGM = 4, WGN = 2;
  static constexpr int WM = BM / (32 * WGM), WN = BN / (32 * WGN);
  static constexpr int BK = 32;
  static constexpr int STAGES = 3;
  static constexpr int OCC = 1;
};
template <>
struct Cfg<MODE_UPDATE> {
  static constexpr int BM = kUpdTileM, BN = kUpdTileN, NW = kUpdWaves, WGM = MUON_UPD_WGM,
                       WGN = NW / WGM;
  static constexpr int WM = BM / (32 * WGM), WN = BN / (32 * WGN);
  static constexpr int BK = 32;
  static constexpr int STAGES = MUON_UPD_STAGES;
  static constexpr int OCC = kUpdBlocksPerCU;
};

// LDS banking measured on gfx950 (bank-conflict counters over single-pattern
// probes): 64 banks of 4 bytes; a 16-byte read serves 16 lanes per clock
// (lanes 0-31 and 32-63 each in two sets of four quads, split by the parity
// of the quad index), an 8-byte read (plain or transposing) 32 lanes.
//
// Row swizzle of K-contiguous tiles: 4 chunks of 16 B per row (K step 32:
// rows m, m+4, m+8, m+12 of 64 bytes fall on the same banks, so the chunk
// index is XORed with (m >> 2) & 3), or 8 chunks (K step 64: rows r and r+1
// fill one 256-byte bank window, so (r >> 1) & 7 spreads 16 consecutive rows
// over 16 distinct slots).  Both are conflict-free for the fragment reads
// (32 consecutive rows, one chunk per half wave); ((m >> 1) + (m >> 3)) & 3,
// the first choice for 4 chunks, met 2-way conflicts.
template <int CPR>
__device__ __forceinline__ int rswz(int m) {
  if constexpr (CPR == 4)
    return (m >> 2) & 3;
  else
    return (m >> 1) & 7;
}
// Chunk swizzle of the update's N-contiguous X tile (K-rows of 256 bytes, all
// on the same banks): chunk c of K-row k is stored at c ^ {0, 6, 12, 10}[k & 3],
// so the 4 K-rows x 64 bytes that 32 lanes of a transposing read take cover
// the 64 banks once.
__device__ __forceinline__ int gswz(int k) { return (0xAC60 >> ((k & 3) * 4)) & 15; }

// vmcnt-only wait (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 16-byte direct-to-LDS load: lane L's 16 bytes from `base + off` land at
// LDS address lds_base + 16 L (lds_base wave-uniform, passed in m0; base a
// 64-bit scalar address, off the lane's 32-bit byte offset).  Written as asm
// so that the compiler does not treat every later LDS read as possibly
// aliasing it (which would make it wait for all loads in flight, prefetches
// included); completion is tracked explicitly with wait_vmcnt before the
// barrier that publishes a K step.  The instruction has no result register.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(uint32_t off, const char* base, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(lds_base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// 16-byte store marked nontemporal (evict first), for the update's X'.
// Measured against plain stores on one box: update launches MoE-1B -2.5 %,
// GPT-400M -1 %, the stress set -2 %, GPT-160M -1.5 %.  The same for the
// polynomial's B (only where a launch's B's exceed the Infinity Cache) made
// it slower on the stress set (+10 %) and no faster on MoE-1B; for the
// Gram's A, +44 % to +54 %: both keep plain stores.
typedef unsigned int u32x4_nt_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt16(void* p, const uint4& v) {
  const u32x4_nt_t x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4_nt_t*>(p));
}

// Workgroup barrier that publishes this wave's LDS traffic (lgkmcnt(0): its
// LDS reads and writes are complete) but leaves global loads in flight (no
// vmcnt wait, unlike a fence); the empty asm statements keep the compiler
// from moving LDS accesses across it in either direction.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((7 << 4) | (0 << 8) | 15 | (3 << 14));  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Completes this wave's LDS writes before its following LDS reads of other
// lanes' data (a wave-private exchange: no other wave takes part), and keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((7 << 4) | (0 << 8) | 15 | (3 << 14));  // lgkmcnt(0) only
  asm volatile("" ::: "memory");
}

// Lower-triangle block index t -> (ti, tj), ti >= tj, row-major over ti.
__device__ __forceinline__ void tri_decode(int t, int& ti, int& tj) {
  int i = int((sqrtf(8.f * float(t) + 1.f) - 1.f) * 0.5f);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

template <int BK>
__device__ __forceinline__ bf16x8_t lds_frag_rows(const LDS_AS char* tile, int row, int chunk) {
  return *reinterpret_cast<const LDS_AS bf16x8_t*>(tile + row * (BK * 2) +
                                                   ((chunk ^ rswz<BK / 8>(row)) << 4));
}

template <int BN>
__device__ __forceinline__ bf16x8_t lds_frag_xT(const LDS_AS char* tile, int kb, int nb, int lane) {
  const int s = lane & 15;
  const int n = nb + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
  const int k = kb + 8 * (lane >> 5) + (s >> 2);
  const LDS_AS char* p0 = tile + k * (BN * 2) + (((n >> 3) ^ gswz(k)) << 4) + (n & 7) * 2;
  const LDS_AS char* p1 = tile + (k + 4) * (BN * 2) + (((n >> 3) ^ gswz(k + 4)) << 4) + (n & 7) * 2;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)p0);
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)p1);
  const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// LAST: the update launch of the last iteration, whose groups apply the step
// (LAST == kLastApply, groups with g.fuse) or write the tail's partial sums
// (LAST == kLastReduce, groups with g.red) in the epilogue; separate
// instantiations, so that the other launches carry none of that code (one
// call never needs both: the step is applied only when nothing is reduced).
template <int MODE, class C, int LAST = 0>
__global__ __launch_bounds__(64 * C::NW, C::OCC) void ns_bf16_kernel(
    Batch bt, TileList tl, int iter, float ca, float cb, float cc) {
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN, S = C::STAGES, BK = C::BK;
  constexpr int KS = BK / 16;                        // MFMA sub-steps per K step
  constexpr int CPK = BK / 8;                        // 16-byte chunks per operand row
  static_assert(KS == 2 || KS == 4, "K step of 32 or 64");
  static_assert(MODE != MODE_UPDATE || BK == 32, "the update's X tile has 32 K-rows");
  constexpr int NT = 64 * C::NW;                     // threads per block
  constexpr int A_BYTES = BM * BK * 2;
  constexpr int B_BYTES = BN * BK * 2;
  constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  constexpr int A_INSTR = A_BYTES / WAVE_BYTES / C::NW;  // per wave
  constexpr int B_INSTR = B_BYTES / WAVE_BYTES / C::NW;
  constexpr int LOADS = A_INSTR + B_INSTR;          // vmcnt per stage per wave
  static_assert(A_BYTES % (C::NW * WAVE_BYTES) == 0 && B_BYTES % (C::NW * WAVE_BYTES) == 0, "tiling");
  static_assert((S - 1) * LOADS < 64, "vmcnt field");
  __shared__ __attribute__((aligned(1024))) char smem_raw[S * STAGE_BYTES];
  LDS_AS char* smem = (LDS_AS char*)(smem_raw);
  (void)ca;
  (void)cb;
  (void)cc;

  // Persistent blocks: XCD x (= blockIdx % 8, the hardware's round-robin)
  // owns the contiguous slice [n x/8, n (x+1)/8) of every group's n tiles,
  // groups taken in the order of tl.group (longest K first); the
  // blocks_per_xcd blocks of an XCD walk the concatenated slices with a
  // stride of blocks_per_xcd, so at any time they hold consecutive tiles (one
  // matrix's, sharing that XCD's L2).  A block's next tile starts loading
  // while the stores of its previous tile drain.
  const int xcd = int(blockIdx.x & 7);
  const int64_t nbx = tl.blocks_per_xcd;
  int64_t l = int64_t(blockIdx.x >> 3), base = 0;
  bool first_tile = true;
  for (int oi = 0; oi < tl.ngroups; ++oi) {
  const int64_t lo = tl.n[oi] * xcd / 8, cnt = tl.n[oi] * (xcd + 1) / 8 - lo;
  const int gi = tl.group[oi];
  const MatGroup& g = bt.g[gi];
  const int tiles = tl.tiles[oi];
  for (; l < base + cnt; l += nbx) {
  const int64_t local = lo + (l - base);
  const int64_t m = local / tiles;
  const int tile = int(local - m * tiles);
  // the previous tile's epilogue has finished reading LDS
  if (!first_tile) block_barrier();
  first_tile = false;
  int ti, tj;
  if (MODE == MODE_UPDATE) {
    const int ntn = g.q_pad / BN;
    ti = tile / ntn;
    tj = tile - ti * ntn;
  } else {
    tri_decode(tile, ti, tj);
  }
  const int i0 = ti * BM, j0 = tj * BN;
  const int64_t qp = g.q_pad, pp = g.p_pad;

  const uint16_t* Xin = reinterpret_cast<const uint16_t*>((iter & 1) ? g.X1 : g.X0) + m * g.x_stride;
  uint16_t* Xout = reinterpret_cast<uint16_t*>((iter & 1) ? g.X0 : g.X1) + m * g.x_stride;
  uint16_t* Am = reinterpret_cast<uint16_t*>(g.A) + m * g.a_stride;
  uint16_t* Bm = reinterpret_cast<uint16_t*>(g.B) + m * g.a_stride;

  const uint16_t* Pa;
  const uint16_t* Pb;
  int64_t lda, ldb;
  int K;
  if (MODE == MODE_GRAM) {
    Pa = Xin + i0 * qp;
    Pb = Xin + j0 * qp;
    lda = ldb = qp;
    // X's padding columns (q .. q_pad) hold zeros: the contraction stops at
    // the first K step boundary past q (and past p below, for A and B,
    // whose padding rows and columns are zero as well)
    K = (g.q + BK - 1) / BK * BK;
  } else if (MODE == MODE_POLY) {
    Pa = Am + i0 * pp;
    Pb = Am + j0 * pp;
    lda = ldb = pp;
    K = (g.p + BK - 1) / BK * BK;
  } else {
    // B is stored in panels of 32 columns ([p/32][p][32]): the 128 rows of
    // one K step are 8 contiguous KiB, loaded as whole cache lines
    Pa = Bm + i0 * kPanel;
    lda = kPanel;
    Pb = Xin + j0;
    ldb = qp;
    K = (g.p + BK - 1) / BK * BK;
  }
  const int nk = K / BK;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  static_assert(C::WGM * C::WGN == C::NW && BM % 64 == 0, "wave grid; 64-row epilogue passes");
  // 32x32 accumulator blocks of a wave: tile row block rblk(mi), column
  // block cblk(ni).  The 256x256 symmetric tiles (8 x 8 blocks, waves of 4
  // row blocks by 2 column blocks) take rows {0,1,5,6} (wm 0) or {2,3,4,7}
  // (wm 1) and columns {wn, 7-wn}: on a diagonal tile, whose 28 blocks
  // above the diagonal are not computed (their values are the transposes of
  // the blocks below it), every wave of the first group then has 4 blocks
  // to compute and every wave of the second 5, against 8 for the
  // consecutive rows and columns of the other tiles (where the two
  // assignments do the same work).
  constexpr bool kBal = MODE != MODE_UPDATE && C::NW == 8 && C::WGM == 2 && C::WGN == 4 &&
                        WM == 4 && WN == 2;
  auto rblk = [&](int mi) -> int {
    if constexpr (kBal) return mi < 2 ? 2 * wm + mi : (mi == 2 ? 5 - wm : 6 + wm);
    else return wm * WM + mi;
  };
  auto cblk = [&](int ni) -> int {
    if constexpr (kBal) return ni == 0 ? wn : 7 - wn;
    else return wn * WN + ni;
  };
  // Blocks (mi, ni) of this wave strictly above a diagonal tile's diagonal
  // (bit mi * WN + ni): not computed there.
  uint32_t upper = 0;
  if constexpr (kBal) {
#pragma unroll
    for (int mi = 0; mi < WM; ++mi)
#pragma unroll
      for (int ni = 0; ni < WN; ++ni)
        if (rblk(mi) < cblk(ni)) upper |= 1u << (mi * WN + ni);
  }
  const uint32_t smem_base = uint32_t(reinterpret_cast<uintptr_t>(smem));

  // LDS holds the A tiles of all stages, then the B tiles (stage s of A at
  // s*A_BYTES, of B at S*A_BYTES + s*B_BYTES), so that a lane's address in
  // any stage is its stage-0 address plus a small compile-time immediate.
  // DMA sources are a 64-bit scalar base per operand, advanced by one K step
  // per step, plus a per-lane 32-bit byte offset fixed for the whole tile:
  // no per-step vector address arithmetic.
  uint32_t offA[A_INSTR], offB[B_INSTR];
#pragma unroll
  for (int i = 0; i < A_INSTR; ++i) {
    // one instruction: 64/CPK rows of CPK 16-byte chunks (whole rows)
    const int row = (wave * A_INSTR + i) * (64 / CPK) + lane / CPK;
    const int c = (lane % CPK) ^ rswz<CPK>(row);
    offA[i] = uint32_t((int64_t(row) * lda + c * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < B_INSTR; ++i) {
    if (MODE == MODE_UPDATE) {
      // K-rows of 2 BN bytes; lane L takes K-row kr0 + L/(BN/8), chunk L%(BN/8)
      constexpr int CPR = BN / 8;
      const int k = (wave * B_INSTR + i) * (WAVE_BYTES / (BN * 2)) + lane / CPR;
      const int c = (lane % CPR) ^ gswz(k);
      offB[i] = uint32_t((int64_t(k) * ldb + c * 8) * 2);
    } else {
      const int row = (wave * B_INSTR + i) * (64 / CPK) + lane / CPK;
      const int c = (lane % CPK) ^ rswz<CPK>(row);
      offB[i] = uint32_t((int64_t(row) * ldb + c * 8) * 2);
    }
  }
  const char* gA = reinterpret_cast<const char*>(Pa);
  const char* gB = reinterpret_cast<const char*>(Pb);
  const int64_t stepA = MODE == MODE_UPDATE ? pp * kPanel * 2 : BK * 2;
  const int64_t stepB = MODE == MODE_UPDATE ? int64_t(BK) * ldb * 2 : int64_t(BK) * 2;

  // Issue the loads of K step `kt` into stage buffer J (= kt % S).  Each wave
  // moves A_INSTR + B_INSTR KiB-sized pieces.  A diagonal tile of a
  // symmetric product (D: both operands are the same rows) loads only A and
  // reads its B fragments from the A buffers.
  auto issue = [&](auto bufc, auto diagc, int kt) {
    constexpr int J = decltype(bufc)::value;
    constexpr bool D = decltype(diagc)::value;
    const char* a = gA + kt * stepA;
    const char* b = gB + kt * stepB;
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i)
      dma16(offA[i], a, smem_base + uint32_t(J * A_BYTES + (wave * A_INSTR + i) * WAVE_BYTES));
    if constexpr (!D) {
#pragma unroll
      for (int i = 0; i < B_INSTR; ++i)
        dma16(offB[i], b,
              smem_base + uint32_t(S * A_BYTES + J * B_BYTES + (wave * B_INSTR + i) * WAVE_BYTES));
    }
  };

  f32x16_t acc[WM][WN];
#pragma unroll
  for (int mi = 0; mi < WM; ++mi)
#pragma unroll
    for (int ni = 0; ni < WN; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  // The 128x128 polynomial takes its linear term b*A from the K loop: the
  // tile's columns j0 .. j0+127 are K columns of its own operand rows
  // i0 .., and a wave's 64 columns are exactly K step klin, so during that
  // step each lane reads from the A stage the 4 consecutive elements of A
  // at each group of 4 accumulator registers (one 8-byte LDS read each).
  // No A tile is read again from memory in the epilogue.
  constexpr bool kLinK = MODE == MODE_POLY && C::NW == 4 && BM == BN && BK == 32 * WN;
  u32x2_t linr[kLinK ? WM : 1][kLinK ? WN : 1][4];
  const int klin = kLinK ? (j0 + wn * 32 * WN) / BK : -1;
  if constexpr (kLinK) {
#pragma unroll
    for (int mi = 0; mi < WM; ++mi)
#pragma unroll
      for (int ni = 0; ni < WN; ++ni)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) linr[mi][ni][g4] = u32x2_t{0u, 0u};  // K step past p: zeros
  }
  auto read_lin = [&](auto bufc) {
    if constexpr (kLinK) {
      constexpr int J = decltype(bufc)::value;
      const LDS_AS char* sA = smem + J * A_BYTES;
#pragma unroll
      for (int mi = 0; mi < WM; ++mi) {
        const int row = rblk(mi) * 32 + (lane & 31);
#pragma unroll
        for (int ni = 0; ni < WN; ++ni)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int kc = ni * 32 + 8 * g4 + 4 * (lane >> 5);  // K column in the step
            linr[mi][ni][g4] = *reinterpret_cast<const LDS_AS u32x2_t*>(
                sA + row * (BK * 2) + (((kc >> 3) ^ rswz<CPK>(row)) << 4) + (kc & 7) * 2);
          }
      }
    }
  };

  // Fragments of one 16-deep K sub-step of stage buffer J.
  auto load_frags = [&](auto bufc, auto diagc, int ks, bf16x8_t (&af)[WM], bf16x8_t (&bfr)[WN]) {
    constexpr int J = decltype(bufc)::value;
    const LDS_AS char* sA = smem + J * A_BYTES;
    const LDS_AS char* sB = decltype(diagc)::value ? sA : smem + S * A_BYTES + J * B_BYTES;
    const int ch = ks * 2 + (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < WM; ++mi)
      af[mi] = lds_frag_rows<BK>(sA, rblk(mi) * 32 + (lane & 31), ch);
#pragma unroll
    for (int ni = 0; ni < WN; ++ni) {
      if (MODE == MODE_UPDATE)
        bfr[ni] = lds_frag_xT<BN>(sB, ks * 16, wn * 32 * WN + ni * 32, lane);
      else
        bfr[ni] = lds_frag_rows<BK>(sB, cblk(ni) * 32 + (lane & 31), ch);
    }
  };
  // The B fragment goes in the MFMA's first operand slot: the accumulator
  // then holds the tile transposed, so that lane l, register 4g + jj is row
  // l%32, column 8g + 4(l/32) + jj of its 32x32 block: 4 consecutive columns
  // of one row per 4 registers (16-byte LDS writes in the epilogue).
  // On a diagonal tile (dgc) of the balanced layout the blocks above the
  // diagonal are skipped (a wave-uniform branch).
  auto mfmas = [&](auto dgc, const bf16x8_t (&af)[WM], const bf16x8_t (&bfr)[WN]) {
#pragma unroll
    for (int mi = 0; mi < WM; ++mi)
#pragma unroll
      for (int ni = 0; ni < WN; ++ni) {
        if constexpr (kBal && decltype(dgc)::value)
          if ((upper >> (mi * WN + ni)) & 1u) continue;
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
      }
  };
  // Waits until the loads of `stage` are done, given that the last stage
  // issued so far is `issued` (capped at nk-1): exactly the loads of the
  // stages issued after `stage` may stay in flight (vmcnt counts in order).
  auto wait_stage = [&](auto diagc, int stage, int issued) {
    constexpr int L = decltype(diagc)::value ? A_INSTR : LOADS;  // loads per stage
    const int younger = (issued < nk - 1 ? issued : nk - 1) - stage;
    if (S > 3 && younger >= 3)
      wait_vmcnt<(S > 3 ? 3 : 0) * L>();
    else if (younger == 2)
      wait_vmcnt<2 * L>();
    else if (younger == 1)
      wait_vmcnt<L>();
    else
      wait_vmcnt<0>();
  };
  static_assert(S >= 2 && S <= 4, "wait_stage covers at most 3 younger stages");

  // Software pipeline over K steps (KS 16-deep sub-steps each): the LDS
  // reads of the next sub-step are always in flight while the MFMAs of the
  // current one issue.  One barrier per K step, before its last sub-step's
  // MFMAs: all reads of step kt are complete there (lgkmcnt 0), so its buffer
  // is refilled with step kt+S right after it, and step kt+1 (waited for by
  // every wave) becomes readable.  The loop is unrolled by S so that every
  // stage buffer index is a compile-time constant.
  bf16x8_t a0[WM], b0[WN], a1[WM], b1[WN];
  auto kloop = [&](auto dg) {
  if constexpr (C::NW == 8 && KS == 2) {
  // Eight waves, two per SIMD: the waves 0-3 and 4-7 run half a K step
  // apart, so that on every SIMD one wave issues its MFMAs while the other
  // reads its next fragments from LDS and issues its loads.  Each K step is
  // a memory phase (fragments of both 16-deep sub-steps, the loads of step
  // kt+S-1 into the buffer step kt-1 used) and a compute phase (all MFMAs of
  // the step), each closed by a barrier; the second group enters the loop
  // one barrier late and the first leaves it one barrier late, so both pass
  // the same barriers.  Between consecutive barriers one group reads and
  // loads while the other multiplies.  Step kt+1 is complete before the
  // barrier after which the first group reads it: each wave waits for its
  // own loads of it at the end of its phase before that barrier.
  const bool late = wave >= 4;
  issue(std::integral_constant<int, 0>{}, dg, 0);
  if constexpr (S > 2) if (1 < nk) issue(std::integral_constant<int, 1>{}, dg, 1);
  if constexpr (S > 3) if (2 < nk) issue(std::integral_constant<int, (S > 3 ? 2 : 0)>{}, dg, 2);
  wait_stage(dg, 0, S - 2);  // the prologue issued steps 0 .. S-2
  block_barrier();
  if (late) block_barrier();
  static_assert(KS == 2, "the ping-pong loop holds the fragments of one 32-deep K step");
  auto pp = [&](auto bufc, int kt) {
    constexpr int J = decltype(bufc)::value;
    load_frags(bufc, dg, 0, a0, b0);
    load_frags(bufc, dg, 1, a1, b1);
    if (kt + S - 1 < nk) issue(std::integral_constant<int, (J + S - 1) % S>{}, dg, kt + S - 1);
    if (late && kt + 1 < nk) wait_stage(dg, kt + 1, kt + S - 1);
    block_barrier();
    mfmas(dg, a0, b0);
    mfmas(dg, a1, b1);
    if (!late && kt + 1 < nk) wait_stage(dg, kt + 1, kt + S - 1);
    block_barrier();
  };
  for (int kt = 0; kt < nk; kt += S) {
    pp(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 < nk) pp(std::integral_constant<int, 1>{}, kt + 1);
    if constexpr (S > 2) if (kt + 2 < nk) pp(std::integral_constant<int, (S > 2 ? 2 : 0)>{}, kt + 2);
    if constexpr (S > 3) if (kt + 3 < nk) pp(std::integral_constant<int, (S > 3 ? 3 : 0)>{}, kt + 3);
  }
  if (!late) block_barrier();
  } else {
  issue(std::integral_constant<int, 0>{}, dg, 0);
  if (1 < nk) issue(std::integral_constant<int, 1>{}, dg, 1);
  if constexpr (S > 2) if (2 < nk) issue(std::integral_constant<int, (S > 2 ? 2 : 0)>{}, dg, 2);
  if constexpr (S > 3) if (3 < nk) issue(std::integral_constant<int, (S > 3 ? 3 : 0)>{}, dg, 3);
  wait_stage(dg, 0, S - 1);  // the prologue issued steps 0 .. S-1
  block_barrier();
  load_frags(std::integral_constant<int, 0>{}, dg, 0, a0, b0);
  auto step = [&](auto bufc, int kt) {
    constexpr int J = decltype(bufc)::value;
    if (kLinK && kt == klin) read_lin(bufc);
    load_frags(bufc, dg, 1, a1, b1);
    mfmas(dg, a0, b0);
    if constexpr (KS == 4) {
      load_frags(bufc, dg, 2, a0, b0);
      mfmas(dg, a1, b1);
      load_frags(bufc, dg, 3, a1, b1);
      mfmas(dg, a0, b0);
    }
    if (kt + 1 < nk) {
      wait_stage(dg, kt + 1, kt + S - 1);  // steps up to kt+S-1 issued so far
      block_barrier();
      if (kt + S < nk) issue(bufc, dg, kt + S);
      load_frags(std::integral_constant<int, (J + 1) % S>{}, dg, 0, a0, b0);
    }
    mfmas(dg, a1, b1);
  };
  for (int kt = 0; kt < nk; kt += S) {
    step(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 < nk) step(std::integral_constant<int, 1>{}, kt + 1);
    if constexpr (S > 2) if (kt + 2 < nk) step(std::integral_constant<int, (S > 2 ? 2 : 0)>{}, kt + 2);
    if constexpr (S > 3) if (kt + 3 < nk) step(std::integral_constant<int, (S > 3 ? 3 : 0)>{}, kt + 3);
  }
  }
  };
  if constexpr (MODE != MODE_UPDATE) {
    if (ti == tj)
      kloop(std::true_type{});
    else
      kloop(std::false_type{});
  } else {
    kloop(std::false_type{});
  }

  // ---- Epilogue: the final fp32 tile is staged through LDS in two passes
  // of 64 rows and stored as 16-byte vectors of 8 bf16.  The mirrored half
  // of an off-diagonal symmetric tile is written from the same staged
  // values read column-wise, so both halves hold identical bits.
  const float* sc = g.scal + m * kScal;
  float alpha = 1.f;
  if (MODE == MODE_GRAM) {
    const float inv = iter == 0 ? sc[SC_INV] : 1.f;
    alpha = inv * inv;
  } else if (MODE == MODE_UPDATE) {
    alpha = iter == 0 ? sc[SC_INV] : 1.f;
  }
  const bool mirror = (MODE != MODE_UPDATE) && (ti != tj);
  // A diagonal tile of the balanced layout computed only the blocks on and
  // below the diagonal: the direct pass writes those, the mirrored pass the
  // transposes of the blocks strictly below it.  (Chunks of 8 columns, or 8
  // rows, never straddle a 32x32 block.)
  const bool dtri = kBal && ti == tj;
  // Final values in fp32, before one rounding: Gram alpha*(X X^T),
  // polynomial c*(A A) + b*A + a*I, update alpha*(B X).
#pragma unroll
  for (int mi = 0; mi < WM; ++mi)
#pragma unroll
    for (int ni = 0; ni < WN; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[mi][ni][r] *= (MODE == MODE_POLY ? cc : alpha);
        if constexpr (kLinK) {
          const u32x2_t w = linr[mi][ni][r >> 2];
          const uint32_t h = (r & 2) ? w[1] : w[0];
          const float a = __uint_as_float((r & 1) ? (h & 0xffff0000u) : (h << 16));
          acc[mi][ni][r] = fmaf(cb, a, acc[mi][ni][r]);
        }
      }
  // fp32 staging row pitch (floats): 4 mod 64 banks, so the 16-byte writes of
  // 16 lanes (16 consecutive rows, one column) cover all banks once.  Passes
  // of PR rows: 64, or 128 for the 512-row tiles (the same bytes per pass).
  constexpr int TP = BN + 4;
  constexpr int PR = BM == 512 ? 128 : 64;
  static_assert(PR * TP * 4 <= S * STAGE_BYTES, "staging");
  LDS_AS float* T = (LDS_AS float*)smem;
  auto tix = [](int r, int c) { return r * TP + c; };   // staging element (r, c)
  constexpr int CPR = BN / 8;                // 8-element chunks per row
  constexpr int CHUNKS = PR * CPR / NT;      // per thread per pass
  uint16_t* Cout = MODE == MODE_UPDATE ? Xout : (MODE == MODE_GRAM ? Am : Bm);
  const int64_t ldc = MODE == MODE_UPDATE ? qp : pp;
  // Output element (r, c): row-major, except the polynomial's B, which the
  // update reads in panels of 32 columns (8 aligned columns stay contiguous).
  auto out_at = [&](int64_t r, int64_t c) -> uint16_t* {
    if constexpr (MODE == MODE_POLY)
      return Cout + (c / kPanel) * (pp * kPanel) + r * kPanel + (c % kPanel);
    else
      return Cout + r * ldc + c;
  };


  // Pass `pass` stages tile rows PR pass .. +PR-1: the 32-row accumulator
  // blocks wm*WM + mi with (wm*WM + mi) / (PR/32) == pass.
  auto stage = [&](int pass) {
#pragma unroll
    for (int mi = 0; mi < WM; ++mi) {
      const int blk = rblk(mi);
      if (blk / (PR / 32) != pass) continue;
      const int row = (blk % (PR / 32)) * 32 + (lane & 31);
#pragma unroll
      for (int ni = 0; ni < WN; ++ni)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int col = cblk(ni) * 32 + 8 * g4 + 4 * (lane >> 5);
          *(LDS_AS f32x4_t*)(T + tix(row, col)) =
              f32x4_t{acc[mi][ni][4 * g4], acc[mi][ni][4 * g4 + 1], acc[mi][ni][4 * g4 + 2],
                      acc[mi][ni][4 * g4 + 3]};
        }
    }
  };
  // Mirrored blocks of symmetric tiles: the pass's accumulators are staged a
  // second time, transposed (Tt[c][r], c < BN tile columns, r < 64 rows of
  // the pass), so that the mirrored rows are read as 16-byte vectors and
  // written as whole 128-byte row runs.  Row pitch 68: the 16-byte reads of
  // 8 lanes per row over two rows hit distinct banks.
  // (The 8-wave 256x256 tiles read the mirrored block by columns from the
  // normal staging instead: the second staging costs them more than the
  // scattered stores; lanes then take consecutive c, so the column reads
  // hit distinct banks.)
  constexpr bool kStageT = C::NW == 4;
  constexpr int TPT = 68;
  static_assert(MODE == MODE_UPDATE || BN * TPT * 4 <= S * STAGE_BYTES, "transposed staging");
  static_assert(MODE == MODE_UPDATE || PR == 64, "symmetric tiles stage 64-row passes");
  // Mirrored chunk q: tile column c (a row of the mirrored block), rows
  // r8 .. r8+7 of the pass.
  auto mirror_pos = [&](int q, int& c, int& r8) {
    if constexpr (kStageT) {
      c = q >> 3;
      r8 = (q & 7) * 8;
    } else {
      c = q % BN;
      r8 = (q / BN) * 8;
    }
  };
  auto stage_t = [&](int pass) {
#pragma unroll
    for (int mi = 0; mi < WM; ++mi) {
      const int blk = rblk(mi);
      if ((blk >> 1) != pass) continue;
      const int row = (blk & 1) * 32 + (lane & 31);
#pragma unroll
      for (int ni = 0; ni < WN; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int col = cblk(ni) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          T[col * TPT + row] = acc[mi][ni][r];
        }
    }
  };
  auto pack8 = [](const float (&v)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = f2bf2(v[2 * e], v[2 * e + 1]);
    return make_uint4(w[0], w[1], w[2], w[3]);
  };
  // The 256x256 polynomial's linear term b*A at the output positions, read
  // as 16-byte rows of A in the epilogue.  A is symmetric, so a mirrored
  // chunk's term is again a row segment of A.
  constexpr bool kLin = MODE == MODE_POLY && !kLinK;
  constexpr int MCH = BN * (PR / 8) / NT;    // mirrored chunks per thread per pass
  const uint16_t* Lin = Am;
  const float lin_coef = cb;
  auto add_lin = [&](float (&v)[8], const uint4& x) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = fmaf(lin_coef, __uint_as_float(w[e] << 16), v[2 * e]);
      v[2 * e + 1] = fmaf(lin_coef, __uint_as_float(w[e] & 0xffff0000u), v[2 * e + 1]);
    }
  };
  // Loads of the linear term for one pass, issued before the pass's LDS
  // staging and barriers so that their latency overlaps them.
  auto load_lin = [&](int pass, uint4 (&lin)[kLin ? CHUNKS : 1], uint4 (&lin_m)[kLin ? MCH : 1]) {
    if (kLin) {
#pragma unroll
      for (int u = 0; u < CHUNKS; ++u) {
        const int q = t + NT * u;
        const int row = q / CPR, col = (q % CPR) * 8;
        lin[u] = *reinterpret_cast<const uint4*>(Lin + (i0 + PR * pass + row) * ldc + j0 + col);
      }
      if (mirror || dtri) {
#pragma unroll
        for (int u = 0; u < MCH; ++u) {
          int c, r8;
          mirror_pos(t + NT * u, c, r8);
          lin_m[u] = *reinterpret_cast<const uint4*>(Lin + (j0 + c) * ldc + i0 + PR * pass + r8);
        }
      }
    }
  };
  auto finish = [&](int pass, const uint4 (&lin)[kLin ? CHUNKS : 1],
                    const uint4 (&lin_m)[kLin ? MCH : 1]) {
#pragma unroll
    for (int u = 0; u < CHUNKS; ++u) {
      const int q = t + NT * u;
      const int row = q / CPR, col = (q % CPR) * 8;
      if (dtri && (PR * pass + row) / 32 < col / 32) continue;
      float v[8];
      const f32x4_t v0 = *(const LDS_AS f32x4_t*)(T + tix(row, col));
      const f32x4_t v1 = *(const LDS_AS f32x4_t*)(T + tix(row, col + 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = v0[e];
        v[e + 4] = v1[e];
      }
      if (kLin) add_lin(v, lin[u]);
      if constexpr (MODE == MODE_UPDATE)
        store_nt16(out_at(i0 + PR * pass + row, j0 + col), pack8(v));
      else
        *reinterpret_cast<uint4*>(out_at(i0 + PR * pass + row, j0 + col)) = pack8(v);
    }
  };
  // Mirrored block: rows j0 + c of C (c < BN), columns i0 + 64*pass + r8 ..
  // +7, from the transposed staging; 8 consecutive lanes cover the 64
  // columns of one row (a whole 128-byte line per row and instruction).
  auto finish_mirror = [&](int pass, const uint4 (&lin_m)[kLin ? MCH : 1]) {
#pragma unroll
    for (int u = 0; u < MCH; ++u) {
      int c, r8;
      mirror_pos(t + NT * u, c, r8);
      if (dtri && (PR * pass + r8) / 32 <= c / 32) continue;
      float v[8];
      if constexpr (kStageT) {
        const f32x4_t v0 = *(const LDS_AS f32x4_t*)(T + c * TPT + r8);
        const f32x4_t v1 = *(const LDS_AS f32x4_t*)(T + c * TPT + r8 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = v0[e];
          v[e + 4] = v1[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = T[tix(r8 + e, c)];
      }
      if (kLin) add_lin(v, lin_m[u]);
      *reinterpret_cast<uint4*>(out_at(j0 + c, i0 + PR * pass + r8)) = pack8(v);
    }
  };

  // Fused tail (last iteration, plain Muon): W' = decay W - step O with O
  // this tile's final fp32 values, which are never stored.  O is the tile in
  // short-side-first orientation: O[i][j] is W[i][j], or W[j][i] for a tall
  // W (trans).  The host enables it only for bf16 weights whose column count
  // is a multiple of 8, so every 8-element chunk along W's rows is entirely
  // inside or outside the matrix.
  const bool fuse = MODE == MODE_UPDATE && LAST == kLastApply && g.fuse;
  // Fused reduction (last iteration of MuonGS, MuonH, or any step with
  // statistics): O is stored as usual, and the tile's partial sums of
  // <W,O>, ||W||^2 and ||O||^2 over the stored bf16 O (what the apply pass
  // reads) are written to the tail partials, so that no separate pass reads
  // W and O again before the per-matrix totals.
  const bool fred = MODE == MODE_UPDATE && LAST == kLastReduce && g.red;
  float red_dot = 0.f, red_ww = 0.f, red_oo = 0.f;
  // W' = decay W + (-step) O for one 8-element chunk of W at wp (16-byte
  // access when W is 16-byte aligned, element by element otherwise).
  auto w_update = [&](uint16_t* wp, bool wvec, const float (&o)[8]) {
    const float dec = g.decay, stp = g.step;
    float v[8];
    if (wvec) {
      const uint4 w = *reinterpret_cast<const uint4*>(wp);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = fmaf(dec, __uint_as_float(ww[e] << 16), -stp * o[2 * e]);
        v[2 * e + 1] = fmaf(dec, __uint_as_float(ww[e] & 0xffff0000u), -stp * o[2 * e + 1]);
      }
      *reinterpret_cast<uint4*>(wp) = pack8(v);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) wp[e] = f2bf(fmaf(dec, bf2f(wp[e]), -stp * o[e]));
    }
  };
  // W' chunk from a W chunk loaded beforehand.
  auto w_apply = [&](const uint4& w, const float (&o)[8]) {
    const float dec = g.decay, stp = g.step;
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = fmaf(dec, __uint_as_float(ww[e] << 16), -stp * o[2 * e]);
      v[2 * e + 1] = fmaf(dec, __uint_as_float(ww[e] & 0xffff0000u), -stp * o[2 * e + 1]);
    }
    return pack8(v);
  };
  // Adds one 8-element chunk's terms: o holds the fp32 values, which are
  // rounded to bf16 first (the stored O), w the W chunk.
  auto red_add = [&](const float (&o)[8], const uint4& w) {
    const uint32_t ww4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float o0 = bf2f(f2bf(o[2 * e])), o1 = bf2f(f2bf(o[2 * e + 1]));
      const float w0 = __uint_as_float(ww4[e] << 16), w1 = __uint_as_float(ww4[e] & 0xffff0000u);
      red_dot = fmaf(w0, o0, fmaf(w1, o1, red_dot));
      red_ww = fmaf(w0, w0, fmaf(w1, w1, red_ww));
      red_oo = fmaf(o0, o0, fmaf(o1, o1, red_oo));
    }
  };
  // W chunk of 8 elements at wp: one 16-byte load when W is 16-byte aligned.
  auto w_chunk = [&](const uint16_t* wp, bool wvec) {
    if (wvec) return *reinterpret_cast<const uint4*>(wp);
    uint32_t ww4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) ww4[e] = uint32_t(wp[2 * e]) | (uint32_t(wp[2 * e + 1]) << 16);
    return make_uint4(ww4[0], ww4[1], ww4[2], ww4[3]);
  };
  // The fused reduction's pass: O stored by rows (as finish does), the terms
  // taken by rows for a wide W (W[i][j] = O[i][j]) and by staged columns for
  // a tall one (W[j][i] = O[i][j]: 8 lanes per W row, as in finish_tail).
  // The host enables it for row lengths that are multiples of 8 only, so
  // every chunk along a W row is entirely inside or outside the matrix.
  auto finish_red = [&](int pass) {
    const uint16_t* Wm = mat_cptr<uint16_t>(reinterpret_cast<const void* const*>(g.W_tab), g.W, m,
                                            int64_t(g.rows) * g.cols);
    const int64_t wld = g.cols;
    const bool wvec = (reinterpret_cast<uintptr_t>(Wm) & 15) == 0;
    // all of the pass's W loads are issued together (groups of them made the
    // register allocation of the 4-wave update spill: 56 to 244 bytes per
    // lane, none this way)
    constexpr int RG = CHUNKS;
    static_assert(CHUNKS % RG == 0, "chunk groups");
#pragma unroll
    for (int u0 = 0; u0 < CHUNKS; u0 += RG) {
      uint4 wv[RG];
      if (!g.trans) {
#pragma unroll
        for (int u = 0; u < RG; ++u) {
          const int q = t + NT * (u0 + u);
          const int row = q / CPR, col = (q % CPR) * 8;
          const int i = i0 + PR * pass + row, j = j0 + col;
          wv[u] = make_uint4(0, 0, 0, 0);
          if (i < g.p && j < g.q) wv[u] = w_chunk(Wm + int64_t(i) * wld + j, wvec);
        }
      }
#pragma unroll
      for (int u = 0; u < RG; ++u) {
        const int q = t + NT * (u0 + u);
        const int row = q / CPR, col = (q % CPR) * 8;
        float v[8];
        const f32x4_t v0 = *(const LDS_AS f32x4_t*)(T + tix(row, col));
        const f32x4_t v1 = *(const LDS_AS f32x4_t*)(T + tix(row, col + 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = v0[e];
          v[e + 4] = v1[e];
        }
        *reinterpret_cast<uint4*>(out_at(i0 + PR * pass + row, j0 + col)) = pack8(v);
        // padding rows and columns of O are zero: nothing to add there
        if (!g.trans) red_add(v, wv[u]);
      }
    }
    if (g.trans) {
      constexpr int MC = BN * (PR / 8) / NT;
      constexpr int MRG = MC;
      static_assert(MC % MRG == 0, "mirrored chunk groups");
#pragma unroll
      for (int u0 = 0; u0 < MC; u0 += MRG) {
        uint4 wt[MRG];
#pragma unroll
        for (int u = 0; u < MRG; ++u) {
          const int q = t + NT * (u0 + u);
          const int c = (q >> 3) % BN, r8 = ((q & 7) + 8 * (q / (8 * BN))) * 8;
          const int i = i0 + PR * pass + r8, j = j0 + c;
          wt[u] = make_uint4(0, 0, 0, 0);
          if (j < g.q && i < g.p) wt[u] = w_chunk(Wm + int64_t(j) * wld + i, wvec);
        }
#pragma unroll
        for (int u = 0; u < MRG; ++u) {
          const int q = t + NT * (u0 + u);
          const int c = (q >> 3) % BN, r8 = ((q & 7) + 8 * (q / (8 * BN))) * 8;
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = T[tix(r8 + e, c)];
          red_add(v, wt[u]);
        }
      }
    }
  };
  auto finish_tail = [&](int pass) {
    uint16_t* Wm = mat_ptr<uint16_t>(g.W_tab, g.W, m, int64_t(g.rows) * g.cols);
    const int64_t wld = g.cols;
    const bool wvec = (reinterpret_cast<uintptr_t>(Wm) & 15) == 0;
    // All 16-byte W chunks of a group are loaded before the group's first W'
    // store (which the compiler may not move loads across), so that their
    // latencies overlap: by rows for a wide W, by columns for a tall one.
    // The 8-wave tiles take the pass in one group; the 4-wave update, which
    // has fewer registers to spare, in groups of GS chunks.
    constexpr int GS = (C::NW == 8 || CHUNKS < MUON_TAIL_GS) ? CHUNKS : MUON_TAIL_GS;
    static_assert(CHUNKS % GS == 0, "chunk groups");
    // (a tall W reads the staged tile by columns below; nothing to do by rows)
    if (!g.trans)
#pragma unroll
    for (int u0 = 0; u0 < CHUNKS; u0 += GS) {
      uint4 wv[GS];
#pragma unroll
      for (int u = 0; u < GS; ++u) {
        const int q = t + NT * (u0 + u);
        const int row = q / CPR, col = (q % CPR) * 8;
        const int i = i0 + PR * pass + row, j = j0 + col;
        wv[u] = make_uint4(0, 0, 0, 0);
        if (!g.trans && wvec && i < g.p && j < g.q)
          wv[u] = *reinterpret_cast<const uint4*>(Wm + int64_t(i) * wld + j);
      }
#pragma unroll
      for (int u = 0; u < GS; ++u) {
        const int q = t + NT * (u0 + u);
        const int row = q / CPR, col = (q % CPR) * 8;
        float v[8];
        const f32x4_t v0 = *(const LDS_AS f32x4_t*)(T + tix(row, col));
        const f32x4_t v1 = *(const LDS_AS f32x4_t*)(T + tix(row, col + 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = v0[e];
          v[e + 4] = v1[e];
        }
        const int i = i0 + PR * pass + row, j = j0 + col;
        if (!g.trans) {
          if (i < g.p && j < g.q) {
            uint16_t* wp = Wm + int64_t(i) * wld + j;
            if (wvec)
              *reinterpret_cast<uint4*>(wp) = w_apply(wv[u], v);
            else
              w_update(wp, false, v);
          }
        }
      }
    }
    if (g.trans) {
      constexpr int MC = BN * (PR / 8) / NT;
      constexpr int MGS = (C::NW == 8 || MC < MUON_TAIL_GS) ? MC : MUON_TAIL_GS;
      static_assert(MC % MGS == 0, "mirrored chunk groups");
      // W row j0 + c, columns i0 + PR pass + r8 .. +7, from staged column c;
      // 8 consecutive lanes take 8 chunks of one row (the pass's first 64
      // columns, then the next 64 when PR = 128), so that every W load and
      // W' store instruction covers 8 whole 128-byte row runs (the
      // column reads of T then meet 4-way bank conflicts; measured faster
      // than one row per lane: GPT-160M last update 221 -> 214 us).  The
      // first group's W loads are issued before the barrier.
      uint4 wt[MGS];
      auto load_wt = [&](int u0) {
#pragma unroll
        for (int u = 0; u < MGS; ++u) {
          const int q = t + NT * (u0 + u);
          const int c = (q >> 3) % BN, r8 = ((q & 7) + 8 * (q / (8 * BN))) * 8;
          const int i = i0 + PR * pass + r8, j = j0 + c;
          wt[u] = make_uint4(0, 0, 0, 0);
          if (wvec && j < g.q && i < g.p) wt[u] = *reinterpret_cast<const uint4*>(Wm + int64_t(j) * wld + i);
        }
      };
      load_wt(0);
      block_barrier();
#pragma unroll
      for (int u0 = 0; u0 < MC; u0 += MGS) {
        if (u0 > 0) load_wt(u0);
#pragma unroll
        for (int u = 0; u < MGS; ++u) {
          const int q = t + NT * (u0 + u);
          const int c = (q >> 3) % BN, r8 = ((q & 7) + 8 * (q / (8 * BN))) * 8;
          const int i = i0 + PR * pass + r8, j = j0 + c;
          if (j >= g.q || i >= g.p) continue;
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = T[tix(r8 + e, c)];
          uint16_t* wp = Wm + int64_t(j) * wld + i;
          if (wvec)
            *reinterpret_cast<uint4*>(wp) = w_apply(wt[u], v);
          else
            w_update(wp, false, v);
        }
      }
    }
  };

  // Plain updates of the 8-wave tiles: each wave stages and stores its own
  // 128x64 accumulators through a private LDS window of 32 rows, so that
  // the epilogue needs one barrier (every wave's last K-step reads are done)
  // and the waves then store independently.  Window pitch 68 floats; in each
  // 8-row round a lane reads row (lane >> 2) & 7, 8-column chunk {lane bits
  // 5, 0, 1}: both the 16-byte writes (accumulator layout) and the reads are
  // conflict-free on gfx950, and each store instruction covers 8 rows of 128
  // bytes.  (MoE-1B update -0.7 % against the shared 128-row passes.)
  constexpr bool kPriv = MODE == MODE_UPDATE && LAST == 0 && C::NW == 8 && WM == 4 && WN == 2;
  if constexpr (kPriv) {
    constexpr int PP = 68;
    static_assert(C::NW * 32 * PP * 4 <= S * STAGE_BYTES, "private windows");
    block_barrier();
    LDS_AS float* Pw = (LDS_AS float*)smem + wave * (32 * PP);
    const int rr = (lane >> 2) & 7;
    const int c8 = (((lane >> 5) & 1) | ((lane & 1) << 1) | (((lane >> 1) & 1) << 2)) * 8;
#pragma unroll
    for (int mi = 0; mi < WM; ++mi) {
#pragma unroll
      for (int ni = 0; ni < WN; ++ni)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *(LDS_AS f32x4_t*)(Pw + (lane & 31) * PP + ni * 32 + 8 * g4 + 4 * (lane >> 5)) =
              f32x4_t{acc[mi][ni][4 * g4], acc[mi][ni][4 * g4 + 1], acc[mi][ni][4 * g4 + 2],
                      acc[mi][ni][4 * g4 + 3]};
      wave_lds_sync();
#pragma unroll
      for (int rnd = 0; rnd < 4; ++rnd) {
        const int row = rnd * 8 + rr;
        const f32x4_t v0 = *(const LDS_AS f32x4_t*)(Pw + row * PP + c8);
        const f32x4_t v1 = *(const LDS_AS f32x4_t*)(Pw + row * PP + c8 + 4);
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = v0[e];
          v[e + 4] = v1[e];
        }
        store_nt16(out_at(i0 + wm * 32 * WM + mi * 32 + row, j0 + wn * 32 * WN + c8), pack8(v));
      }
      wave_lds_sync();  // the window's reads are done before the next block's writes
    }
  } else
#pragma unroll
  for (int pass = 0; pass < BM / PR; ++pass) {
    // The 256x256 polynomial's b*A loads are issued before the pass's
    // staging and barriers: its one block per CU has no other block to hide
    // their latency behind.
    uint4 lin[kLin ? CHUNKS : 1], lin_m[kLin ? MCH : 1];
    constexpr bool kEarlyLin = kLin;
    if (kEarlyLin && !fuse) load_lin(pass, lin, lin_m);
    block_barrier();  // stage buffers (pass 0) / the previous pass's T no longer read
    stage(pass);
    block_barrier();
    if (MODE == MODE_POLY && ti == tj) {
      // a*I on a diagonal tile (i0 == j0): staged row r of this pass holds
      // its diagonal element in column PR pass + r; the padding rows beyond
      // p keep a zero diagonal
      if (t < PR && i0 + PR * pass + t < g.p) T[tix(t, PR * pass + t)] += ca;
      block_barrier();
    }
    if (fuse) {
      finish_tail(pass);
    } else if (fred) {
      finish_red(pass);
    } else {
      if (!kEarlyLin) load_lin(pass, lin, lin_m);
      finish(pass, lin, lin_m);
      if constexpr (MODE != MODE_UPDATE) {
        if (mirror || dtri) {
          if constexpr (kStageT) {
            block_barrier();  // the row reads of T are done
            stage_t(pass);
            block_barrier();
          }
          finish_mirror(pass, lin_m);
        }
      }
    }
  }
  if (fred) {
    // the tile's three sums, in a fixed order and in fp64 beyond the lanes'
    // own: wave shuffles, then the waves' values through LDS
    double rd = red_dot, rw = red_ww, ro = red_oo;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      rd += __shfl_xor(rd, off, 64);
      rw += __shfl_xor(rw, off, 64);
      ro += __shfl_xor(ro, off, 64);
    }
    __shared__ double red_lds[3 * C::NW];
    if (lane == 0) {
      red_lds[wave] = rd;
      red_lds[C::NW + wave] = rw;
      red_lds[2 * C::NW + wave] = ro;
    }
    block_barrier();
    if (t < 3) {
      double sum = 0.0;
#pragma unroll
      for (int w = 0; w < C::NW; ++w) sum += red_lds[t * C::NW + w];
      g.tail_part[(m * g.red_tiles + tile) * 3 + t] = sum;
    }
    red_dot = red_ww = red_oo = 0.f;
  }
  }  // tiles of group oi
  base += cnt;
  }  // groups
}

inline dim3 grid_of(const TileList& tl) { return dim3(unsigned(8 * tl.blocks_per_xcd)); }

}  // namespace

hipError_t launch_gram_bf16(const Batch& bt, const TileList& tl, int iter, bool big, hipStream_t s) {
  if (big)
    hipLaunchKernelGGL((ns_bf16_kernel<MODE_GRAM, CfgSyrkBig>), grid_of(tl), dim3(64 * CfgSyrkBig::NW),
                       0, s, bt, tl, iter, 0.f, 0.f, 0.f);
  else
    hipLaunchKernelGGL((ns_bf16_kernel<MODE_GRAM, Cfg<MODE_GRAM>>), grid_of(tl),
                       dim3(64 * Cfg<MODE_GRAM>::NW), 0, s, bt, tl, iter, 0.f, 0.f, 0.f);
  return hipGetLastError();
}
hipError_t launch_poly_bf16(const Batch& bt, const TileList& tl, float a, float b, float c, bool big,
                            hipStream_t s) {
  if (big)
    hipLaunchKernelGGL((ns_bf16_kernel<MODE_POLY, CfgSyrkBig>), grid_of(tl), dim3(64 * CfgSyrkBig::NW),
                       0, s, bt, tl, 0, a, b, c);
  else
    hipLaunchKernelGGL((ns_bf16_kernel<MODE_POLY, Cfg<MODE_POLY>>), grid_of(tl),
                       dim3(64 * Cfg<MODE_POLY>::NW), 0, s, bt, tl, 0, a, b, c);
  return hipGetLastError();
}
template <class C>
void launch_update_cfg(const Batch& bt, const TileList& tl, int iter, hipStream_t s) {
  if (tl.fuse_tail == kLastApply)
    hipLaunchKernelGGL((ns_bf16_kernel<MODE_UPDATE, C, kLastApply>), grid_of(tl), dim3(64 * C::NW), 0,
                       s, bt, tl, iter, 0.f, 0.f, 0.f);
  else if (tl.fuse_tail == kLastReduce)
    hipLaunchKernelGGL((ns_bf16_kernel<MODE_UPDATE, C, kLastReduce>), grid_of(tl), dim3(64 * C::NW), 0,
                       s, bt, tl, iter, 0.f, 0.f, 0.f);
  else
    hipLaunchKernelGGL((ns_bf16_kernel<MODE_UPDATE, C, 0>), grid_of(tl), dim3(64 * C::NW), 0, s, bt, tl,
                       iter, 0.f, 0.f, 0.f);
}
hipError_t launch_update_bf16(const Batch& bt, const TileList& tl, int iter, int cfg, hipStream_t s) {
  if (cfg == kUpdCfg512)
    launch_update_cfg<CfgUpd512>(bt, tl, iter, s);
  else if (cfg == kUpdCfg256)
    launch_update_cfg<CfgUpdBig>(bt, tl, iter, s);
  else
    launch_update_cfg<Cfg<MODE_UPDATE>>(bt, tl, iter, s);
  return hipGetLastError();
}

}  // namespace muon
