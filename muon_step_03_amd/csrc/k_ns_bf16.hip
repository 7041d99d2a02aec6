// Newton-Schulz products on bf16 matrix cores (gfx950 MFMA 32x32x16 bf16,
// float32 accumulation, float32 epilogues, one round-to-nearest-even per
// stored operand).
//
// One iteration, on X (p x q, short side first):
//   A = X X^T                 symmetric: only lower-triangle block tiles are
//                             computed, each written to both triangles
//   B = b*A + c*A A^T         A is symmetric, so A A = A A^T: the same
//                             symmetric form with K = p and the b*A epilogue
//   X' = a*X + B X            full p x q output
// which is X_k = aX + b(XX^T)X + c(XX^T)^2 X of "[논문 AI 리뷰] MUON IS
// SCALABLE FOR LLM TRAINING TECHNICAL REPORT", section 2, and the three-line
// Newton-Schulz code block of "LLM Pretraining Loss Spike 진단과 처방 ... Muon
// 전환 판단", section "Muon head의 실체는 하이브리드 옵티마이저다".
//
// The first iteration receives the unnormalised U (the head cannot know
// ||U|| while it writes X0): its Gram is scaled by inv^2 and its update by
// inv, inv = 1/(||U||_F + 1e-7), which is the iteration applied to U*inv.
//
// Kernel structure (256 threads = 4 waves in a 2x2 grid):
//  * Block tiles are compile-time (defaults: symmetric products 128x128,
//    64x64 per wave; update 128x256, 64x128 per wave, fewer LDS reads per
//    MFMA).
//  * K steps of 32, staged through LDS by 16-byte direct-to-LDS loads
//    (global_load_lds): STAGES buffers, loads for up to STAGES-1 later steps
//    in flight while step k is multiplied; one barrier per K step, and the
//    MFMA fragments double-buffered in registers.
//  * K-contiguous operand tiles: rows of 32 bf16 (64 B, 4 chunks of 16 B),
//    chunk c of row m stored at c ^ f(m), f(m) = ((m>>1) + (m>>3)) & 3,
//    so the fragment reads (32 consecutive rows, one chunk) do not collide
//    in 32- or 64-bank LDS.  The swizzle is applied by choosing which
//    global chunk each lane fetches (a direct-to-LDS load writes lane L's
//    16 bytes at base + 16 L).
//  * The update's X operand is N-contiguous: its tile is kept as 32 K-rows
//    of BN bf16 (chunk c of row k stored at c ^ g(k), g = {0,6,12,10}[k&3])
//    and MFMA B fragments are read with the transposing LDS read
//    ds_read_b64_tr_b16: within a 16-lane group, output lane i element j
//    comes from source lane 4j + i/4, element i%4, so lane s addresses
//    X[k0 + s/4][n0 + 4 (s%4)] and two reads give 8 consecutive k.
//  * Blocks are renumbered so that consecutive tiles (same matrix) land on
//    the same XCD (hardware dispatches block b to XCD b % 8), keeping one
//    matrix's operands in one XCD's L2.
#include "muon_internal.h"

namespace muon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int BK = 32;
constexpr int WAVE_BYTES = 1024;    // bytes one direct-to-LDS instruction moves

enum { MODE_GRAM = 0, MODE_POLY = 1, MODE_UPDATE = 2 };

template <int MODE>
struct Cfg;
#ifndef MUON_SYRK_STAGES
#define MUON_SYRK_STAGES 4
#endif
#ifndef MUON_UPD_STAGES
#define MUON_UPD_STAGES 3
#endif
#ifndef MUON_SYRK_OCC
#define MUON_SYRK_OCC 2
#endif
#ifndef MUON_UPD_OCC
#define MUON_UPD_OCC 2
#endif
template <>
struct Cfg<MODE_GRAM> {
  static constexpr int BM = kSyrkTile, BN = kSyrkTile, WM = BM / 64, WN = BN / 64;
  static constexpr int STAGES = MUON_SYRK_STAGES;
  static constexpr int OCC = MUON_SYRK_OCC;  // blocks per CU the register budget targets
};
template <>
struct Cfg<MODE_POLY> : Cfg<MODE_GRAM> {};
template <>
struct Cfg<MODE_UPDATE> {
  static constexpr int BM = kUpdTileM, BN = kUpdTileN, WM = BM / 64, WN = BN / 64;
  static constexpr int STAGES = MUON_UPD_STAGES;
  static constexpr int OCC = MUON_UPD_OCC;
};

__device__ __forceinline__ int fswz(int m) { return ((m >> 1) + (m >> 3)) & 3; }
__device__ __forceinline__ int gswz(int k) { return (0xACE0 >> ((k & 3) * 4)) & 15; }  // {0,6,12,10}

// vmcnt-only wait (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 16-byte direct-to-LDS load: lane L's 16 bytes from `src` land at LDS
// address lds_base + 16 L (lds_base wave-uniform, passed in m0).  Written as
// asm so that the compiler does not treat every later LDS read as possibly
// aliasing it (which would make it wait for all loads in flight, prefetches
// included); completion is tracked explicitly with wait_vmcnt before the
// barrier that publishes a K step.  The instruction has no result register.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

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

// Lower-triangle block index t -> (ti, tj), ti >= tj, row-major over ti.
__device__ __forceinline__ void tri_decode(int t, int& ti, int& tj) {
  int i = int((sqrtf(8.f * float(t) + 1.f) - 1.f) * 0.5f);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

// Within one group's block range (padded to a multiple of 8 and starting at a
// multiple of 8), block j runs on XCD j % 8 (hardware round-robin); renumber
// so that XCD x takes the contiguous tile range [x*n/8, (x+1)*n/8): every
// XCD gets the same share of every group, and consecutive tiles (one
// matrix's) share an XCD's L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t j, int64_t npad) {
#ifdef MUON_NO_XCD_REMAP
  return j;
#endif
  return (j & 7) * (npad >> 3) + (j >> 3);
}

// One direct-to-LDS instruction of a K-contiguous tile: 16 rows x 64 bytes.
// Lane L takes row r0 + L/4, physical chunk L%4, i.e. logical chunk
// (L%4) ^ f(row).
__device__ __forceinline__ void dma_rows(const uint16_t* base, int64_t ld, int k0, int r0,
                                         uint32_t tile, int lane) {
  const int row = r0 + (lane >> 2);
  const int c = (lane & 3) ^ fswz(row);
  dma16(base + int64_t(row) * ld + k0 + c * 8, tile + r0 * (BK * 2));
}

// One direct-to-LDS instruction of the update's X tile: 1024/(2 BN) K-rows
// of 2 BN bytes.  Lane L takes K-row kr0 + L/(BN/8), physical chunk L%(BN/8).
template <int BN>
__device__ __forceinline__ void dma_xrows(const uint16_t* base, int64_t ld, int k0, int kr0,
                                          uint32_t tile, int lane) {
  constexpr int CPR = BN / 8;  // 16-byte chunks per row
  const int k = kr0 + lane / CPR;
  const int c = (lane % CPR) ^ gswz(k);
  dma16(base + int64_t(k0 + k) * ld + c * 8, tile + kr0 * (BN * 2));
}

__device__ __forceinline__ bf16x8_t lds_frag_rows(const LDS_AS char* tile, int row, int chunk) {
  return *reinterpret_cast<const LDS_AS bf16x8_t*>(tile + row * (BK * 2) + ((chunk ^ fswz(row)) << 4));
}

// Four consecutive K-rows at one column of the update's X tile, in the
// MFMA accumulator's row pattern: lane l (s = l % 16) gets
// X[kb + 4 (l/32) + j][nb + 16 ((l/16) % 2) + s], j = 0..3 (one transposing
// read; source lane s addresses X[k + s/4][n + 4 (s%4)]).
template <int BN>
__device__ __forceinline__ i16x4_t lds_rows4_xT(const LDS_AS char* tile, int kb, int nb, int lane) {
  const int s = lane & 15;
  const int n = nb + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
  const int k = kb + 4 * (lane >> 5) + (s >> 2);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (LDS_AS i16x4_t*)(tile + k * (BN * 2) + (((n >> 3) ^ gswz(k)) << 4) + (n & 7) * 2));
}

// Four consecutive K values (kb + 4 (l/32) .. +3) of row `row` of a
// K-contiguous tile: one 8-byte read.
__device__ __forceinline__ i16x4_t lds_k4_rows(const LDS_AS char* tile, int row, int kb, int lane) {
  const int k = kb + 4 * (lane >> 5);
  return *(const LDS_AS i16x4_t*)(tile + row * (BK * 2) + (((k >> 3) ^ fswz(row)) << 4) + (k & 7) * 2);
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

template <int MODE>
__global__ __launch_bounds__(256, Cfg<MODE>::OCC) void ns_bf16_kernel(Batch bt, Work wk, int iter,
                                                                     float c1, float c2) {
  using C = Cfg<MODE>;
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN, S = C::STAGES;
  constexpr int A_BYTES = BM * BK * 2;
  constexpr int B_BYTES = BN * BK * 2;
  constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  constexpr int A_INSTR = A_BYTES / WAVE_BYTES / 4;  // per wave
  constexpr int B_INSTR = B_BYTES / WAVE_BYTES / 4;
  constexpr int LOADS = A_INSTR + B_INSTR;          // vmcnt per stage per wave
  static_assert(A_BYTES % (4 * WAVE_BYTES) == 0 && B_BYTES % (4 * WAVE_BYTES) == 0, "tiling");
  static_assert((S - 1) * LOADS < 64, "vmcnt field");
  __shared__ __attribute__((aligned(1024))) char smem_raw[S * STAGE_BYTES];
  LDS_AS char* smem = (LDS_AS char*)(smem_raw);
  (void)c2;

  const int64_t bid = blockIdx.x;
  const int gi = find_group(wk, bid);
  const MatGroup& g = bt.g[gi];
  const int tiles = wk.tiles[gi];
  const int64_t local = xcd_remap(bid - wk.begin[gi], wk.begin[gi + 1] - wk.begin[gi]);
  if (local >= g.count * tiles) return;  // padding block
  const int64_t m = local / tiles;
  const int tile = int(local - m * tiles);
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
    K = g.q_pad;
  } else if (MODE == MODE_POLY) {
    Pa = Am + i0 * pp;
    Pb = Am + j0 * pp;
    lda = ldb = pp;
    K = g.p_pad;
  } else {
    Pa = Bm + i0 * pp;
    lda = pp;
    Pb = Xin + j0;
    ldb = qp;
    K = g.p_pad;
  }
  const int nk = K / BK;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t smem_base = uint32_t(reinterpret_cast<uintptr_t>(smem));

  // Issue the loads of K step `kt` into stage buffer kt % S.  Each wave moves
  // A_INSTR + B_INSTR KiB-sized pieces.
  auto issue = [&](int kt) {
    const uint32_t st = smem_base + uint32_t((kt % S) * STAGE_BYTES);
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) dma_rows(Pa, lda, k0, (wave * A_INSTR + i) * 16, st, lane);
#pragma unroll
    for (int i = 0; i < B_INSTR; ++i) {
      if (MODE == MODE_UPDATE)
        dma_xrows<BN>(Pb, ldb, k0, (wave * B_INSTR + i) * (1024 / (BN * 2)), st + A_BYTES, lane);
      else
        dma_rows(Pb, ldb, k0, (wave * B_INSTR + i) * 16, st + A_BYTES, lane);
    }
  };

#pragma unroll
  for (int s = 0; s < S; ++s)
    if (s < nk) issue(s);

  f32x16_t acc[WM][WN];
  float pre[MODE == MODE_POLY ? WM : 1][MODE == MODE_POLY ? WN : 1][16];  // b*A term
#pragma unroll
  for (int mi = 0; mi < WM; ++mi)
#pragma unroll
    for (int ni = 0; ni < WN; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  // The a*X term of the update and the b*A term of the polynomial need the
  // tile's own rows i0 .. i0+127 of X (resp. A, symmetric: A[i][j] =
  // A[j][i]); those rows pass through LDS as the B operand's K rows of K
  // steps i0/32 .. i0/32+3.  While K step kt is resident, the wave picks up
  // the values for its accumulator rows 32 (2 wm + mi) .. +31 when
  // kt == i0/32 + 2 wm + mi, so the epilogue reads nothing from memory.
  auto pick_diag = [&](int kt, const LDS_AS char* sB) {
    if (MODE == MODE_GRAM) return;
    const int mi = kt - i0 / BK - 2 * wm;
    if (mi < 0 || mi >= WM) return;
#pragma unroll
    for (int m2 = 0; m2 < WM; ++m2) {
      if (m2 != mi) continue;
#pragma unroll
      for (int ni = 0; ni < WN; ++ni)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          i16x4_t v;
          if (MODE == MODE_UPDATE)
            v = lds_rows4_xT<BN>(sB, 8 * g4, wn * 32 * WN + ni * 32, lane);
          else
            v = lds_k4_rows(sB, wn * 32 * WN + ni * 32 + (lane & 31), 8 * g4, lane);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x = __uint_as_float(uint32_t(uint16_t(v[j])) << 16);
            if (MODE == MODE_UPDATE)
              acc[m2][ni][4 * g4 + j] = fmaf(c1, x, acc[m2][ni][4 * g4 + j]);
            else
              pre[m2][ni][4 * g4 + j] = x;
          }
        }
    }
  };

  // Fragments of one 16-deep K sub-step of stage buffer `buf`.
  auto load_frags = [&](int buf, int ks, bf16x8_t (&af)[WM], bf16x8_t (&bfr)[WN]) {
    const LDS_AS char* sA = smem + buf * STAGE_BYTES;
    const LDS_AS char* sB = sA + A_BYTES;
    const int ch = ks * 2 + (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < WM; ++mi) af[mi] = lds_frag_rows(sA, wm * 32 * WM + mi * 32 + (lane & 31), ch);
#pragma unroll
    for (int ni = 0; ni < WN; ++ni) {
      if (MODE == MODE_UPDATE)
        bfr[ni] = lds_frag_xT<BN>(sB, ks * 16, wn * 32 * WN + ni * 32, lane);
      else
        bfr[ni] = lds_frag_rows(sB, wn * 32 * WN + ni * 32 + (lane & 31), ch);
    }
  };
  auto mfmas = [&](const bf16x8_t (&af)[WM], const bf16x8_t (&bfr)[WN]) {
#pragma unroll
    for (int mi = 0; mi < WM; ++mi)
#pragma unroll
      for (int ni = 0; ni < WN; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
  };
  // Waits until the loads of `stage` are done, given that the last stage
  // issued so far is `issued` (capped at nk-1): exactly the loads of the
  // stages issued after `stage` may stay in flight (vmcnt counts in order).
  auto wait_stage = [&](int stage, int issued) {
    const int younger = (issued < nk - 1 ? issued : nk - 1) - stage;
    if (S > 3 && younger >= 3)
      wait_vmcnt<(S > 3 ? 3 : 0) * LOADS>();
    else if (younger == 2)
      wait_vmcnt<2 * LOADS>();
    else if (younger == 1)
      wait_vmcnt<LOADS>();
    else
      wait_vmcnt<0>();
  };
  static_assert(S <= 4, "wait_stage covers at most 3 younger stages");

  // Software pipeline over K steps (two 16-deep sub-steps each): the LDS
  // reads of the next sub-step are always in flight while the MFMAs of the
  // current one issue.  One barrier per K step, between its sub-steps: all
  // reads of step kt are complete there (lgkmcnt 0), so its buffer is
  // refilled with step kt+S right after it, and step kt+1 (waited for by
  // every wave) becomes readable.
  bf16x8_t a0[WM], b0[WN], a1[WM], b1[WN];
  wait_stage(0, S - 1);  // the prologue issued steps 0 .. S-1
  block_barrier();
  load_frags(0, 0, a0, b0);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt % S;
    load_frags(buf, 1, a1, b1);
    mfmas(a0, b0);
    pick_diag(kt, smem + buf * STAGE_BYTES + A_BYTES);
    if (kt + 1 < nk) {
      wait_stage(kt + 1, kt + S - 1);  // steps up to kt+S-1 issued so far
      block_barrier();
      if (kt + S < nk) issue(kt + S);
      load_frags((kt + 1) % S, 0, a0, b0);
    }
    mfmas(a1, b1);
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
  // Final values in fp32, before one rounding: Gram alpha*(X X^T),
  // polynomial c*(A A) + b*A, update alpha*(a*X + B X).
#pragma unroll
  for (int mi = 0; mi < WM; ++mi)
#pragma unroll
    for (int ni = 0; ni < WN; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (MODE == MODE_POLY)
          acc[mi][ni][r] = fmaf(c2, acc[mi][ni][r], c1 * pre[mi][ni][r]);
        else
          acc[mi][ni][r] *= alpha;
      }
  constexpr int TP = BN + 8;                 // fp32 staging row pitch (floats)
  static_assert(64 * TP * 4 <= S * STAGE_BYTES, "staging");
  LDS_AS float* T = (LDS_AS float*)smem;
  constexpr int CPR = BN / 8;                // 8-element chunks per row
  constexpr int CHUNKS = 64 * CPR / 256;     // per thread per pass
  uint16_t* Cout = MODE == MODE_UPDATE ? Xout : (MODE == MODE_GRAM ? Am : Bm);
  const int64_t ldc = MODE == MODE_UPDATE ? qp : pp;

  auto stage = [&](int pass) {
    if (wm == pass) {
      // MFMA 32x32 output layout: lane l, register r holds row
      // 8*(r/4) + 4*(l/32) + r%4, column l%32 of a 32x32 block.
#pragma unroll
      for (int mi = 0; mi < WM; ++mi)
#pragma unroll
        for (int ni = 0; ni < WN; ++ni)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int col = wn * 32 * WN + ni * 32 + (lane & 31);
            T[row * TP + col] = acc[mi][ni][r];
          }
    }
  };
  auto pack8 = [](const float (&v)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = f2bf2(v[2 * e], v[2 * e + 1]);
    return make_uint4(w[0], w[1], w[2], w[3]);
  };
  auto finish = [&](int pass) {
#pragma unroll
    for (int u = 0; u < CHUNKS; ++u) {
      const int q = t + 256 * u;
      const int row = q / CPR, col = (q % CPR) * 8;
      float v[8];
      const f32x4_t v0 = *(const LDS_AS f32x4_t*)(T + row * TP + col);
      const f32x4_t v1 = *(const LDS_AS f32x4_t*)(T + row * TP + col + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = v0[e];
        v[e + 4] = v1[e];
      }
      *reinterpret_cast<uint4*>(Cout + (i0 + 64 * pass + row) * ldc + j0 + col) = pack8(v);
    }
    if (mirror) {
      // Mirrored block: rows j0 + c of C (c < BN), columns i0 + 64*pass + r8
      // .. +7, from staged column c; lanes take consecutive c, so the
      // column reads hit distinct banks.
#pragma unroll
      for (int u = 0; u < BN * 8 / 256; ++u) {
        const int q = t + 256 * u;
        const int c = q % BN, r8 = (q / BN) * 8;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = T[(r8 + e) * TP + c];
        *reinterpret_cast<uint4*>(Cout + (j0 + c) * ldc + i0 + 64 * pass + r8) = pack8(v);
      }
    }
  };

  block_barrier();  // stage buffers no longer read
  stage(0);
  block_barrier();
  finish(0);
  block_barrier();  // T is rewritten by the next pass
  stage(1);
  block_barrier();
  finish(1);
}

inline dim3 grid_of(const Work& wk) { return dim3(unsigned(wk.begin[wk.ngroups])); }

}  // namespace

hipError_t launch_gram_bf16(const Batch& bt, const Work& wk, int iter, hipStream_t s) {
  hipLaunchKernelGGL(ns_bf16_kernel<MODE_GRAM>, grid_of(wk), dim3(256), 0, s, bt, wk, iter, 0.f, 0.f);
  return hipGetLastError();
}
hipError_t launch_poly_bf16(const Batch& bt, const Work& wk, float b, float c, hipStream_t s) {
  hipLaunchKernelGGL(ns_bf16_kernel<MODE_POLY>, grid_of(wk), dim3(256), 0, s, bt, wk, 0, b, c);
  return hipGetLastError();
}
hipError_t launch_update_bf16(const Batch& bt, const Work& wk, int iter, float a, hipStream_t s) {
  hipLaunchKernelGGL(ns_bf16_kernel<MODE_UPDATE>, grid_of(wk), dim3(256), 0, s, bt, wk, iter, a, 0.f);
  return hipGetLastError();
}

}  // namespace muon
