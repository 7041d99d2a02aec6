// Newton-Schulz products on bf16 matrix cores (gfx950 MFMA 32x32x16 bf16,
// float32 accumulation, float32 epilogues, one round-to-nearest-even per
// stored operand).
//
// One iteration, on X (p x q, short side first):
//   A = X X^T                 symmetric: only lower-triangle block tiles are
//                             computed, each written to both triangles
//   B = b*A + c*A A^T         A is symmetric, so A A = A A^T: the same
//                             symmetric form with K = p and the b*A epilogue
//   X' = a*X + B X            full p x q output; X is N-contiguous, so its
//                             tiles are transposed in registers on the way
//                             into LDS
// which is X_k = aX + b(XX^T)X + c(XX^T)^2 X of "[논문 AI 리뷰] MUON IS
// SCALABLE FOR LLM TRAINING TECHNICAL REPORT", section 2, and the three-line
// Newton-Schulz code block of "LLM Pretraining Loss Spike 진단과 처방 ... Muon
// 전환 판단", section "Muon head의 실체는 하이브리드 옵티마이저다".
//
// The first iteration receives the unnormalised U (the head cannot know
// ||U|| while it writes X0): its Gram is scaled by inv^2 and its update by
// inv, inv = 1/(||U||_F + 1e-7), which is the iteration applied to U*inv.
//
// Block tile 128x128, K step 64, 256 threads = 4 waves in a 2x2 grid, each
// wave a 64x64 sub-tile of 2x2 MFMA 32x32 outputs.  LDS rows hold 64 bf16
// (128 bytes) of one operand row; 16-byte chunks are XOR-swizzled by
// (row + row/8) mod 8 so that fragment reads (32 consecutive rows, one chunk)
// and the transposing 8-byte writes are bank-conflict free.
#include "muon_internal.h"

namespace muon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int BM = kBf16Tile;      // 128
constexpr int BK = 64;
constexpr int ROWB = BK * 2;       // bytes per LDS row
constexpr int TILEB = BM * ROWB;   // 16 KB per operand tile

enum { MODE_GRAM = 0, MODE_POLY = 1, MODE_UPDATE = 2 };

__device__ __forceinline__ int swz(int row) { return (row + (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * ROWB + ((chunk ^ swz(row)) << 4);
}

// Lower-triangle block index t -> (ti, tj), ti >= tj, row-major over ti.
__device__ __forceinline__ void tri_decode(int t, int& ti, int& tj) {
  int i = int((sqrtf(8.f * float(t) + 1.f) - 1.f) * 0.5f);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

// 128 rows x 64 K-contiguous bf16 from global: thread t takes rows
// t/8 + 32*r, 16-byte chunk t%8 (8 threads per 128-byte row segment).
__device__ __forceinline__ void gload_rows(const uint16_t* base, int64_t ld, int k0,
                                           u32x4_t (&r)[4]) {
  const int t = threadIdx.x;
  const int row = t >> 3, ch = t & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = *reinterpret_cast<const u32x4_t*>(base + int64_t(row + 32 * i) * ld + k0 + ch * 8);
}
__device__ __forceinline__ void sstore_rows(char* lds, const u32x4_t (&r)[4]) {
  const int t = threadIdx.x;
  const int row = t >> 3, ch = t & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4_t*>(lds + lds_off(row + 32 * i, ch)) = r[i];
}

// X tile of the update: 64 K-rows x 128 N-columns, N contiguous in memory.
// Thread t loads rows k0 + 4*(t/16) + i (i = 0..3), columns 8*(t%16) .. +7.
__device__ __forceinline__ void gload_xT(const uint16_t* base, int64_t ld, int k0,
                                         u32x4_t (&r)[4]) {
  const int t = threadIdx.x;
  const int nb = t & 15, kq = t >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = *reinterpret_cast<const u32x4_t*>(base + int64_t(k0 + 4 * kq + i) * ld + nb * 8);
}
// ... and stores it as 128 N-rows of 64 K-contiguous bf16: for each of its 8
// columns the thread packs its 4 K values into 8 bytes.
__device__ __forceinline__ void sstore_xT(char* lds, const u32x4_t (&r)[4]) {
  const int t = threadIdx.x;
  const int nb = t & 15, kq = t >> 4;
  const int chunk = kq >> 1, sub = (kq & 1) * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = e >> 1;
    uint32_t lo, hi;
    if (e & 1) {
      lo = (r[0][d] >> 16) | (r[1][d] & 0xffff0000u);
      hi = (r[2][d] >> 16) | (r[3][d] & 0xffff0000u);
    } else {
      lo = (r[0][d] & 0xffffu) | (r[1][d] << 16);
      hi = (r[2][d] & 0xffffu) | (r[3][d] << 16);
    }
    const int n = nb * 8 + e;
    u32x2_t v;
    v[0] = lo;
    v[1] = hi;
    *reinterpret_cast<u32x2_t*>(lds + lds_off(n, chunk) + sub) = v;
  }
}

template <int MODE>
__global__ __launch_bounds__(256, 2) void ns_bf16_kernel(Batch bt, Work wk, int iter, float c1,
                                                         float c2) {
  __shared__ __attribute__((aligned(16))) char lds[2 * TILEB];
  char* sA = lds;
  char* sB = lds + TILEB;

  const int64_t bid = blockIdx.x;
  const int gi = find_group(wk, bid);
  const MatGroup& g = bt.g[gi];
  const int64_t local = bid - wk.begin[gi];
  const int tiles = wk.tiles[gi];
  const int64_t m = local / tiles;
  const int tile = int(local - m * tiles);
  int ti, tj;
  if (MODE == MODE_UPDATE) {
    const int ntn = g.q_pad / BM;
    ti = tile / ntn;
    tj = tile - ti * ntn;
  } else {
    tri_decode(tile, ti, tj);
  }
  const int i0 = ti * BM, j0 = tj * BM;
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

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16_t acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  u32x4_t ra[4], rb[4];
  gload_rows(Pa, lda, 0, ra);
  if (MODE == MODE_UPDATE)
    gload_xT(Pb, ldb, 0, rb);
  else
    gload_rows(Pb, ldb, 0, rb);

  for (int k0 = 0; k0 < K; k0 += BK) {
    sstore_rows(sA, ra);
    if (MODE == MODE_UPDATE)
      sstore_xT(sB, rb);
    else
      sstore_rows(sB, rb);
    __syncthreads();
    if (k0 + BK < K) {  // next K tile in flight while this one is multiplied
      gload_rows(Pa, lda, k0 + BK, ra);
      if (MODE == MODE_UPDATE)
        gload_xT(Pb, ldb, k0 + BK, rb);
      else
        gload_rows(Pb, ldb, k0 + BK, rb);
    }
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int ch = ks * 2 + (lane >> 5);
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        af[mi] = *reinterpret_cast<const bf16x8_t*>(sA + lds_off(wm * 64 + mi * 32 + (lane & 31), ch));
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bfr[ni] = *reinterpret_cast<const bf16x8_t*>(sB + lds_off(wn * 64 + ni * 32 + (lane & 31), ch));
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    __syncthreads();
  }

  // Epilogue.  MFMA 32x32 output layout: lane l, register r holds row
  // 8*(r/4) + 4*(l/32) + r%4, column l%32 of the 32x32 block.
  const float* sc = g.scal + m * kScal;
  float alpha = 1.f, beta = 0.f;
  if (MODE == MODE_GRAM) {
    const float inv = iter == 0 ? sc[SC_INV] : 1.f;
    alpha = inv * inv;
  } else if (MODE == MODE_POLY) {
    alpha = c2;  // c
    beta = c1;   // b
  } else {
    alpha = iter == 0 ? sc[SC_INV] : 1.f;
  }
  const bool mirror = (MODE != MODE_UPDATE) && (ti != tj);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i0 + wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = j0 + wn * 64 + ni * 32 + (lane & 31);
        float v = acc[mi][ni][r];
        if (MODE == MODE_GRAM) {
          const uint16_t h = f2bf(alpha * v);
          Am[row * pp + col] = h;
          if (mirror) Am[col * pp + row] = h;
        } else if (MODE == MODE_POLY) {
          const uint16_t h = f2bf(fmaf(alpha, v, beta * bf2f(Am[row * pp + col])));
          Bm[row * pp + col] = h;
          if (mirror) Bm[col * pp + row] = h;
        } else {
          const float x = bf2f(Xin[row * qp + col]);
          Xout[row * qp + col] = f2bf(alpha * fmaf(c1, x, v));
        }
      }
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
