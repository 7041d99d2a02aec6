// Newton-Schulz products in true float32 (fused multiply-add on the vector
// ALUs, no reduced-precision matrix modes), for the float32 path whose
// results must track an fp64 computation to about 1e-5.
//
// Same three products and first-iteration scaling as the bf16 path:
//   A = X X^T (lower-triangle tiles, mirrored), B = b*A + c*A A^T,
//   X' = a*X + B X
// ("[논문 AI 리뷰] MUON IS SCALABLE FOR LLM TRAINING TECHNICAL REPORT",
// section 2; the Newton-Schulz code block of "LLM Pretraining Loss Spike
// 진단과 처방 ... Muon 전환 판단", section "Muon head의 실체는 하이브리드
// 옵티마이저다").
//
// Block tile 64x64, K step 32, 1024 threads in four groups of 256: group g
// multiplies the g-th quarter of the K steps (each thread a 4x4 output
// patch, two LDS stages per group, the next K step's operands loaded into
// registers while the current one is multiplied), and the four partial
// tiles are summed through LDS in group order.  Small float32 matrices give
// these launches few blocks, so a tile's chain of K steps sets their time:
// the split shortens it four-fold (bitwise reproducible: a fixed order).
#include "muon_internal.h"

namespace muon {
namespace {

constexpr int TB = kF32Tile;  // 64
constexpr int BKF = 32;

enum { MODE_GRAM = 0, MODE_POLY = 1, MODE_UPDATE = 2 };

__device__ __forceinline__ void tri_decode(int t, int& ti, int& tj) {
  int i = int((sqrtf(8.f * float(t) + 1.f) - 1.f) * 0.5f);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

constexpr int KGROUPS = 4;

template <int MODE>
__global__ __launch_bounds__(256 * KGROUPS) void ns_f32_kernel(Batch bt, Work wk, int iter,
                                                               float c1, float c2) {
  __shared__ __attribute__((aligned(16))) float As[KGROUPS][2][BKF][TB + 4];
  __shared__ __attribute__((aligned(16))) float Bs[KGROUPS][2][BKF][TB + 4];

  const int64_t bid = blockIdx.x;
  const int gi = find_group(wk, bid);
  const MatGroup& g = bt.g[gi];
  const int64_t local = bid - wk.begin[gi];
  const int tiles = wk.tiles[gi];
  const int64_t m = local / tiles;
  const int tile = int(local - m * tiles);
  int ti, tj;
  if (MODE == MODE_UPDATE) {
    const int ntn = g.q_pad / TB;
    ti = tile / ntn;
    tj = tile - ti * ntn;
  } else {
    tri_decode(tile, ti, tj);
  }
  const int i0 = ti * TB, j0 = tj * TB;
  const int64_t qp = g.q_pad, pp = g.p_pad;

  const float* Xin = reinterpret_cast<const float*>((iter & 1) ? g.X1 : g.X0) + m * g.x_stride;
  float* Xout = reinterpret_cast<float*>((iter & 1) ? g.X0 : g.X1) + m * g.x_stride;
  float* Am = reinterpret_cast<float*>(g.A) + m * g.a_stride;
  float* Bm = reinterpret_cast<float*>(g.B) + m * g.a_stride;

  const float* Pa;
  const float* Pb;
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

  const int kg = int(threadIdx.x) >> 8;   // K group
  const int t = int(threadIdx.x) & 255;
  const int tm = t >> 4, tn = t & 15;
  float acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;

  // Operand loads of one K step: the K-contiguous tiles (A, and the Gram's
  // and polynomial's B) as 64 rows x 32 k, two float4 per thread, stored
  // transposed (k-major) in LDS; the update's X tile as 32 k-rows x 64.
  const int lrow = t >> 2, lkq = (t & 3) * 8;
  const int lkk = t >> 3, lnq = (t & 7) * 8;
  float4 ra0, ra1, rb0, rb1;
  auto gload = [&](int k0) {
    const float* pa = Pa + lrow * lda + k0 + lkq;
    ra0 = *reinterpret_cast<const float4*>(pa);
    ra1 = *reinterpret_cast<const float4*>(pa + 4);
    if (MODE != MODE_UPDATE) {
      const float* pb = Pb + lrow * ldb + k0 + lkq;
      rb0 = *reinterpret_cast<const float4*>(pb);
      rb1 = *reinterpret_cast<const float4*>(pb + 4);
    } else {
      const float* pb = Pb + (k0 + lkk) * ldb + lnq;
      rb0 = *reinterpret_cast<const float4*>(pb);
      rb1 = *reinterpret_cast<const float4*>(pb + 4);
    }
  };
  auto sstore = [&](int buf) {
    const float a8[8] = {ra0.x, ra0.y, ra0.z, ra0.w, ra1.x, ra1.y, ra1.z, ra1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) As[kg][buf][lkq + j][lrow] = a8[j];
    if (MODE != MODE_UPDATE) {
      const float b8[8] = {rb0.x, rb0.y, rb0.z, rb0.w, rb1.x, rb1.y, rb1.z, rb1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) Bs[kg][buf][lkq + j][lrow] = b8[j];
    } else {
      *reinterpret_cast<float4*>(&Bs[kg][buf][lkk][lnq]) = rb0;
      *reinterpret_cast<float4*>(&Bs[kg][buf][lkk][lnq + 4]) = rb1;
    }
  };
  // this group's K steps: [s0, s1) of the K / BKF steps (possibly none)
  const int nsteps = K / BKF;
  const int s0 = nsteps * kg / KGROUPS, s1 = nsteps * (kg + 1) / KGROUPS;
  if (s0 < s1) {
    gload(s0 * BKF);
    sstore(0);
  }
  __syncthreads();
  int buf = 0;
  for (int st = s0; st < s1; ++st) {
    const int k0 = st * BKF;
    const bool more = st + 1 < s1;
    if (more) gload(k0 + BKF);   // in flight during this step's products
#pragma unroll 8
    for (int k = 0; k < BKF; ++k) {
      const float4 a = *reinterpret_cast<const float4*>(&As[kg][buf][k][tm * 4]);
      const float4 b = *reinterpret_cast<const float4*>(&Bs[kg][buf][k][tn * 4]);
      const float av[4] = {a.x, a.y, a.z, a.w};
      const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(av[r], bv[c], acc[r][c]);
    }
    // the other stage was last read before the previous barrier
    if (more) sstore(buf ^ 1);
    // (groups run different step counts: a group-local barrier would do, but
    // the block barrier keeps the code plain; a group past its last step
    // still passes it)
    __syncthreads();
    buf ^= 1;
  }
  // groups with fewer steps meet the others' remaining barriers here
  for (int st = s1 - s0; st < (nsteps + KGROUPS - 1) / KGROUPS; ++st) __syncthreads();

  // The four partial tiles, summed in group order (As is free again).
  float* R = &As[0][0][0][0];
  static_assert(sizeof(As) >= sizeof(float) * (KGROUPS - 1) * TB * TB, "partials fit");
  if (kg > 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      *reinterpret_cast<float4*>(&R[((kg - 1) * TB + tm * 4 + r) * TB + tn * 4]) =
          make_float4(acc[r][0], acc[r][1], acc[r][2], acc[r][3]);
  }
  __syncthreads();
  if (kg > 0) return;
#pragma unroll
  for (int q = 0; q < KGROUPS - 1; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float4 v = *reinterpret_cast<const float4*>(&R[(q * TB + tm * 4 + r) * TB + tn * 4]);
      acc[r][0] += v.x;
      acc[r][1] += v.y;
      acc[r][2] += v.z;
      acc[r][3] += v.w;
    }

  const float* sc = g.scal + m * kScal;
  float alpha = 1.f, beta = 0.f;
  if (MODE == MODE_GRAM) {
    const float inv = iter == 0 ? sc[SC_INV] : 1.f;
    alpha = inv * inv;
  } else if (MODE == MODE_POLY) {
    alpha = c2;
    beta = c1;
  } else {
    alpha = iter == 0 ? sc[SC_INV] : 1.f;
  }
  const bool mirror = (MODE != MODE_UPDATE) && (ti != tj);
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int row = i0 + tm * 4 + r;
      const int col = j0 + tn * 4 + c;
      const float v = acc[r][c];
      if (MODE == MODE_GRAM) {
        const float h = alpha * v;
        Am[row * pp + col] = h;
        if (mirror) Am[col * pp + row] = h;
      } else if (MODE == MODE_POLY) {
        const float h = fmaf(alpha, v, beta * Am[row * pp + col]);
        Bm[row * pp + col] = h;
        if (mirror) Bm[col * pp + row] = h;
      } else {
        Xout[row * qp + col] = alpha * fmaf(c1, Xin[row * qp + col], v);
      }
    }
}

inline dim3 grid_of(const Work& wk) { return dim3(unsigned(wk.begin[wk.ngroups])); }

}  // namespace

hipError_t launch_gram_f32(const Batch& bt, const Work& wk, int iter, hipStream_t s) {
  hipLaunchKernelGGL(ns_f32_kernel<MODE_GRAM>, grid_of(wk), dim3(256 * KGROUPS), 0, s, bt, wk, iter, 0.f, 0.f);
  return hipGetLastError();
}
hipError_t launch_poly_f32(const Batch& bt, const Work& wk, float b, float c, hipStream_t s) {
  hipLaunchKernelGGL(ns_f32_kernel<MODE_POLY>, grid_of(wk), dim3(256 * KGROUPS), 0, s, bt, wk, 0, b, c);
  return hipGetLastError();
}
hipError_t launch_update_f32(const Batch& bt, const Work& wk, int iter, float a, hipStream_t s) {
  hipLaunchKernelGGL(ns_f32_kernel<MODE_UPDATE>, grid_of(wk), dim3(256 * KGROUPS), 0, s, bt, wk, iter, a, 0.f);
  return hipGetLastError();
}

}  // namespace muon
