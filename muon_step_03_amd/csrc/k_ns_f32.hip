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
// Block tile 64x64, K step 16, 256 threads each owning a 4x4 output patch.
#include "muon_internal.h"

namespace muon {
namespace {

constexpr int TB = kF32Tile;  // 64
constexpr int BKF = 16;

enum { MODE_GRAM = 0, MODE_POLY = 1, MODE_UPDATE = 2 };

__device__ __forceinline__ void tri_decode(int t, int& ti, int& tj) {
  int i = int((sqrtf(8.f * float(t) + 1.f) - 1.f) * 0.5f);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

template <int MODE>
__global__ __launch_bounds__(256) void ns_f32_kernel(Batch bt, Work wk, int iter, float c1,
                                                     float c2) {
  __shared__ __attribute__((aligned(16))) float As[BKF][TB + 4];
  __shared__ __attribute__((aligned(16))) float Bs[BKF][TB + 4];

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

  const int t = threadIdx.x;
  const int tm = t >> 4, tn = t & 15;
  float acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;

  for (int k0 = 0; k0 < K; k0 += BKF) {
    {
      const int row = t >> 2, kq = (t & 3) * 4;
      const float4 v = *reinterpret_cast<const float4*>(Pa + row * lda + k0 + kq);
      As[kq + 0][row] = v.x;
      As[kq + 1][row] = v.y;
      As[kq + 2][row] = v.z;
      As[kq + 3][row] = v.w;
      if (MODE != MODE_UPDATE) {
        const float4 w = *reinterpret_cast<const float4*>(Pb + row * ldb + k0 + kq);
        Bs[kq + 0][row] = w.x;
        Bs[kq + 1][row] = w.y;
        Bs[kq + 2][row] = w.z;
        Bs[kq + 3][row] = w.w;
      }
    }
    if (MODE == MODE_UPDATE) {
      const int kk = t >> 4, nq = (t & 15) * 4;
      *reinterpret_cast<float4*>(&Bs[kk][nq]) =
          *reinterpret_cast<const float4*>(Pb + (k0 + kk) * ldb + nq);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BKF; ++k) {
      const float4 a = *reinterpret_cast<const float4*>(&As[k][tm * 4]);
      const float4 b = *reinterpret_cast<const float4*>(&Bs[k][tn * 4]);
      const float av[4] = {a.x, a.y, a.z, a.w};
      const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(av[r], bv[c], acc[r][c]);
    }
    __syncthreads();
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
  hipLaunchKernelGGL(ns_f32_kernel<MODE_GRAM>, grid_of(wk), dim3(256), 0, s, bt, wk, iter, 0.f, 0.f);
  return hipGetLastError();
}
hipError_t launch_poly_f32(const Batch& bt, const Work& wk, float b, float c, hipStream_t s) {
  hipLaunchKernelGGL(ns_f32_kernel<MODE_POLY>, grid_of(wk), dim3(256), 0, s, bt, wk, 0, b, c);
  return hipGetLastError();
}
hipError_t launch_update_f32(const Batch& bt, const Work& wk, int iter, float a, hipStream_t s) {
  hipLaunchKernelGGL(ns_f32_kernel<MODE_UPDATE>, grid_of(wk), dim3(256), 0, s, bt, wk, iter, a, 0.f);
  return hipGetLastError();
}

}  // namespace muon
