// Elementwise phases of the Muon step: the head (momentum, Nesterov
// look-ahead, Frobenius-norm partials, X0 write in short-side orientation)
// and the tail (MuonGS reductions, projection, RMS scale, decoupled weight
// decay, W update).  Both are HBM-bound; each block moves one tile of 4096
// elements with coalesced accesses (16x256 for a wide matrix, 64x64
// transposed through LDS for a tall one, which is iterated as its
// transpose).
//
// Passages: update order — "[Deep Learning] Muon — 행렬 업데이트를 직교화하는
// 옵티마이저", section 3; SGD-momentum/Nesterov defaults and the 1e-7
// normaliser — "LLM Pretraining Loss Spike 진단과 처방 ... Muon 전환 판단",
// section "Muon head의 실체는 하이브리드 옵티마이저다"; 0.2*sqrt(max(A,B)) —
// "[논문 AI 리뷰] MUON IS SCALABLE FOR LLM TRAINING", section 2, eq. 4;
// Gram-Schmidt projection — "MuonGS: Pretraining LLMs with Relaxed
// Weight-Norm Control", section "전제와 한계".
#include "muon_internal.h"

namespace muon {
namespace {

constexpr int T = kEwTile;  // 64

struct TileRef {
  const MatGroup* g;
  int64_t m;     // matrix index within the group
  int tile;      // tile (block) index within the matrix
  int per;       // tiles (blocks) per matrix in this launch
};

__device__ __forceinline__ TileRef decode(const Batch& bt, const Work& wk, int64_t bid) {
  const int gi = find_group(wk, bid);
  const int64_t local = bid - wk.begin[gi];
  const int tiles = wk.tiles[gi];
  TileRef r;
  r.g = &bt.g[gi];
  r.m = local / tiles;
  r.tile = int(local - r.m * tiles);
  r.per = tiles;
  return r;
}

__device__ __forceinline__ bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

template <bool BF16>
struct Vec4;
template <>
struct Vec4<true> {  // 4 bf16 = 8 bytes
  static __device__ __forceinline__ void load(const uint16_t* p, float* v) {
    const uint2 d = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(d.x << 16);
    v[1] = __uint_as_float(d.x & 0xffff0000u);
    v[2] = __uint_as_float(d.y << 16);
    v[3] = __uint_as_float(d.y & 0xffff0000u);
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float* v) {
    uint2 d;
    d.x = f2bf2(v[0], v[1]);
    d.y = f2bf2(v[2], v[3]);
    *reinterpret_cast<uint2*>(p) = d;
  }
};
template <>
struct Vec4<false> {  // 4 floats = 16 bytes
  static __device__ __forceinline__ void load(const float* p, float* v) {
    const float4 d = *reinterpret_cast<const float4*>(p);
    v[0] = d.x; v[1] = d.y; v[2] = d.z; v[3] = d.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// Streams touched once per step (the gradient, the momentum buffer) use
// nontemporal accesses: they are marked evict-first in the caches, which
// keeps L2 and the Infinity Cache for X0, read next by the Gram product
// (measured: head 5.5 -> 6.1 TB/s on 1024x4096 matrices).  Whole 64-byte
// runs per row only: the same hint on scattered 16-byte writes of the
// weights (the fused last update of a tall matrix) halved their speed.
typedef unsigned int nt_u32x2 __attribute__((ext_vector_type(2)));
typedef float nt_f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void load4_nt(const uint16_t* p, float* v) {
  const nt_u32x2 d = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x2*>(p));
  v[0] = __uint_as_float(d.x << 16);
  v[1] = __uint_as_float(d.x & 0xffff0000u);
  v[2] = __uint_as_float(d.y << 16);
  v[3] = __uint_as_float(d.y & 0xffff0000u);
}
__device__ __forceinline__ void load4_nt(const float* p, float* v) {
  const nt_f32x4 d = __builtin_nontemporal_load(reinterpret_cast<const nt_f32x4*>(p));
  v[0] = d.x;
  v[1] = d.y;
  v[2] = d.z;
  v[3] = d.w;
}
__device__ __forceinline__ void store4_nt(float* p, const float* v) {
  const nt_f32x4 d = {v[0], v[1], v[2], v[3]};
  __builtin_nontemporal_store(d, reinterpret_cast<nt_f32x4*>(p));
}

// ------------------------------------------------------------------- head
// M' = mu*M + G, U = G + mu*M' on one 64x64 tile of X (X = U, or U^T for a
// tall matrix); writes M' in place, U (rounded to X's type) into X0 with
// zeros in the padding, and the tile's sum of u^2 (unrounded u, summed in
// fp64: the total then hardly depends on how the matrix is cut into tiles,
// which differs between a matrix and its transpose, so that the step of W^T
// is the transpose of W's bit for bit).
template <bool BF16>
__global__ __launch_bounds__(256) void head_kernel(Batch bt, Work wk, float mu) {
  using E = Elem<BF16>;
  using TE = typename E::T;
  __shared__ float S[T][T + 1];
  __shared__ double red[4];

  const TileRef tr = decode(bt, wk, blockIdx.x);
  const MatGroup& g = *tr.g;
  const int t = threadIdx.x;
  if (!g.trans && g.q_pad == g.cols && g.p_pad == g.rows) {
    // No transpose and no padding: X0 = U has G's and M's layout, so the
    // matrix is one contiguous run and a tile is 4096 consecutive elements
    // (4 sweeps of 1024; runs of 2 / 4 KiB of G / M per sweep).  rows x cols
    // is then a multiple of 4096 (both padded sides are multiples of 64).
    const int64_t elems = int64_t(g.rows) * g.cols;
    const TE* G = mat_cptr<TE>(g.G_tab, g.G, tr.m, elems);
    float* M = mat_ptr<float>(reinterpret_cast<void* const*>(g.M_tab), reinterpret_cast<char*>(g.M),
                              tr.m, elems);
    TE* X = reinterpret_cast<TE*>(g.X0) + tr.m * g.x_stride;
    const bool vec = aligned16(M) && ((reinterpret_cast<uintptr_t>(G) & (BF16 ? 7u : 15u)) == 0);
    const int64_t base = int64_t(tr.tile) * (4 * 4 * 256) + 4 * t;
    float u[4][4];
    double ss = 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t off = base + 1024 * k;
      if (vec) {
        float gv[4], mv[4];
        load4_nt(G + off, gv);
        load4_nt(M + off, mv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mv[e] = fmaf(mu, mv[e], gv[e]);
          u[k][e] = fmaf(mu, mv[e], gv[e]);
        }
        store4_nt(M + off, mv);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gv = E::load(G + off + e);
          const float mv = fmaf(mu, M[off + e], gv);
          M[off + e] = mv;
          u[k][e] = fmaf(mu, mv, gv);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) ss = fma(double(u[k][e]), double(u[k][e]), ss);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) Vec4<BF16>::store(X + base + 1024 * k, u[k]);
    const double tot = block_sum_256(ss, red);
    if (t == 0) g.head_part[tr.m * g.head_tiles + tr.tile] = tot;
    return;
  }
  // A wide matrix (X = U, no transpose) is taken in tiles of 16 rows x 256
  // columns (row runs of 512 / 1024 bytes of G / M), or of 32 x 128 when its
  // padded row length is a multiple of 128 only; a tall one in 64 x 64
  // tiles transposed through LDS.  All give the same tile count.
  const int flat = g.trans ? 1 : (g.q_pad % (4 * T)) == 0 ? 4 : (g.q_pad % (2 * T)) == 0 ? 2 : 1;
  const int TR = T / flat, TC = T * flat;
  const int ntj = g.q_pad / TC;
  const int ti = tr.tile / ntj;
  const int tj = tr.tile - ti * ntj;
  const int i0 = ti * TR, j0 = tj * TC;          // X-orientation origin
  const int sr0 = g.trans ? j0 : i0;             // weight-orientation origin
  const int sc0 = g.trans ? i0 : j0;
  const int64_t elems = int64_t(g.rows) * g.cols;
  const TE* G = mat_cptr<TE>(g.G_tab, g.G, tr.m, elems);
  float* M = mat_ptr<float>(reinterpret_cast<void* const*>(g.M_tab),
                            reinterpret_cast<char*>(g.M), tr.m, elems);
  TE* X = reinterpret_cast<TE*>(g.X0) + tr.m * g.x_stride;

  // 4 consecutive elements per thread; TC/4 threads per row, 4 sweeps
  const int tpr = TC / 4;
  const int rb = t / tpr;         // 0..15 (64x64) or 0..3 (16x256)
  const int cq = (t % tpr) * 4;   // 0..60 or 0..252
  const int rstep = 256 / tpr;
  const bool vec = (sc0 + cq + 4 <= g.cols) && ((g.cols & 3) == 0) && aligned16(M) &&
                   ((reinterpret_cast<uintptr_t>(G) & (BF16 ? 7u : 15u)) == 0);

  float u[4][4];
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = sr0 + rb + rstep * k;
#pragma unroll
    for (int e = 0; e < 4; ++e) u[k][e] = 0.f;
    if (r < g.rows) {
      const int64_t off = int64_t(r) * g.cols + sc0 + cq;
      if (vec) {
        float gv[4], mv[4];
        load4_nt(G + off, gv);
        load4_nt(M + off, mv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mv[e] = fmaf(mu, mv[e], gv[e]);
          u[k][e] = fmaf(mu, mv[e], gv[e]);
        }
        store4_nt(M + off, mv);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (sc0 + cq + e < g.cols) {
            const float gv = E::load(G + off + e);
            const float mv = fmaf(mu, M[off + e], gv);
            M[off + e] = mv;
            u[k][e] = fmaf(mu, mv, gv);
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) ss = fma(double(u[k][e]), double(u[k][e]), ss);
  }

  if (!g.trans) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      Vec4<BF16>::store(X + int64_t(i0 + rb + rstep * k) * g.q_pad + j0 + cq, u[k]);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[rb + 16 * k][cq + e] = u[k][e];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int xi = rb + 16 * k;  // X row offset = source column offset
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = S[cq + e][xi];
      Vec4<BF16>::store(X + int64_t(i0 + xi) * g.q_pad + j0 + cq, v);
    }
  }

  const double tot = block_sum_256(ss, red);
  if (t == 0) g.head_part[tr.m * g.head_tiles + tr.tile] = tot;
}

// ||U||_F and 1/(||U||_F + 1e-7) from the head partials of one matrix (one
// block per matrix, fixed summation order, fp64 until the two scalars are
// rounded to fp32).
__global__ __launch_bounds__(256) void norm_finalize_kernel(Batch bt, Work wk) {
  __shared__ double red[4];
  const TileRef tr = decode(bt, wk, blockIdx.x);
  const MatGroup& g = *tr.g;
  const double* part = g.head_part + tr.m * g.head_tiles;
  double s = 0.0;
  for (int i = threadIdx.x; i < g.head_tiles; i += 256) s += part[i];
  s = block_sum_256(s, red);
  if (threadIdx.x == 0) {
    const double n = sqrt(s);
    float* sc = g.scal + tr.m * kScal;
    sc[SC_NORM] = float(n);
    sc[SC_INV] = float(1.0 / (n + double(kEpsNorm)));
    if (g.stats) g.stats[tr.m * MUON_STATS_PER_MATRIX + 0] = float(n);
  }
}

// ------------------------------------------------------------------- tail
// A tail tile is 64x64 in weight orientation, or, for a wide matrix whose
// rows are a multiple of 64 and columns a multiple of 256 (and no row/column
// statistics wanted), 16 rows x 256 columns: row runs of 512 bytes of W and
// O, and the same tile count.  Each thread holds 4 consecutive columns of 4
// rows, rstep rows apart.
struct TailTile {
  int r0, c0;   // weight-orientation origin
  int rb, cq;   // thread's first row offset and column offset
  int rstep;    // row distance between the thread's 4 rows
  int tc;       // tile columns (64 or 256)
};

__device__ __forceinline__ TailTile tail_tile(const MatGroup& g, int tile, bool allow_flat) {
  const int t = threadIdx.x;
  TailTile tt;
  if (allow_flat && !g.trans && (g.rows % T) == 0 && (g.cols % (4 * T)) == 0) {
    const int ntc = g.cols / (4 * T);
    const int ti = tile / ntc;
    tt.r0 = ti * (T / 4);
    tt.c0 = (tile - ti * ntc) * (4 * T);
    tt.rb = t >> 6;
    tt.cq = (t & 63) * 4;
    tt.rstep = 4;
    tt.tc = 4 * T;
  } else {
    const int ti = tile / g.tail_tiles_c;
    tt.r0 = ti * T;
    tt.c0 = (tile - ti * g.tail_tiles_c) * T;
    tt.rb = t >> 4;
    tt.cq = (t & 15) * 4;
    tt.rstep = 16;
    tt.tc = T;
  }
  return tt;
}

// Gathers the thread's 4x4 elements of the Newton-Schulz output O in weight
// orientation (through LDS when the iterate is the transpose; such tiles are
// always 64x64).  Every X access lies inside the padded extents.
template <bool BF16, bool NT>
__device__ __forceinline__ void load_o_tile(const MatGroup& g, const typename Elem<BF16>::T* X,
                                            const TailTile& tt, float (*S)[T + 1], float o[4][4]) {
  if (!g.trans) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const auto* p = X + int64_t(tt.r0 + tt.rb + tt.rstep * k) * g.q_pad + tt.c0 + tt.cq;
      if (NT) load4_nt(p, o[k]); else Vec4<BF16>::load(p, o[k]);
    }
  } else {
    // X rows are weight columns: read X[c0 + i][r0 + j] coalesced, then
    // transpose through LDS.
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float v[4];
      const auto* p = X + int64_t(tt.c0 + tt.rb + 16 * k) * g.q_pad + tt.r0 + tt.cq;
      if (NT) load4_nt(p, v); else Vec4<BF16>::load(p, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) S[tt.rb + 16 * k][tt.cq + e] = v[e];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[k][e] = S[tt.cq + e][tt.rb + 16 * k];
  }
}

template <bool BF16, bool NT>
__device__ __forceinline__ void load_w_tile(const MatGroup& g, const typename Elem<BF16>::T* W,
                                            const TailTile& tt, float w[4][4], bool valid[4][4]) {
  using E = Elem<BF16>;
  const bool vec = (tt.c0 + tt.tc <= g.cols) && ((g.cols & 3) == 0) &&
                   ((reinterpret_cast<uintptr_t>(W) & (BF16 ? 7u : 15u)) == 0);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = tt.r0 + tt.rb + tt.rstep * k;
    const int64_t off = int64_t(r) * g.cols + tt.c0 + tt.cq;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[k][e] = 0.f;
      valid[k][e] = (r < g.rows) && (tt.c0 + tt.cq + e < g.cols);
    }
    if (r < g.rows) {
      if (vec) {
        if (NT) load4_nt(W + off, w[k]); else Vec4<BF16>::load(W + off, w[k]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (valid[k][e]) w[k][e] = E::load(W + off + e);
      }
    }
  }
}

// Block sums of three values with one pair of barriers.
template <typename F>
__device__ __forceinline__ void block_sum3_256(F& a, F& b, F& c, F* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    a += __shfl_xor(a, off, 64);
    b += __shfl_xor(b, off, 64);
    c += __shfl_xor(c, off, 64);
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    red[wave] = a;
    red[4 + wave] = b;
    red[8 + wave] = c;
  }
  __syncthreads();
  a = (red[0] + red[1]) + (red[2] + red[3]);
  b = (red[4] + red[5]) + (red[6] + red[7]);
  c = (red[8] + red[9]) + (red[10] + red[11]);
}

// Per-tile partials of <W,O>, ||W||^2, ||O||^2 (O scaled by 1/(||U||+eps)
// when no Newton-Schulz step ran, since X0 holds the unnormalised U).
template <bool BF16>
__global__ __launch_bounds__(256) void tail_reduce_kernel(Batch bt, Work wk, int ns_steps, int rc) {
  using TE = typename Elem<BF16>::T;
  __shared__ float S[T][T + 1];
  __shared__ double red[12];
  const TileRef tr = decode(bt, wk, blockIdx.x);
  const MatGroup& g = *tr.g;
  const TailTile tt = tail_tile(g, tr.tile, !rc);
  const int64_t elems = int64_t(g.rows) * g.cols;
  const TE* W = mat_cptr<TE>(reinterpret_cast<const void* const*>(g.W_tab), g.W, tr.m, elems);
  const TE* X = reinterpret_cast<const TE*>((ns_steps & 1) ? g.X1 : g.X0) + tr.m * g.x_stride;
  const float oscale = ns_steps == 0 ? g.scal[tr.m * kScal + SC_INV] : 1.0f;

  float w[4][4], o[4][4];
  bool valid[4][4];
  // nontemporal: the reduction reads W and O at 5.2 instead of 4.3 TB/s
  // (the apply, which reads them again, is no slower for it)
  load_w_tile<BF16, true>(g, W, tt, w, valid);
  load_o_tile<BF16, true>(g, X, tt, S, o);
  // (sums in fp64, as the head's: W's and W^T's tiles then give the same
  // totals to the last bit of their fp32 rounding)
  double dot = 0.0, ww = 0.0, oo = 0.0;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double wv = w[k][e], ov = valid[k][e] ? o[k][e] * oscale : 0.f;
      dot = fma(wv, ov, dot);
      ww = fma(wv, wv, ww);
      oo = fma(ov, ov, oo);
    }
  block_sum3_256(dot, ww, oo, red);
  if (threadIdx.x == 0) {
    double* p = g.tail_part + (tr.m * g.red_tiles + tr.tile) * 3;
    p[0] = dot;
    p[1] = ww;
    p[2] = oo;
  }
  if (rc) {
    // Row and column sums of O^2 over this 64x64 tile: 64 + 64 partials.
    // A row's 64 values sit in 16 consecutive threads (shuffle reduction);
    // a column's in the 16 row groups (through LDS).
    const int t = threadIdx.x;
    const int rb = tt.rb, cq = tt.cq;
    float* out = g.rc_part + (tr.m * g.tail_tiles + tr.tile) * (2 * T);
    float rs[4], cs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      rs[k] = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ov = valid[k][e] ? o[k][e] * oscale : 0.f;
        rs[k] = fmaf(ov, ov, rs[k]);
        cs[e] = fmaf(ov, ov, cs[e]);
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) rs[k] += __shfl_xor(rs[k], off, 16);
    if ((t & 15) == 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k) out[rb + 16 * k] = rs[k];
    }
    __syncthreads();  // S is free again (load_o_tile may have used it)
#pragma unroll
    for (int e = 0; e < 4; ++e) S[rb][cq + e] = cs[e];
    __syncthreads();
    if (t < T) {
      float c = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) c += S[r][t];
      out[T + t] = c;
    }
  }
}

// NorMuon / MeqMuon, first step: one block per chunk of kRcChunk rows (or
// columns) of one matrix.  Each thread sums its row's (column's) squared
// norm of O over the tile partials (tile order; unrolled by 8 so that the
// loads are in flight together) and stores it; the block stores the
// chunk's count, mean norm, sum of squared deviations from that mean, sum
// of squared norms and count of non-zero norms.
__global__ __launch_bounds__(256) void rc_sum_kernel(Batch bt, Work wk) {
  __shared__ float red[12];
  const TileRef tr = decode(bt, wk, blockIdx.x);
  const MatGroup& g = *tr.g;
  const int ncr = (g.rows + kRcChunk - 1) / kRcChunk;
  const bool is_row = tr.tile < ncr;
  const int chunk = is_row ? tr.tile : tr.tile - ncr;
  const int n = is_row ? g.rows : g.cols;
  const int idx = chunk * kRcChunk + int(threadIdx.x);
  const bool valid = idx < n;
  const int tcn = g.tail_tiles_c, trn = g.tail_tiles / g.tail_tiles_c;
  const float* part = g.rc_part + tr.m * g.tail_tiles * (2 * T);
  float* srow = g.rc_norm2 + tr.m * (int64_t(g.rows) + g.cols);
  float* scol = srow + g.rows;
  float a = 0.f;
  if (valid) {
    if (is_row) {
      const int ti = idx / T, ri = idx - ti * T;
      const float* pr = part + int64_t(ti) * tcn * (2 * T) + ri;
#pragma unroll 8
      for (int tc = 0; tc < tcn; ++tc) a += pr[tc * (2 * T)];
      srow[idx] = a;
    } else {
      const int tc = idx / T, ci = idx - tc * T;
      const float* pc = part + int64_t(tc) * (2 * T) + T + ci;
#pragma unroll 8
      for (int ti = 0; ti < trn; ++ti) a += pc[int64_t(ti) * tcn * (2 * T)];
      scol[idx] = a;
    }
  }
  const int cnt = min(kRcChunk, n - chunk * kRcChunk);
  const float nrm = valid ? sqrtf(a) : 0.f;
  float sn = nrm, sa = a, nz = (valid && a > 0.f) ? 1.f : 0.f;
  block_sum3_256(sn, sa, nz, red);
  const float mean = sn / float(cnt);
  const float dv = valid ? nrm - mean : 0.f;
  const float m2 = block_sum_256(dv * dv, red);
  if (threadIdx.x == 0) {
    float* st = g.rc_stat + (tr.m * tr.per + tr.tile) * 5;
    st[0] = float(cnt);
    st[1] = mean;
    st[2] = m2;
    st[3] = sa;
    st[4] = nz;
  }
}

// Second step, by one thread per matrix (in tail_finalize_kernel): the chunk
// statistics of the rows and of the columns merged in chunk order (count,
// mean and sum of squared deviations by the pairwise update of Chan et
// al.), the direction to equalise (NorMuon: rows; MeqMuon: the one whose
// norms have the larger std/mean, rows on a tie) and the common norm
// target = ||O||_F / sqrt(count along it).  The apply kernel scales O by
// target/norm along that direction (0 for a zero row or column).
__device__ void rc_merge(const MatGroup& g, int64_t m, int variant) {
  const int ncr = (g.rows + kRcChunk - 1) / kRcChunk;
  const int nch = rc_chunks(g.rows, g.cols);
  const float* st = g.rc_stat + m * nch * 5;
  float spread[2], sum_a[2], nz[2];
  for (int side = 0; side < 2; ++side) {
    const int c0 = side == 0 ? 0 : ncr, c1 = side == 0 ? ncr : nch;
    float n = 0.f, mean = 0.f, m2 = 0.f, sa = 0.f, z = 0.f;
    for (int c = c0; c < c1; ++c) {
      const float* q = st + c * 5;
      const float nb = q[0], nab = n + nb, delta = q[1] - mean;
      mean = mean + delta * (nb / nab);
      m2 = m2 + q[2] + delta * delta * (n * nb / nab);
      n = nab;
      sa += q[3];
      z += q[4];
    }
    spread[side] = mean > 0.f ? sqrtf(m2 / n) / mean : 0.f;
    sum_a[side] = sa;
    nz[side] = z;
  }
  const bool rows_dir = variant == MUON_VARIANT_NORMUON || spread[0] >= spread[1];
  const float target = sqrtf(sum_a[0] / float(rows_dir ? g.rows : g.cols));
  float* sc = g.scal + m * kScal;
  sc[SC_RC_TARGET] = target;
  sc[SC_RC_ROWS] = rows_dir ? 1.f : 0.f;
  if (g.stats) g.stats[m * MUON_STATS_PER_MATRIX + 4] = target * target * nz[rows_dir ? 0 : 1];
}

// Per-matrix totals: ||W||^2, <W,O>, ||O||^2, the MuonGS coefficient and the
// optional stats; with rc (NorMuon, MeqMuon) also the equalisation's
// direction and target (rc_sum_kernel ran before).
__global__ __launch_bounds__(256) void tail_finalize_kernel(Batch bt, Work wk, int variant, int rc) {
  __shared__ double red[12];
  const TileRef tr = decode(bt, wk, blockIdx.x);
  const MatGroup& g = *tr.g;
  const double* part = g.tail_part + tr.m * g.red_tiles * 3;
  double dot = 0.0, ww = 0.0, oo = 0.0;
  for (int i = threadIdx.x; i < g.red_tiles; i += 256) {
    dot += part[3 * i + 0];
    ww += part[3 * i + 1];
    oo += part[3 * i + 2];
  }
  block_sum3_256(dot, ww, oo, red);
  if (threadIdx.x == 0) {
    // totals in fp64; each scalar rounded to fp32 once
    const double coef = (variant == MUON_VARIANT_MUONGS && ww > 0.0) ? dot / ww : 0.0;
    float hscale = 1.f;
    if (variant == MUON_VARIANT_MUONH) {
      // ||W^||^2 = ||d W - step O||^2 = d^2 ||W||^2 - 2 d step <W,O> + step^2 ||O||^2
      const double d = g.decay, st = g.step;
      const double h2 = d * d * ww - 2.0 * d * st * dot + st * st * oo;
      if (h2 > 0.0) hscale = float(sqrt(ww / h2));
    }
    float* sc = g.scal + tr.m * kScal;
    sc[SC_R2] = float(ww);
    sc[SC_DOT] = float(dot);
    sc[SC_O2] = float(oo);
    sc[SC_COEF] = float(coef);
    sc[SC_HSCALE] = hscale;
    if (g.stats) {
      float* st = g.stats + tr.m * MUON_STATS_PER_MATRIX;
      st[1] = float(ww);
      st[2] = float(dot);
      st[3] = float(oo);
      st[4] = float(fmax(oo - 2.0 * coef * dot + coef * coef * ww, 0.0));
    }
    if (rc) rc_merge(g, tr.m, variant);
  }
}

// W' = h * ((1 - lr*wd) W - lr*s*(O - coef*W)): coef the MuonGS projection
// coefficient, h the MuonH renormalisation (coef = 0, h = 1 for plain Muon).
// Blocks run in the reverse of the reduction's order, so that the first
// ones find the W and O tiles that the reduction read last still in the
// Infinity Cache.
template <bool BF16>
__global__ __launch_bounds__(256) void tail_apply_kernel(Batch bt, Work wk, int ns_steps,
                                                         int reduced, int rc) {
  using E = Elem<BF16>;
  using TE = typename E::T;
  __shared__ float S[T][T + 1];
  const TileRef tr = decode(bt, wk, reduced ? gridDim.x - 1 - blockIdx.x : blockIdx.x);
  const MatGroup& g = *tr.g;
  const TailTile tt = tail_tile(g, tr.tile, !rc);
  const int64_t elems = int64_t(g.rows) * g.cols;
  TE* W = mat_ptr<TE>(g.W_tab, g.W, tr.m, elems);
  const TE* X = reinterpret_cast<const TE*>((ns_steps & 1) ? g.X1 : g.X0) + tr.m * g.x_stride;
  const float* sc = g.scal + tr.m * kScal;
  const float oscale = ns_steps == 0 ? sc[SC_INV] : 1.0f;
  const float coef = reduced ? sc[SC_COEF] : 0.f;
  const float h = reduced ? sc[SC_HSCALE] : 1.f;
  const float step = g.step;
  const float wcoef = h * (g.decay + step * coef);
  const float ocoef = h * step * oscale;

  float w[4][4], o[4][4];
  bool valid[4][4];
  load_w_tile<BF16, false>(g, W, tt, w, valid);
  load_o_tile<BF16, false>(g, X, tt, S, o);

  if (rc) {
    // NorMuon / MeqMuon: O scaled by target/norm along the equalised
    // direction (0 for a zero row or column), by 1 along the other; indices
    // clamped so that a ragged tile reads inside the matrix's norms (the
    // clamped products are never stored).
    const float* srow = g.rc_norm2 + tr.m * (int64_t(g.rows) + g.cols);
    const float* scol = srow + g.rows;
    // (both sets of norms loaded unconditionally, beside the two scalars,
    // so that no load waits for another)
    float ra[4], ca[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) ra[k] = srow[min(tt.r0 + tt.rb + tt.rstep * k, g.rows - 1)];
#pragma unroll
    for (int e = 0; e < 4; ++e) ca[e] = scol[min(tt.c0 + tt.cq + e, g.cols - 1)];
    const float target = sc[SC_RC_TARGET];
    const bool rows_dir = sc[SC_RC_ROWS] != 0.f;
    auto scale_of = [&](float a) { return a > 0.f ? target / sqrtf(a) : 0.f; };
    float rsc[4], csc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) rsc[k] = rows_dir ? scale_of(ra[k]) : 1.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) csc[e] = rows_dir ? 1.f : scale_of(ca[e]);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[k][e] *= rsc[k] * csc[e];
  }
  const bool vec = (tt.c0 + tt.tc <= g.cols) && ((g.cols & 3) == 0) &&
                   ((reinterpret_cast<uintptr_t>(W) & (BF16 ? 7u : 15u)) == 0);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = tt.r0 + tt.rb + tt.rstep * k;
    if (r >= g.rows) continue;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = fmaf(wcoef, w[k][e], -ocoef * o[k][e]);
    const int64_t off = int64_t(r) * g.cols + tt.c0 + tt.cq;
    if (vec) {
      Vec4<BF16>::store(W + off, v);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (valid[k][e]) W[off + e] = E::cvt(v[e]);
    }
  }
}

inline dim3 grid_of(const Work& wk) { return dim3(unsigned(wk.begin[wk.ngroups])); }

}  // namespace

hipError_t launch_head(const Batch& bt, const Work& wk, bool bf16, float momentum, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(head_kernel<true>, grid_of(wk), dim3(256), 0, s, bt, wk, momentum);
  else
    hipLaunchKernelGGL(head_kernel<false>, grid_of(wk), dim3(256), 0, s, bt, wk, momentum);
  return hipGetLastError();
}

hipError_t launch_norm_finalize(const Batch& bt, const Work& wk, hipStream_t s) {
  hipLaunchKernelGGL(norm_finalize_kernel, grid_of(wk), dim3(256), 0, s, bt, wk);
  return hipGetLastError();
}

hipError_t launch_tail_reduce(const Batch& bt, const Work& wk, bool bf16, int ns_steps, bool rc,
                              hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(tail_reduce_kernel<true>, grid_of(wk), dim3(256), 0, s, bt, wk, ns_steps, int(rc));
  else
    hipLaunchKernelGGL(tail_reduce_kernel<false>, grid_of(wk), dim3(256), 0, s, bt, wk, ns_steps, int(rc));
  return hipGetLastError();
}

hipError_t launch_tail_finalize(const Batch& bt, const Work& wk, int variant, bool rc, hipStream_t s) {
  hipLaunchKernelGGL(tail_finalize_kernel, grid_of(wk), dim3(256), 0, s, bt, wk, variant, int(rc));
  return hipGetLastError();
}

hipError_t launch_rc_sum(const Batch& bt, const Work& wk, hipStream_t s) {
  hipLaunchKernelGGL(rc_sum_kernel, grid_of(wk), dim3(256), 0, s, bt, wk);
  return hipGetLastError();
}

hipError_t launch_tail_apply(const Batch& bt, const Work& wk, bool bf16, const Hyper& h,
                             bool reduced, hipStream_t s) {
  const int rc = (h.variant == MUON_VARIANT_NORMUON || h.variant == MUON_VARIANT_MEQMUON) ? 1 : 0;
  if (bf16)
    hipLaunchKernelGGL(tail_apply_kernel<true>, grid_of(wk), dim3(256), 0, s, bt, wk, h.ns_steps,
                       int(reduced), rc);
  else
    hipLaunchKernelGGL(tail_apply_kernel<false>, grid_of(wk), dim3(256), 0, s, bt, wk, h.ns_steps,
                       int(reduced), rc);
  return hipGetLastError();
}

}  // namespace muon
