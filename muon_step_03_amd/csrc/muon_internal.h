// Internal structures shared by the host dispatcher and the HIP kernels.
//
// Data layout in HBM (per shape group; every region 256-byte aligned):
//   X0, X1  [count][p_pad][q_pad]   Newton-Schulz iterate, ping-pong
//                                   (p_pad, q_pad: multiples of the GEMM
//                                   block tiles).  X is
//                                   the momentum look-ahead U in "short side
//                                   first" orientation: X = U if rows <= cols,
//                                   X = U^T otherwise.  Rows/cols beyond p/q
//                                   are zero, and stay zero under the
//                                   iteration, so the GEMM kernels need no
//                                   edge masking.
//   A, B    [count][p_pad][p_pad]   Gram matrix X X^T and polynomial a I + b A + c A A
//                                   (bf16 path; b A + c A A on the fp32 path)
//   head    [count][head_tiles]     per-tile partial sums of u^2 (fp64)
//   tail    [count][tail_tiles][3]  per-tile partials of <W,O>, ||W||^2, ||O||^2 (fp64)
//                                   (red_tiles <= tail_tiles of them are used)
//   scal    [count][kScal]          per-matrix scalars (norm, 1/(norm+eps), ...)
//   rc      [count][tail_tiles][128] per-tile row and column sums of O^2
//   rcs     [count][rows + cols]    squared row and column norms of O (NorMuon, MeqMuon)
//   rcst    [count][rc_chunks][5]   per-chunk statistics of those norms
// Element type of X, A, B is bf16 (bit pattern in uint16_t) on the bf16 path
// and float on the fp32 path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muon.h"

namespace muon {

constexpr int kMaxGroups = MUON_GROUPS_PER_LAUNCH;
constexpr int kEwTile = 64;
// Rows or columns per block of the NorMuon/MeqMuon norm sums.
constexpr int kRcChunk = 256;
inline __host__ __device__ int rc_chunks(int rows, int cols) {
  return (rows + kRcChunk - 1) / kRcChunk + (cols + kRcChunk - 1) / kRcChunk;
}        // head/tail tile edge (elements)
// bf16 Newton-Schulz block tiles (wave tile = block tile / 2 in each
// dimension, 4 waves per block).
#ifndef MUON_SYRK_TILE
#define MUON_SYRK_TILE 128
#endif
#ifndef MUON_UPD_TILE_M
#define MUON_UPD_TILE_M 128
#endif
#ifndef MUON_UPD_TILE_N
#define MUON_UPD_TILE_N 256
#endif
// Waves per update block (4: 128x256 tiles, two blocks per CU; 8: larger
// tiles, one block per CU).
#ifndef MUON_UPD_WAVES
#define MUON_UPD_WAVES 4
#endif
constexpr int kUpdWaves = MUON_UPD_WAVES;
constexpr int kUpdBlocksPerCU = kUpdWaves == 8 ? 1 : 2;
// Blocks per CU of the symmetric products (2: four stages of 16 KB each).
#ifndef MUON_SYRK_OCC
#define MUON_SYRK_OCC 2
#endif
constexpr int kSyrkBlocksPerCU = MUON_SYRK_OCC;
constexpr int kSyrkTile = MUON_SYRK_TILE;   // symmetric products: square tiles
// 256x256 tiles (8 waves, one block per CU) for matrices whose short side
// is at least kBigMinP and whose padded sides are multiples of 256, in a
// launch that then holds at least kSyrkBigMinRounds (symmetric products) or
// kUpdBigMinRounds (update) tiles per CU; otherwise the 128-wide tiles.
#ifndef MUON_SYRK_BIG_MIN_P
#define MUON_SYRK_BIG_MIN_P 512
#endif
constexpr int kBigTile = 256;
constexpr int kBigMinP = MUON_SYRK_BIG_MIN_P;
constexpr int kBigBlocksPerCU = 1;
// Short side from which the polynomial also takes 256x256 tiles.
#ifndef MUON_POLY_BIG_MIN_P
#define MUON_POLY_BIG_MIN_P 2048
#endif
constexpr int kPolyBigMinP = MUON_POLY_BIG_MIN_P;
#ifndef MUON_SYRK_BIG_MIN_ROUNDS
#define MUON_SYRK_BIG_MIN_ROUNDS 4
#endif
#ifndef MUON_UPD_BIG_MIN_ROUNDS
#define MUON_UPD_BIG_MIN_ROUNDS 8
#endif
constexpr int kSyrkBigMinRounds = MUON_SYRK_BIG_MIN_ROUNDS;
constexpr int kUpdBigMinRounds = MUON_UPD_BIG_MIN_ROUNDS;
constexpr int kSyrkBigTile = kBigTile;
constexpr int kUpdBigTile = kBigTile;
constexpr int kUpdTileM = MUON_UPD_TILE_M;  // update: rows (along p)
constexpr int kUpdTileN = MUON_UPD_TILE_N;  // update: columns (along q)
constexpr int kBf16PadP = kSyrkTile > kUpdTileM ? kSyrkTile : kUpdTileM;
constexpr int kBf16PadQ = kUpdTileN > kSyrkTile ? kUpdTileN : kSyrkTile;
constexpr int kF32Tile = 64;       // fp32 GEMM block tile edge
constexpr double kEpsNorm = 1e-7;  // added to ||U||_F before dividing

// Per-matrix scalar slots.
enum : int {
  SC_NORM = 0,   // ||U||_F
  SC_INV = 1,    // 1 / (||U||_F + eps)
  SC_R2 = 2,     // ||W||_F^2
  SC_DOT = 3,    // <W, O>_F
  SC_O2 = 4,     // ||O||_F^2
  SC_COEF = 5,   // MuonGS projection coefficient <W,O>/||W||^2 (0 otherwise)
  SC_HSCALE = 6, // MuonH renormalisation ||W|| / ||W^|| (1 otherwise)
  SC_RC_TARGET = 7,  // NorMuon/MeqMuon: the common norm ||O||_F / sqrt(count)
  SC_RC_ROWS = 8,    // NorMuon/MeqMuon: 1 if the rows are equalised, 0 if the columns
  kScal = 10
};

// One shape group as the kernels see it.
struct MatGroup {
  void* const* W_tab;
  const void* const* G_tab;
  float* const* M_tab;
  char* W;
  const char* G;
  float* M;
  int64_t count;
  int rows, cols;      // weight orientation
  int p, q;            // short side, long side
  int p_pad, q_pad;    // padded X extents
  int trans;           // 1 when rows > cols (X = U^T)
  int head_tiles;      // head tiles per matrix (X orientation, 64x64)
  int tail_tiles;      // tail tiles per matrix (W orientation, 64x64)
  int tail_tiles_c;    // tail tiles along cols
  char* X0;
  char* X1;
  char* A;
  char* B;
  int64_t x_stride;    // elements between matrices in X0/X1
  int64_t a_stride;    // elements between matrices in A/B
  double* head_part;   // [count][head_tiles]: per-tile sums of u^2 (fp64)
  double* tail_part;   // [count][red_tiles][3]: per-tile <W,O>, ||W||^2, ||O||^2 (fp64)
  float* rc_part;      // [count][tail_tiles][128]: per-tile row and column sums of O^2
  float* rc_norm2;     // [count][rows + cols]: squared row, then column norms of O
  float* rc_stat;      // [count][rc_chunks(rows, cols)][5]: per-chunk norm statistics
  float* scal;
  float* stats;        // MUON_STATS_PER_MATRIX per matrix, or null
  float decay;         // 1 - lr*wd
  float step;          // lr * s, s = 0.2*sqrt(max(rows, cols)) or max(1, rows/cols)^0.5
  int fuse;            // 1: the last update applies W' = decay W - step O itself
  int red;             // 1: the last update writes the tail partials of <W,O>,
                       //    ||W||^2, ||O||^2 (one triple per update tile)
  int red_tiles;       // tail partials per matrix: update tiles when red, tail tiles otherwise
};

struct Batch {
  MatGroup g[kMaxGroups];
  int ngroups;
};

// How one launch splits into blocks: `tiles[g]` blocks per matrix of group g,
// blocks of group g are [begin[g], begin[g+1]).
struct Work {
  int64_t begin[kMaxGroups + 1];
  int tiles[kMaxGroups];
  int ngroups;
};

// Static tile list of a persistent Newton-Schulz launch: groups in processing
// order (longest K first), n[i] tiles (count x tiles per matrix) of group
// group[i]; 8 * blocks_per_xcd blocks.
struct TileList {
  int64_t n[kMaxGroups];
  int tiles[kMaxGroups];
  int group[kMaxGroups];
  int ngroups;
  int blocks_per_xcd;
  int fuse_tail;   // update launch of the last iteration: kLastApply (groups with
                   // fuse set write W' instead of X') or kLastReduce (groups with
                   // red set also write the tail partials); 0 otherwise
};
enum : int { kLastApply = 1, kLastReduce = 2 };

struct Hyper {
  float lr;
  float momentum;
  float wd;
  float a, b, c;
  int ns_steps;
  int variant;
};

// ---------------------------------------------------------------- device side
__device__ __forceinline__ int find_group(const Work& w, int64_t bid) {
  int g = 0;
  while (g + 1 < w.ngroups && bid >= w.begin[g + 1]) ++g;
  return g;
}

template <typename T>
__device__ __forceinline__ T* mat_ptr(void* const* tab, char* base, int64_t m, int64_t elems) {
  return tab ? reinterpret_cast<T*>(tab[m]) : reinterpret_cast<T*>(base) + m * elems;
}
template <typename T>
__device__ __forceinline__ const T* mat_cptr(const void* const* tab, const char* base, int64_t m,
                                             int64_t elems) {
  return tab ? reinterpret_cast<const T*>(tab[m]) : reinterpret_cast<const T*>(base) + m * elems;
}

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// float -> bf16, round to nearest even (the hardware conversion
// v_cvt_pk_bf16_f32); NaN stays NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// Two floats -> two bf16 packed in one word (a in the low half), one instruction.
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
  using T = uint16_t;
  static __device__ __forceinline__ float load(const T* p) { return bf2f(*p); }
  static __device__ __forceinline__ T cvt(float f) { return f2bf(f); }
  static __device__ __forceinline__ float to_f(T v) { return bf2f(v); }
};
template <>
struct Elem<false> {
  using T = float;
  static __device__ __forceinline__ float load(const T* p) { return *p; }
  static __device__ __forceinline__ T cvt(float f) { return f; }
  static __device__ __forceinline__ float to_f(T v) { return v; }
};

// Sum of v over the 256-thread block, in a fixed order (deterministic).
// `red` must hold 4 values of LDS.  Result valid in every thread.
template <typename F>
__device__ __forceinline__ F block_sum_256(F v, F* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// ---------------------------------------------------------------- AdamW
// One launch covers up to kAdamSegs parameter tensors; each block updates
// kAdamChunk consecutive elements of one tensor.
constexpr int kAdamSegs = MUON_ADAMW_TENSORS_PER_LAUNCH;
constexpr int kAdamVec = 4;                    // elements per vector access
constexpr int kAdamVecPerThread = 4;           // vectors per thread per block
constexpr int kAdamChunk = 256 * kAdamVec * kAdamVecPerThread;

struct AdamSeg {
  void* P;              // parameters (bf16 bits or float)
  const void* G;        // gradients, same dtype as P
  float* m;             // first moment
  float* v;             // second moment
  int64_t n;            // elements
  float decay;          // 1 - lr*wd
  float step_size;      // lr / (1 - beta1^t)
  int vec;              // 1: all four pointers allow kAdamVec-wide accesses
  int pad_;
};

struct AdamBatch {
  AdamSeg seg[kAdamSegs];
  int64_t begin[kAdamSegs + 1];  // blocks of tensor s are [begin[s], begin[s+1])
  int nseg;
  float beta1, beta2, eps;
  float one_minus_beta1, one_minus_beta2;  // rounded once from double (not 1 - float(beta))
  float inv_sqrt_bc2;            // 1 / sqrt(1 - beta2^t)
};

// ------------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error.
hipError_t launch_head(const Batch& bt, const Work& wk, bool bf16, float momentum, hipStream_t s);
hipError_t launch_norm_finalize(const Batch& bt, const Work& wk, hipStream_t s);
// `rc`: also the per-tile row and column sums of O^2 (NorMuon, MeqMuon).
hipError_t launch_tail_reduce(const Batch& bt, const Work& wk, bool bf16, int ns_steps, bool rc,
                              hipStream_t s);
hipError_t launch_tail_finalize(const Batch& bt, const Work& wk, int variant, bool rc, hipStream_t s);
// NorMuon / MeqMuon: row and column norms of O, the direction to equalise and
// the per-row and per-column scales (one block per matrix).
hipError_t launch_rc_sum(const Batch& bt, const Work& wk, hipStream_t s);
// `reduced`: tail_finalize ran, so the per-matrix coefficient and MuonH
// scale are read from the scalars (otherwise 0 and 1).
hipError_t launch_tail_apply(const Batch& bt, const Work& wk, bool bf16, const Hyper& h,
                             bool reduced, hipStream_t s);
// Newton-Schulz products.  `iter` selects X0/X1 and the first-iteration norm
// scaling.
hipError_t launch_gram_bf16(const Batch& bt, const TileList& tl, int iter, bool big, hipStream_t s);
// The bf16 polynomial stores B = a*I + b*A + c*A*A, so that the bf16 update
// is the plain product X' = B X.
hipError_t launch_poly_bf16(const Batch& bt, const TileList& tl, float a, float b, float c, bool big,
                            hipStream_t s);
// Update tile configurations: 128x256 (two blocks per CU), 256x256 (one
// block per CU) and 512x128 (one block per CU, matrices whose padded short
// side is 512: their long side is padded to a multiple of 128 only).
enum : int { kUpdCfg128 = 0, kUpdCfg256 = 1, kUpdCfg512 = 2 };
constexpr int kUpd512P = 512;
constexpr int kUpd512TileN = 128;
hipError_t launch_update_bf16(const Batch& bt, const TileList& tl, int iter, int cfg, hipStream_t s);
hipError_t launch_gram_f32(const Batch& bt, const Work& wk, int iter, hipStream_t s);
hipError_t launch_poly_f32(const Batch& bt, const Work& wk, float b, float c, hipStream_t s);
hipError_t launch_update_f32(const Batch& bt, const Work& wk, int iter, float a, hipStream_t s);
// AdamW over the tensors of `bt`: begin[nseg] blocks.
hipError_t launch_adamw(const AdamBatch& bt, bool bf16, hipStream_t s);

}  // namespace muon
