// AdamW for the parameters a hybrid Muon optimizer keeps off Muon (input
// embedding, output head, gains and biases): "LLM Pretraining Loss Spike 진단과
// 처방" (juhoplayground.github.io), section "Muon head의 실체는 하이브리드
// 옵티마이저다"; betas, eps and weight decay from the experiments paragraph of
// "MuonGS: Pretraining LLMs with Relaxed Weight-Norm Control" (onedev.kr).
// Decoupled AdamW with bias correction, per element, in float32:
//
//   m' = b1 m + (1 - b1) g
//   v' = b2 v + (1 - b2) g^2
//   p' = (1 - lr wd) p - (lr / (1 - b1^t)) m' / (sqrt(v') / sqrt(1 - b2^t) + eps)
//
// Purely HBM-bound: 22 bytes per element with bf16 p and g (p r/w, g r, m r/w,
// v r/w), 28 with float32.  One launch covers many tensors; every block owns
// kAdamChunk consecutive elements of one tensor.  Each thread handles
// kAdamVecPerThread vectors of 4 elements at a stride of 256 vectors, so every
// wave instruction reads or writes one contiguous run; all loads of a thread
// are issued before its arithmetic.
#include "muon_internal.h"

namespace muon {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

struct Coef {
  float b1, omb1, b2, omb2, eps, inv_sqrt_bc2, decay, step_size;
};

// Every rounding is spelled out (explicit fused multiply-adds, contraction
// off), so the vector and per-element paths give identical bits.
__device__ __forceinline__ float adam_elem(float p, float g, float& m, float& v, const Coef& c) {
#pragma clang fp contract(off)
  m = __builtin_fmaf(c.b1, m, c.omb1 * g);
  v = __builtin_fmaf(c.b2, v, c.omb2 * (g * g));
  const float denom = __builtin_fmaf(__builtin_sqrtf(v), c.inv_sqrt_bc2, c.eps);
  return __builtin_fmaf(c.decay, p, -(c.step_size * (m / denom)));
}

// Every stream is read and written once per step: nontemporal accesses
// (evict-first in the caches).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <bool BF16>
__device__ __forceinline__ f32x4 load4(const void* base, int64_t e) {
  if constexpr (BF16) {
    const u16x4 h = __builtin_nontemporal_load(
        reinterpret_cast<const u16x4*>(static_cast<const uint16_t*>(base) + e));
    return f32x4{bf2f(h.x), bf2f(h.y), bf2f(h.z), bf2f(h.w)};
  } else {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + e));
  }
}

template <bool BF16>
__device__ __forceinline__ void store4(void* base, int64_t e, f32x4 x) {
  if constexpr (BF16) {
    const u32x2 w = {f2bf2(x.x, x.y), f2bf2(x.z, x.w)};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + e));
  } else {
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(static_cast<float*>(base) + e));
  }
}
__device__ __forceinline__ f32x4 load4f(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void store4f(float* p, f32x4 x) {
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}

template <bool BF16>
__global__ __launch_bounds__(256) void adamw_kernel(const AdamBatch bt) {
  const int64_t b = blockIdx.x;
  int s = 0;
  while (s + 1 < bt.nseg && b >= bt.begin[s + 1]) ++s;
  const AdamSeg& sg = bt.seg[s];
  const int64_t base = (b - bt.begin[s]) * int64_t(kAdamChunk);
  const Coef c{bt.beta1, bt.one_minus_beta1, bt.beta2, bt.one_minus_beta2, bt.eps, bt.inv_sqrt_bc2,
               sg.decay, sg.step_size};
  const int t = threadIdx.x;

  if (sg.vec && base + kAdamChunk <= sg.n) {
    f32x4 p[kAdamVecPerThread], g[kAdamVecPerThread], m[kAdamVecPerThread], v[kAdamVecPerThread];
#pragma unroll
    for (int j = 0; j < kAdamVecPerThread; ++j) {
      const int64_t e = base + int64_t(j * 256 + t) * kAdamVec;
      p[j] = load4<BF16>(sg.P, e);
      g[j] = load4<BF16>(sg.G, e);
      m[j] = load4f(sg.m + e);
      v[j] = load4f(sg.v + e);
    }
#pragma unroll
    for (int j = 0; j < kAdamVecPerThread; ++j) {
      const int64_t e = base + int64_t(j * 256 + t) * kAdamVec;
      f32x4 r;
#pragma unroll
      for (int k = 0; k < kAdamVec; ++k) {
        float mk = m[j][k], vk = v[j][k];
        r[k] = adam_elem(p[j][k], g[j][k], mk, vk, c);
        m[j][k] = mk;
        v[j][k] = vk;
      }
      store4<BF16>(sg.P, e, r);
      store4f(sg.m + e, m[j]);
      store4f(sg.v + e, v[j]);
    }
    return;
  }
  // The last, partial chunk of a tensor (or a tensor whose pointers do not
  // allow vector accesses): one element per thread per pass.
  const int64_t end = base + kAdamChunk < sg.n ? base + kAdamChunk : sg.n;
  using E = Elem<BF16>;
  typename E::T* P = static_cast<typename E::T*>(sg.P);
  const typename E::T* G = static_cast<const typename E::T*>(sg.G);
  for (int64_t e = base + t; e < end; e += 256) {
    float m = sg.m[e], v = sg.v[e];
    const float r = adam_elem(E::load(P + e), E::load(G + e), m, v, c);
    P[e] = E::cvt(r);
    sg.m[e] = m;
    sg.v[e] = v;
  }
}

}  // namespace

hipError_t launch_adamw(const AdamBatch& bt, bool bf16, hipStream_t s) {
  const dim3 grid(unsigned(bt.begin[bt.nseg]));
  if (bf16)
    hipLaunchKernelGGL(adamw_kernel<true>, grid, dim3(256), 0, s, bt);
  else
    hipLaunchKernelGGL(adamw_kernel<false>, grid, dim3(256), 0, s, bt);
  return hipGetLastError();
}

}  // namespace muon
