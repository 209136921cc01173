// AdamW for the parameters outside the Muon groups.  "Muon Meets Mamba"
// (abstract and experiments) compares Muon with AdamW and keeps AdamW for
// the parameters that are not projection weights; the formula is the usual
// one with decoupled weight decay and bias-corrected moments (step t from 1):
//   m' = b1 m + (1 - b1) g,   v' = b2 v + (1 - b2) g^2,
//   p' = p (1 - lr wd) - (lr / (1 - b1^t)) m' / (sqrt(v') / sqrt(1 - b2^t) + eps).
// One launch covers up to kAdamwMax tensors of any sizes: the grid is cut into
// blocks of kAdamwBlock elements, each block finds its tensor in the prefix
// table of block offsets.  Purely elementwise and HBM-bound (26 bytes per
// element with bf16 gradients: p, m, v read and written, g read).
#include "common.cuh"
#include "launch.h"

namespace muon {
namespace {

__device__ __forceinline__ void adamw1(float& p, float& m, float& v, float g, const AdamwLaunch& A) {
  m = fmaf(A.beta1, m, A.one_m_b1 * g);
  v = fmaf(A.beta2, v, A.one_m_b2 * g * g);
  const float denom = sqrtf(v) * A.inv_sqrt_bc2 + A.eps;
  p = fmaf(p, A.decay, -A.lr_bc * (m / denom));
}

template <typename GT>
__device__ __forceinline__ float gval(const void* g, long long i);
template <> __device__ __forceinline__ float gval<float>(const void* g, long long i) {
  return static_cast<const float*>(g)[i];
}
template <> __device__ __forceinline__ float gval<bf16_t>(const void* g, long long i) {
  return bf16_to_f32(static_cast<const bf16_t*>(g)[i]);
}

template <typename GT>
__global__ void __launch_bounds__(256) adamw_kernel(AdamwLaunch A) {
  int t = 0;
  while (t + 1 < A.nt && static_cast<long long>(blockIdx.x) >= A.t[t + 1].block0) ++t;
  const AdamwTensor& T = A.t[t];
  const long long e0 = (static_cast<long long>(blockIdx.x) - T.block0) * kAdamwBlock;
  const long long e1 = e0 + kAdamwBlock < T.n ? e0 + kAdamwBlock : T.n;
  const uintptr_t al = reinterpret_cast<uintptr_t>(T.p) | reinterpret_cast<uintptr_t>(T.m) |
                       reinterpret_cast<uintptr_t>(T.v) |
                       (reinterpret_cast<uintptr_t>(T.g) & (sizeof(GT) == 2 ? 7u : 15u));
  if ((al & 15u) == 0 && e1 - e0 == kAdamwBlock) {
    // full block, aligned: 4 consecutive elements per thread and load, every
    // load of the block issued before the first store (the tensors may not
    // be proven disjoint, so the compiler would not reorder them itself);
    // non-temporal, since every element is touched once per step (+12% over
    // cached accesses on the Mamba-2-130M parameter set)
    constexpr int U = kAdamwBlock / (256 * 4);
    f32x4_t p[U], m[U], v[U];
    float g[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long i = e0 + (static_cast<long long>(u) * 256 + threadIdx.x) * 4;
      p[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(T.p + i));
      m[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(T.m + i));
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(T.v + i));
      if constexpr (sizeof(GT) == 2) {
        const u32x2_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(static_cast<const bf16_t*>(T.g) + i));
        g[u][0] = lo_bf16(w[0]); g[u][1] = hi_bf16(w[0]); g[u][2] = lo_bf16(w[1]); g[u][3] = hi_bf16(w[1]);
      } else {
        const f32x4_t w = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(T.g) + i);
        g[u][0] = w[0]; g[u][1] = w[1]; g[u][2] = w[2]; g[u][3] = w[3];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float pe = p[u][e], me = m[u][e], ve = v[u][e];
        adamw1(pe, me, ve, g[u][e], A);
        p[u][e] = pe; m[u][e] = me; v[u][e] = ve;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long i = e0 + (static_cast<long long>(u) * 256 + threadIdx.x) * 4;
      __builtin_nontemporal_store(p[u], reinterpret_cast<f32x4_t*>(T.p + i));
      __builtin_nontemporal_store(m[u], reinterpret_cast<f32x4_t*>(T.m + i));
      __builtin_nontemporal_store(v[u], reinterpret_cast<f32x4_t*>(T.v + i));
    }
  } else {
    for (long long i = e0 + threadIdx.x; i < e1; i += 256) {
      float p = T.p[i], m = T.m[i], v = T.v[i];
      adamw1(p, m, v, gval<GT>(T.g, i), A);
      T.p[i] = p; T.m[i] = m; T.v[i] = v;
    }
  }
}

}  // namespace

hipError_t launch_adamw(const AdamwLaunch& A, bool grad_bf16, int blocks, hipStream_t st) {
  if (blocks == 0) return hipSuccess;
  if (grad_bf16) hipLaunchKernelGGL(adamw_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, A);
  else hipLaunchKernelGGL(adamw_kernel<float>, dim3(blocks), dim3(256), 0, st, A);
  return hipGetLastError();
}

}  // namespace muon
