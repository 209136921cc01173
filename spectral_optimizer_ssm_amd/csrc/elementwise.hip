// HBM-bound passes of the Muon step: the fused momentum / Nesterov /
// Frobenius-partials pass that opens the step and the apply pass that closes
// it.  The momentum rule is heavy-ball without dampening with the Nesterov
// look-ahead, the plain reading taken for the optimizer momentum that
// "Muon Meets Mamba" (abstract) leaves unstated; the descent step is the
// "steepest descent under the spectral norm" of the same abstract.
//
// Both passes also move between the user's m x n layout and the oriented
// iterate X (s x l, s = min(m, n)) that the Newton-Schulz kernels work on:
// for a tall matrix X = U^T, transposed through an LDS tile so that global
// reads and writes stay coalesced.  X is zero-padded to s_pad x ld.
#include "common.cuh"
#include "launch.h"

namespace muon {

// 16-byte vector loads and stores; NT marks data touched once in the step
// (read once, or written and not read again by this step) as non-temporal.
// A contiguous momentum-shaped stream reached 6.1 TB/s with it against 5.3
// plain, but the momentum passes themselves measured slower with it (their
// 32-byte-per-lane M accesses), so only the apply passes use it.
template <bool NT, typename V>
__device__ __forceinline__ V ld16(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
  else return *reinterpret_cast<const V*>(p);
}
template <bool NT, typename V>
__device__ __forceinline__ void st16(void* p, V v) {
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
  else *reinterpret_cast<V*>(p) = v;
}

template <typename T> struct Vec8;
template <> struct Vec8<float> {
  template <bool NT = false>
  __device__ static void load(const float* p, float* v) {
    const f32x4_t a = ld16<NT, f32x4_t>(p);
    const f32x4_t b = ld16<NT, f32x4_t>(p + 4);
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  }
  template <bool NT = false>
  __device__ static void store(float* p, const float* v) {
    f32x4_t a = {v[0], v[1], v[2], v[3]};
    f32x4_t b = {v[4], v[5], v[6], v[7]};
    st16<NT>(p, a);
    st16<NT>(p + 4, b);
  }
};
template <> struct Vec8<bf16_t> {
  template <bool NT = false>
  __device__ static void load(const bf16_t* p, float* v) {
    const u32x4_t a = ld16<NT, u32x4_t>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = lo_bf16(a[i]); v[2 * i + 1] = hi_bf16(a[i]); }
  }
  template <bool NT = false>
  __device__ static void store(bf16_t* p, const float* v) {
    u32x4_t a;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    st16<NT>(p, a);
  }
};

__device__ __forceinline__ bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename T> __device__ __forceinline__ float ld1(const T* p);
template <> __device__ __forceinline__ float ld1<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld1<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }
template <typename T> __device__ __forceinline__ void st1(T* p, float v);
template <> __device__ __forceinline__ void st1<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st1<bf16_t>(bf16_t* p, float v) { *p = f32_to_bf16(v); }

// M' = beta M + G;  U = G + beta M' (nesterov) or M';  no momentum: U = G.
__device__ __forceinline__ float momentum1(float g, float* mp, bool has_m, float beta, bool nesterov) {
  if (!has_m) return g;
  const float mn = fmaf(beta, *mp, g);
  *mp = mn;
  return nesterov ? fmaf(beta, mn, g) : mn;
}

// ---------------------------------------------------------------------------
// Wide matrices (m <= n): X = U, elementwise.  grid = (P, matrices).
// ---------------------------------------------------------------------------
template <typename GT, typename XT>
__global__ void __launch_bounds__(256) momentum_wide_kernel(PtrTable G, MutPtrTable M, XT* X, long long xstride,
                                                            int m, int n, int ldg, int s_pad, int ld, float beta,
                                                            int nesterov, float* partials, int P) {
  __shared__ float red[8];
  const int z = blockIdx.y;
  const GT* g = static_cast<const GT*>(G.p[z]);
  float* mm = static_cast<float*>(M.p[z]);
  XT* x = X + z * xstride;
  const bool has_m = mm != nullptr;
  const bool nest = nesterov != 0;
  const long long chunks = static_cast<long long>(s_pad) * (ld / 8);
  const int cpr = ld / 8;
  const bool vec = (n % 8) == 0 && (ldg % 8) == 0 && a16(g) && (!has_m || a16(mm));
  float ss = 0.0f;
  for (long long c = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; c < chunks;
       c += static_cast<long long>(gridDim.x) * blockDim.x) {
    const int r = static_cast<int>(c / cpr);
    const int c0 = static_cast<int>(c % cpr) * 8;
    float u[8];
    if (r < m && c0 < n && vec) {
      float gv[8], mv[8];
      const long long off = static_cast<long long>(r) * n + c0;
      Vec8<GT>::load(g + static_cast<long long>(r) * ldg + c0, gv);
      if (has_m) Vec8<float>::load(mm + off, mv);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u[j] = momentum1(gv[j], &mv[j], has_m, beta, nest);
        ss = fmaf(u[j], u[j], ss);
      }
      if (has_m) Vec8<float>::store(mm + off, mv);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u[j] = 0.0f;
        if (r < m && c0 + j < n) {
          const long long off = static_cast<long long>(r) * n + c0 + j;
          u[j] = momentum1(ld1<GT>(g + static_cast<long long>(r) * ldg + c0 + j), mm + off, has_m, beta, nest);
          ss = fmaf(u[j], u[j], ss);
        }
      }
    }
    Vec8<XT>::store(x + static_cast<long long>(r) * ld + c0, u);
  }
  ss = block_sum(ss, red);
  if (threadIdx.x == 0) partials[static_cast<long long>(z) * P + blockIdx.x] = ss;
}

// ---------------------------------------------------------------------------
// Tall matrices (m > n): X = U^T through a 64 x 64 LDS tile.  A workgroup
// takes kTallTiles consecutive tiles along X's long side and writes one
// partial; grid = (row blocks x tile groups, matrices), P = workgroups per
// matrix.
// ---------------------------------------------------------------------------
constexpr int kTallTiles = 2;
template <typename GT, typename XT>
__global__ void __launch_bounds__(256) momentum_tall_kernel(PtrTable G, MutPtrTable M, XT* X, long long xstride,
                                                            int m, int n, int ldg, int s_pad, int ld, float beta,
                                                            int nesterov, float* partials, int P) {
  __shared__ float tile[64][65];
  __shared__ float red[8];
  const int z = blockIdx.y;
  const GT* g = static_cast<const GT*>(G.p[z]);
  float* mm = static_cast<float*>(M.p[z]);
  XT* x = X + z * xstride;
  const bool has_m = mm != nullptr;
  const bool nest = nesterov != 0;
  const int tiles_k = (ld + 63) / 64;
  const int groups_k = (tiles_k + kTallTiles - 1) / kTallTiles;
  const int i0 = (blockIdx.x / groups_k) * 64;  // X rows  = U columns (short side)
  const int kt0 = (blockIdx.x % groups_k) * kTallTiles;
  const int kt1 = kt0 + kTallTiles < tiles_k ? kt0 + kTallTiles : tiles_k;
  const bool vec = (n % 8) == 0 && (ldg % 8) == 0 && a16(g) && (!has_m || a16(mm));
  const int t = threadIdx.x;
  float ss = 0.0f;
  for (int kt = kt0; kt < kt1; ++kt) {
  const int k0 = kt * 64;                          // X cols  = U rows    (long side)
  if (kt != kt0) __syncthreads();                  // the previous tile's transposed reads are done
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int kr = t / 8 + 32 * pass;
    const int ic = (t % 8) * 8;
    const int ur = k0 + kr, uc = i0 + ic;
    float u[8];
    if (ur < m && uc + 7 < n && vec) {
      float gv[8], mv[8];
      const long long off = static_cast<long long>(ur) * n + uc;
      Vec8<GT>::load(g + static_cast<long long>(ur) * ldg + uc, gv);
      if (has_m) Vec8<float>::load(mm + off, mv);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u[j] = momentum1(gv[j], &mv[j], has_m, beta, nest);
        ss = fmaf(u[j], u[j], ss);
      }
      if (has_m) Vec8<float>::store(mm + off, mv);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u[j] = 0.0f;
        if (ur < m && uc + j < n) {
          const long long off = static_cast<long long>(ur) * n + uc + j;
          u[j] = momentum1(ld1<GT>(g + static_cast<long long>(ur) * ldg + uc + j), mm + off, has_m, beta, nest);
          ss = fmaf(u[j], u[j], ss);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[kr][ic + j] = u[j];
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int ir = t / 8 + 32 * pass;
    const int kc = (t % 8) * 8;
    if (i0 + ir < s_pad && k0 + kc < ld) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = tile[kc + j][ir];
      Vec8<XT>::store(x + static_cast<long long>(i0 + ir) * ld + k0 + kc, v);
    }
  }
  }
  ss = block_sum(ss, red);
  if (threadIdx.x == 0) partials[static_cast<long long>(z) * P + blockIdx.x] = ss;
}

// ---------------------------------------------------------------------------
// Apply: O = X (or X^T), optionally scaled by 1/(nu+eps) when no Newton-Schulz
// step ran; W -= lr*scale*O; optional copy of O to the user.
// ---------------------------------------------------------------------------
struct ApplyArgs {
  const float* partials;  // non-null: scale X by 1/(nu+eps) (zero-step case)
  int P;
  float eps;
  float neg_lr_scale;
  const float* cap_part;  // spectral cap (see ApplyLaunch)
  int cap_P;
  const float* cap_sigma;
  float cap;
  PtrTable cu, cv;
};

__device__ __forceinline__ float apply_prologue(const ApplyArgs& a, int z, float* red) {
  if (a.partials == nullptr) return 1.0f;
  return inv_norm_from_partials(a.partials + static_cast<long long>(z) * a.P, a.P, a.eps, red, nullptr);
}

// gamma of the spectral cap for matrix z (0 when the cap is off or inactive):
// c = u^T O v from fixed-order partial sums.
__device__ __forceinline__ float cap_gamma(const ApplyArgs& a, int z, float* red) {
  if (a.cap_part == nullptr) return 0.0f;
  float c = 0.0f;
  for (int i = threadIdx.x; i < a.cap_P; i += blockDim.x) c += a.cap_part[static_cast<long long>(z) * a.cap_P + i];
  c = block_sum(c, red);
  return (a.cap_sigma[z] >= a.cap && c < 0.0f) ? c : 0.0f;
}

template <typename XT>
__global__ void __launch_bounds__(256) apply_wide_kernel(const XT* X, long long xstride, int m, int n, int ld,
                                                         int ldo, MutPtrTable W, MutPtrTable O, ApplyArgs a) {
  __shared__ float red[8];
  const int z = blockIdx.y;
  const XT* x = X + z * xstride;
  float* w = static_cast<float*>(W.p[z]);
  XT* o = static_cast<XT*>(O.p[z]);
  const float inv = apply_prologue(a, z, red);
  const float gamma = cap_gamma(a, z, red);
  const float* cu = static_cast<const float*>(a.cu.p[z]);
  const float* cv = static_cast<const float*>(a.cv.p[z]);
  const int cpr = (n + 7) / 8;
  const long long chunks = static_cast<long long>(m) * cpr;
  const bool vec = (n % 8) == 0 && (ldo % 8) == 0 && (!w || a16(w)) && (!o || a16(o));
  for (long long c = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; c < chunks;
       c += static_cast<long long>(gridDim.x) * blockDim.x) {
    const int r = static_cast<int>(c / cpr);
    const int c0 = static_cast<int>(c % cpr) * 8;
    const long long off = static_cast<long long>(r) * n + c0;
    const long long ooff = static_cast<long long>(r) * ldo + c0;
    if (vec) {
      float ov[8], wv[8];
      Vec8<XT>::template load<true>(x + static_cast<long long>(r) * ld + c0, ov);
#pragma unroll
      for (int j = 0; j < 8; ++j) ov[j] *= inv;
      if (gamma != 0.0f) {
        const float gu = gamma * cu[r];
#pragma unroll
        for (int j = 0; j < 8; ++j) ov[j] = fmaf(-gu, cv[c0 + j], ov[j]);
      }
      if (o) Vec8<XT>::template store<true>(o + ooff, ov);
      if (w) {
        Vec8<float>::template load<true>(w + off, wv);
#pragma unroll
        for (int j = 0; j < 8; ++j) wv[j] = fmaf(a.neg_lr_scale, ov[j], wv[j]);
        Vec8<float>::template store<true>(w + off, wv);
      }
    } else {
      for (int j = 0; j < 8 && c0 + j < n; ++j) {
        float ov = ld1<XT>(x + static_cast<long long>(r) * ld + c0 + j) * inv;
        if (gamma != 0.0f) ov = fmaf(-gamma * cu[r], cv[c0 + j], ov);
        if (o) st1<XT>(o + ooff + j, ov);
        if (w) w[off + j] = fmaf(a.neg_lr_scale, ov, w[off + j]);
      }
    }
  }
}

template <typename XT>
__global__ void __launch_bounds__(256) apply_tall_kernel(const XT* X, long long xstride, int m, int n, int ld,
                                                         int ldo, MutPtrTable W, MutPtrTable O, ApplyArgs a) {
  __shared__ float tile[64][65];
  __shared__ float red[8];
  const int z = blockIdx.y;
  const XT* x = X + z * xstride;
  float* w = static_cast<float*>(W.p[z]);
  XT* o = static_cast<XT*>(O.p[z]);
  const float inv = apply_prologue(a, z, red);
  const float gamma = cap_gamma(a, z, red);
  const float* cu = static_cast<const float*>(a.cu.p[z]);
  const float* cv = static_cast<const float*>(a.cv.p[z]);
  // tiles over U = X^T (m x n): rows k (long side), cols i (short side)
  const int tiles_i = (n + 63) / 64;
  const int k0 = (blockIdx.x / tiles_i) * 64;
  const int i0 = (blockIdx.x % tiles_i) * 64;
  const int t = threadIdx.x;
  // read X rows i0.., cols k0.. (coalesced along k)
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int ir = t / 8 + 32 * pass;
    const int kc = (t % 8) * 8;
    float v[8];
    if (i0 + ir < n && k0 + kc + 7 < ld) {
      Vec8<XT>::template load<true>(x + static_cast<long long>(i0 + ir) * ld + k0 + kc, v);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[kc + j][ir] = v[j] * inv;
  }
  __syncthreads();
  const bool vec = (n % 8) == 0 && (ldo % 8) == 0 && (!w || a16(w)) && (!o || a16(o));
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int kr = t / 8 + 32 * pass;
    const int ic = (t % 8) * 8;
    const int ur = k0 + kr, uc = i0 + ic;
    if (ur >= m) continue;
    const long long off = static_cast<long long>(ur) * n + uc;
    const long long ooff = static_cast<long long>(ur) * ldo + uc;
    if (vec && uc + 7 < n) {
      float ov[8], wv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) ov[j] = tile[kr][ic + j];
      if (gamma != 0.0f) {
        const float gu = gamma * cu[ur];
#pragma unroll
        for (int j = 0; j < 8; ++j) ov[j] = fmaf(-gu, cv[uc + j], ov[j]);
      }
      if (o) Vec8<XT>::template store<true>(o + ooff, ov);
      if (w) {
        Vec8<float>::template load<true>(w + off, wv);
#pragma unroll
        for (int j = 0; j < 8; ++j) wv[j] = fmaf(a.neg_lr_scale, ov[j], wv[j]);
        Vec8<float>::template store<true>(w + off, wv);
      }
    } else {
      for (int j = 0; j < 8 && uc + j < n; ++j) {
        float ov = tile[kr][ic + j];
        if (gamma != 0.0f) ov = fmaf(-gamma * cu[ur], cv[uc + j], ov);
        if (o) st1<XT>(o + ooff + j, ov);
        if (w) w[off + j] = fmaf(a.neg_lr_scale, ov, w[off + j]);
      }
    }
  }
}

// nu per matrix from the partials (used for norms_out).
__global__ void __launch_bounds__(256) norms_kernel(const float* partials, int P, float* out) {
  __shared__ float red[8];
  const int z = blockIdx.x;
  float nu = 0.0f;
  inv_norm_from_partials(partials + static_cast<long long>(z) * P, P, 0.0f, red, &nu);
  if (threadIdx.x == 0) out[z] = nu;
}

// Non-finite flag of a call: any partial sum of squares of the update
// direction that is not finite (a NaN or Inf in G or M, or an overflow of
// ||U||^2).  One workgroup; every thread issues all of its loads before it
// tests them; the flag is written with a plain store.
__global__ void __launch_bounds__(1024) flags_kernel(const float* partials, long long n, unsigned* flag) {
  __shared__ int any;
  if (threadIdx.x == 0) any = 0;
  __syncthreads();
  constexpr int U = 16;
  int bad = 0;
  for (long long i0 = 0; i0 < n; i0 += static_cast<long long>(U) * blockDim.x) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long i = i0 + static_cast<long long>(u) * blockDim.x + threadIdx.x;
      v[u] = i < n ? partials[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) bad |= !__builtin_isfinite(v[u]);
  }
  if (bad) any = 1;
  __syncthreads();
  if (threadIdx.x == 0) *flag = static_cast<unsigned>(any);
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
int momentum_blocks_per_matrix(bool tall, int s_pad, int ld) {
  if (tall) return ((s_pad + 63) / 64) * (((ld + 63) / 64 + kTallTiles - 1) / kTallTiles);
  const long long chunks = static_cast<long long>(s_pad) * (ld / 8);
  long long b = (chunks + 256 * 8 - 1) / (256 * 8);  // about 8 chunks per thread
  if (b < 1) b = 1;
  if (b > 1024) b = 1024;
  return static_cast<int>(b);
}

hipError_t launch_momentum(const MomentumLaunch& L, hipStream_t st) {
  const dim3 grid(L.P, L.count);
  const dim3 block(256);
#define MUON_MOM(GT, XT)                                                                            \
  do {                                                                                              \
    if (L.tall)                                                                                     \
      hipLaunchKernelGGL((momentum_tall_kernel<GT, XT>), grid, block, 0, st, L.G, L.M,              \
                         static_cast<XT*>(L.X), L.xstride, L.m, L.n, L.ldg, L.s_pad, L.ld, L.beta,  \
                         L.nesterov, L.partials, L.P);                                              \
    else                                                                                            \
      hipLaunchKernelGGL((momentum_wide_kernel<GT, XT>), grid, block, 0, st, L.G, L.M,              \
                         static_cast<XT*>(L.X), L.xstride, L.m, L.n, L.ldg, L.s_pad, L.ld, L.beta,  \
                         L.nesterov, L.partials, L.P);                                              \
  } while (0)
  if (L.grad_bf16 && L.x_bf16) MUON_MOM(bf16_t, bf16_t);
  else if (L.grad_bf16) MUON_MOM(bf16_t, float);
  else if (L.x_bf16) MUON_MOM(float, bf16_t);
  else MUON_MOM(float, float);
#undef MUON_MOM
  return hipGetLastError();
}

hipError_t launch_apply(const ApplyLaunch& L, hipStream_t st) {
  ApplyArgs a{L.partials, L.P, L.eps, L.neg_lr_scale, L.cap_part, L.cap_P, L.cap_sigma, L.cap, L.cu, L.cv};
  const dim3 block(256);
  if (L.tall) {
    const dim3 grid(((L.m + 63) / 64) * ((L.n + 63) / 64), L.count);
    if (L.x_bf16)
      hipLaunchKernelGGL((apply_tall_kernel<bf16_t>), grid, block, 0, st, static_cast<const bf16_t*>(L.X),
                         L.xstride, L.m, L.n, L.ld, L.ldo, L.W, L.O, a);
    else
      hipLaunchKernelGGL((apply_tall_kernel<float>), grid, block, 0, st, static_cast<const float*>(L.X),
                         L.xstride, L.m, L.n, L.ld, L.ldo, L.W, L.O, a);
  } else {
    const long long chunks = static_cast<long long>(L.m) * ((L.n + 7) / 8);
    long long b = (chunks + 256 * 8 - 1) / (256 * 8);
    if (b < 1) b = 1;
    if (b > 1024) b = 1024;
    const dim3 grid(static_cast<unsigned>(b), L.count);
    if (L.x_bf16)
      hipLaunchKernelGGL((apply_wide_kernel<bf16_t>), grid, block, 0, st, static_cast<const bf16_t*>(L.X),
                         L.xstride, L.m, L.n, L.ld, L.ldo, L.W, L.O, a);
    else
      hipLaunchKernelGGL((apply_wide_kernel<float>), grid, block, 0, st, static_cast<const float*>(L.X),
                         L.xstride, L.m, L.n, L.ld, L.ldo, L.W, L.O, a);
  }
  return hipGetLastError();
}

hipError_t launch_norms(const float* partials, int P, int count, float* out, hipStream_t st) {
  hipLaunchKernelGGL(norms_kernel, dim3(count), dim3(256), 0, st, partials, P, out);
  return hipGetLastError();
}

hipError_t launch_flags(const float* partials, long long n, unsigned* flag, hipStream_t st) {
  hipLaunchKernelGGL(flags_kernel, dim3(1), dim3(1024), 0, st, partials, n, flag);
  return hipGetLastError();
}

}  // namespace muon
