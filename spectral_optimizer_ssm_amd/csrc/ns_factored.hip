// Newton-Schulz of low-rank matrices given by their factors.
//
// "MuonSSM: Orthogonalizing State Space Models" (method section on the
// value-key injections and their light Newton-Schulz step): every injection
// is a sum of r outer products, X = V K^T with V m x r and K n x r.  Each NS
// step keeps that form, X_k = V C_k K^T, with an r x r core:
//   P = V^T V,  S = K^T K,  nu = ||X||_F = sqrt(tr(P S)),  C_0 = I / (nu + eps),
//   N = C S C^T P   (so that X X^T X = V (N C) K^T),
//   C <- a C + b N C + c N N C.
// So the kernel reads the factors (3 KB for a 64 x 128 rank-8 injection,
// against 16 KB dense), computes P and S on the matrix cores and runs the
// r x r recurrence in float32 (factored_core.cuh); it writes the core (256 B)
// and, on request, the dense result O = (V C) K^T.
//
// Layout and work split: one wavefront owns four consecutive matrices, staged
// in LDS side by side as factored_core.cuh lays them out.
//
// Waves are persistent and walk the groups of four with a stride of the grid.
// For 64 x 128 rank-8 injections with aligned factors (the MuonSSM shape) a
// wave loads the next group's factors into registers (12 x 16 bytes per lane)
// while it computes the current one, so the load latency overlaps the
// recurrence; other shapes stage each group from memory in turn.
#include "common.cuh"
#include "factored_core.cuh"
#include "launch.h"

namespace muon {
namespace {

using fact::kMats;
using fact::kRow;
using fact::wave_sync;
using fact::WaveLds;

// Persistent grid: four workgroups of four waves per CU, each walking an equal
// share of the groups (two are resident at a time at 204 registers per lane; a
// grid of three per CU at three waves per SIMD measured no faster).
constexpr int kFactWgPerCu = 4;

// Steps 2-6 for the four matrices b0 .. b0 + nm - 1 staged in L.vk.
template <bool FAST>
__device__ __forceinline__ void factored_compute(const FactLaunch& F, const WaveLds& L, long long b0, int nm,
                                                 int lane);

// Factors of one full group (four 64 x 128 rank-8 injections) in registers:
// lane l holds V rows l + 64 e (e < 4) and K rows l + 64 e (e < 8) of the
// group's concatenated rows, 16 bytes each.
constexpr int kFastM = 64, kFastN = 128, kFastV = kMats * kFastM / 64, kFastK = kMats * kFastN / 64;
struct FastRegs {
  u32x4_t v[kFastV], k[kFastK];
};
__device__ __forceinline__ void fast_load(const FactLaunch& F, long long b0, int lane, FastRegs& R) {
  const u32x4_t* Vg = reinterpret_cast<const u32x4_t*>(F.V + b0 * kFastM * 8);
  const u32x4_t* Kg = reinterpret_cast<const u32x4_t*>(F.K + b0 * kFastN * 8);
#pragma unroll
  for (int e = 0; e < kFastV; ++e) R.v[e] = Vg[lane + 64 * e];
#pragma unroll
  for (int e = 0; e < kFastK; ++e) R.k[e] = Kg[lane + 64 * e];
}
// Row t of matrix q (t = e % m, q = e / m for concatenated row e) goes to
// staged row t, bytes 16 q: with four full matrices every staged byte is
// written, so no zero padding is needed.
__device__ __forceinline__ void fast_stage(const WaveLds& L, int lane, const FastRegs& R) {
#pragma unroll
  for (int e = 0; e < kFastV; ++e) {
    const int c = lane + 64 * e, q = c / kFastM, t = c % kFastM;
    *reinterpret_cast<u32x4_t*>(L.vk + fact::slot(t, q)) = R.v[e];
  }
#pragma unroll
  for (int e = 0; e < kFastK; ++e) {
    const int c = lane + 64 * e, q = c / kFastN, u = c % kFastN;
    *reinterpret_cast<u32x4_t*>(L.vk + fact::slot(kFastM + u, q)) = R.k[e];
  }
}

__global__ void __launch_bounds__(256) ns_factored_kernel(FactLaunch F) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rows = F.m_pad + F.n_pad;
  char* base = lds + wave * F.per_wave;
  WaveLds L;
  L.vk = base;
  L.f = reinterpret_cast<float*>(base + F.f_off);
  L.t = reinterpret_cast<float*>(base + rows * kRow + fact::kWorkBytes);
  const int m = F.m, n = F.n, r = F.r;
  // groups of four matrices, walked by every wave of the grid in turn
  const long long groups = (F.batch + kMats - 1) / kMats;
  const long long gstride = static_cast<long long>(gridDim.x) * F.waves;
  long long gi = static_cast<long long>(blockIdx.x) * F.waves + wave;

  // fast path (64 x 128, rank 8, aligned factors, full groups): the next
  // group's factors are loaded into registers while this group is computed
  if (F.vec && m == kFastM && n == kFastN && r == 8 && F.m_pad == kFastM && F.n_pad == kFastN) {
    const long long full = F.batch / kMats;
    if (gi < full) {
      FastRegs R;
      fast_load(F, gi * kMats, lane, R);
      for (; gi < full; gi += gstride) {
        fast_stage(L, lane, R);
        wave_sync();
        if (gi + gstride < full) fast_load(F, (gi + gstride) * kMats, lane, R);
        factored_compute<true>(F, L, gi * kMats, kMats, lane);
      }
    }
    // the remaining partial group (at most one) takes the general path
    if (gi != full || full * kMats == F.batch) return;
  }
  for (; gi < groups; gi += gstride) {
  const long long b0 = gi * kMats;
  const int nm = F.batch - b0 < kMats ? static_cast<int>(F.batch - b0) : kMats;

  // 1. stage V and K (zero padded) as [rows][32 bf16]
  for (int o = lane * 16; o < rows * kRow; o += 64 * 16)
    *reinterpret_cast<u32x4_t*>(L.vk + o) = u32x4_t{0u, 0u, 0u, 0u};
  wave_sync();
  const bf16_t* Vg = F.V + b0 * m * r;
  const bf16_t* Kg = F.K + b0 * n * r;
  if (F.vec) {
    // one 16-byte row per lane and load: row t of matrix q -> staged row t, bytes 16q
    for (int e = lane; e < nm * m; e += 64) {
      const int q = e / m, t = e - q * m;
      *reinterpret_cast<u32x4_t*>(L.vk + fact::slot(t, q)) = *reinterpret_cast<const u32x4_t*>(Vg + e * 8);
    }
    for (int e = lane; e < nm * n; e += 64) {
      const int q = e / n, u = e - q * n;
      *reinterpret_cast<u32x4_t*>(L.vk + fact::slot(F.m_pad + u, q)) =
          *reinterpret_cast<const u32x4_t*>(Kg + e * 8);
    }
  } else {
    for (int e = lane; e < nm * m * r; e += 64) {
      const int q = e / (m * r), rem = e - q * m * r, t = rem / r, c = rem - t * r;
      *reinterpret_cast<bf16_t*>(L.vk + fact::slot(t, q) + 2 * c) = Vg[e];
    }
    for (int e = lane; e < nm * n * r; e += 64) {
      const int q = e / (n * r), rem = e - q * n * r, u = rem / r, c = rem - u * r;
      *reinterpret_cast<bf16_t*>(L.vk + fact::slot(F.m_pad + u, q) + 2 * c) = Kg[e];
    }
  }
  wave_sync();
  factored_compute<false>(F, L, b0, nm, lane);
  }
}

template <bool FAST>
__device__ __forceinline__ void factored_compute(const FactLaunch& F, const WaveLds& L, long long b0, int nm,
                                                 int lane) {
  const int m = F.m, n = F.n, r = F.r;
  // 2-4. Grams, normalisation and the r x r recurrence (the fast shape's row
  // counts as constants)
  if constexpr (FAST) fact::core<kFastM, kFastN>(F, L, lane);
  else fact::core(F, L, lane);
  const int q = lane >> 4, i = (lane & 15) >> 1, j0 = 4 * (lane & 1);

  // 5. the core, r x r float32 per matrix
  if (F.C != nullptr && q < nm && i < r) {
    const float* C = L.mat(q, fact::kC);
    float* dst = F.C + (b0 + q) * r * r + i * r;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (j0 + e < r) dst[j0 + e] = C[i * fact::kLd + j0 + e];
  }
  if (F.O == nullptr) return;

  // 6. dense O = (V C) K^T: T = V C staged in LDS (rows t, 8 floats per
  // matrix), then lane p of matrix q writes 8 consecutive columns of each row
  {
    const float* C = L.mat(q, fact::kC);
    const int p = lane & 15;
    for (int t = p; t < m; t += 16) {
      float acc[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const float v = bf16_to_f32(*reinterpret_cast<const bf16_t*>(L.vk + fact::slot(t, q) + 2 * d));
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = fmaf(v, C[d * fact::kLd + c], acc[c]);
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) L.t[t * 32 + 8 * q + c] = acc[c];
    }
    wave_sync();
    if (q < nm) {
      bf16_t* Og = F.O + (b0 + q) * m * n;
      for (int u0 = 8 * p; u0 < n; u0 += 128) {
        float kv[8][8];  // K rows u0 .. u0 + 7 of matrix q
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int c = 0; c < 8; ++c)
            kv[e][c] = bf16_to_f32(*reinterpret_cast<const bf16_t*>(L.vk + fact::slot(F.m_pad + u0 + e, q) + 2 * c));
        for (int t = 0; t < m; ++t) {
          float o[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float s = 0.0f;
#pragma unroll
            for (int c = 0; c < 8; ++c) s = fmaf(L.t[t * 32 + 8 * q + c], kv[e][c], s);
            o[e] = s;
          }
          u32x4_t w;
#pragma unroll
          for (int h = 0; h < 4; ++h) w[h] = pack_bf16x2(o[2 * h], o[2 * h + 1]);
          *reinterpret_cast<u32x4_t*>(Og + static_cast<long long>(t) * n + u0) = w;
        }
      }
    }
  }
}

}  // namespace

// Without the dense output the r x r work matrices share the staging area:
// the Gram has read the staged factors before the recurrence writes them, and
// the next group is staged only after the core has been stored (one wave, LDS
// operations in order).
int factored_lds_per_wave(int m_pad, int n_pad, bool dense, int* f_off) {
  const int stage = (m_pad + n_pad) * kRow, work = fact::kWorkBytes;
  if (!dense) {
    if (f_off) *f_off = 0;
    return stage > work ? stage : work;
  }
  if (f_off) *f_off = stage;
  return stage + work + m_pad * 32 * 4;
}

hipError_t launch_ns_factored(const FactLaunch& F, hipStream_t st) {
  const long long groups = (F.batch + kMats - 1) / kMats;
  // persistent waves: a few resident workgroups per CU walk the groups
  const int cus = device_cus();
  const long long need = (groups + F.waves - 1) / F.waves;
  const long long cap = static_cast<long long>(cus) * kFactWgPerCu;
  const long long blocks = need < cap ? need : cap;
  const size_t lds = static_cast<size_t>(F.waves) * F.per_wave;
  hipLaunchKernelGGL(ns_factored_kernel, dim3(static_cast<unsigned>(blocks)), dim3(64 * F.waves), lds, st, F);
  return hipGetLastError();
}

}  // namespace muon
