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
// r x r recurrence in float32; it writes the core (256 B) and, on request,
// the dense result O = (V C) K^T.
//
// Layout and work split: one wavefront owns four consecutive matrices.  Their
// V and K are staged in LDS side by side as [rows][32 columns] bf16 (matrix q
// in columns 8q .. 8q + 7, zero padded), so one v_mfma_f32_32x32x16_bf16 per
// 16 rows gives the four Gram matrices at once on its diagonal 8 x 8 blocks;
// the MFMA operand (one column of 8 consecutive rows per lane) comes from
// two ds_read_b64_tr_b16.  The r x r recurrence then runs on 16 lanes per
// matrix, each lane owning 4 entries of one row, through LDS.
//
// Waves are persistent and walk the groups of four with a stride of the grid.
// For 64 x 128 rank-8 injections with aligned factors (the MuonSSM shape) a
// wave loads the next group's factors into registers (12 x 16 bytes per lane)
// while it computes the current one, so the load latency overlaps the
// recurrence; other shapes stage each group from memory in turn.
#include "common.cuh"
#include "launch.h"

namespace muon {
namespace {

constexpr int kMats = 4;          // matrices per wavefront
// Persistent grid: four workgroups of four waves per CU, each walking an equal
// share of the groups (two are resident at a time at 204 registers per lane; a
// grid of three per CU at three waves per SIMD measured no faster).
constexpr int kFactWgPerCu = 4;
constexpr int kRow = 64;          // bytes per staged row (32 bf16 columns)

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// LDS of one wavefront.
struct WaveLds {
  char* vk;      // (m_pad + n_pad) x kRow: V rows, then K rows
  float* f;      // kMats x 6 x 64: P, S, C, T1, N, T2
  float* t;      // m_pad x 32 floats: V C of the four matrices (dense output)
  __device__ float* mat(int q, int which) const { return f + (q * 6 + which) * 64; }
};
enum { kP = 0, kS, kC, kT1, kN, kT2 };

// Gram of the 32 staged columns over rows [row0, row0 + rows): lane l holds
// column l % 32, rows 8 (g / 4) + 4 (l / 32) + g % 4 of the 32 x 32 result.
__device__ f32x16_t gram32(const char* vk, int row0, int rows, int lane) {
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
  const int g = lane >> 4;
  const int colbase = 16 * (g & 1);
  const int rr = (lane & 15) >> 2, u = lane & 3;
  for (int k0 = 0; k0 < rows; k0 += 16) {
    // A operand: row (= staged column) lane % 32, contraction index
    // k0 + 8 (lane / 32) + 0..7; lane 16g + 4rr + u addresses staged row
    // k0 + 8 (g >> 1) + 4h + rr, columns colbase + 4u .. + 3.
    u32x2_t part[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = row0 + k0 + 8 * (g >> 1) + 4 * h + rr;
      const char* p = vk + row * kRow + (colbase + 4 * u) * 2;
      const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p);
      part[h] = __builtin_bit_cast(u32x2_t, v);
    }
    const u32x4_t w = {part[0][0], part[0][1], part[1][0], part[1][1]};
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, w);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc, 0, 0, 0);
  }
  return acc;
}

// Keep the diagonal 8 x 8 blocks of a gram32 result: lane l writes rows
// 4 (l / 32) + 0..3, column l % 8 of matrix (l % 32) / 8.
__device__ void store_blocks(const f32x16_t& acc, const WaveLds& L, int which, int lane) {
  const int q = (lane & 31) >> 3, j = lane & 7, i0 = 4 * (lane >> 5);
  float* dst = L.mat(q, which);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float v = q == 0 ? acc[e] : q == 1 ? acc[4 + e] : q == 2 ? acc[8 + e] : acc[12 + e];
    dst[(i0 + e) * 8 + j] = v;
  }
}

// Z = X Y (or X Y^T) for the wave's four 8 x 8 matrices; lane l handles
// matrix l / 16, row i = (l % 16) / 2, columns j0 .. j0 + 3 with j0 = 4 (l % 2).
template <bool TRANS_Y>
__device__ void mm8(const WaveLds& L, int x, int y, int z, int lane) {
  const int q = lane >> 4, i = (lane & 15) >> 1, j0 = 4 * (lane & 1);
  const float* X = L.mat(q, x);
  const float* Y = L.mat(q, y);
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float xv = X[i * 8 + c];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(xv, TRANS_Y ? Y[(j0 + e) * 8 + c] : Y[c * 8 + j0 + e], acc[e]);
  }
  wave_sync();  // every lane has read X and Y before Z (which may alias neither) is written
  float* Z = L.mat(q, z);
#pragma unroll
  for (int e = 0; e < 4; ++e) Z[i * 8 + j0 + e] = acc[e];
  wave_sync();
}

// Steps 2-6 for the four matrices b0 .. b0 + nm - 1 staged in L.vk.
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
    *reinterpret_cast<u32x4_t*>(L.vk + t * kRow + 16 * q) = R.v[e];
  }
#pragma unroll
  for (int e = 0; e < kFastK; ++e) {
    const int c = lane + 64 * e, q = c / kFastN, u = c % kFastN;
    *reinterpret_cast<u32x4_t*>(L.vk + (kFastM + u) * kRow + 16 * q) = R.k[e];
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
  L.t = reinterpret_cast<float*>(base + rows * kRow + kMats * 6 * 64 * 4);
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
        factored_compute(F, L, gi * kMats, kMats, lane);
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
      *reinterpret_cast<u32x4_t*>(L.vk + t * kRow + 16 * q) = *reinterpret_cast<const u32x4_t*>(Vg + e * 8);
    }
    for (int e = lane; e < nm * n; e += 64) {
      const int q = e / n, u = e - q * n;
      *reinterpret_cast<u32x4_t*>(L.vk + (F.m_pad + u) * kRow + 16 * q) =
          *reinterpret_cast<const u32x4_t*>(Kg + e * 8);
    }
  } else {
    for (int e = lane; e < nm * m * r; e += 64) {
      const int q = e / (m * r), rem = e - q * m * r, t = rem / r, c = rem - t * r;
      *reinterpret_cast<bf16_t*>(L.vk + t * kRow + (8 * q + c) * 2) = Vg[e];
    }
    for (int e = lane; e < nm * n * r; e += 64) {
      const int q = e / (n * r), rem = e - q * n * r, u = rem / r, c = rem - u * r;
      *reinterpret_cast<bf16_t*>(L.vk + (F.m_pad + u) * kRow + (8 * q + c) * 2) = Kg[e];
    }
  }
  wave_sync();
  factored_compute(F, L, b0, nm, lane);
  }
}

__device__ __forceinline__ void factored_compute(const FactLaunch& F, const WaveLds& L, long long b0, int nm,
                                                 int lane) {
  const int m = F.m, n = F.n, r = F.r;
  // 2. P = V^T V and S = K^T K on the matrix cores; both are read before
  // either is stored (the work matrices may share the staging area)
  const f32x16_t gp = gram32(L.vk, 0, F.m_pad, lane);
  const f32x16_t gq = gram32(L.vk, F.m_pad, F.n_pad, lane);
  wave_sync();
  store_blocks(gp, L, kP, lane);
  store_blocks(gq, L, kS, lane);
  wave_sync();

  // 3. nu^2 = tr(P S) per matrix (16 lanes each), C_0 = I_r / (nu + eps)
  const int q = lane >> 4, i = (lane & 15) >> 1, j0 = 4 * (lane & 1);
  {
    const float* P = L.mat(q, kP);
    const float* S = L.mat(q, kS);
    float t2 = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) t2 = fmaf(P[i * 8 + j0 + e], S[(j0 + e) * 8 + i], t2);
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) t2 += __shfl_xor(t2, d, 64);
    const float inv = 1.0f / (sqrtf(t2) + F.eps);
    float* C = L.mat(q, kC);
#pragma unroll
    for (int e = 0; e < 4; ++e) C[i * 8 + j0 + e] = (i == j0 + e && i < r) ? inv : 0.0f;
  }
  wave_sync();

  // 4. the r x r recurrence (zero padding stays zero)
  for (int k = 0; k < F.steps; ++k) {
    mm8<false>(L, kC, kS, kT1, lane);   // C S
    mm8<true>(L, kT1, kC, kT2, lane);   // C S C^T
    mm8<false>(L, kT2, kP, kN, lane);   // N = C S C^T P
    mm8<false>(L, kN, kC, kT1, lane);   // N C
    const bool quintic = F.c[k] != 0.0f;
    if (quintic) mm8<false>(L, kN, kT1, kT2, lane);  // N N C
    float* C = L.mat(q, kC);
    const float* NC = L.mat(q, kT1);
    const float* NNC = L.mat(q, kT2);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int o = i * 8 + j0 + e;
      float v = fmaf(F.a[k], C[o], F.b[k] * NC[o]);
      if (quintic) v = fmaf(F.c[k], NNC[o], v);
      C[o] = v;
    }
    wave_sync();
  }

  // 5. the core, r x r float32 per matrix
  if (F.C != nullptr && q < nm && i < r) {
    const float* C = L.mat(q, kC);
    float* dst = F.C + (b0 + q) * r * r + i * r;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (j0 + e < r) dst[j0 + e] = C[i * 8 + j0 + e];
  }
  // 5'. W = V C (bf16, m x 8) for the momentum pathway: lane p of matrix q
  // forms rows p, p + 16, ... from the staged V rows (kept: the work
  // matrices sit over the staged K rows in this mode)
  if (F.W != nullptr) {
    const float* C = L.mat(q, kC);
    const int p = lane & 15;
    if (q < nm) {
      for (int t = p; t < m; t += 16) {
        const u32x4_t vv = *reinterpret_cast<const u32x4_t*>(L.vk + t * kRow + 16 * q);
        float v[8];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          v[2 * h] = lo_bf16(vv[h]);
          v[2 * h + 1] = hi_bf16(vv[h]);
        }
        float o[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] = 0.0f;
#pragma unroll
        for (int d = 0; d < 8; ++d)
#pragma unroll
          for (int c = 0; c < 8; ++c) o[c] = fmaf(v[d], C[d * 8 + c], o[c]);
        u32x4_t w;
#pragma unroll
        for (int h = 0; h < 4; ++h) w[h] = pack_bf16x2(o[2 * h], o[2 * h + 1]);
        *reinterpret_cast<u32x4_t*>(F.W + ((b0 + q) * m + t) * 8) = w;
      }
    }
    wave_sync();  // V read before the next group is staged
  }
  if (F.O == nullptr) return;

  // 6. dense O = (V C) K^T: T = V C staged in LDS (rows t, 8 floats per
  // matrix), then lane p of matrix q writes 8 consecutive columns of each row
  {
    const float* C = L.mat(q, kC);
    const int p = lane & 15;
    for (int t = p; t < m; t += 16) {
      float acc[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const float v = bf16_to_f32(*reinterpret_cast<const bf16_t*>(L.vk + t * kRow + (8 * q + d) * 2));
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = fmaf(v, C[d * 8 + c], acc[c]);
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
            kv[e][c] = bf16_to_f32(*reinterpret_cast<const bf16_t*>(L.vk + (F.m_pad + u0 + e) * kRow + (8 * q + c) * 2));
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
int factored_lds_per_wave(int m_pad, int n_pad, bool dense, int* f_off, bool keep_v) {
  const int stage = (m_pad + n_pad) * kRow, work = kMats * 6 * 64 * 4;
  if (keep_v && !dense && n_pad * kRow >= work) {  // work matrices over the staged K rows
    if (f_off) *f_off = m_pad * kRow;
    return stage;
  }
  if (keep_v && !dense) {
    if (f_off) *f_off = stage;
    return stage + work;
  }
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
