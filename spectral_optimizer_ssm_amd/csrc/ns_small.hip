// Whole Newton-Schulz iteration on chip for small matrices.
//
// "MuonSSM" (method section on light Newton-Schulz orthogonalisation) runs a
// single Newton-Schulz step, with no explicit SVD, on the low-rank injection of
// every token and head; its ablation on the number of Newton-Schulz steps
// compares one step with five.  Each matrix (s x l, s <= 64) is loaded once,
// normalised by its Frobenius norm, iterated in LDS and registers, and stored
// once, so the pass streams HBM exactly once each way.
//
// bf16 kernel: one wavefront per matrix, several matrices per workgroup.
//  * X lives in LDS (row-major, 16-byte chunks XOR-swizzled per row).
//  * Gram A = X X^T on v_mfma_f32_32x32x16_bf16 from ds_read_b128 fragments.
//  * A never touches memory: by symmetry the Gram accumulators already hold,
//    lane by lane, the operand fragments of A that the combine needs, after a
//    permutation of the contraction index (a sum is invariant under one).
//  * Combine D[k][i] = sum_j X[j][k] A[i][j] with the X operand gathered from
//    LDS in the same contraction order; each lane then holds 4 consecutive
//    columns of one row of Y = a X + b A X.
//  * Y overwrites X in LDS one 32-column block at a time (same wave, in
//    order) and leaves through coalesced 16-byte stores.
// fp32 kernel: one workgroup per matrix, plain FMA dot products in LDS.
#include "common.cuh"
#include "launch.h"

namespace muon {
namespace {

constexpr int WPB = 4;  // waves (matrices) per workgroup, bf16 kernel

// Lanes of one wavefront exchange data through LDS between phases.  LDS
// instructions of a wavefront execute in order; the fence keeps the compiler
// from moving accesses across the phase boundary.  (Waves leave the matrix
// loop independently, so a workgroup barrier is not an option here.)
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int S, int L>
struct SmallGeo {
  static constexpr int CPR = L / 8;                       // 16-B chunks per row
  static constexpr int RPS = L >= 128 ? 1 : 128 / L;      // rows per 256-B bank sweep
  // XOR only inside an aligned power-of-two group of chunks that divides the
  // row, so the swizzled chunk never leaves its row
  static constexpr int SWM = (CPR % 16 == 0) ? 16 : (CPR % 8 == 0) ? 8 : (CPR % 4 == 0) ? 4 : 1;
  static constexpr int BYTES = S * L * 2;
  static constexpr int CHUNKS = S * CPR;
  __device__ static int chunk_off(int r, int c) { return r * (L * 2) + ((c ^ ((r / RPS) % SWM)) << 4); }
  __device__ static int elem_off(int r, int k) { return chunk_off(r, k >> 3) + ((k & 7) << 1); }
};

// Two waves per SIMD where the registers allow it without spilling (up to
// 64 x 128; larger shapes hold more accumulators).
template <int S, int L> struct SmallWpe { static constexpr int v = S * L <= 64 * 128 ? 2 : 1; };

template <int S, int L>
__global__ void __launch_bounds__(WPB * 64) __attribute__((amdgpu_waves_per_eu(SmallWpe<S, L>::v)))
ns_small_bf16_kernel(NsSmallLaunch P) {
  using Geo = SmallGeo<S, L>;
  constexpr int NB = S / 32;      // 32-row blocks of X (and of A)
  constexpr int NJ = S / 16;      // contraction steps over j in the combine
  constexpr int NK = L / 32;      // 32-column blocks of X
  __shared__ __attribute__((aligned(16))) char lds_all[WPB][Geo::BYTES];
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  char* lds = lds_all[wid];
  const int G = lane >> 5, l32 = lane & 31;
  const long long nwaves = static_cast<long long>(gridDim.x) * WPB;

  for (long long mat = static_cast<long long>(blockIdx.x) * WPB + wid; mat < P.count; mat += nwaves) {
    const bf16_t* src = static_cast<const bf16_t*>(P.X) + mat * P.in_stride;
    bf16_t* dst = static_cast<bf16_t*>(P.Y) + mat * P.out_stride;

    // ---- load X, sum of squares -------------------------------------------
    float ss = 0.0f;
#pragma unroll
    for (int p = 0; p < Geo::CHUNKS / 64; ++p) {
      const int q = lane + 64 * p;
      const int r = q / Geo::CPR, c = q % Geo::CPR;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src + static_cast<long long>(r) * P.ld_in + c * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = lo_bf16(v[e]), b = hi_bf16(v[e]);
        ss = fmaf(a, a, ss);
        ss = fmaf(b, b, ss);
      }
      *reinterpret_cast<u32x4_t*>(lds + Geo::chunk_off(r, c)) = v;
    }
    wave_lds_sync();
    float inv;
    if (P.partials != nullptr) {
      float s2 = 0.0f;
      for (int i = lane; i < P.P; i += 64) s2 += P.partials[mat * P.P + i];
      inv = 1.0f / (sqrtf(wave_sum(s2)) + P.eps);
    } else {
      inv = 1.0f / (sqrtf(wave_sum(ss)) + P.eps);
    }

    for (int step = 0; step < P.steps; ++step) {
      const float sc = step == 0 ? inv : 1.0f;
      // ---- Gram: all NB x NB blocks ---------------------------------------
      f32x16_t g[NB][NB];
#pragma unroll
      for (int bm = 0; bm < NB; ++bm)
#pragma unroll
        for (int bn = 0; bn < NB; ++bn)
#pragma unroll
          for (int r = 0; r < 16; ++r) g[bm][bn][r] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < L / 16; ++ks) {
        bf16x8_t f[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
          f[b] = *reinterpret_cast<const bf16x8_t*>(lds + Geo::chunk_off(b * 32 + l32, ks * 2 + G));
#pragma unroll
        for (int bm = 0; bm < NB; ++bm)
#pragma unroll
          for (int bn = 0; bn < NB; ++bn)
            g[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[bm], f[bn], g[bm][bn], 0, 0, 0);
      }
      // ---- A fragments for the combine (B operand, column i, 8 j's) --------
      // block (bm, ib), lane: A[bm*32 + 8g' + 4G + r][ib*32 + l32]
      //   = A[ib*32 + l32][j], j = 16*js + 8*(t/4) + 4G + t%4, js = 2bm + kappa
      const float gs = sc * sc;
      u32x4_t af[NB][NJ];
#pragma unroll
      for (int ib = 0; ib < NB; ++ib)
#pragma unroll
        for (int js = 0; js < NJ; ++js) {
          const int bm = js >> 1, kap = js & 1;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int gp = 2 * kap + h;
            af[ib][js][2 * h] = pack_bf16x2(g[bm][ib][4 * gp + 0] * gs, g[bm][ib][4 * gp + 1] * gs);
            af[ib][js][2 * h + 1] = pack_bf16x2(g[bm][ib][4 * gp + 2] * gs, g[bm][ib][4 * gp + 3] * gs);
          }
        }
      // ---- combine, one 32-column block of X at a time ----------------------
      // Column block kb of X is read only by block kb of the combine, so Y's
      // block kb replaces it in LDS right away (this wave's region; LDS
      // operations of a wave execute in order) and only one block of Y is
      // held in registers: two waves per SIMD instead of one.
      const float alpha = P.a[step] * sc, beta = P.b[step] * sc;
#pragma unroll 1
      for (int kb = 0; kb < NK; ++kb) {
        u32x2_t ypk[NB][4];
        f32x16_t c[NB];
#pragma unroll
        for (int ib = 0; ib < NB; ++ib)
#pragma unroll
          for (int r = 0; r < 16; ++r) c[ib][r] = 0.0f;
        const int kcol = kb * 32 + l32;
#pragma unroll
        for (int js = 0; js < NJ; ++js) {
          bf16x8_t xf;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int j = 16 * js + 8 * (t >> 2) + 4 * G + (t & 3);
            xf[t] = *reinterpret_cast<const __bf16*>(lds + Geo::elem_off(j, kcol));
          }
#pragma unroll
          for (int ib = 0; ib < NB; ++ib)
            c[ib] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf, __builtin_bit_cast(bf16x8_t, af[ib][js]), c[ib], 0, 0, 0);
        }
        // lane: row i = ib*32 + l32, columns k = kb*32 + 8q + 4G + 0..3
#pragma unroll
        for (int ib = 0; ib < NB; ++ib)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int i = ib * 32 + l32, k = kb * 32 + 8 * q + 4 * G;
            const u32x2_t xv = *reinterpret_cast<const u32x2_t*>(lds + Geo::elem_off(i, k));
            const float y0 = fmaf(alpha, lo_bf16(xv[0]), beta * c[ib][4 * q + 0]);
            const float y1 = fmaf(alpha, hi_bf16(xv[0]), beta * c[ib][4 * q + 1]);
            const float y2 = fmaf(alpha, lo_bf16(xv[1]), beta * c[ib][4 * q + 2]);
            const float y3 = fmaf(alpha, hi_bf16(xv[1]), beta * c[ib][4 * q + 3]);
            ypk[ib][q] = u32x2_t{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
          }
        wave_lds_sync();
#pragma unroll
        for (int ib = 0; ib < NB; ++ib)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int i = ib * 32 + l32, k = kb * 32 + 8 * q + 4 * G;
            *reinterpret_cast<u32x2_t*>(lds + Geo::elem_off(i, k)) = ypk[ib][q];
          }
        wave_lds_sync();
      }
    }

    // ---- store (zero steps: the normalised input) ---------------------------
#pragma unroll
    for (int p = 0; p < Geo::CHUNKS / 64; ++p) {
      const int q = lane + 64 * p;
      const int r = q / Geo::CPR, c = q % Geo::CPR;
      u32x4_t v = *reinterpret_cast<const u32x4_t*>(lds + Geo::chunk_off(r, c));
      if (P.steps == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = pack_bf16x2(lo_bf16(v[e]) * inv, hi_bf16(v[e]) * inv);
      }
      *reinterpret_cast<u32x4_t*>(dst + static_cast<long long>(r) * P.ld_out + c * 8) = v;
    }
    wave_lds_sync();  // the next matrix overwrites this region
  }
}

// ---- float32: one workgroup per matrix --------------------------------------
template <int LMAX>
__global__ void __launch_bounds__(256) ns_small_f32_kernel(NsSmallLaunch P) {
  constexpr int SMAX = 64;
  __shared__ float xa[SMAX][LMAX + 1];
  __shared__ float xb[SMAX][LMAX + 1];
  __shared__ float am[SMAX][SMAX + 1];
  __shared__ float red[4];
  const int S = P.s, Lw = P.l, tid = threadIdx.x;
  for (long long mat = blockIdx.x; mat < P.count; mat += gridDim.x) {
    const float* src = static_cast<const float*>(P.X) + mat * P.in_stride;
    float* dst = static_cast<float*>(P.Y) + mat * P.out_stride;
    float ss = 0.0f;
    for (int e = tid; e < S * Lw; e += 256) {
      int i, k;
      float v;
      if (P.transposed) {  // stored as l x s: consecutive threads read consecutive i
        i = e % S; k = e / S;
        v = src[static_cast<long long>(k) * P.ld_in + i];
      } else {
        i = e / Lw; k = e % Lw;
        v = src[static_cast<long long>(i) * P.ld_in + k];
      }
      xa[i][k] = v;
      ss = fmaf(v, v, ss);
    }
    float inv;
    if (P.partials != nullptr) {
      float s2 = 0.0f;
      for (int i = tid; i < P.P; i += 256) s2 += P.partials[mat * P.P + i];
      inv = 1.0f / (sqrtf(block_sum(s2, red)) + P.eps);
    } else {
      inv = 1.0f / (sqrtf(block_sum(ss, red)) + P.eps);
    }
    __syncthreads();
    for (int e = tid; e < S * Lw; e += 256) xa[e / Lw][e % Lw] *= inv;
    __syncthreads();
    float (*cur)[LMAX + 1] = xa;
    float (*nxt)[LMAX + 1] = xb;
    for (int step = 0; step < P.steps; ++step) {
      for (int e = tid; e < S * S; e += 256) {
        const int i = e / S, j = e % S;
        float acc = 0.0f;
        for (int k = 0; k < Lw; ++k) acc = fmaf(cur[i][k], cur[j][k], acc);
        am[i][j] = acc;
      }
      __syncthreads();
      const float a = P.a[step], b = P.b[step];
      for (int e = tid; e < S * Lw; e += 256) {
        const int i = e / Lw, k = e % Lw;
        float acc = 0.0f;
        for (int j = 0; j < S; ++j) acc = fmaf(am[i][j], cur[j][k], acc);
        nxt[i][k] = fmaf(a, cur[i][k], b * acc);
      }
      __syncthreads();
      float (*t)[LMAX + 1] = cur;
      cur = nxt;
      nxt = t;
    }
    for (int e = tid; e < S * Lw; e += 256) {
      if (P.transposed) {
        const int i = e % S, k = e / S;
        dst[static_cast<long long>(k) * P.ld_out + i] = cur[i][k];
      } else {
        const int i = e / Lw, k = e % Lw;
        dst[static_cast<long long>(i) * P.ld_out + k] = cur[i][k];
      }
    }
    __syncthreads();
  }
}

long long small_grid(long long units, long long cap) { return units < cap ? (units < 1 ? 1 : units) : cap; }

}  // namespace

bool ns_small_supported(bool bf16, int s, int l) {
  if (bf16) return (s == 32 || s == 64) && l % 32 == 0 && l >= s && l <= 256;
  return s >= 1 && s <= 64 && l >= s && l <= 256;
}

hipError_t launch_ns_small(const NsSmallLaunch& P, bool bf16, hipStream_t st) {
  if (bf16) {
    const long long blocks = small_grid((P.count + WPB - 1) / WPB, 1LL << 16);
    const dim3 grid(static_cast<unsigned>(blocks)), block(WPB * 64);
#define MUON_SMALL(SS, LL)                                                                 \
  if (P.s == SS && P.l == LL) {                                                            \
    hipLaunchKernelGGL((ns_small_bf16_kernel<SS, LL>), grid, block, 0, st, P);             \
    return hipGetLastError();                                                              \
  }
    MUON_SMALL(32, 32) MUON_SMALL(32, 64) MUON_SMALL(32, 96) MUON_SMALL(32, 128)
    MUON_SMALL(32, 160) MUON_SMALL(32, 192) MUON_SMALL(32, 224) MUON_SMALL(32, 256)
    MUON_SMALL(64, 64) MUON_SMALL(64, 96) MUON_SMALL(64, 128) MUON_SMALL(64, 160)
    MUON_SMALL(64, 192) MUON_SMALL(64, 224) MUON_SMALL(64, 256)
#undef MUON_SMALL
    return hipErrorInvalidValue;
  }
  const long long blocks = small_grid(P.count, 1LL << 16);
  if (P.l <= 128)
    hipLaunchKernelGGL((ns_small_f32_kernel<128>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, P);
  else
    hipLaunchKernelGGL((ns_small_f32_kernel<256>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, P);
  return hipGetLastError();
}

}  // namespace muon
