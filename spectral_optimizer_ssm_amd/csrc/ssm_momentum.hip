// Momentum pathway of MuonSSM over sequences of factored injections.
//
// "MuonSSM: Orthogonalizing State Space Models" (method section on the
// momentum-augmented state update; theory section, parallelism): beside the
// memory state S_t a momentum state M_t accumulates the Newton-Schulz
// conditioned injections, and the pair follows a block-affine recurrence.
// Read as heavy-ball momentum on the memory:
//   U_t = NS(V_t K_t^T) = V_t C_t K_t^T = W_t K_t^T   (r x r core C_t, ns_factored.hip)
//   M_t = beta M_{t-1} + U_t,   S_t = a_t S_{t-1} + M_t.
// The dense U_t (16 KB for a 64 x 128 injection) never reaches memory: the
// factored kernel writes W_t = V_t C_t (1 KB per token) and this file turns
// the recurrence into weighted sums of rank-r products W_t K_t^T.
//
// Chunks.  Over a chunk of L tokens u = 0..L-1 entered with (S, M):
//   M' = beta^L M + sum_u beta^(L-1-u) U_u
//   S' = A S + B M + sum_u w_u U_u,   A = prod_u a_u,   B = beta w_0,
//   w_u = g_u + beta w_{u+1} (w_L = 0),   g_u = prod_{s>u} a_s.
// ssm_momentum_accum_kernel forms the two sums of one (sequence, chunk) as
// float32 partials; ssm_momentum_combine_kernel applies the chunk maps in
// token order to the caller's (S, M).  Sums and maps are the same
// recurrence regrouped (the block-affine structure the pages point to).
//
// Accumulation kernel: one workgroup of 4 waves per (sequence, chunk), the
// 64 x 128 state tile (zero padded) split into four 32-column blocks, one per
// wave.  The factored kernel has written W_u = V_u C_u (m x 8 bf16) for every
// token, so
//   P[i][j] += sum_{u, r} W_u[i][r] (w_u K_u[j][r])
// runs on v_mfma_f32_32x32x16_bf16 with the contraction index (token pair,
// rank): each lane loads its two 16-byte rows of W and its 16-byte row of K
// straight from memory, scales the K row by the token's weight (one per
// partial sum) and rounds it to bf16.  No LDS staging and no barriers in the
// token loop; the four waves read the same W rows (L2 serves three of them).
#include "common.cuh"
#include "launch.h"

namespace muon {
namespace {

constexpr int kTileM = 64, kTileN = 128, kTile = kTileM * kTileN;

__global__ void __launch_bounds__(256) ssm_momentum_accum_kernel(SsmMomLaunch P) {
  __shared__ float wgt[2][kSsmMomQ];
  __shared__ float dec[kSsmMomQ];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int G = lane >> 5, l32 = lane & 31;
  const long long seq = blockIdx.x / P.nchunks;
  const int ch = static_cast<int>(blockIdx.x - seq * P.nchunks);
  const int t0 = ch * P.Q;
  const int len = P.T - t0 < P.Q ? P.T - t0 : P.Q;
  const bool with_s = P.S != nullptr;
  const long long tok0 = seq * P.T + t0;

  // per-token weights by the backward recurrence (one thread, decays staged)
  if (with_s)
    for (int u = tid; u < len; u += 256) dec[u] = P.a[tok0 + u];
  __syncthreads();
  if (tid == 0) {
    float wmv = 1.0f, g = 1.0f, ws = 0.0f;
    for (int u = len - 1; u >= 0; --u) {
      wgt[0][u] = wmv;
      wmv *= P.beta;
      if (with_s) {
        ws = g + P.beta * ws;
        wgt[1][u] = ws;
        g *= dec[u];
      }
    }
    float* cf = P.coef + (seq * P.nchunks + ch) * 4;
    cf[0] = wmv;                          // beta^L
    cf[1] = with_s ? g : 0.0f;            // A = prod a
    cf[2] = with_s ? P.beta * ws : 0.0f;  // B = beta w_0
    cf[3] = 0.0f;
  }
  __syncthreads();

  const bf16_t* Ws = P.W + tok0 * P.m * 8;
  const bf16_t* Ks = P.K + tok0 * P.n * 8;
  f32x16_t accM[2], accS[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) accM[rb][r] = accS[rb][r] = 0.0f;
  const int col = 32 * w + l32;
  const bool row0 = l32 < P.m, row1 = l32 + 32 < P.m, colok = col < P.n;
  auto scaled = [](const u32x4_t& k, float s) {
    u32x4_t o;
#pragma unroll
    for (int h = 0; h < 4; ++h) o[h] = pack_bf16x2(lo_bf16(k[h]) * s, hi_bf16(k[h]) * s);
    return __builtin_bit_cast(bf16x8_t, o);
  };
#pragma unroll 4
  for (int tp = 0; tp < len; tp += 2) {
    const int t = tp + G;
    const bool ok = t < len;
    const u32x4_t z = {0u, 0u, 0u, 0u};
    const long long wt = static_cast<long long>(t) * P.m, kt = static_cast<long long>(t) * P.n;
    const u32x4_t a0 = (ok && row0) ? *reinterpret_cast<const u32x4_t*>(Ws + (wt + l32) * 8) : z;
    const u32x4_t a1 = (ok && row1) ? *reinterpret_cast<const u32x4_t*>(Ws + (wt + l32 + 32) * 8) : z;
    const u32x4_t kv = (ok && colok) ? *reinterpret_cast<const u32x4_t*>(Ks + (kt + col) * 8) : z;
    const float sm = ok ? wgt[0][t] : 0.0f;
    const bf16x8_t A0 = __builtin_bit_cast(bf16x8_t, a0), A1 = __builtin_bit_cast(bf16x8_t, a1);
    const bf16x8_t km = scaled(kv, sm);
    accM[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, km, accM[0], 0, 0, 0);
    accM[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, km, accM[1], 0, 0, 0);
    if (with_s) {
      const bf16x8_t ks = scaled(kv, ok ? wgt[1][t] : 0.0f);
      accS[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, ks, accS[0], 0, 0, 0);
      accS[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, ks, accS[1], 0, 0, 0);
    }
  }

  // partials: lane (G, l32), register 4 q + e holds row 32 rb + 8 q + 4 G + e,
  // column 32 w + l32 of the padded 64 x 128 tile
  float* pm = P.part + (seq * P.nchunks + ch) * (with_s ? 2 : 1) * static_cast<long long>(kTile);
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 32 * rb + 8 * q + 4 * G + e;
        pm[row * kTileN + col] = accM[rb][4 * q + e];
        if (with_s) pm[kTile + row * kTileN + col] = accS[rb][4 * q + e];
      }
}

// (S, M) <- chunk maps in token order; one thread per state element.
__global__ void __launch_bounds__(256) ssm_momentum_combine_kernel(SsmMomLaunch P) {
  const long long mn = static_cast<long long>(P.m) * P.n;
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= P.nseq * mn) return;
  const long long seq = idx / mn;
  const int e = static_cast<int>(idx - seq * mn);
  const int i = e / P.n, j = e - i * P.n;
  const bool with_s = P.S != nullptr;
  const int nout = with_s ? 2 : 1;
  float M = P.M[idx];
  float S = with_s ? P.S[idx] : 0.0f;
  for (int c = 0; c < P.nchunks; ++c) {
    const float* cf = P.coef + (seq * P.nchunks + c) * 4;
    const float* pb = P.part + (seq * P.nchunks + c) * nout * static_cast<long long>(kTile) + i * kTileN + j;
    if (with_s) S = fmaf(cf[1], S, fmaf(cf[2], M, pb[kTile]));
    M = fmaf(cf[0], M, pb[0]);
  }
  P.M[idx] = M;
  if (with_s) P.S[idx] = S;
}

}  // namespace

hipError_t launch_ssm_momentum(const SsmMomLaunch& P, hipStream_t st, int phase) {
  if (phase == 0) {
    const long long blocks = P.nseq * P.nchunks;
    hipLaunchKernelGGL(ssm_momentum_accum_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, P);
  } else {
    const long long blocks = (P.nseq * P.m * P.n + 255) / 256;
    hipLaunchKernelGGL(ssm_momentum_combine_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, P);
  }
  return hipGetLastError();
}

}  // namespace muon
