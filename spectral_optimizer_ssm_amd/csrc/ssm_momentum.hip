// Momentum pathway of MuonSSM over sequences of factored injections.
//
// "MuonSSM: Orthogonalizing State Space Models" (method section on the
// momentum-augmented state update; theory section, parallelism): beside the
// memory state S_t a momentum state M_t accumulates the Newton-Schulz
// conditioned injections, and the pair follows a block-affine recurrence.
// Read as heavy-ball momentum on the memory:
//   U_t = NS(V_t K_t^T) = V_t C_t K_t^T   (r x r core C_t, ns_factored.hip)
//   M_t = beta M_{t-1} + U_t,   S_t = a_t S_{t-1} + M_t.
// The dense U_t (16 KB for a 64 x 128 injection) never reaches memory: the
// cores come from the factored kernel (256 B per token) and this file turns
// the recurrence into weighted sums of rank-r products.
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
// wave.  Per sub-batch of 16 tokens the workgroup forms W_u = V_u C_u (64 x 8,
// float32 FMAs, every row once) scaled by the token's two weights, rounds it
// to bf16 in LDS, and each wave accumulates
//   P[i][j] += sum_{u, r} (w_u W_u)[i][r] K_u[j][r]
// on v_mfma_f32_32x32x16_bf16: the contraction index is (token pair, rank),
// its A operand a 16-byte LDS row of W, its B operand a 16-byte row of K
// straight from memory.
#include "common.cuh"
#include "launch.h"

namespace muon {
namespace {

constexpr int kSub = 16;        // tokens per sub-batch
constexpr int kTileM = 64, kTileN = 128, kTile = kTileM * kTileN;

__global__ void __launch_bounds__(256) ssm_momentum_accum_kernel(SsmMomLaunch P) {
  __shared__ __attribute__((aligned(16))) float cs[kSub][64];
  __shared__ __attribute__((aligned(16))) bf16_t wm[kSub][kTileM][8];
  __shared__ __attribute__((aligned(16))) bf16_t wsh[kSub][kTileM][8];
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
    cf[0] = wmv;                        // beta^L
    cf[1] = with_s ? g : 0.0f;          // A = prod a
    cf[2] = with_s ? P.beta * ws : 0.0f;  // B = beta w_0
    cf[3] = 0.0f;
  }

  const bf16_t* Vs = P.V + tok0 * P.m * 8;
  const bf16_t* Ks = P.K + tok0 * P.n * 8;
  const float* Cs = P.C + tok0 * 64;
  f32x16_t accM[2], accS[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) accM[rb][r] = accS[rb][r] = 0.0f;
  const int col = 32 * w + l32;
  const int tt = tid >> 4, rsub = tid & 15;  // W rows: token tt, rows rsub + 16 e

  for (int tb = 0; tb < len; tb += kSub) {
    const int nt = len - tb < kSub ? len - tb : kSub;
    // loads: the core (16 B per thread), this thread's 4 rows of V, and the
    // wave's K rows for the 8 token pairs (token tb + 2 p + G, row col)
    f32x4_t cv = {0.0f, 0.0f, 0.0f, 0.0f};
    if (tt < nt) cv = *reinterpret_cast<const f32x4_t*>(Cs + static_cast<long long>(tb + tt) * 64 + 4 * rsub);
    u32x4_t vr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = rsub + 16 * e;
      vr[e] = u32x4_t{0u, 0u, 0u, 0u};
      if (tt < nt && row < P.m)
        vr[e] = *reinterpret_cast<const u32x4_t*>(Vs + (static_cast<long long>(tb + tt) * P.m + row) * 8);
    }
    u32x4_t kf[kSub / 2];
#pragma unroll
    for (int p = 0; p < kSub / 2; ++p) {
      const int t = 2 * p + G;
      kf[p] = u32x4_t{0u, 0u, 0u, 0u};
      if (t < nt && col < P.n)
        kf[p] = *reinterpret_cast<const u32x4_t*>(Ks + (static_cast<long long>(tb + t) * P.n + col) * 8);
    }
    *reinterpret_cast<f32x4_t*>(&cs[tt][4 * rsub]) = cv;
    __syncthreads();  // cores staged (and the weights, on the first pass)

    // W = V C for 4 rows of token tt, scaled by the token's two weights
    const float sm = tt < nt ? wgt[0][tb + tt] : 0.0f;
    const float ss = (with_s && tt < nt) ? wgt[1][tb + tt] : 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v[8];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        v[2 * h] = lo_bf16(vr[e][h]);
        v[2 * h + 1] = hi_bf16(vr[e][h]);
      }
      float o[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) o[c] = 0.0f;
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] = fmaf(v[r], cs[tt][r * 8 + c], o[c]);
      const int row = rsub + 16 * e;
      u32x4_t pm, ps;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        pm[h] = pack_bf16x2(o[2 * h] * sm, o[2 * h + 1] * sm);
        ps[h] = pack_bf16x2(o[2 * h] * ss, o[2 * h + 1] * ss);
      }
      *reinterpret_cast<u32x4_t*>(&wm[tt][row][0]) = pm;
      if (with_s) *reinterpret_cast<u32x4_t*>(&wsh[tt][row][0]) = ps;
    }
    __syncthreads();  // W of the sub-batch staged

#pragma unroll
    for (int p = 0; p < kSub / 2; ++p) {
      const bf16x8_t kb = __builtin_bit_cast(bf16x8_t, kf[p]);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const bf16x8_t am = *reinterpret_cast<const bf16x8_t*>(&wm[2 * p + G][32 * rb + l32][0]);
        accM[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, kb, accM[rb], 0, 0, 0);
        if (with_s) {
          const bf16x8_t as = *reinterpret_cast<const bf16x8_t*>(&wsh[2 * p + G][32 * rb + l32][0]);
          accS[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as, kb, accS[rb], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // every wave has read the sub-batch before it is replaced
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
