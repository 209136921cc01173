// Momentum pathway of MuonSSM over sequences of factored injections.
//
// "MuonSSM: Orthogonalizing State Space Models" (method section on the
// momentum-augmented state update; theory section, parallelism): beside the
// memory state S_t a momentum state M_t accumulates the Newton-Schulz
// conditioned injections, and the pair follows a block-affine recurrence.
// Read as heavy-ball momentum on the memory:
//   U_t = NS(V_t K_t^T) = V_t C_t K_t^T = W_t K_t^T   (r x r core C_t, factored_core.cuh)
//   M_t = beta M_{t-1} + U_t,   S_t = a_t S_{t-1} + M_t.
// Neither U_t (16 KB dense for a 64 x 128 injection) nor W_t = V_t C_t ever
// reaches memory: one kernel forms every token's core from its factors and
// folds W_t K_t^T into float32 partial sums on the matrix cores.
//
// Regrouping.  Over L tokens u = 0..L-1 entered with (S, M):
//   M' = beta^L M + sum_u beta^(L-1-u) U_u
//   S' = A S + B M + sum_u w_u U_u,   A = prod_u a_u,   B = beta w_0,
//   w_u = g_u + beta w_{u+1} (w_L = 0),   g_u = prod_{s>u} a_s.
// The fused kernel forms the two sums of a chunk of 256 tokens with the
// weights taken relative to the chunk's end, and the chunk's map (beta^L, A,
// B); the combine kernel applies the chunk maps in token order to the
// caller's (S, M).  Maps and sums are the recurrence regrouped (the
// block-affine structure the pages point to).
//
// Fused kernel: one workgroup of four waves per (sequence, chunk), persistent
// over chunks, two workgroups per CU.  At a chunk's start every wave computes
// its weights by suffix scans over the chunk's decays.  In a round of 16
// tokens each wave stages four tokens' V and K in its own LDS area
// (factored_core.cuh layout), loads the next round's factors into registers,
// runs the core and forms the weighted factors W_M = V (wm C) over its V rows
// and W_S = V (ws C) in its work area on the matrix cores.  After a barrier
// wave w accumulates the column block 32 w .. 32 w + 31 (both 32-row blocks)
// of the zero-padded 64 x 128 tiles of both sums over the round's tokens on
// v_mfma_f32_32x32x16_bf16, the contraction index being (token pair, rank):
// weighted-factor rows are the A operand, K rows the B operand.  The next
// round's barrier keeps the areas until every wave has read them.
#include "common.cuh"
#include "factored_core.cuh"
#include "launch.h"

namespace muon {
namespace {

using fact::kRow;
using fact::slot;
using fact::wave_sync;

constexpr int kTileM = 64, kTileN = 128, kTile = kTileM * kTileN;
constexpr int kWaves = 4;                          // waves per workgroup
constexpr int kRound = kWaves * fact::kMats;       // tokens per round
constexpr int kStage = (kTileM + kTileN) * kRow;   // staged V and K rows of a wave
constexpr int kArea = kStage + fact::kWorkBytes;   // LDS of a wave
constexpr int kFusedLds = kWaves * kArea;          // 75.5 KB: two workgroups per CU
static_assert(kSsmMomQ % kRound == 0, "chunks are whole rounds");
static_assert(kTileM * kRow <= fact::kWorkBytes, "the work area holds the 64 rows of W_S");
static_assert(2 * kFusedLds <= 160 * 1024, "two workgroups fit a CU");

// Factors of a wave's four tokens: lane l holds rows l + 64 e of their
// concatenated V rows (e < 4) and K rows (e < 8), zero past the valid tokens.
struct RoundRegs {
  u32x4_t v[4], k[8];
};

// tokr: first token of the round (index into [nseq * T]); nvr: its valid
// tokens.  Buffer loads through resources that end with the wave's valid
// tokens: rows past them read as zero without a select.
template <bool FIXED>
__device__ __forceinline__ void load_round(const SsmMomLaunch& P, long long tokr, int nvr, int w, int lane,
                                           RoundRegs& R) {
  const int m = FIXED ? kTileM : P.m, n = FIXED ? kTileN : P.n;
  // the clamp compiles to a vector-unit median; moved back to a scalar so
  // that the resources below stay in scalar registers (a resource in vector
  // registers is wrapped in a loop over the lanes' distinct values)
  const int nv0 = nvr - fact::kMats * w;
  const int nv = __builtin_amdgcn_readfirstlane(nv0 < 0 ? 0 : nv0 > fact::kMats ? fact::kMats : nv0);
  const long long tok = tokr + fact::kMats * w;
  // one 16-byte row per rank-8 row
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(P.V) + tok * m * 8, static_cast<short>(0), nv * m * 16, 0x00020000);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(P.K) + tok * n * 8, static_cast<short>(0), nv * n * 16, 0x00020000);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    R.v[e] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, (lane + 64 * e) * 16, 0, 0));
#pragma unroll
  for (int e = 0; e < 8; ++e)
    R.k[e] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, (lane + 64 * e) * 16, 0, 0));
}

// Row t of token q goes to staged row t, slot q; K rows after the 64 V rows.
// Rows past m and n are never written (zero from the start).
template <bool FIXED>
__device__ __forceinline__ void stage_round(const SsmMomLaunch& P, char* vk, const RoundRegs& R, int lane) {
  const int m = FIXED ? kTileM : P.m, n = FIXED ? kTileN : P.n;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = lane + 64 * e;
    if (c < fact::kMats * m) {
      const int q = c / m, t = c - q * m;
      *reinterpret_cast<u32x4_t*>(vk + slot(t, q)) = R.v[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = lane + 64 * e;
    if (c < fact::kMats * n) {
      const int q = c / n, u = c - q * n;
      *reinterpret_cast<u32x4_t*>(vk + slot(kTileM + u, q)) = R.k[e];
    }
  }
}

// The round's weighted factors of the wave's nv valid tokens q (token
// 4 w + q of the round), on the matrix cores:
//   W_M = V (wm C) over the staged V rows (in place),
//   W_S = V (ws C) into the wave's work area (same row and slot layout),
// so that token q adds W_M K^T to the momentum sum and W_S K^T to the memory
// sum.  Per 32-row block, W^T (rows (token q, rank c), columns the block's V
// rows) = BD^T V^T with BD the block-diagonal of the four weighted cores, the
// contraction (token, rank d) taken 16 at a time (two tokens).  The weighted
// core enters as two bf16 terms (hi + lo, to about 2^-17 relative), so with
// the exact bf16 V the float32 products and sums match a float32 V (w C) to
// about 2^-16 before the one rounding of W to bf16.  Every V row and core is
// read before any W row is written; rows past m stay zero.
__device__ __forceinline__ void write_w(const fact::WaveLds& L, int nv, float wmq, float wsq, bool with_s,
                                        int lane) {
  const int i = lane & 31, kg = lane >> 5;
  const int qc = i >> 3, c = i & 7;        // A operand row: core qc, column c
  const bool live = qc < nv;
  const float* C = L.mat(qc, fact::kC);
  float col[8];                            // column c of core qc (rows d), or zeros
#pragma unroll
  for (int d = 0; d < 8; ++d) col[d] = live ? C[d * fact::kLd + c] : 0.0f;
  const float sw[2] = {wmq, wsq};   // the two weights of core qc
  // A operands for the token pairs (0, 1) and (2, 3): lane (i, kg) holds the
  // weighted column when core qc is the pair's token kg
  bf16x8_t ahi[2][2], alo[2][2];   // [sum][pair]
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bool mine = qc == 2 * h + kg;
      u32x4_t hv, lv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = mine ? col[2 * e] * sw[u] : 0.0f, x1 = mine ? col[2 * e + 1] * sw[u] : 0.0f;
        hv[e] = pack_bf16x2(x0, x1);
        lv[e] = pack_bf16x2(x0 - lo_bf16(hv[e]), x1 - hi_bf16(hv[e]));
      }
      ahi[u][h] = __builtin_bit_cast(bf16x8_t, hv);
      alo[u][h] = __builtin_bit_cast(bf16x8_t, lv);
    }
  // B operands: lane (j, kg) holds V row 32 rb + j of token 2 h + kg (one slot)
  u32x4_t bv[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      bv[rb][h] = *reinterpret_cast<const u32x4_t*>(L.vk + slot(32 * rb + i, 2 * h + kg));
  wave_sync();  // every V row and core read before W overwrites them
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (u == 1 && !with_s) break;
    char* dst = u == 0 ? L.vk : reinterpret_cast<char*>(L.f);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      f32x16_t acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bv[rb][h]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[u][h], b, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[u][h], b, acc, 0, 0, 0);
      }
      // lane (j, kg), registers 4 q + e: row 32 rb + j, token q, ranks 4 kg + e
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2_t wv = {pack_bf16x2(acc[4 * q], acc[4 * q + 1]), pack_bf16x2(acc[4 * q + 2], acc[4 * q + 3])};
        *reinterpret_cast<u32x2_t*>(dst + slot(32 * rb + i, q) + 8 * kg) = wv;
      }
    }
  }
}

// Weights of a chunk's len tokens relative to its end, token t = 4 l + i on
// lane l (i < 4), and the chunk's map:
//   wm_t = beta^(len-1-t),  ws_t = w_t = sum_{v=t}^{len-1} beta^(v-t) g_v,
//   g_v = prod_{s>v} a_s;  map: bl = beta^len, A = prod a, B = beta w_0.
// Each lane summarises its four tokens as (pa, pf, s) = (prod a, beta^(its
// tokens), w of its first token counting only its own tokens); a suffix scan
// over the lanes joins a segment L with the one after it, R, as
// (pa_L pa_R, pf_L pf_R, pa_R s_L + pf_L s_R); each lane then walks its four
// tokens backwards from the summary of the lanes after it.  Every wave of the
// workgroup computes the same values.
struct ChunkW {
  float wm[4], ws[4];
  float bl, A, B;
};
template <bool WITH_S>
__device__ __forceinline__ ChunkW chunk_weights(const SsmMomLaunch& P, long long tok0, int len, int lane) {
  const float beta = P.beta;
  float a[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 4 * lane + i;
    a[i] = (WITH_S && t < len) ? P.a[tok0 + t] : 1.0f;
  }
  float pa = 1.0f, pf = 1.0f, sv = 0.0f;
#pragma unroll
  for (int i = 3; i >= 0; --i)
    if (4 * lane + i < len) {
      sv = fmaf(beta, sv, pa);
      pa *= a[i];
      pf *= beta;
    }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float oa = __shfl_down(pa, d, 64), of = __shfl_down(pf, d, 64), os = __shfl_down(sv, d, 64);
    if (lane + d < 64) {
      sv = fmaf(pf, os, sv * oa);
      pa *= oa;
      pf *= of;
    }
  }
  // the lanes after this one: exclusive values
  float ga = __shfl_down(pa, 1, 64), gf = __shfl_down(pf, 1, 64), w = __shfl_down(sv, 1, 64);
  if (lane == 63) {
    ga = 1.0f;
    gf = 1.0f;
    w = 0.0f;
  }
  ChunkW C;
#pragma unroll
  for (int i = 3; i >= 0; --i) {
    const bool valid = 4 * lane + i < len;   // tokens past len: no term, no factor
    if (valid) w = fmaf(beta, w, ga);
    C.wm[i] = valid ? gf : 0.0f;
    C.ws[i] = valid ? w : 0.0f;
    if (valid) {
      ga *= a[i];
      gf *= beta;
    }
  }
  C.bl = __shfl(pf, 0, 64);
  C.A = WITH_S ? __shfl(pa, 0, 64) : 0.0f;
  C.B = WITH_S ? beta * __shfl(C.ws[0], 0, 64) : 0.0f;
  return C;
}

// Workgroup barrier for the hand-over of LDS areas: this wave's LDS accesses
// complete (lgkmcnt(0)) and the barrier; the next round's factor loads stay in
// flight (vmcnt not waited for), where __syncthreads() would drain them.  The
// registers they fill are waited for where they are used.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // vmcnt(63) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// FIXED: the 64 x 128 shape; WITH_S: the memory state is carried (P.S given).
template <bool FIXED, bool WITH_S>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
ssm_momentum_fused_kernel(SsmMomLaunch P) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long nitems = P.nseq * P.nchunks;
  long long it = blockIdx.x;
  if (it >= nitems) return;  // (the grid holds no more workgroups than items)
  constexpr bool with_s = WITH_S;
  char* area = lds + w * kArea;
  fact::WaveLds L;
  L.vk = area;
  L.f = reinterpret_cast<float*>(area + kStage);
  L.t = nullptr;
  for (int o = lane * 16; o < kStage; o += 64 * 16) *reinterpret_cast<u32x4_t*>(area + o) = u32x4_t{0u, 0u, 0u, 0u};

  // chunk `it` of sequence it / nchunks: its first token and length
  auto chunk = [&](long long i, long long& tok0, int& len) {
    const long long seq = i / P.nchunks;
    const int t0 = static_cast<int>(i - seq * P.nchunks) * P.Q;
    len = P.T - t0 < P.Q ? P.T - t0 : P.Q;
    tok0 = seq * P.T + t0;
  };
  long long tok0;
  int len;
  chunk(it, tok0, len);
  RoundRegs R;
  load_round<FIXED>(P, tok0, len < kRound ? len : kRound, w, lane, R);

  const int G = lane >> 5, l32 = lane & 31;
  const int krow = kTileM + 32 * w + l32;   // wave w: tile columns 32 w .. 32 w + 31
  const int qc = l32 >> 3;                  // the core whose weights this lane applies
  for (;;) {
    const int nr = (len + kRound - 1) / kRound;
    const ChunkW cw = chunk_weights<WITH_S>(P, tok0, len, lane);
    f32x16_t accM[2], accS[2];   // row blocks 0 and 1
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) accM[rb][r] = accS[rb][r] = 0.0f;
    for (int rd = 0; rd < nr; ++rd) {
      const int nvr = len - kRound * rd < kRound ? len - kRound * rd : kRound;
      lds_barrier();  // every wave is done with the previous round's areas
      stage_round<FIXED>(P, area, R, lane);
      wave_sync();
      // the next round's factors load while this round is computed
      if (rd + 1 < nr) {
        const int nv2 = len - kRound * (rd + 1);
        load_round<FIXED>(P, tok0 + kRound * (rd + 1), nv2 < kRound ? nv2 : kRound, w, lane, R);
      } else if (it + gridDim.x < nitems) {
        long long tok2;
        int len2;
        chunk(it + gridDim.x, tok2, len2);
        load_round<FIXED>(P, tok2, len2 < kRound ? len2 : kRound, w, lane, R);
      }
      // weights of the wave's tokens 16 rd + 4 w + i (i < 4), held by lane
      // 4 rd + w; this lane applies those of its core qc
      const int src_lane = fact::kMats * rd + w;
      float wm_r[4], ws_r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wm_r[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cw.wm[i]), src_lane));
        ws_r[i] = WITH_S ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cw.ws[i]), src_lane)) : 0.0f;
      }
      const float wmq = qc == 0 ? wm_r[0] : qc == 1 ? wm_r[1] : qc == 2 ? wm_r[2] : wm_r[3];
      const float wsq = qc == 0 ? ws_r[0] : qc == 1 ? ws_r[1] : qc == 2 ? ws_r[2] : ws_r[3];
      fact::core<kTileM, kTileN>(P.ns, L, lane);   // V rows and K rows padded to the 64 x 128 tile
      int nv = nvr - fact::kMats * w;
      nv = nv < 0 ? 0 : nv;
      write_w(L, nv, wmq, wsq, with_s, lane);
      lds_barrier();  // every wave's weighted factors and K rows are staged

      for (int tp = 0; 2 * tp < nvr; ++tp) {
        // token 2 tp + G lives in wave tp / 2's area, slot q; tokens past nvr
        // have zero factors
        const int q = 2 * (tp & 1) + G;
        const char* src = lds + (tp >> 1) * kArea;
        const bf16x8_t km = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(src + slot(krow, q)));
        const bf16x8_t m0 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(src + slot(l32, q)));
        const bf16x8_t m1 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(src + slot(32 + l32, q)));
        accM[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(m0, km, accM[0], 0, 0, 0);
        accM[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(m1, km, accM[1], 0, 0, 0);
        if (with_s) {
          const char* ss = src + kStage;   // W_S rows in the work area
          const bf16x8_t s0 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(ss + slot(l32, q)));
          const bf16x8_t s1 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(ss + slot(32 + l32, q)));
          accS[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(s0, km, accS[0], 0, 0, 0);
          accS[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(s1, km, accS[1], 0, 0, 0);
        }
      }
    }

    // partials: lane (G, l32), register 4 q + e of row block rb holds row
    // 32 rb + 8 q + 4 G + e, column 32 w + l32 of the padded 64 x 128 tile;
    // stored through a buffer resource (one per-lane offset, the row offsets
    // scalar)
    {
      const int nout = with_s ? 2 : 1;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          P.part + it * nout * static_cast<long long>(kTile), static_cast<short>(0), nout * kTile * 4, 0x00020000);
      const int voff = ((4 * G) * kTileN + 32 * w + l32) * 4;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int soff = (32 * rb + 8 * q + e) * kTileN * 4;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(accM[rb][4 * q + e]), rs, voff, soff, 0);
            if (with_s)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(accS[rb][4 * q + e]), rs, voff, soff + kTile * 4,
                                                    0);
          }
    }
    if (tid == 0) {
      float* cf = P.coef + it * 4;
      cf[0] = cw.bl;
      cf[1] = cw.A;
      cf[2] = cw.B;
      cf[3] = 0.0f;
    }
    it += gridDim.x;
    if (it >= nitems) break;
    chunk(it, tok0, len);
  }
}

// (S, M) <- chunk maps in token order; one thread per state element, the
// partials of four chunks loaded before they are applied.
__global__ void __launch_bounds__(256) ssm_momentum_combine_kernel(SsmMomLaunch P) {
  const long long mn = static_cast<long long>(P.m) * P.n;
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= P.nseq * mn) return;
  const long long seq = idx / mn;
  const int e = static_cast<int>(idx - seq * mn);
  const int i = e / P.n, j = e - i * P.n;
  const bool with_s = P.S != nullptr;
  const long long stride = (with_s ? 2 : 1) * static_cast<long long>(kTile);   // floats per chunk
  const float* pb = P.part + seq * P.nchunks * stride + i * kTileN + j;
  const float4* cf = reinterpret_cast<const float4*>(P.coef) + seq * P.nchunks;
  float M = P.M[idx];
  float S = with_s ? P.S[idx] : 0.0f;
  int c = 0;
  for (; c + 4 <= P.nchunks; c += 4) {
    float pm[4], ps[4];
    float4 k[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      pm[u] = pb[(c + u) * stride];
      ps[u] = with_s ? pb[(c + u) * stride + kTile] : 0.0f;
      k[u] = cf[c + u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (with_s) S = fmaf(k[u].y, S, fmaf(k[u].z, M, ps[u]));
      M = fmaf(k[u].x, M, pm[u]);
    }
  }
  for (; c < P.nchunks; ++c) {
    const float4 k = cf[c];
    if (with_s) S = fmaf(k.y, S, fmaf(k.z, M, pb[c * stride + kTile]));
    M = fmaf(k.x, M, pb[c * stride]);
  }
  P.M[idx] = M;
  if (with_s) P.S[idx] = S;
}

}  // namespace

hipError_t launch_ssm_momentum(const SsmMomLaunch& P, hipStream_t st, int phase) {
  if (P.m > kTileM || P.n > kTileN || P.ns.r != 8 || P.ns.m_pad != kTileM || P.ns.n_pad != kTileN ||
      P.Q % kRound != 0)
    return hipErrorInvalidValue;
  if (phase == 0) {
    const long long items = P.nseq * P.nchunks;
    const long long slots = 2LL * device_cus();  // 75.5 KB of LDS: two workgroups per CU
    const unsigned blocks = static_cast<unsigned>(items < slots ? items : slots);
    const bool fixed = P.m == kTileM && P.n == kTileN, with_s = P.S != nullptr;
    const void* fn = fixed ? (with_s ? reinterpret_cast<const void*>(ssm_momentum_fused_kernel<true, true>)
                                     : reinterpret_cast<const void*>(ssm_momentum_fused_kernel<true, false>))
                           : (with_s ? reinterpret_cast<const void*>(ssm_momentum_fused_kernel<false, true>)
                                     : reinterpret_cast<const void*>(ssm_momentum_fused_kernel<false, false>));
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kFusedLds) != hipSuccess)
      return hipErrorInvalidValue;
    const dim3 grid(blocks), block(kWaves * 64);
    if (fixed && with_s)
      hipLaunchKernelGGL((ssm_momentum_fused_kernel<true, true>), grid, block, kFusedLds, st, P);
    else if (fixed)
      hipLaunchKernelGGL((ssm_momentum_fused_kernel<true, false>), grid, block, kFusedLds, st, P);
    else if (with_s)
      hipLaunchKernelGGL((ssm_momentum_fused_kernel<false, true>), grid, block, kFusedLds, st, P);
    else
      hipLaunchKernelGGL((ssm_momentum_fused_kernel<false, false>), grid, block, kFusedLds, st, P);
  } else {
    const long long blocks = (P.nseq * P.m * P.n + 255) / 256;
    hipLaunchKernelGGL(ssm_momentum_combine_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, P);
  }
  return hipGetLastError();
}

}  // namespace muon
