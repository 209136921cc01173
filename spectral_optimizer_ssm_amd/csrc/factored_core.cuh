// The r x r Newton-Schulz core of four factored injections on one wavefront,
// shared by the factored kernel (ns_factored.hip) and the fused momentum
// pathway (ssm_momentum.hip).
//
// "MuonSSM: Orthogonalizing State Space Models" (method section on the
// value-key injections and their light Newton-Schulz step): for X = V K^T
// with V m x r and K n x r every NS step keeps the form X_k = V C_k K^T,
//   P = V^T V,  S = K^T K,  nu = ||X||_F = sqrt(tr(P S)),  C_0 = I / (nu + eps),
//   N = C S C^T P   (so that X X^T X = V (N C) K^T),
//   C <- a C + b N C + c N N C.
//
// LDS of a wavefront: the four matrices' V and K side by side as 64-byte rows
// of four 16-byte slots (matrix q's r = 8 bf16 in slot q, zero padded), V
// rows first, so one v_mfma_f32_32x32x16_bf16 per 16 rows gives the four
// Gram matrices at once on its diagonal 8 x 8 blocks (operands from two
// ds_read_b64_tr_b16 per lane); the 8 x 8 recurrence then runs on 16 lanes
// per matrix, each lane owning 4 entries of one row, through LDS.  Slot q of
// row t sits at position q ^ x(t), with bit 0 of x(t) bit 2 of t and bit 1
// of x(t) bit 1 of t xor bit 3: the rows of equal parity among eight
// consecutive ones (the rows of a 16-byte access served together by 32
// four-byte banks) and those of equal residue mod 4 among sixteen (the same
// by 64 banks) get distinct positions, and rows t and t + 2 of a transposing
// read's four-row group get disjoint position pairs.
#pragma once

#include "common.cuh"

namespace muon {
namespace fact {

constexpr int kMats = 4;   // matrices per wavefront
constexpr int kRow = 64;   // bytes per staged row (32 bf16 columns)

// Byte offset of slot q (matrix q's 16 bytes) of staged row t.
__device__ __forceinline__ int slot(int t, int q) {
  const int x = ((t >> 2) & 1) | (((t >> 1) ^ (t >> 3)) & 1) << 1;
  return t * kRow + 16 * (q ^ x);
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// The 8 x 8 float32 work matrices: rows kLd = 9 floats apart, so the eight
// rows' entries of one column fall on distinct banks; each matrix's six in a
// block of 440 floats, so the four matrices of a wave start 24 banks apart
// (mod 32) and an access to the same entry of all four, or to one column of
// each, does not collide.
constexpr int kLd = 9;
constexpr int kMatF = 8 * kLd, kGroupF = 6 * kMatF + 8;

// LDS of one wavefront.
struct WaveLds {
  char* vk;      // (m_pad + n_pad) x kRow: V rows, then K rows
  float* f;      // kMats x 6 matrices: P, S, C, T1, N, T2
  float* t;      // m_pad x 32 floats: V C of the four matrices (dense output only)
  __device__ float* mat(int q, int which) const { return f + q * kGroupF + which * kMatF; }
};
enum { kP = 0, kS, kC, kT1, kN, kT2 };
constexpr int kWorkBytes = kMats * kGroupF * 4;

// Gram of the 32 staged columns over rows [row0, row0 + rows): lane l holds
// column l % 32, rows 8 (g / 4) + 4 (l / 32) + g % 4 of the 32 x 32 result.
__device__ __forceinline__ bf16x8_t gram_operand(const char* vk, int k0, int lane) {
  // A operand: row (= staged column) lane % 32, contraction index
  // k0 + 8 (lane / 32) + 0..7; lane 16g + 4rr + u addresses staged row
  // k0 + 8 (g >> 1) + 4h + rr, columns colbase + 4u .. + 3 (slot
  // colbase / 8 + u / 2, bytes 8 (u % 2) ..).
  const int g = lane >> 4;
  const int colbase = 16 * (g & 1);
  const int rr = (lane & 15) >> 2, u = lane & 3;
  u32x2_t part[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = k0 + 8 * (g >> 1) + 4 * h + rr;
    const char* p = vk + slot(row, (colbase >> 3) + (u >> 1)) + 8 * (u & 1);
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p);
    part[h] = __builtin_bit_cast(u32x2_t, v);
  }
  const u32x4_t w = {part[0][0], part[0][1], part[1][0], part[1][1]};
  return __builtin_bit_cast(bf16x8_t, w);
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
  return acc;
}

__device__ __forceinline__ f32x16_t gram32(const char* vk, int row0, int rows, int lane) {
  f32x16_t acc = zero16();
  for (int k0 = 0; k0 < rows; k0 += 16) {
    const bf16x8_t a = gram_operand(vk, row0 + k0, lane);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc, 0, 0, 0);
  }
  return acc;
}

// Both Grams for row counts known at compile time, their k-steps interleaved
// (two independent accumulation chains); each accumulates in the same order
// as gram32.
template <int MP, int NP>
__device__ __forceinline__ void gram32_pair(const char* vk, int lane, f32x16_t& gp, f32x16_t& gq) {
  static_assert(MP % 16 == 0 && NP % 16 == 0 && MP <= NP, "padded row counts");
  gp = zero16();
  gq = zero16();
#pragma unroll
  for (int k0 = 0; k0 < NP; k0 += 16) {
    if (k0 < MP) {
      const bf16x8_t a = gram_operand(vk, k0, lane);
      gp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, gp, 0, 0, 0);
    }
    const bf16x8_t b = gram_operand(vk, MP + k0, lane);
    gq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, gq, 0, 0, 0);
  }
}

// Sum over the 16 lanes of each row of the wave (DPP: no LDS round trip).
// The pairing is that of a butterfly over lane bits 0, 1, 2, 3 (the mirrors
// pair the same groups as bits 2 and 3), so every lane ends with the same
// sum a shuffle butterfly gives.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f32<0xb1>(v);     // quad_perm [1, 0, 3, 2]: lane ^ 1
  v += dpp_f32<0x4e>(v);     // quad_perm [2, 3, 0, 1]: lane ^ 2
  v += dpp_f32<0x141>(v);    // row_half_mirror: lane i <-> 7 - i within 8
  v += dpp_f32<0x140>(v);    // row_mirror: lane i <-> 15 - i within 16
  return v;
}

// Keep the diagonal 8 x 8 blocks of a gram32 result: lane l writes rows
// 4 (l / 32) + 0..3, column l % 8 of matrix (l % 32) / 8.
// (Each lane stores under its own matrix's branch: a select of the register
// group by lane compiles to a 16-way select chain per value.)
__device__ __forceinline__ void store_blocks(const f32x16_t& acc, const WaveLds& L, int which, int lane) {
  const int q = (lane & 31) >> 3, j = lane & 7, i0 = 4 * (lane >> 5);
#pragma unroll
  for (int qq = 0; qq < kMats; ++qq)
    if (q == qq) {
      float* dst = L.mat(qq, which);
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(i0 + e) * kLd + j] = acc[4 * qq + e];
    }
}

// Z = X Y (or X Y^T) for the wave's four 8 x 8 matrices; lane l handles
// matrix l / 16, row i = (l % 16) / 2, columns j0 .. j0 + 3 with j0 = 4 (l % 2).
template <bool TRANS_Y>
__device__ __forceinline__ void mm8(const WaveLds& L, int x, int y, int z, int lane) {
  const int q = lane >> 4, i = (lane & 15) >> 1, j0 = 4 * (lane & 1);
  const float* X = L.mat(q, x);
  const float* Y = L.mat(q, y);
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float xv = X[i * kLd + c];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(xv, TRANS_Y ? Y[(j0 + e) * kLd + c] : Y[c * kLd + j0 + e], acc[e]);
  }
  wave_sync();  // every lane has read X and Y before Z (which may alias neither) is written
  float* Z = L.mat(q, z);
#pragma unroll
  for (int e = 0; e < 4; ++e) Z[i * kLd + j0 + e] = acc[e];
  wave_sync();
}

// The cores C of the four matrices staged in L.vk (V rows 0 .. m_pad - 1, K
// rows m_pad .. m_pad + n_pad - 1), left in L.mat(q, kC).  Args supplies
// m_pad, n_pad (multiples of 16), r, eps, steps and the per-step
// coefficients a[], b[], c[]; MP and NP, when nonzero, are m_pad and n_pad
// known at compile time (the Gram loops then unroll, so the staged rows of
// later k-steps are read while earlier ones are multiplied).  Both Grams are
// read before either is stored, so the work matrices may lie over the staged
// rows.
template <int MP = 0, int NP = 0, class Args>
__device__ __forceinline__ void core(const Args& F, const WaveLds& L, int lane) {
  const int r = F.r;
  // P = V^T V and S = K^T K on the matrix cores
  f32x16_t gp, gq;
  if constexpr (MP > 0 && NP > 0) {
    gram32_pair<MP, NP>(L.vk, lane, gp, gq);
  } else {
    gp = gram32(L.vk, 0, F.m_pad, lane);
    gq = gram32(L.vk, F.m_pad, F.n_pad, lane);
  }
  wave_sync();
  store_blocks(gp, L, kP, lane);
  store_blocks(gq, L, kS, lane);
  wave_sync();

  // nu^2 = tr(P S) per matrix (16 lanes each), C_0 = I_r / (nu + eps)
  const int q = lane >> 4, i = (lane & 15) >> 1, j0 = 4 * (lane & 1);
  float inv;
  {
    const float* P = L.mat(q, kP);
    const float* S = L.mat(q, kS);
    float t2 = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) t2 = fmaf(P[i * kLd + j0 + e], S[(j0 + e) * kLd + i], t2);
    t2 = row_sum16(t2);
    inv = 1.0f / (sqrtf(t2) + F.eps);
  }
  if (F.steps == 0) {
    float* C = L.mat(q, kC);
#pragma unroll
    for (int e = 0; e < 4; ++e) C[i * kLd + j0 + e] = (i == j0 + e && i < r) ? inv : 0.0f;
    wave_sync();
    return;
  }

  // The first step from C_0 = inv I_r (P and S vanish outside the leading
  // r x r block): C S C^T = inv^2 S, so N = inv^2 S P, N C = inv^3 S P and
  // N N C = inv^5 (S P)^2 -- one product (two for a quintic step) instead of
  // four (five).  The powers of inv are applied one factor at a time, so a
  // zero product stays zero however large 1 / eps is.
  {
    const bool quintic = F.c[0] != 0.0f;
    mm8<false>(L, kS, kP, kT1, lane);                 // S P
    if (quintic) mm8<false>(L, kT1, kT1, kT2, lane);  // (S P)^2
    float* C = L.mat(q, kC);
    const float* SP = L.mat(q, kT1);
    const float* SP2 = L.mat(q, kT2);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int o = i * kLd + j0 + e;
      const float c0 = (i == j0 + e && i < r) ? inv : 0.0f;
      const float nc = ((SP[o] * inv) * inv) * inv;
      float v = fmaf(F.a[0], c0, F.b[0] * nc);
      if (quintic) v = fmaf(F.c[0], ((((SP2[o] * inv) * inv) * inv) * inv) * inv, v);
      C[o] = v;
    }
    wave_sync();
  }

  // later steps: the r x r recurrence in full (zero padding stays zero)
  for (int k = 1; k < F.steps; ++k) {
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
      const int o = i * kLd + j0 + e;
      float v = fmaf(F.a[k], C[o], F.b[k] * NC[o]);
      if (quintic) v = fmaf(F.c[k], NNC[o], v);
      C[o] = v;
    }
    wave_sync();
  }
}

}  // namespace fact
}  // namespace muon
