// Newton-Schulz matrix products on the gfx950 matrix cores, bf16 inputs and
// fp32 accumulation (v_mfma_f32_32x32x16_bf16).
//
// "Muon Meets Mamba" (abstract) orthogonalises each weight update with a
// Newton-Schulz iteration; "MuonSSM" (section on convergence and complexity)
// notes that its matrix products are the constant-factor cost of the method.
// One cubic step on the oriented iterate X (s x l, s <= l) is
//     A = X X^T            (symmetric Gram, s x s)        -> gram kernel
//     X' = a X + b A X     (polynomial combine, s x l)    -> combine kernel
// The Gram kernel computes only tiles on or above the diagonal and writes
// each one twice (in place and mirrored).  The combine kernel fuses the
// a X + b (.) epilogue.  On the first step the Frobenius normalisation is
// folded in: the Gram scales by 1/(nu+eps)^2, the combine's a and b by
// 1/(nu+eps), nu re-reduced from the momentum pass's per-block partials.
//
// Layout: X [count][s_pad][ld] and A [count][s_pad][s_pad], bf16, row-major,
// zero-padded so every tile is full (s_pad % 128 == 0, ld % 128 == 0); the
// padding stays zero through every step because padded rows and columns of A
// are zero.
//
// Main loop: 128 x 128 workgroup tile, BK = 64, four waves of 64 x 64 (2 x 2
// MFMA blocks of 32 x 32), global -> registers -> LDS double buffering with
// one barrier per K-tile.  LDS rows are 128 B (64 bf16); 16-byte chunks are
// XOR-swizzled by (row >> 1) & 7 so that the fragment reads of 16 lanes cover
// all 64 banks.
#include "common.cuh"
#include "launch.h"

namespace muon {
namespace {

constexpr int BK = 64;             // K per LDS stage (64 bf16 = 128 B per row)
constexpr int TM = 128, TN = 128;  // workgroup tile
constexpr int WM = 64, WN = 64;    // wave tile
constexpr int FM = WM / 32, FN = WN / 32;
constexpr int NWAVE = (TM / WM) * (TN / WN);
constexpr int NTHR = NWAVE * kWave;
constexpr int STAGE_A = TM * BK;   // bf16 elements per operand tile
constexpr int STAGE_B = TN * BK;

__device__ __forceinline__ int swz(int r, int c) {  // 16-B chunk index -> byte offset in a 128-B row
  return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
}

// Fragment (8 bf16) for a 32-row MFMA block at k-step ks (16 K) of a tile.
__device__ __forceinline__ bf16x8_t lds_frag(const char* tile, int row0, int ks, int lane) {
  const int r = row0 + (lane & 31);
  const int c = ks * 2 + (lane >> 5);
  return *reinterpret_cast<const bf16x8_t*>(tile + swz(r, c));
}

// --- loaders ----------------------------------------------------------------
// K-contiguous source: R rows of 64 bf16 starting at src (row stride ld).
template <int R>
struct RowLoader {
  static constexpr int N = R * 8 / NTHR;  // 16-B chunks per thread
  u32x4_t v[N];
  __device__ void load(const bf16_t* src, long long ld, int k0) {
#pragma unroll
    for (int p = 0; p < N; ++p) {
      const int q = threadIdx.x + NTHR * p;
      const int r = q >> 3, c = q & 7;
      v[p] = *reinterpret_cast<const u32x4_t*>(src + r * ld + k0 + c * 8);
    }
  }
  __device__ void store(char* tile) const {
#pragma unroll
    for (int p = 0; p < N; ++p) {
      const int q = threadIdx.x + NTHR * p;
      const int r = q >> 3, c = q & 7;
      *reinterpret_cast<u32x4_t*>(tile + swz(r, c)) = v[p];
    }
  }
};

// N-contiguous source transposed into a K-contiguous LDS tile: the tile row
// is the source column (R of them, from col0), its 64 K values are source
// rows j0..j0+63.  Each thread moves 4 source rows x 8 source columns.
template <int R>
struct TransLoader {
  static constexpr int NB = (BK / 4) * (R / 8) / NTHR;  // 4x8 blocks per thread
  u32x4_t v[NB][4];
  __device__ void load(const bf16_t* src, long long ld, int j0, int col0) {
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      const int q = threadIdx.x + NTHR * p;
      const int cc = q % (R / 8), jq = q / (R / 8);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[p][i] = *reinterpret_cast<const u32x4_t*>(src + (j0 + jq * 4 + i) * ld + col0 + cc * 8);
    }
  }
  __device__ void store(char* tile) const {
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      const int q = threadIdx.x + NTHR * p;
      const int cc = q % (R / 8), jq = q / (R / 8);
      const int jchunk = jq >> 1, half = jq & 1;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int sh = 16 * h;
          const uint32_t c0 = (v[p][0][d] >> sh) & 0xFFFFu, c1 = (v[p][1][d] >> sh) & 0xFFFFu;
          const uint32_t c2 = (v[p][2][d] >> sh) & 0xFFFFu, c3 = (v[p][3][d] >> sh) & 0xFFFFu;
          u32x2_t w = {c0 | (c1 << 16), c2 | (c3 << 16)};
          const int row = cc * 8 + 2 * d + h;
          *reinterpret_cast<u32x2_t*>(tile + swz(row, jchunk) + half * 8) = w;
        }
      }
    }
  }
};

// --- main loop ----------------------------------------------------------------
struct Acc {
  f32x16_t c[FM][FN];
};

__device__ __forceinline__ void mma_stage(const char* ta, const char* tb, int wm, int wn, Acc& acc) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    bf16x8_t fa[FM], fb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = lds_frag(ta, wm * WM + i * 32, ks, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = lds_frag(tb, wn * WN + j * 32, ks, lane);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc.c[i][j], 0, 0, 0);
  }
}

__device__ __forceinline__ float step1_inv(const NsGemmLaunch& L, int z, float* red) {
  if (L.partials == nullptr) return 1.0f;
  return inv_norm_from_partials(L.partials + static_cast<long long>(z) * L.P, L.P, L.eps, red, nullptr);
}

// --- Gram: A = X X^T, tiles bi <= bj only ------------------------------------
__global__ void __launch_bounds__(NTHR) gram_bf16_kernel(NsGemmLaunch L) {
  __shared__ __attribute__((aligned(16))) char lds[2][(STAGE_A + STAGE_B) * 2];
  __shared__ float red[NWAVE];
  const int z = blockIdx.y;
  const int nt = L.s_pad / TM;
  // linear upper-triangle index -> (bi, bj)
  int t = blockIdx.x, bi = 0;
  while (t >= nt - bi) { t -= nt - bi; ++bi; }
  const int bj = bi + t;
  const bf16_t* X = static_cast<const bf16_t*>(L.X) + z * L.xstride;
  bf16_t* A = static_cast<bf16_t*>(L.A) + z * L.astride;
  const float inv = step1_inv(L, z, red);
  const float scale = inv * inv;

  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wid / (TN / WN), wn = wid % (TN / WN);
  Acc acc;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.c[i][j][r] = 0.0f;

  const bf16_t* srcA = X + static_cast<long long>(bi) * TM * L.ld;
  const bf16_t* srcB = X + static_cast<long long>(bj) * TN * L.ld;
  RowLoader<TM> la;
  RowLoader<TN> lb;
  const int nk = L.ld / BK;
  la.load(srcA, L.ld, 0);
  lb.load(srcB, L.ld, 0);
  la.store(lds[0]);
  lb.store(lds[0] + STAGE_A * 2);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      la.load(srcA, L.ld, (kt + 1) * BK);
      lb.load(srcB, L.ld, (kt + 1) * BK);
    }
    mma_stage(lds[cur], lds[cur] + STAGE_A * 2, wm, wn, acc);
    if (kt + 1 < nk) {
      la.store(lds[cur ^ 1]);
      lb.store(lds[cur ^ 1] + STAGE_A * 2);
    }
    __syncthreads();
  }

  // D[m][n] = A[bi*TM + m][bj*TN + n]; lane holds 4 consecutive m at one n.
  const int col = lane & 31, rq = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int gn = bj * TN + wn * WN + j * 32 + col;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int gm = bi * TM + wm * WM + i * 32 + g * 8 + rq;
        const float v0 = acc.c[i][j][4 * g + 0] * scale, v1 = acc.c[i][j][4 * g + 1] * scale;
        const float v2 = acc.c[i][j][4 * g + 2] * scale, v3 = acc.c[i][j][4 * g + 3] * scale;
        // mirrored tile: A[gn][gm .. gm+3], contiguous
        u32x2_t w = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
        *reinterpret_cast<u32x2_t*>(A + static_cast<long long>(gn) * L.s_pad + gm) = w;
        if (bi != bj) {
          bf16_t* p = A + static_cast<long long>(gm) * L.s_pad + gn;
          p[0] = static_cast<bf16_t>(w[0] & 0xFFFF);
          p[L.s_pad] = static_cast<bf16_t>(w[0] >> 16);
          p[2 * L.s_pad] = static_cast<bf16_t>(w[1] & 0xFFFF);
          p[3 * L.s_pad] = static_cast<bf16_t>(w[1] >> 16);
        }
      }
    }
  }
}

// --- combine: Y = alpha X + beta A X ------------------------------------------
// MFMA M-dim = columns k of X (the long side), N-dim = rows i; the operand
// from X is its transpose (k rows, j contiguous), the operand from A is A's
// rows (A symmetric).  D[k][i] = (A X)[i][k]: each lane holds 4 consecutive k
// of one row i, so X is read and Y written 8 bytes at a time.
__global__ void __launch_bounds__(NTHR) combine_bf16_kernel(NsGemmLaunch L) {
  __shared__ __attribute__((aligned(16))) char lds[2][(STAGE_A + STAGE_B) * 2];
  __shared__ float red[NWAVE];
  const int z = blockIdx.y;
  const int tiles_k = L.ld / TM;
  const int tk = blockIdx.x % tiles_k;  // column block of X (M-dim)
  const int ti = blockIdx.x / tiles_k;  // row block of X / A (N-dim)
  const bf16_t* X = static_cast<const bf16_t*>(L.X) + z * L.xstride;
  bf16_t* Y = static_cast<bf16_t*>(L.Y) + z * L.xstride;
  const bf16_t* A = static_cast<const bf16_t*>(L.A) + z * L.astride;
  const float inv = step1_inv(L, z, red);
  const float alpha = L.alpha * inv, beta = L.beta * inv;

  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wid / (TN / WN), wn = wid % (TN / WN);
  Acc acc;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.c[i][j][r] = 0.0f;

  const bf16_t* srcA = A + static_cast<long long>(ti) * TN * L.s_pad;  // rows i of A
  TransLoader<TM> lx;
  RowLoader<TN> la;
  const int nk = L.s_pad / BK;
  lx.load(X, L.ld, 0, tk * TM);
  la.load(srcA, L.s_pad, 0);
  lx.store(lds[0]);
  la.store(lds[0] + STAGE_A * 2);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      lx.load(X, L.ld, (kt + 1) * BK, tk * TM);
      la.load(srcA, L.s_pad, (kt + 1) * BK);
    }
    mma_stage(lds[cur], lds[cur] + STAGE_A * 2, wm, wn, acc);
    if (kt + 1 < nk) {
      lx.store(lds[cur ^ 1]);
      la.store(lds[cur ^ 1] + STAGE_A * 2);
    }
    __syncthreads();
  }

  const int col = lane & 31, rq = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int gi = ti * TN + wn * WN + j * 32 + col;  // row of X / Y
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int gk = tk * TM + wm * WM + i * 32 + g * 8 + rq;  // 4 consecutive columns
        const long long off = static_cast<long long>(gi) * L.ld + gk;
        const u32x2_t xv = *reinterpret_cast<const u32x2_t*>(X + off);
        const float y0 = fmaf(alpha, lo_bf16(xv[0]), beta * acc.c[i][j][4 * g + 0]);
        const float y1 = fmaf(alpha, hi_bf16(xv[0]), beta * acc.c[i][j][4 * g + 1]);
        const float y2 = fmaf(alpha, lo_bf16(xv[1]), beta * acc.c[i][j][4 * g + 2]);
        const float y3 = fmaf(alpha, hi_bf16(xv[1]), beta * acc.c[i][j][4 * g + 3]);
        u32x2_t w = {pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
        *reinterpret_cast<u32x2_t*>(Y + off) = w;
      }
    }
  }
}

}  // namespace

hipError_t launch_gram_bf16(const NsGemmLaunch& L, hipStream_t st) {
  const int nt = L.s_pad / TM;
  const dim3 grid(nt * (nt + 1) / 2, L.count);
  hipLaunchKernelGGL(gram_bf16_kernel, grid, dim3(NTHR), 0, st, L);
  return hipGetLastError();
}

hipError_t launch_combine_bf16(const NsGemmLaunch& L, hipStream_t st) {
  const dim3 grid((L.ld / TM) * (L.s_pad / TN), L.count);
  hipLaunchKernelGGL(combine_bf16_kernel, grid, dim3(NTHR), 0, st, L);
  return hipGetLastError();
}

}  // namespace muon
