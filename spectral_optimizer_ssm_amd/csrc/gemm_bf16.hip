// Newton-Schulz matrix products on the gfx950 matrix cores: bf16 inputs,
// fp32 accumulation (v_mfma_f32_32x32x16_bf16).
//
// "Muon Meets Mamba" (abstract) orthogonalises each weight update with a
// Newton-Schulz iteration; "MuonSSM" (section on convergence and complexity)
// notes that its matrix products are the method's constant-factor cost.  One
// cubic step on the oriented iterate X (s x l, s <= l) is
//     X' = a X + b (X X^T) X = A' X,   A' = a I + b X X^T   (symmetric)
// computed as two launches:
//   gram    : A' = alpha I + beta X X^T, only tiles on or above the diagonal,
//             each stored in place and mirrored;
//   combine : Y  = A' X, a plain product.
// On the first step X holds the unnormalised U and the Frobenius
// normalisation is folded in: alpha = a / (nu + eps), beta = b / (nu + eps)^3,
// with nu re-reduced from the momentum pass's per-block partial sums.
//
// Layout: X [count][s_pad][ld], A' [count][s_pad][s_pad], bf16 row-major,
// s_pad % 256 == 0, ld % 256 == 0, zero padding (stays zero: padded rows and
// columns of A' are zero).  The Gram's contraction stops at kdim, the first
// multiple of 64 >= l.
//
// Tiling: 256 x 256 workgroup tile, four waves of 128 x 128 (4 x 4 MFMA blocks
// of 32 x 32), BK = 64, two LDS stages of 64 KB filled by
// global_load_lds_dwordx4 (each lane's 16 bytes land at base + 16 * lane, so a
// wave writes 1 KB of LDS per instruction; the global address each lane
// fetches implements the swizzle).
//  * K-contiguous operands (rows of X in the Gram, rows of A' in the combine)
//    sit as [256 rows][64 K] with 16-byte chunks XOR-swizzled by (row>>1)&7
//    and are read as ds_read_b128 fragments.
//  * The combine's X operand is contracted over X's row index: it sits
//    row-major as [64 rows j][256 columns k] (chunks swizzled by 4*(j&3)) and
//    its fragments come from ds_read_b64_tr_b16: 16 lanes each address 4
//    elements of a 4 x 16 block and every lane receives one column's 4
//    consecutive rows, exactly the MFMA operand layout.
// The MFMA's M side is X's column index in the combine, so each lane ends up
// with 4 consecutive columns of one output row (8-byte stores).
//
// Work distribution: one launch covers every shape group of the step
// (segments).  Workgroups are dealt to the 8 XCDs round-robin by hardware;
// each segment's tiles are cut into 8 contiguous shares and XCD x runs share x
// of every segment, heaviest segment first, so the tiles of a matrix share an
// L2 and long tiles start early.
#include "common.cuh"
#include "launch.h"

namespace muon {
namespace {

constexpr int T = 256;          // workgroup tile (both dims)
constexpr int BK = 64;          // K per LDS stage
constexpr int WT = 128;         // wave tile
constexpr int F = WT / 32;      // MFMA blocks per wave dimension
constexpr int NTHR = 256;
constexpr int OPB = T * BK * 2; // bytes of one operand tile per stage (32 KB)
constexpr int NXCD = 8;

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void dma16(const void* src, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_wave_base, 16, 0, 0);
}

// ---- K-contiguous operand: [256 rows][64 K], 128-byte rows -------------------
__device__ __forceinline__ int rswz(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

// Each of the 4 waves issues 8 instructions = 512 chunks of the 2048.
__device__ __forceinline__ void load_rows(char* op, const bf16_t* src, long long ld, int k0) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int blk = w * 8 + i;
    const int P = blk * 64 + lane;
    const int r = P >> 3, pc = P & 7;
    const int c = pc ^ ((r >> 1) & 7);
    dma16(src + r * ld + k0 + c * 8, op + blk * 1024);
  }
}

__device__ __forceinline__ bf16x8_t frag_rows(const char* op, int row0, int ks, int lane) {
  const int r = row0 + (lane & 31);
  return *reinterpret_cast<const bf16x8_t*>(op + rswz(r, ks * 2 + (lane >> 5)));
}

// ---- X operand of the combine: [64 rows j][256 cols k], 512-byte rows -------
__device__ __forceinline__ int xswz(int j, int c) { return j * 512 + ((c ^ ((j & 3) << 2)) << 4); }

__device__ __forceinline__ void load_xrows(char* op, const bf16_t* X, long long ld, int j0, int k0) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int blk = w * 8 + i;
    const int P = blk * 64 + lane;
    const int j = P >> 5, pc = P & 31;
    const int c = pc ^ ((j & 3) << 2);
    dma16(X + (j0 + j) * ld + k0 + c * 8, op + blk * 1024);
  }
}

// MFMA operand with rows = columns k0..k0+31 of X and the 16 contraction
// values j = 16 ks + 8 (lane / 32) + 0..7.
__device__ __forceinline__ bf16x8_t frag_xcols(const char* op, int k0, int ks, int lane) {
  const int g = lane >> 4, jj = lane & 15;
  const int kk = k0 + 16 * (g & 1) + 4 * (jj & 3);
  const int c = kk >> 3, half = (kk >> 2) & 1;
  u32x2_t part[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = ks * 16 + 8 * (g >> 1) + 4 * h + (jj >> 2);
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(op + xswz(j, c) + half * 8));
    part[h] = __builtin_bit_cast(u32x2_t, v);
  }
  // whole-register repacking: 4 + 4 contraction values -> one 8-value operand
  const u32x4_t w = {part[0][0], part[0][1], part[1][0], part[1][1]};
  return __builtin_bit_cast(bf16x8_t, w);
}

struct Acc {
  f32x16_t c[F][F];
  __device__ void zero() {
#pragma unroll
    for (int i = 0; i < F; ++i)
#pragma unroll
      for (int j = 0; j < F; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) c[i][j][r] = 0.0f;
  }
};

__device__ __forceinline__ void wait_dma_and_sync() {
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) lgkmcnt(0) expcnt(0): this wave's LDS fills landed
  __syncthreads();
}

// ---- segment table ----------------------------------------------------------
__device__ __forceinline__ bool find_tile(const GemmArgs& G, int& seg, int& tile) {
  const int x = blockIdx.x % NXCD;
  int local = blockIdx.x / NXCD;
  for (int s = 0; s < G.nseg; ++s) {
    const int tot = G.seg[s].count * G.seg[s].tiles_per_mat;
    const int q = (tot + NXCD - 1) / NXCD;
    const int lo = x * q;
    const int len = lo >= tot ? 0 : (lo + q <= tot ? q : tot - lo);
    if (local < len) {
      seg = s;
      tile = lo + local;
      return true;
    }
    local -= len;
  }
  return false;
}

__device__ __forceinline__ float seg_inv(const GemmSeg& S, int z, float* red) {
  if (S.partials == nullptr) return 1.0f;
  return inv_norm_from_partials(S.partials + static_cast<long long>(z) * S.P, S.P, S.eps, red, nullptr);
}

// ---- Gram: A' = alpha I + beta X X^T ------------------------------------------
__global__ void __launch_bounds__(NTHR) gram_bf16_kernel(GemmArgs G) {
  __shared__ __attribute__((aligned(1024))) char lds0[2 * OPB];
  __shared__ __attribute__((aligned(1024))) char lds1[2 * OPB];
  __shared__ float red[NTHR / 64];
  int si, tile;
  if (!find_tile(G, si, tile)) return;
  const GemmSeg& S = G.seg[si];
  const int z = tile / S.tiles_per_mat;
  int t = tile % S.tiles_per_mat, bi = 0;
  const int nt = S.s_pad / T;
  while (t >= nt - bi) { t -= nt - bi; ++bi; }
  const int bj = bi + t;
  const bool diag = bi == bj;
  const bf16_t* X = S.X + z * S.xstride;
  bf16_t* A = S.A + z * S.astride;
  const float inv = seg_inv(S, z, red);
  const float alpha = S.a * inv, beta = S.b * inv * inv * inv;

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  Acc acc;
  acc.zero();
  const bf16_t* srcA = X + static_cast<long long>(bi) * T * S.ld;
  const bf16_t* srcB = X + static_cast<long long>(bj) * T * S.ld;
  const int nk = S.kdim / BK;

  auto stage_load = [&](char* buf, int kt) {
    load_rows(buf, srcA, S.ld, kt * BK);
    if (!diag) load_rows(buf + OPB, srcB, S.ld, kt * BK);
  };
  auto stage_mma = [&](const char* buf) {
    const char* ta = buf;
    const char* tb = diag ? buf : buf + OPB;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t fa[F], fb[F];
#pragma unroll
      for (int i = 0; i < F; ++i) fa[i] = frag_rows(ta, wm * WT + i * 32, ks, lane);
#pragma unroll
      for (int j = 0; j < F; ++j) fb[j] = frag_rows(tb, wn * WT + j * 32, ks, lane);
#pragma unroll
      for (int i = 0; i < F; ++i)
#pragma unroll
        for (int j = 0; j < F; ++j)
          acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc.c[i][j], 0, 0, 0);
    }
  };

  stage_load(lds0, 0);
  wait_dma_and_sync();
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {
    stage_load(lds1, kt + 1);
    stage_mma(lds0);
    wait_dma_and_sync();
    if (kt + 2 < nk) stage_load(lds0, kt + 2);
    stage_mma(lds1);
    wait_dma_and_sync();
  }
  if (kt < nk) stage_mma(lds0);

  // epilogue: D[m][n] = (X X^T)[bi*T + m][bj*T + n]; lane: 4 consecutive m at one n
  const int col = lane & 31, rq = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < F; ++i) {
#pragma unroll
    for (int j = 0; j < F; ++j) {
      const int gn = bj * T + wn * WT + j * 32 + col;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int gm = bi * T + wm * WT + i * 32 + q * 8 + rq;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = beta * acc.c[i][j][4 * q + r] + ((gm + r == gn) ? alpha : 0.0f);
        const u32x2_t w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        *reinterpret_cast<u32x2_t*>(A + static_cast<long long>(gn) * S.s_pad + gm) = w;  // mirrored
        if (!diag) {
          bf16_t* p = A + static_cast<long long>(gm) * S.s_pad + gn;
          p[0] = static_cast<bf16_t>(w[0] & 0xFFFF);
          p[S.s_pad] = static_cast<bf16_t>(w[0] >> 16);
          p[2 * S.s_pad] = static_cast<bf16_t>(w[1] & 0xFFFF);
          p[3 * S.s_pad] = static_cast<bf16_t>(w[1] >> 16);
        }
      }
    }
  }
}

// ---- combine: Y = A' X --------------------------------------------------------
// D[k][i] = sum_j X[j][k] A'[i][j] = (A' X)[i][k]
__global__ void __launch_bounds__(NTHR) combine_bf16_kernel(GemmArgs G) {
  __shared__ __attribute__((aligned(1024))) char lds0[2 * OPB];
  __shared__ __attribute__((aligned(1024))) char lds1[2 * OPB];
  int si, tile;
  if (!find_tile(G, si, tile)) return;
  const GemmSeg& S = G.seg[si];
  const int z = tile / S.tiles_per_mat;
  const int t = tile % S.tiles_per_mat;
  const int tiles_k = S.ld / T;
  const int tk = t % tiles_k, ti = t / tiles_k;
  const bf16_t* X = S.X + z * S.xstride;
  bf16_t* Y = S.Y + z * S.xstride;
  const bf16_t* Ap = S.A + z * S.astride + static_cast<long long>(ti) * T * S.s_pad;

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  Acc acc;
  acc.zero();
  const int nk = S.s_pad / BK;

  auto stage_load = [&](char* buf, int kt) {
    load_xrows(buf, X, S.ld, kt * BK, tk * T);
    load_rows(buf + OPB, Ap, S.s_pad, kt * BK);
  };
  auto stage_mma = [&](const char* buf) {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t fx[F], fa[F];
#pragma unroll
      for (int i = 0; i < F; ++i) fx[i] = frag_xcols(buf, wm * WT + i * 32, ks, lane);
#pragma unroll
      for (int j = 0; j < F; ++j) fa[j] = frag_rows(buf + OPB, wn * WT + j * 32, ks, lane);
#pragma unroll
      for (int i = 0; i < F; ++i)
#pragma unroll
        for (int j = 0; j < F; ++j)
          acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fx[i], fa[j], acc.c[i][j], 0, 0, 0);
    }
  };

  stage_load(lds0, 0);
  wait_dma_and_sync();
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {
    stage_load(lds1, kt + 1);
    stage_mma(lds0);
    wait_dma_and_sync();
    if (kt + 2 < nk) stage_load(lds0, kt + 2);
    stage_mma(lds1);
    wait_dma_and_sync();
  }
  if (kt < nk) stage_mma(lds0);

  // lane: row i = ti*T + wn*WT + j*32 + (lane & 31); columns k = ... + 8q + 4 (lane >> 5) + 0..3
  const int col = lane & 31, rq = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < F; ++i) {
#pragma unroll
    for (int j = 0; j < F; ++j) {
      const int gi = ti * T + wn * WT + j * 32 + col;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int gk = tk * T + wm * WT + i * 32 + q * 8 + rq;
        const u32x2_t w = {pack_bf16x2(acc.c[i][j][4 * q + 0], acc.c[i][j][4 * q + 1]),
                           pack_bf16x2(acc.c[i][j][4 * q + 2], acc.c[i][j][4 * q + 3])};
        *reinterpret_cast<u32x2_t*>(Y + static_cast<long long>(gi) * S.ld + gk) = w;
      }
    }
  }
}

int grid_for(const GemmArgs& G) {
  int per_xcd = 0;
  for (int s = 0; s < G.nseg; ++s) {
    const int tot = G.seg[s].count * G.seg[s].tiles_per_mat;
    per_xcd += (tot + NXCD - 1) / NXCD;
  }
  return per_xcd * NXCD;
}

}  // namespace

int gram_tiles_per_matrix(int s_pad) {
  const int nt = s_pad / T;
  return nt * (nt + 1) / 2;
}
int combine_tiles_per_matrix(int s_pad, int ld) { return (s_pad / T) * (ld / T); }

hipError_t launch_gram_bf16(const GemmArgs& G, hipStream_t st) {
  const int grid = grid_for(G);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(gram_bf16_kernel, dim3(grid), dim3(NTHR), 0, st, G);
  return hipGetLastError();
}

hipError_t launch_combine_bf16(const GemmArgs& G, hipStream_t st) {
  const int grid = grid_for(G);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_bf16_kernel, dim3(grid), dim3(NTHR), 0, st, G);
  return hipGetLastError();
}

}  // namespace muon
