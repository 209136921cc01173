// Newton-Schulz matrix products on the gfx950 matrix cores: bf16 inputs,
// fp32 accumulation (v_mfma_f32_32x32x16_bf16).
//
// "Muon Meets Mamba" (abstract) orthogonalises each weight update with a
// Newton-Schulz iteration; "MuonSSM" (section on convergence and complexity)
// notes that its matrix products are the method's constant-factor cost.  One
// cubic step on the oriented iterate X (s x l, s <= l) is
//     X' = a X + b (X X^T) X = A' X,   A' = a I + b X X^T   (symmetric).
// Two kernels:
//   symprod_bf16_kernel : products L R^T whose result is symmetric, so only
//       tiles on or above the diagonal are computed, each stored in place and
//       mirrored, with O1 = a1 I + b1 L R^T and an optional affine second
//       output O2 = a2 I + b2 O1.  It serves the Gram X X^T (L = R = X,
//       contraction over the long side) and the products of the accumulated
//       schedule (L, R polynomials in one Gram matrix, which commute).
//   combine_bf16_kernel : Y = A' X, a plain product.
// On the first step X holds the unnormalised U and the Frobenius
// normalisation is folded into the coefficients as powers of 1/(nu + eps),
// with nu re-reduced from the momentum pass's per-block partial sums.
//
// Layout: X [count][s_pad][ld], s x s matrices [count][s_pad][s_pad], bf16
// row-major, s_pad % 256 == 0, ld % 256 == 0, zero padding (stays zero:
// padded rows of X are zero).  The Gram's contraction stops at kdim, the
// first multiple of 64 >= l.
//
// Combine tiling: 128 (i) x 256 (k) workgroup tile, four waves of 64 x 128
// made of 32 x 32 MFMA blocks, two workgroups per CU.  The contraction runs in
// stages of BK = 32 through three LDS buffers of 24 KB: the fill of stage
// kt + 2 is issued while stage kt is multiplied, so an L2 miss to MALL or HBM
// does not stall the matrix pipes.  Fills use buffer_load ... lds (each
// lane's 16 bytes land at base + 16 * lane; the per-lane source offset
// implements the swizzle).  Stage hand-over is an explicit s_waitcnt
// vmcnt(<loads of younger stages>) + s_barrier, because __syncthreads() would
// drain every outstanding fill.
//  * K-contiguous operands (rows of A' in the combine, both operands of the
//    symmetric products) sit as [rows][32 K] (64-byte rows, 16-byte chunks
//    XOR-swizzled by (row >> 2) & 3) and are read as ds_read_b128 fragments.
//  * The combine's X operand is contracted over X's row index: it sits
//    row-major as [32 rows j][256 columns k] (chunks swizzled by 4*(j&3)) and
//    its fragments come from ds_read_b64_tr_b16: 16 lanes each address 4
//    elements of a 4 x 16 block and every lane receives one column's 4
//    consecutive rows, exactly the MFMA operand layout.
// Outputs leave through LDS as whole rows.
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

constexpr int BK = 32;            // K per LDS stage
constexpr int KS = BK / 16;       // MFMA k-steps per stage
constexpr int NXCD = 8;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Wave index as a scalar: everything derived from it (LDS block bases, buffer
// soffsets) stays in SGPRs instead of being treated as divergent.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// 16-byte buffer load written straight into LDS: lane l's data lands at
// lds_wave_base + 16 * l.  The per-lane byte offset is a VGPR, everything that
// is uniform (row block, stage) goes into the SGPR soffset.
//
// The LDS destination goes through an empty asm, so the compiler cannot tie
// the fill to a stage buffer: otherwise its own wait insertion, which merges
// the pending fills imprecisely at control-flow joins, makes some stages wait
// for every fill in flight (vmcnt(0)) before reading LDS.  Every read of a
// stage is ordered after its fills by the explicit vmcnt + barrier hand-over.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, int voff, int soff, char* lds_wave_base) {
  unsigned a = static_cast<unsigned>(reinterpret_cast<unsigned long long>((lds_ptr_t)lds_wave_base));
  asm volatile("" : "+s"(a));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)static_cast<unsigned long long>(a), 16, voff, soff, 0, 0);
}

// ---- K-contiguous operand: [256 rows][32 K], 64-byte rows ------------------
__device__ __forceinline__ int rswz(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }

// Per-lane byte offset of the K-contiguous fill: 1 KB block b holds rows
// 16b + (lane >> 2); LDS chunk (lane & 3) of a row holds source chunk
// (lane & 3) ^ ((row >> 2) & 3), and (row >> 2) & 3 = (lane >> 4) & 3 for
// every b.
__device__ __forceinline__ int row_voff(int ld_bytes) {
  const int lane = threadIdx.x & 63;
  return (lane >> 2) * ld_bytes + (((lane & 3) ^ ((lane >> 4) & 3)) << 4);
}

// Two 1 KB blocks (16 rows each) per wave: 128 rows with four waves.  soff0:
// byte offset of (first row, first K of the stage).
__device__ __forceinline__ void load_rows(char* op, __amdgpu_buffer_rsrc_t rsrc, int voff, int ld_bytes, int soff0) {
  const int w = wave_id();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int blk = w * 2 + i;
    dma16(rsrc, voff, soff0 + blk * 16 * ld_bytes, op + blk * 1024);
  }
}

// Lane part of a K-contiguous fragment address for k-step ks: row (lane & 31)
// of a 32-row block, chunk 2 ks + (lane >> 5).  A block's first row is a
// multiple of 32, which leaves the swizzle unchanged, so the full address is
// tile + r0 * 64 + rfrag_off(ks) with r0 * 64 a constant offset.
__device__ __forceinline__ int rfrag_off(int ks, int lane) {
  const int r = lane & 31;
  return r * 64 + (((ks * 2 + (lane >> 5)) ^ ((r >> 2) & 3)) << 4);
}

__device__ __forceinline__ bf16x8_t frag_at(const char* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

// ---- X operand of the combine: [32 rows j][256 cols k], 512-byte rows -------
__device__ __forceinline__ int xswz(int j, int c) { return j * 512 + ((c ^ ((j & 3) << 2)) << 4); }

// Block b holds rows 2b, 2b+1 (lane >> 5); chunk (lane & 31) of LDS row j
// holds source chunk (lane & 31) ^ ((j & 3) << 2), which depends on b only
// through its parity.
struct XOffs {
  int even, odd;
  __device__ explicit XOffs(int ld_bytes) {
    const int lane = threadIdx.x & 63;
    const int base = (lane >> 5) * ld_bytes;
    even = base + (((lane & 31) ^ ((lane >> 5) << 2)) << 4);
    odd = base + (((lane & 31) ^ ((2 + (lane >> 5)) << 2)) << 4);
  }
};


// MFMA operand with rows = columns 32 i .. 32 i + 31 of the wave's X columns
// and the 16 contraction values j = 16 ks + 8 (lane / 32) + 0..7, from two
// transposing reads (4 rows each).  Lane part of the address of block i:
// the row-in-quad (lane >> 2) & 3 of the 16-lane group fixes the swizzle, so
// ks and the half h only add constants (16 ks rows, 4 h rows).
__device__ __forceinline__ int xfrag_off(int wcol0, int i, int lane) {
  const int g = lane >> 4, jj = lane & 15;
  const int kk = wcol0 + i * 32 + 16 * (g & 1) + 4 * (jj & 3);
  const int j = 8 * (g >> 1) + (jj >> 2);
  return xswz(j, kk >> 3) + ((kk >> 2) & 1) * 8;
}

__device__ __forceinline__ bf16x8_t frag_xcols(const char* p) {
  u32x2_t part[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(p + h * 4 * 512));
    part[h] = __builtin_bit_cast(u32x2_t, v);
  }
  // whole-register repacking: 4 + 4 contraction values -> one 8-value operand
  const u32x4_t w = {part[0][0], part[0][1], part[1][0], part[1][1]};
  return __builtin_bit_cast(bf16x8_t, w);
}

// The same transposing read for a K-major tile of RS-byte rows (the
// symmetric products' transposed operand blocks, rows = contraction index).
template <int RS>
__device__ __forceinline__ bf16x8_t frag_tr(const char* p) {
  u32x2_t part[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(p + h * 4 * RS));
    part[h] = __builtin_bit_cast(u32x2_t, v);
  }
  const u32x4_t w = {part[0][0], part[0][1], part[1][0], part[1][1]};
  return __builtin_bit_cast(bf16x8_t, w);
}

template <int FM, int FN>
struct Acc {
  f32x16_t c[FM][FN];
  __device__ void zero() {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) c[i][j][r] = 0.0f;
  }
};

// The MFMAs of one stage with one set of fragments (for accumulator tiles too
// large to leave registers for a second set).  SWAP: the B fragment is the
// MFMA's first operand, so acc.c[i][j] holds the transpose of block (i, j).
template <int FM, int FN, bool SWAP = false, class FragA, class FragB>
__device__ __forceinline__ void stage_mma_single(Acc<FM, FN>& acc, FragA fra, FragB frb) {
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bf16x8_t fa[FM], fb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = fra(ks, i);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = frb(ks, j);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc.c[i][j] = SWAP ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc.c[i][j], 0, 0, 0)
                           : __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc.c[i][j], 0, 0, 0);
  }
}

// The MFMAs of one stage; fragments of k-step ks+1 are read while ks runs.
// SWAP as in stage_mma_single.
template <int FM, int FN, bool SWAP = false, class FragA, class FragB>
__device__ __forceinline__ void stage_mma(Acc<FM, FN>& acc, FragA fra, FragB frb) {
  bf16x8_t fa[2][FM], fb[2][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) fa[0][i] = fra(0, i);
#pragma unroll
  for (int j = 0; j < FN; ++j) fb[0][j] = frb(0, j);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int c = ks & 1;
    if (ks + 1 < KS) {
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[c ^ 1][i] = fra(ks + 1, i);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[c ^ 1][j] = frb(ks + 1, j);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc.c[i][j] = SWAP ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[c][j], fa[c][i], acc.c[i][j], 0, 0, 0)
                           : __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][i], fb[c][j], acc.c[i][j], 0, 0, 0);
  }
}

// Stage hand-over: wait until this wave's fills of the stage about to be used
// have landed (`younger` fills of later stages may stay in flight; fills
// complete in issue order), finish this wave's LDS reads, then barrier so
// every wave's part is visible and the buffer being refilled next is free.
template <int YOUNGER>
__device__ __forceinline__ void stage_sync() {
  static_assert(YOUNGER >= 0 && YOUNGER < 16, "vmcnt immediate");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070 | YOUNGER);  // vmcnt(YOUNGER) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Loads per wave per stage are LPS (2 per operand); `ahead` = stages whose
// fills were issued after the one needed now (0, 1 or 2).
template <int LPS>
__device__ __forceinline__ void stage_sync_ahead(int ahead) {
  if (ahead >= 2) stage_sync<2 * LPS>();
  else if (ahead == 1) stage_sync<LPS>();
  else stage_sync<0>();
}

// The stage buffers are separate LDS arrays (so the compiler can tell a fill
// of one from reads of another); a buffer is chosen by a wave-uniform index.
template <int N>
struct BufsN {
  char* b[N];
  __device__ char* operator[](int p) const {
    if constexpr (N == 3) return p == 0 ? b[0] : p == 1 ? b[1] : b[2];
    else return p == 0 ? b[0] : p == 1 ? b[1] : p == 2 ? b[2] : b[3];
  }
};

// The pipelined contraction: stages 0..nk-1 through N buffers, N - 1 fills in
// flight.  fill(buf, kt) issues this wave's fills of stage kt, mma(buf, kt)
// multiplies it.
template <int LPS, int N, class Fill, class Mma>
__device__ __forceinline__ void pipeline(const BufsN<N>& bufs, int nk, Fill fill, Mma mma) {
  static_assert(N == 3 || N == 4, "stage count");
#pragma unroll
  for (int p = 0; p < N - 1; ++p)
    if (p < nk) fill(bufs[p], p);
  for (int kt0 = 0; kt0 < nk; kt0 += N) {
#pragma unroll
    for (int b = 0; b < N; ++b) {
      const int kt = kt0 + b;
      if (kt < nk) {
        const int issued_after = (nk - 1 - kt) < (N - 2) ? (nk - 1 - kt) : (N - 2);
        stage_sync_ahead<LPS>(issued_after);
        if (kt + N - 1 < nk) fill(bufs[(b + N - 1) % N], kt + N - 1);
        mma(bufs[b], kt);
      }
    }
  }
}

// The same pipeline over three consecutive stage ranges [0, k2), [k2, k1),
// [k1, nk), each multiplied by its own straight-line body (mma0, mma1, mma2
// in range order).  k2 and k1 must be multiples of N, so that stage kt sits in
// buffer kt % N with a static choice in every range.
template <int LPS, int N, class Fill, class MmaA, class MmaB, class MmaC>
__device__ __forceinline__ void pipeline3(const BufsN<N>& bufs, int nk, int k2, int k1, Fill fill, MmaA mma0,
                                          MmaB mma1, MmaC mma2) {
  static_assert(N == 3 || N == 4, "stage count");
#pragma unroll
  for (int p = 0; p < N - 1; ++p)
    if (p < nk) fill(bufs[p], p);
  auto range = [&](int kbeg, int kend, auto mma) {
    for (int kt0 = kbeg; kt0 < kend; kt0 += N) {
#pragma unroll
      for (int b = 0; b < N; ++b) {
        const int kt = kt0 + b;
        if (kt < kend) {
          const int issued_after = (nk - 1 - kt) < (N - 2) ? (nk - 1 - kt) : (N - 2);
          stage_sync_ahead<LPS>(issued_after);
          if (kt + N - 1 < nk) fill(bufs[(b + N - 1) % N], kt + N - 1);
          mma(bufs[b], kt);
        }
      }
    }
  };
  range(0, k2, mma0);
  range(k2, k1, mma1);
  range(k1, nk, mma2);
}

// A copy of v the compiler cannot see through: epilogue addresses derived from
// it are computed after the main loop instead of being hoisted above it (where
// they would occupy registers for the whole loop).
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// ---- output staging ------------------------------------------------------------
// The combine's bf16 output tile leaves through LDS as 32-row slabs (512-byte
// rows, 16-byte chunks XOR-swizzled by row & 31), so that global stores are
// whole rows: each wave instruction writes two contiguous 512-byte rows.
// (Stores of 8 bytes per lane scattered over 32 rows were not merged into
// full lines and cost more than the main loop.)
__device__ __forceinline__ int slab_off(int r, int col) {
  return r * 512 + ((((col >> 3) ^ (r & 31))) << 4) + (col & 7) * 2;
}

// Affine image of 8 staged bf16 values: b x, plus a for the element e == dcol
// (the one on the matrix diagonal; dcol < 0 or > 7: none).
__device__ __forceinline__ u32x4_t affine8(u32x4_t v, float a, float b, int dcol) {
  u32x4_t o;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float x0 = __uint_as_float(v[h] << 16), x1 = __uint_as_float(v[h] & 0xffff0000u);
    o[h] = pack_bf16x2(b * x0 + (dcol == 2 * h ? a : 0.0f), b * x1 + (dcol == 2 * h + 1 ? a : 0.0f));
  }
  return o;
}

// ---- segment table ----------------------------------------------------------
template <class Args>
__device__ __forceinline__ bool find_tile_at(const Args& G, int x, int local, int& seg, int& tile) {
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

// Segment runs [s, e] chained by zip_next share their matrix index range:
// each XCD takes a contiguous share of the matrices and walks them one by
// one, all segments' tiles of a matrix together (operands they share, such
// as a common factor, stay in that XCD's L2).
__device__ __forceinline__ bool find_tile_zip(const SymArgs& G, int x, int local, int& seg, int& tile) {
  for (int s = 0; s < G.nseg;) {
    int e = s;
    while (e + 1 < G.nseg && G.seg[e].zip_next) ++e;
    const int cnt = G.seg[s].count, tpm = G.seg[s].tiles_per_mat, per = (e - s + 1) * tpm;
    const int q = (cnt + NXCD - 1) / NXCD, z0 = x * q;
    const int nz = z0 >= cnt ? 0 : (z0 + q <= cnt ? q : cnt - z0);
    if (local < nz * per) {
      const int z = z0 + local / per, rem = local % per;
      seg = s + rem / tpm;
      tile = z * tpm + rem % tpm;
      return true;
    }
    local -= nz * per;
    s = e + 1;
  }
  return false;
}

template <class Args>
__device__ __forceinline__ bool find_tile(const Args& G, int& seg, int& tile) {
  return find_tile_at(G, blockIdx.x % NXCD, blockIdx.x / NXCD, seg, tile);
}

template <class Seg>
__device__ __forceinline__ float seg_inv(const Seg& S, int z, float* red) {
  if (S.partials == nullptr) return 1.0f;
  return inv_norm_from_partials(S.partials + static_cast<long long>(z) * S.P, S.P, S.eps, red, nullptr);
}

__device__ __forceinline__ float ipow(float x, int p) {
  float r = 1.0f;
  for (int i = 0; i < p; ++i) r *= x;
  return r;
}

// Upper-triangle tile t of an nt x nt tile grid -> (bi, bj), bi <= bj.
__device__ __forceinline__ void upper_tile(int t, int nt, int& bi, int& bj) {
  bi = 0;
  while (t >= nt - bi) { t -= nt - bi; ++bi; }
  bj = bi + t;
}

// ---- combine: Y = A' X, 128 x 256 tiles ----------------------------------------
// D[k][i] = sum_j X[j][k] A'[i][j] = (A' X)[i][k].  Four waves of 64 (k) x
// 128 (i), three LDS stages of 24 KB (X rows j x 256 k and A' rows i x 32 K):
// two workgroups share a CU.  The output leaves through 32-row slabs in two
// rounds (rows 0..95 through the three buffers, then rows 96..127).
// FUSE: the apply is fused into the epilogue (GemmSeg.fuse).
constexpr int C2_TI = 128, C2_TK = 256, C2_NTHR = 256;
constexpr int C2_OPX = BK * C2_TK * 2;      // 16 KB
constexpr int C2_OPA = C2_TI * BK * 2;      // 8 KB
constexpr int C2_STAGE = C2_OPX + C2_OPA;   // 24 KB

// Copy NS staged 32-row slabs (bufs[p] holds tile rows 32 (j0 + p) + r) out:
// to Y (row stride ldy) or, fused, into W and O of a wide matrix.
template <int NS, bool FUSE>
__device__ __forceinline__ void slabs32_out(const BufsN<3>& bufs, int j0, bf16_t* Y, long long ldy, float* W,
                                            bf16_t* O, long long n, int i0, int k0, int s, int l, float nls) {
  constexpr int PER = 32 * 32 / C2_NTHR;  // 16-byte chunks per thread per slab
  const int tid = opaque(threadIdx.x);
  if constexpr (!FUSE) {
#pragma unroll
    for (int p = 0; p < NS; ++p)
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int q = tid + C2_NTHR * u, r = q >> 5, c = q & 31;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(bufs[p] + r * 512 + ((c ^ (r & 31)) << 4));
        *reinterpret_cast<u32x4_t*>(Y + static_cast<long long>(i0 + (j0 + p) * 32 + r) * ldy + k0 + c * 8) = v;
      }
  } else {
    const bool full = i0 + (j0 + NS) * 32 <= s && k0 + C2_TK <= l && (W == nullptr || ((n % 4) == 0 &&
                      (reinterpret_cast<uintptr_t>(W) & 15u) == 0)) &&
                      (O == nullptr || ((n % 8) == 0 && (reinterpret_cast<uintptr_t>(O) & 15u) == 0));
    u32x4_t v[NS][PER];
    f32x4_t w[NS][PER][2];
#pragma unroll
    for (int p = 0; p < NS; ++p)
#pragma unroll
      for (int u = 0; u < PER; ++u) {  // every W load of this thread before its first store
        const int q = tid + C2_NTHR * u, r = q >> 5, c = q & 31;
        v[p][u] = *reinterpret_cast<const u32x4_t*>(bufs[p] + r * 512 + ((c ^ (r & 31)) << 4));
        if (full && W != nullptr) {  // W is read once and written once: non-temporal
          const long long off = static_cast<long long>(i0 + (j0 + p) * 32 + r) * n + k0 + c * 8;
          w[p][u][0] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(W + off));
          w[p][u][1] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(W + off + 4));
        }
      }
#pragma unroll
    for (int p = 0; p < NS; ++p)
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int q = tid + C2_NTHR * u, r = q >> 5, c = q & 31;
        const int i = i0 + (j0 + p) * 32 + r, k = k0 + c * 8;
        const long long off = static_cast<long long>(i) * n + k;
        const u32x4_t vv = v[p][u];
        if (full) {
          if (O != nullptr) __builtin_nontemporal_store(vv, reinterpret_cast<u32x4_t*>(O + off));
          if (W != nullptr) {
            f32x4_t w0 = w[p][u][0], w1 = w[p][u][1];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              w0[2 * h] = fmaf(nls, lo_bf16(vv[h]), w0[2 * h]);
              w0[2 * h + 1] = fmaf(nls, hi_bf16(vv[h]), w0[2 * h + 1]);
              w1[2 * h] = fmaf(nls, lo_bf16(vv[2 + h]), w1[2 * h]);
              w1[2 * h + 1] = fmaf(nls, hi_bf16(vv[2 + h]), w1[2 * h + 1]);
            }
            __builtin_nontemporal_store(w0, reinterpret_cast<f32x4_t*>(W + off));
            __builtin_nontemporal_store(w1, reinterpret_cast<f32x4_t*>(W + off + 4));
          }
        } else if (i < s) {  // edge tiles: element by element within the matrix
          for (int e = 0; e < 8 && k + e < l; ++e) {
            const uint32_t word = vv[e >> 1];
            const float o = (e & 1) ? hi_bf16(word) : lo_bf16(word);
            if (O != nullptr) O[off + e] = static_cast<bf16_t>((e & 1) ? (word >> 16) : (word & 0xffffu));
            if (W != nullptr) W[off + e] = fmaf(nls, o, W[off + e]);
          }
        }
      }
  }
}

template <bool FUSE>
__global__ void __launch_bounds__(C2_NTHR) __attribute__((amdgpu_waves_per_eu(2, 2)))
combine_bf16_kernel(GemmArgs G) {
  __shared__ __attribute__((aligned(1024))) char lds0[C2_STAGE];
  __shared__ __attribute__((aligned(1024))) char lds1[C2_STAGE];
  __shared__ __attribute__((aligned(1024))) char lds2[C2_STAGE];
  int si, tile;
  if (!find_tile(G, si, tile)) return;
  const GemmSeg& S = G.seg[si];
  // the integer divisions run on the vector unit: their results are moved
  // back to scalars, so that everything derived from them (matrix bases,
  // buffer descriptors) is provably uniform
  const int z = __builtin_amdgcn_readfirstlane(tile / S.tiles_per_mat);
  const int t = __builtin_amdgcn_readfirstlane(tile % S.tiles_per_mat);
  // row tiles innermost: the tiles that share an X column panel run together
  // (on one XCD) and read it once from HBM
  const int tiles_i = S.s_pad / C2_TI;
  const int ti = __builtin_amdgcn_readfirstlane(t % tiles_i), tk = __builtin_amdgcn_readfirstlane(t / tiles_i);
  const bf16_t* X = S.X + z * S.xstride;
  const bf16_t* Am = S.A + z * S.astride;

  // waves: 4 along k (columns of X), each 64 (k) x 128 (i): 2 x 4 MFMA blocks
  constexpr int CM = 64, FM = 2, FN = 4;
  const int lane = threadIdx.x & 63, wm = wave_id();
  Acc<FM, FN> acc;
  acc.zero();
  const int nk = S.s_pad / BK;
  const int ld_bytes = S.ld * 2, sp_bytes = S.s_pad * 2;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, static_cast<long long>(S.s_pad) * ld_bytes);
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(Am, static_cast<long long>(S.s_pad) * sp_bytes);
  const XOffs xo(ld_bytes);
  const int avoff = row_voff(sp_bytes);
  const int offA = ti * C2_TI * sp_bytes;
  int roff[KS], xoff[FM];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) roff[ks] = rfrag_off(ks, lane);
#pragma unroll
  for (int i = 0; i < FM; ++i) xoff[i] = xfrag_off(wm * CM, i, lane);
  const BufsN<3> bufs{{lds0, lds1, lds2}};

  pipeline<6>(
      bufs, nk,
      [&](char* buf, int kt) {
        // X: 16 blocks of two 512-byte rows, 4 per wave; A': 8 blocks of 16
        // 64-byte rows, 2 per wave
        const int soffx = kt * BK * ld_bytes + tk * C2_TK * 2;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int blk = wm * 4 + b;
          dma16(xr, (b & 1) ? xo.odd : xo.even, soffx + blk * 2 * ld_bytes, buf + blk * 1024);
        }
        load_rows(buf + C2_OPX, ar, avoff, sp_bytes, offA + kt * BK * 2);
      },
      [&](const char* buf, int) {
        const char* tb = buf + C2_OPX;
        stage_mma<FM, FN>(acc, [&](int ks, int i) { return frag_xcols(buf + xoff[i] + ks * 16 * 512); },
                          [&](int ks, int j) { return frag_at(tb + roff[ks] + j * 32 * 64); });
      });

  // lane: row i = j*32 + (lane & 31) of the tile, columns
  // k = wm*CM + i*32 + 8q + 4 (lane >> 5) + 0..3
  stage_sync<0>();
  const int lane_e = opaque(lane);
  const int col = lane_e & 31, rq = ((lane_e >> 5) & 1) * 4;
  float* Wz = nullptr;
  bf16_t* Oz = nullptr;
  if constexpr (FUSE) {
    Wz = static_cast<float*>(G.W.p[S.tab0 + z]);
    Oz = static_cast<bf16_t*>(G.O.p[S.tab0 + z]);
    if (S.tall) {
      // W (l x s) row k holds the iterate's column k: the 32 lanes of a half
      // wave own 32 consecutive i at each of their 4 k (two 128-byte row
      // segments per access); per 32-column block i, all 64 of its W loads
      // before any of its stores (memory-level parallelism: the epilogue is
      // bound by the latency of these loads, not by bandwidth)
      const float nls = S.neg_lr_scale;
      const bool full = (ti + 1) * C2_TI <= S.s && (tk + 1) * C2_TK <= S.l;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        float wv[FN][16];
        if (full && Wz != nullptr) {
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const float* wcol = Wz + ti * C2_TI + j * 32 + col;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                wv[j][4 * q + r] = __builtin_nontemporal_load(
                    &wcol[static_cast<long long>(tk * C2_TK + wm * CM + i * 32 + q * 8 + rq + r) * S.n]);
          }
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int gi = ti * C2_TI + j * 32 + col;
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int gk = tk * C2_TK + wm * CM + i * 32 + q * 8 + rq + r;
              const bf16_t ob = f32_to_bf16(acc.c[i][j][4 * q + r]);
              const long long off = static_cast<long long>(gk) * S.n + gi;
              if (full) {
                if (Oz != nullptr) __builtin_nontemporal_store(ob, &Oz[off]);
                if (Wz != nullptr) __builtin_nontemporal_store(fmaf(nls, bf16_to_f32(ob), wv[j][4 * q + r]), &Wz[off]);
              } else if (gi < S.s && gk < S.l) {
                if (Oz != nullptr) Oz[off] = ob;
                if (Wz != nullptr) Wz[off] = fmaf(nls, bf16_to_f32(ob), Wz[off]);
              }
            }
        }
      }
      return;
    }
  }
  // staged: 32-row slabs, rows 0..95 then 96..127
  bf16_t* Y = FUSE ? nullptr : S.Y + z * S.xstride;
  auto stage_block = [&](int j, char* buf) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = wm * CM + i * 32 + q * 8 + rq;
        const u32x2_t w = {pack_bf16x2(acc.c[i][j][4 * q + 0], acc.c[i][j][4 * q + 1]),
                           pack_bf16x2(acc.c[i][j][4 * q + 2], acc.c[i][j][4 * q + 3])};
        *reinterpret_cast<u32x2_t*>(buf + slab_off(col, k)) = w;
      }
  };
  stage_block(0, lds0);
  stage_block(1, lds1);
  stage_block(2, lds2);
  __syncthreads();
  slabs32_out<3, FUSE>(bufs, 0, Y, S.ld, Wz, Oz, S.n, ti * C2_TI, tk * C2_TK, S.s, S.l, S.neg_lr_scale);
  __syncthreads();
  stage_block(3, lds0);
  __syncthreads();
  slabs32_out<1, FUSE>(bufs, 3, Y, S.ld, Wz, Oz, S.n, ti * C2_TI, tk * C2_TK, S.s, S.l, S.neg_lr_scale);
}

// ---- symmetric products: O = alpha I + beta L R ----------------------------------
// L and R are symmetric and commute (polynomials in one Gram matrix), so
// tile (bi, bj) of L R is sum_k L[bi rows][k] R[bj rows][k]: both operands are
// read row-wise (K-contiguous), exactly like the Gram.  The s_pad x s_pad
// matrices are small (768 for the Mamba-2 projections), so the tile is
// TT x TT with TT = 192 when it divides s_pad (10 upper tiles per 768 x 768
// matrix: one wave of workgroups for 48 matrices, and half the operand bytes
// per flop of TT = 128), else 128.  Four waves of TT/2 x TT/2, three LDS
// stages; the stage buffers double as the output staging area.
template <int V> struct IntC { static constexpr int value = V; };
template <int TT> struct SymCfg;
template <> struct SymCfg<128> { static constexpr int kWpe = 3; };  // 48 KB LDS: three workgroups per CU
template <> struct SymCfg<192> { static constexpr int kWpe = 2; };  // 72 KB LDS: two workgroups per CU
constexpr int NTHR2 = 256;
constexpr int SYM_NSTAGE = 3;
constexpr int kSymSingleFragsAbove = 4;  // larger wave tiles read one fragment set per k-step

int sym_tile(int s_pad) { return s_pad % 192 == 0 ? 192 : 128; }

// Operands stored as their upper block triangle (SymSeg.tri_in): block
// (kb, b) with kb < b is read as the transpose of the stored block (kb, b) into
// a K-major tile [32 k rows][TT columns] (TT * 2-byte rows).  The 16-byte
// chunk in position p of row j holds source chunk p ^ sym_tswz(j), which keeps
// the four rows of a transposing read on distinct banks (row strides of 96 or
// 64 banks).
template <int TT>
__device__ __forceinline__ int sym_tswz(int j) {
  return TT == 192 ? (((j >> 1) & 1) << 2) : ((j & 3) << 2);
}

// Lane part of the DMA source offset of fill block blk of a K-major tile:
// LDS chunk position blk * 64 + lane = (row j, position p).
template <int TT>
__device__ __forceinline__ int sym_tvoff(int blk, int lane, int ld_bytes) {
  constexpr int CPR = TT / 8;
  const int idx = blk * 64 + lane, j = idx / CPR, p = idx % CPR;
  return j * ld_bytes + ((p ^ sym_tswz<TT>(j)) << 4);
}

// Lane part of the address of the transposed operand fragment whose rows are
// tile columns col0 .. col0 + 31 (k-step 0; a k-step adds 16 rows, which
// leaves the swizzle unchanged).
template <int TT>
__device__ __forceinline__ int sym_tfrag_off(int col0, int lane) {
  const int g = lane >> 4, jj = lane & 15;
  const int c = col0 + 16 * (g & 1) + 4 * (jj & 3);
  const int j = 8 * (g >> 1) + (jj >> 2);
  return j * (TT * 2) + (((c >> 3) ^ sym_tswz<TT>(j)) << 4) + ((c >> 2) & 1) * 8;
}

// Staging row r (0..63 within one buffer), column col (0..TT-1) of a TT-wide
// bf16 tile: TT * 2-byte rows, 16-byte chunks swizzled by the row (XOR of the
// low four bits for 16 chunks, of the low three within each group of eight for
// 24 chunks).
template <int TT>
__device__ __forceinline__ int sym_slab_off(int r, int col) {
  const int c = col >> 3;
  const int cs = TT == 128 ? (c ^ (r & 15)) : ((c & ~7) | ((c ^ r) & 7));
  return r * (TT * 2) + (cs << 4) + (col & 7) * 2;
}

// Copy a staged TT x TT tile (rows 64p + r in buffer p) to dst + off (row
// stride ld); dst2, when non-null, receives a2 I + b2 dst from the rounded
// values (the identity only on a diagonal tile, dg).  Either may be null.
template <int TT>
__device__ __forceinline__ void sym_to_global(const BufsN<SYM_NSTAGE>& bufs, bf16_t* dst, bf16_t* dst2, long long off,
                                              long long ld, float a2, float b2, bool dg) {
  constexpr int CPR = TT / 8;              // 16-byte chunks per row
  constexpr int PER = 64 * CPR / NTHR2;    // chunks per thread per buffer
  const int tid = opaque(threadIdx.x);     // addresses computed here, not held across the tile loop
#pragma unroll
  for (int p = 0; p < TT / 64; ++p) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = tid + NTHR2 * u;
      const int r = q / CPR, c = q % CPR;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(bufs[p] + sym_slab_off<TT>(r, c * 8));
      const long long o = off + static_cast<long long>(p * 64 + r) * ld + c * 8;
      if (dst != nullptr) *reinterpret_cast<u32x4_t*>(dst + o) = v;
      if (dst2 != nullptr) *reinterpret_cast<u32x4_t*>(dst2 + o) = affine8(v, a2, b2, dg ? p * 64 + r - c * 8 : -1);
    }
  }
}

// F32: the result leaves as float32 straight from the accumulators into F
// (the diagnostics' Gram matrix), exactly symmetric: on a diagonal tile only
// the entries on or above the diagonal are taken and mirrored.
template <int TT, bool F32>
__global__ void __launch_bounds__(NTHR2) __attribute__((amdgpu_waves_per_eu(SymCfg<TT>::kWpe, SymCfg<TT>::kWpe)))
symprod_bf16_kernel(SymArgs G) {
  constexpr int OPBT = TT * BK * 2;  // bytes of one operand per stage
  __shared__ __attribute__((aligned(1024))) char lds0[2 * OPBT];
  __shared__ __attribute__((aligned(1024))) char lds1[2 * OPBT];
  __shared__ __attribute__((aligned(1024))) char lds2[2 * OPBT];
  __shared__ float red[NTHR2 / 64];
  const BufsN<SYM_NSTAGE> bufs{{lds0, lds1, lds2}};
  constexpr int WT = TT / 2, FM = WT / 32, FN = WT / 32;  // waves: 2 x 2 of WT x WT
  constexpr int BPW = TT / 64;                             // 1 KB fill blocks per wave per operand
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int wm = wid >> 1, wn = wid & 1;
  int roff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) roff[ks] = rfrag_off(ks, lane);
  int tfa[FM], tfb[FN];  // transposed-fragment offsets (upper-triangle operands)
#pragma unroll
  for (int i = 0; i < FM; ++i) tfa[i] = sym_tfrag_off<TT>(wm * WT + i * 32, lane);
#pragma unroll
  for (int j = 0; j < FN; ++j) tfb[j] = sym_tfrag_off<TT>(wn * WT + j * 32, lane);

  // Persistent: the workgroups of XCD x walk that XCD's tile list with a
  // stride of their number, so the stores of one tile drain while the next
  // tile's first stages load.
  const int x = blockIdx.x % NXCD, per_xcd = gridDim.x / NXCD;
  for (int local = blockIdx.x / NXCD;; local += per_xcd) {
    int si, tile;
    if (!find_tile_zip(G, x, local, si, tile)) break;
    const SymSeg& S = G.seg[si];
    const int z = tile / S.tiles_per_mat;
    int bi, bj;
    upper_tile(tile % S.tiles_per_mat, S.s_pad / TT, bi, bj);
    const bool diag = bi == bj;
    const bool single = diag && S.L == S.R && (!F32 || S.lmap == S.rmap);  // both operands are the same rows
    // An off-diagonal tile of an upper-triangle output is computed transposed
    // (the B fragment as the MFMA's first operand): lanes then hold four
    // consecutive columns of the tile, which leave in 8-byte stores.  The
    // product of commuting symmetric factors is symmetric and each element is
    // the same products summed in the same k order.
    const bool swap = !F32 && !diag && S.tri_out;
    const long long zoff = z * S.stride;                 // outputs
    const long long zin = z * S.in_stride;               // operands
    const float inv = seg_inv(S, z, red);
    const float ia = ipow(inv, S.pa), ib = ipow(inv, S.pb);

    Acc<FM, FN> acc;
    acc.zero();
    const int sp_bytes = S.ld * 2;  // operand row stride
    const long long mbytes = static_cast<long long>(S.s_pad) * sp_bytes;
    const __amdgpu_buffer_rsrc_t lr = make_rsrc(S.L + zin, mbytes);
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(S.R + zin, mbytes);
    const int voff = row_voff(sp_bytes);
    const int offL = bi * TT * sp_bytes, offR = bj * TT * sp_bytes;
    const int nk = S.kdim / BK;
    auto fill_rows = [&](char* op, __amdgpu_buffer_rsrc_t rs, int soff0) {
#pragma unroll
      for (int b = 0; b < BPW; ++b) {
        const int blk = wid * BPW + b;
        dma16(rs, voff, soff0 + blk * 16 * sp_bytes, op + blk * 1024);
      }
    };
    // upper-triangle operands: stage kt reads block (kt / kb_stages) of the
    // row panels bi and bj; below the diagonal it is a transposed block
    // (bi <= bj, so a transposed L block implies a transposed R block)
    const int tri = S.tri_in;
    const int kbs = TT / BK;  // stages per k block
    auto fill_t = [&](char* op, __amdgpu_buffer_rsrc_t rs, int soff) {
#pragma unroll
      for (int b = 0; b < BPW; ++b) {
        const int blk = wid * BPW + b;
        dma16(rs, sym_tvoff<TT>(blk, lane, sp_bytes), soff, op + blk * 1024);
      }
    };
    // column offset (bytes) of stage kt in the rows of L (map = lmap) or R
    auto kcol = [&](int kt, unsigned map) {
      if constexpr (F32) {
        if (S.kseg > 0) {
          const int per = S.kseg / BK;
          int g = 0;
          while (kt >= (g + 1) * per) ++g;  // at most 7 segments
          return (static_cast<int>((map >> (4 * g)) & 0xfu) * S.kseg + (kt - g * per) * BK) * 2;
        }
      }
      return kt * BK * 2;
    };
    auto fill_op = [&](char* op, __amdgpu_buffer_rsrc_t rs, int b, int off, int kt, unsigned map = 0u) {
      if (tri && kt / kbs < b) fill_t(op, rs, kt * BK * sp_bytes + b * TT * 2);
      else fill_rows(op, rs, off + kcol(kt, map));
    };
    auto mma = [&](const char* buf, int kt, bool one, auto sw) {
      constexpr bool SW = decltype(sw)::value != 0;
      const int kb = kt / kbs;
      const bool lt = tri && kb < bi, rt = tri && kb < bj;  // uniform per stage
      const char* ab = buf;
      const char* bb = one ? buf : buf + OPBT;
      auto fa = [&](int ks, int i) {
        return lt ? frag_tr<TT * 2>(ab + tfa[i] + ks * 16 * TT * 2)
                  : frag_at(ab + wm * WT * 64 + roff[ks] + i * 32 * 64);
      };
      auto fb = [&](int ks, int j) {
        return rt ? frag_tr<TT * 2>(bb + tfb[j] + ks * 16 * TT * 2)
                  : frag_at(bb + wn * WT * 64 + roff[ks] + j * 32 * 64);
      };
      if constexpr (FM * FN > kSymSingleFragsAbove) stage_mma_single<FM, FN, SW>(acc, fa, fb);
      else stage_mma<FM, FN, SW>(acc, fa, fb);
    };
    if constexpr (TT == 192) {
      // the operand modes change only at k-block boundaries (multiples of 6
      // stages): stages below block bi read both operands transposed, those
      // below bj only R; each range runs a straight-line body
      const int k2 = tri ? bi * kbs : 0, k1 = tri ? bj * kbs : 0;
      auto body = [&](const char* buf, bool one, auto lt_rt, auto sw) {
        constexpr int MODE = decltype(lt_rt)::value;
        constexpr bool SW = decltype(sw)::value != 0;
        const char* ab = buf;
        const char* bb = one ? buf : buf + OPBT;
        auto fa_r = [&](int ks, int i) { return frag_at(ab + wm * WT * 64 + roff[ks] + i * 32 * 64); };
        auto fa_t = [&](int ks, int i) { return frag_tr<TT * 2>(ab + tfa[i] + ks * 16 * TT * 2); };
        auto fb_r = [&](int ks, int j) { return frag_at(bb + wn * WT * 64 + roff[ks] + j * 32 * 64); };
        auto fb_t = [&](int ks, int j) { return frag_tr<TT * 2>(bb + tfb[j] + ks * 16 * TT * 2); };
        if constexpr (MODE == 2) stage_mma_single<FM, FN, SW>(acc, fa_t, fb_t);
        else if constexpr (MODE == 1) stage_mma_single<FM, FN, SW>(acc, fa_r, fb_t);
        else stage_mma_single<FM, FN, SW>(acc, fa_r, fb_r);
      };
      auto fill2 = [&](char* buf, int kt) {
        fill_op(buf, lr, bi, offL, kt, S.lmap);
        fill_op(buf + OPBT, rr, bj, offR, kt, S.rmap);
      };
      if (single) {
        pipeline3<BPW>(bufs, nk, k2, k1, [&](char* buf, int kt) { fill_op(buf, lr, bi, offL, kt, S.lmap); },
                       [&](const char* buf, int) { body(buf, true, IntC<2>{}, IntC<0>{}); },
                       [&](const char* buf, int) { body(buf, true, IntC<1>{}, IntC<0>{}); },
                       [&](const char* buf, int) { body(buf, true, IntC<0>{}, IntC<0>{}); });
      } else if (swap) {
        pipeline3<2 * BPW>(bufs, nk, k2, k1, fill2,
                           [&](const char* buf, int) { body(buf, false, IntC<2>{}, IntC<1>{}); },
                           [&](const char* buf, int) { body(buf, false, IntC<1>{}, IntC<1>{}); },
                           [&](const char* buf, int) { body(buf, false, IntC<0>{}, IntC<1>{}); });
      } else {
        pipeline3<2 * BPW>(bufs, nk, k2, k1, fill2,
                           [&](const char* buf, int) { body(buf, false, IntC<2>{}, IntC<0>{}); },
                           [&](const char* buf, int) { body(buf, false, IntC<1>{}, IntC<0>{}); },
                           [&](const char* buf, int) { body(buf, false, IntC<0>{}, IntC<0>{}); });
      }
    } else if (single) {
      pipeline<BPW>(bufs, nk, [&](char* buf, int kt) { fill_op(buf, lr, bi, offL, kt, S.lmap); },
                    [&](const char* buf, int kt) { mma(buf, kt, true, IntC<0>{}); });
    } else {
      auto fill2 = [&](char* buf, int kt) {
        fill_op(buf, lr, bi, offL, kt, S.lmap);
        fill_op(buf + OPBT, rr, bj, offR, kt, S.rmap);
      };
      if (swap)
        pipeline<2 * BPW>(bufs, nk, fill2, [&](const char* buf, int kt) { mma(buf, kt, false, IntC<1>{}); });
      else
        pipeline<2 * BPW>(bufs, nk, fill2, [&](const char* buf, int kt) { mma(buf, kt, false, IntC<0>{}); });
    }

    // epilogue: D[m][n] = (L R)[bi*TT + m][bj*TT + n]; lane: 4 consecutive m
    // at one n.  The mirrored tile is staged (rows n, contiguous m) and
    // written out, then, off the diagonal, the tile itself; both leave as
    // whole rows.  O2 is the affine image of O1's rounded values.  Every
    // 32-row block lies in one 64-row buffer, so buffer choices are uniform.
    stage_sync<0>();
    const float a1 = S.a1 * ia, b1 = S.b1 * ib;
    const int lane_e = opaque(lane);
    const int col = lane_e & 31, rq = ((lane_e >> 5) & 1) * 4;
    if constexpr (F32) {
      // lane: D[m0 + r][n], r = 0..3; the tile row-wise (32 lanes cover 32
      // consecutive n), the mirror as one 16-byte store per lane
      float* F = S.F + zoff;
      const long long sp = S.s_pad;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = wn * WT + j * 32 + col;
        const long long gn = static_cast<long long>(bj) * TT + n;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int m0 = wm * WT + i * 32 + q * 8 + rq;
            const long long gm = static_cast<long long>(bi) * TT + m0;
            f32x4_t v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = b1 * acc.c[i][j][4 * q + r] + ((diag && m0 + r == n) ? a1 : 0.0f);
            if (!diag) {
#pragma unroll
              for (int r = 0; r < 4; ++r) F[(gm + r) * sp + gn] = v[r];
              *reinterpret_cast<f32x4_t*>(F + gn * sp + gm) = v;
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (m0 + r <= n) {
                  F[(gm + r) * sp + gn] = v[r];
                  F[gn * sp + gm + r] = v[r];
                }
            }
          }
        }
      }
      continue;  // the operands' LDS is free: every wave passed the barrier above
    }
    bf16_t* O1 = S.O1 == nullptr ? nullptr : S.O1 + zoff;
    bf16_t* O2 = S.O2 == nullptr ? nullptr : S.O2 + zoff;
    // the mirrored block (bj, bi) is skipped when the output keeps only its
    // upper block triangle (a diagonal block is always whole)
    const bool mirror = diag || !S.tri_out;
    if (mirror) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int nb = wn * WT + j * 32;  // 32-aligned block of n
      char* buf = bufs[nb >> 6];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = wm * WT + i * 32 + q * 8 + rq;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            v[r] = b1 * acc.c[i][j][4 * q + r] + ((diag && m + r == nb + col) ? a1 : 0.0f);
          *reinterpret_cast<u32x2_t*>(buf + sym_slab_off<TT>((nb & 63) + col, m)) =
              u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
      }
    }
    __syncthreads();
    sym_to_global<TT>(bufs, O1, O2, static_cast<long long>(bj) * TT * S.s_pad + bi * TT, S.s_pad, S.a2, S.b2, diag);
    }
    if (swap) {
      // acc.c[i][j] register 4 q + r: tile row m = wm WT + 32 i + col, column
      // n = wn WT + 32 j + 8 q + rq + r (the transposed block)
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int mb = wm * WT + i * 32;  // 32-aligned block of m
        char* buf = bufs[mb >> 6];
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n0 = wn * WT + j * 32 + q * 8 + rq;
            const f32x16_t& c = acc.c[i][j];
            *reinterpret_cast<u32x2_t*>(buf + sym_slab_off<TT>((mb & 63) + col, n0)) =
                u32x2_t{pack_bf16x2(b1 * c[4 * q], b1 * c[4 * q + 1]), pack_bf16x2(b1 * c[4 * q + 2], b1 * c[4 * q + 3])};
          }
      }
      __syncthreads();
      sym_to_global<TT>(bufs, O1, O2, static_cast<long long>(bi) * TT * S.s_pad + bj * TT, S.s_pad, S.a2, S.b2, false);
    } else if (!diag) {
      if (mirror) __syncthreads();
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int mb = wm * WT + i * 32;  // 32-aligned block of m
        char* buf = bufs[mb >> 6];
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              *reinterpret_cast<bf16_t*>(buf + sym_slab_off<TT>((mb & 63) + q * 8 + rq + r, wn * WT + j * 32 + col)) =
                  f32_to_bf16(b1 * acc.c[i][j][4 * q + r]);
      }
      __syncthreads();
      sym_to_global<TT>(bufs, O1, O2, static_cast<long long>(bi) * TT * S.s_pad + bj * TT, S.s_pad, S.a2, S.b2, false);
    }
    __syncthreads();  // staging read out before the next tile's fills land
  }
}

// Tiles per XCD of a segment table walked by find_tile_zip, times the XCDs.
int grid_for_zip(const SymArgs& G) {
  int per_xcd = 0;
  for (int s = 0; s < G.nseg;) {
    int e = s;
    while (e + 1 < G.nseg && G.seg[e].zip_next) ++e;
    per_xcd += (G.seg[s].count + NXCD - 1) / NXCD * (e - s + 1) * G.seg[s].tiles_per_mat;
    s = e + 1;
  }
  return per_xcd * NXCD;
}

template <int TT, bool F32>
hipError_t launch_symprod_tt(const SymArgs& G, hipStream_t st) {
  // persistent: kWpe resident workgroups per CU (LDS bound), a multiple of
  // the XCD count
  const int cus = device_cus();
  const int slots = (SymCfg<TT>::kWpe * cus) / NXCD * NXCD;
  const int need = grid_for_zip(G);
  const int grid = need < slots ? need : slots;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((symprod_bf16_kernel<TT, F32>), dim3(grid), dim3(NTHR2), 0, st, G);
  return hipGetLastError();
}

template <class Args>
int grid_for(const Args& G) {
  int per_xcd = 0;
  for (int s = 0; s < G.nseg; ++s) {
    const int tot = G.seg[s].count * G.seg[s].tiles_per_mat;
    per_xcd += (tot + NXCD - 1) / NXCD;
  }
  return per_xcd * NXCD;
}

}  // namespace

int combine_tiles_per_matrix(int s_pad, int ld) { return (s_pad / C2_TI) * (ld / C2_TK); }
int symprod_tile(int s_pad) { return sym_tile(s_pad); }
int symprod_tiles_per_matrix(int s_pad, int tile) {
  const int nt = s_pad / (tile ? tile : sym_tile(s_pad));
  return nt * (nt + 1) / 2;
}

// One launch per tile size and output type present (zip chains never mix
// them: they share s_pad and outputs).
hipError_t launch_symprod_bf16(const SymArgs& G, hipStream_t st) {
  SymArgs part[4] = {};
  for (int s = 0; s < G.nseg; ++s) {
    const int tt = G.seg[s].tile ? G.seg[s].tile : sym_tile(G.seg[s].s_pad);
    SymArgs& P = part[(tt == 192 ? 1 : 0) + (G.seg[s].F != nullptr ? 2 : 0)];
    P.seg[P.nseg++] = G.seg[s];
  }
  hipError_t e = part[1].nseg ? launch_symprod_tt<192, false>(part[1], st) : hipSuccess;
  if (e == hipSuccess && part[0].nseg) e = launch_symprod_tt<128, false>(part[0], st);
  if (e == hipSuccess && part[3].nseg) e = launch_symprod_tt<192, true>(part[3], st);
  if (e == hipSuccess && part[2].nseg) e = launch_symprod_tt<128, true>(part[2], st);
  return e;
}

// Segments with and without the fused apply go to separate launches.
hipError_t launch_combine_bf16(const GemmArgs& G, hipStream_t st) {
  GemmArgs part[2] = {};
  for (int s = 0; s < G.nseg; ++s) {
    GemmArgs& P = part[G.seg[s].fuse ? 1 : 0];
    P.seg[P.nseg++] = G.seg[s];
  }
  part[1].W = G.W;
  part[1].O = G.O;
  for (int f = 0; f < 2; ++f) {
    const int grid = grid_for(part[f]);
    if (grid == 0) continue;
    if (f) hipLaunchKernelGGL(combine_bf16_kernel<true>, dim3(grid), dim3(C2_NTHR), 0, st, part[f]);
    else hipLaunchKernelGGL(combine_bf16_kernel<false>, dim3(grid), dim3(C2_NTHR), 0, st, part[f]);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace muon
