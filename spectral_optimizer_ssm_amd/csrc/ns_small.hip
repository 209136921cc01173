// Whole Newton-Schulz iteration on chip for small matrices.
//
// "MuonSSM" (method section on light Newton-Schulz orthogonalisation) runs a
// single Newton-Schulz step, with no explicit SVD, on the low-rank injection of
// every token and head; its ablation on the number of Newton-Schulz steps
// compares one step with five.  Each matrix (s x l, s <= 128) is loaded once,
// normalised by its Frobenius norm, iterated in LDS and registers, and stored
// once, so the pass streams HBM exactly once each way (non-temporal loads and
// stores: the matrices are touched once).
//
// bf16 kernel (s = 32 with l <= 256, s = 64 with l <= 128): one wavefront per
// matrix, several matrices per workgroup.
//  * X lives in LDS (row-major, 16-byte chunks XOR-swizzled per row).
//  * Gram A = X X^T on v_mfma_f32_32x32x16_bf16 from ds_read_b128 fragments.
//  * A never touches memory: by symmetry the Gram accumulators already hold,
//    lane by lane, the operand fragments of A that the combine needs, after a
//    permutation of the contraction index (a sum is invariant under one).
//  * Combine D[k][i] = sum_j X[j][k] A[i][j] with the X operand read from
//    LDS in the same contraction order by transposing reads
//    (ds_read_b64_tr_b16); each lane then holds 4 consecutive columns of one
//    row of Y = a X + b A X.
//  * Y overwrites X in LDS one 32-column block at a time (same wave, in
//    order) and leaves through coalesced 16-byte stores.
// Larger bf16 shapes (s up to 128, l up to 512): one matrix per workgroup of
// s / 32 waves, rows of the result split over the waves
// (ns_small_bf16_wgr_kernel) or, for the largest, columns
// (ns_small_bf16_wg_kernel).
// fp32 kernel: one workgroup per matrix, products on the fp32 matrix cores.
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

// ds_read_b64_tr_b16: in each 16-lane group the lanes address a 4 x 16 block
// of 16-bit values (lane 4 r + u: row r, elements 4 u .. 4 u + 3) and lane p
// receives column p's 4 values, rows 0..3 in order.
__device__ __forceinline__ u32x2_t tr_read(const char* p) {
  return __builtin_bit_cast(
      u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p));
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


template <int S, int L>
// Two waves per SIMD: the shapes taken here (up to 32 x 256 and 64 x 128)
// hold few enough accumulators and fragments.
__global__ void __launch_bounds__(WPB * 64) __attribute__((amdgpu_waves_per_eu(2)))
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

  // The first NPRE chunks per lane of a wave's next matrix are loaded into
  // registers while the current one is combined (the Gram accumulators are
  // dead by then), so part of every load latency overlaps the wave's own work.
  constexpr int NPRE = Geo::CHUNKS / 128;
  u32x4_t pre[NPRE];
  bool have_pre = false;
  for (long long mat = static_cast<long long>(blockIdx.x) * WPB + wid; mat < P.count; mat += nwaves) {
    const bf16_t* src = static_cast<const bf16_t*>(P.X) + mat * P.in_stride;
    bf16_t* dst = static_cast<bf16_t*>(P.Y) + mat * P.out_stride;

    // ---- load X, sum of squares -------------------------------------------
    float ss = 0.0f;
#pragma unroll
    for (int p = 0; p < Geo::CHUNKS / 64; ++p) {
      const int q = lane + 64 * p;
      const int r = q / Geo::CPR, c = q % Geo::CPR;
      const u32x4_t v = (p < NPRE && have_pre) ? pre[p < NPRE ? p : 0] : __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + static_cast<long long>(r) * P.ld_in + c * 8));
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
      if (step == P.steps - 1) {
        const long long nxt = mat + nwaves;
        have_pre = nxt < P.count;
        if (have_pre) {
          const bf16_t* nsrc = static_cast<const bf16_t*>(P.X) + nxt * P.in_stride;
#pragma unroll
          for (int p = 0; p < NPRE; ++p) {
            const int q = lane + 64 * p;
            const int r = q / Geo::CPR, c = q % Geo::CPR;
            pre[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(nsrc + static_cast<long long>(r) * P.ld_in + c * 8));
          }
        }
      }
#pragma unroll 1
      for (int kb = 0; kb < NK; ++kb) {
        u32x2_t ypk[NB][4];
        f32x16_t c[NB];
#pragma unroll
        for (int ib = 0; ib < NB; ++ib)
#pragma unroll
          for (int r = 0; r < 16; ++r) c[ib][r] = 0.0f;
        // X operand xf[t] = X[16 js + 8 (t / 4) + 4 G + t % 4][32 kb + l32] from
        // two transposing reads: lane 16 g4 + 4 rr + u addresses row
        // 16 js + 8 h + 4 (g4 / 2) + rr, columns 32 kb + 16 (g4 & 1) + 4 u .. + 3
        const int g4 = lane >> 4, rr = (lane >> 2) & 3, u = lane & 3;
        const int tcol = kb * 32 + 16 * (g4 & 1) + 4 * u;
#pragma unroll
        for (int js = 0; js < NJ; ++js) {
          u32x2_t part[2];
#pragma unroll
          for (int h = 0; h < 2; ++h)
            part[h] = tr_read(lds + Geo::elem_off(16 * js + 8 * h + 4 * (g4 >> 1) + rr, tcol));
          const bf16x8_t xf = __builtin_bit_cast(bf16x8_t, u32x4_t{part[0][0], part[0][1], part[1][0], part[1][1]});
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
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(dst + static_cast<long long>(r) * P.ld_out + c * 8));
    }
    wave_lds_sync();  // the next matrix overwrites this region
  }
}

// ---- bf16, one matrix per workgroup: short sides to 128, long sides to 512 ----
// The same arithmetic as ns_small_bf16_kernel, shared by S / 32 waves (one per
// 32-row block) so that a large matrix is not left to one wave's latency:
//  * X (s x l, l a runtime multiple of 32) sits in LDS, 16-byte chunks
//    XOR-swizzled per row; A = X X^T (s x s bf16) after it.
//  * Gram: wave w accumulates column block w of A over the whole long side and
//    writes it, by symmetry, as rows 32 w .. 32 w + 31 of A (8-byte row
//    segments, chunks swizzled per row).
//  * Combine: wave w takes the 32-column blocks kb = w, w + S/32, ... of
//    Y = a X + b A X.  Its A operand fragments come from A's rows (two 8-byte
//    reads each), its X operand, contracted over X's row index, from two
//    ds_read_b64_tr_b16 per 16 rows: in each 16-lane group the lanes address
//    a 4 x 16 block and every lane receives one column's 4 consecutive rows.
//    Only wave w reads and writes its column blocks, so Y overwrites X in
//    place; two workgroup barriers per step separate the Gram, the combine
//    and the next Gram.
// Zero rows and columns (muon_step's padding of both sides to multiples of
// 32) stay zero through every product.
struct RtGeo {
  int row, cpr, swm1;
  __device__ explicit RtGeo(int l) : row(2 * l), cpr(l / 8) {
    // long sides >= 96 here: one row covers a 256-byte bank sweep, and the
    // XOR key r mod swm (swm = 4, 8 or 16 chunks, dividing 16) is shared by
    // rows 16 apart
    swm1 = ((cpr % 16 == 0) ? 16 : (cpr % 8 == 0) ? 8 : 4) - 1;
  }
  __device__ int chunk_off(int r, int c) const { return r * row + ((c ^ (r & swm1)) << 4); }
};

template <int S>
struct WgGeoA {  // A: S rows of S bf16, 16-byte chunks XOR-swizzled per row
  static constexpr int ROW = 2 * S, CPR = S / 8;
  static constexpr int SW1 = ((CPR % 16 == 0) ? 16 : (CPR % 8 == 0) ? 8 : 4) - 1;
  __device__ static int off(int r, int c) { return r * ROW + ((c ^ (r & SW1)) << 4); }
};

template <int S>
__global__ void __launch_bounds__(256) ns_small_bf16_wg_kernel(NsSmallLaunch P) {
  extern __shared__ __attribute__((aligned(16))) char lds_dyn[];
  constexpr int NB = S / 32, NJ = S / 16, NT = NB * 64;
  using GA = WgGeoA<S>;
  const int L = P.l;
  const RtGeo geo(L);
  const int nk = L / 32, chunks = S * geo.cpr;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  char* xs = lds_dyn;
  char* as = lds_dyn + static_cast<size_t>(S) * L * 2;
  float* red = reinterpret_cast<float*>(as);  // the norm's reduction, before A exists
  const int G = lane >> 5, l32 = lane & 31;
  // Gram operand rows l32 + 32 b and the update's rows share one key
  const int key32 = l32 & geo.swm1, base32 = l32 * geo.row;
  // transposing reads: lane 16 g4 + 4 rr + u addresses row 8 h + 4 (g4 / 2)
  // + rr (+ 16 js), columns 16 (g4 & 1) + 4 u .. + 3 of the block
  const int g4 = lane >> 4, rr = (lane >> 2) & 3, u = lane & 3;
  int trow[2], tkey[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 8 * h + 4 * (g4 >> 1) + rr;
    trow[h] = r * geo.row + 8 * (u & 1);
    tkey[h] = r & geo.swm1;
  }
  const int tchunk = 2 * (g4 & 1) + (u >> 1);

  for (long long mat = blockIdx.x; mat < P.count; mat += gridDim.x) {
    const bf16_t* src = static_cast<const bf16_t*>(P.X) + mat * P.in_stride;
    bf16_t* dst = static_cast<bf16_t*>(P.Y) + mat * P.out_stride;
    // stage X: eight 16-byte loads in flight per thread
    float ss = 0.0f;
    for (int q0 = threadIdx.x; q0 < chunks; q0 += 8 * NT) {
      u32x4_t v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int q = q0 + e * NT;
        if (q < chunks) {
          const int r = q / geo.cpr, c = q - r * geo.cpr;
          v[e] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + static_cast<long long>(r) * P.ld_in + c * 8));
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int q = q0 + e * NT;
        if (q < chunks) {
          const int r = q / geo.cpr, c = q - r * geo.cpr;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float x0 = lo_bf16(v[e][t]), x1 = hi_bf16(v[e][t]);
            ss = fmaf(x0, x0, ss);
            ss = fmaf(x1, x1, ss);
          }
          *reinterpret_cast<u32x4_t*>(xs + geo.chunk_off(r, c)) = v[e];
        }
      }
    }
    float tot;
    if (P.partials != nullptr) {
      float s2 = 0.0f;
      for (int i = threadIdx.x; i < P.P; i += NT) s2 += P.partials[mat * P.P + i];
      tot = block_sum(s2, red);
    } else {
      tot = block_sum(ss, red);
    }
    const float inv = 1.0f / (sqrtf(tot) + P.eps);
    __syncthreads();  // red is read by every thread before A overwrites it

    for (int step = 0; step < P.steps; ++step) {
      const float sc = step == 0 ? inv : 1.0f;
      // Gram column block w
      f32x16_t g[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) g[b][r] = 0.0f;
#pragma unroll 2
      for (int ks = 0; ks < L / 16; ++ks) {
        const int co = ((ks * 2 + G) ^ key32) << 4;
        bf16x8_t f[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) f[b] = *reinterpret_cast<const bf16x8_t*>(xs + base32 + b * 32 * geo.row + co);
        bf16x8_t fw = f[0];
#pragma unroll
        for (int b = 1; b < NB; ++b)
          if (b == w) fw = f[b];
#pragma unroll
        for (int b = 0; b < NB; ++b) g[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[b], fw, g[b], 0, 0, 0);
      }
      // g[b] lane (G, l32), register 4 q + e = A[32 b + 8 q + 4 G + e][32 w + l32]
      // = A[32 w + l32][32 b + 8 q + 4 G + e]: one 8-byte row segment per q
      const float gs = sc * sc;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x2_t v = {pack_bf16x2(g[b][4 * q] * gs, g[b][4 * q + 1] * gs),
                             pack_bf16x2(g[b][4 * q + 2] * gs, g[b][4 * q + 3] * gs)};
          *reinterpret_cast<u32x2_t*>(as + GA::off(32 * w + l32, 4 * b + q) + 8 * G) = v;
        }
      __syncthreads();  // A complete; every Gram read of X done

      // the combine's A operand: af[ib][js] = A[32 ib + l32][16 js + 8 h + 4 G + 0..3], h = 0, 1
      u32x4_t af[NB][NJ];
#pragma unroll
      for (int ib = 0; ib < NB; ++ib)
#pragma unroll
        for (int js = 0; js < NJ; ++js) {
          const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(as + GA::off(32 * ib + l32, 2 * js) + 8 * G);
          const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(as + GA::off(32 * ib + l32, 2 * js + 1) + 8 * G);
          af[ib][js] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        }
      const float alpha = P.a[step] * sc, beta = P.b[step] * sc;
#pragma unroll 1
      for (int kb = w; kb < nk; kb += NB) {
        f32x16_t c[NB];
#pragma unroll
        for (int ib = 0; ib < NB; ++ib)
#pragma unroll
          for (int r = 0; r < 16; ++r) c[ib][r] = 0.0f;
        int xo[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) xo[h] = trow[h] + (((kb * 4 + tchunk) ^ tkey[h]) << 4);
#pragma unroll
        for (int js = 0; js < NJ; ++js) {
          const u32x2_t p0 = tr_read(xs + xo[0] + js * 16 * geo.row);
          const u32x2_t p1 = tr_read(xs + xo[1] + js * 16 * geo.row);
          const bf16x8_t xf = __builtin_bit_cast(bf16x8_t, u32x4_t{p0[0], p0[1], p1[0], p1[1]});
#pragma unroll
          for (int ib = 0; ib < NB; ++ib)
            c[ib] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf, __builtin_bit_cast(bf16x8_t, af[ib][js]), c[ib], 0,
                                                            0, 0);
        }
        // c[ib] lane (G, l32), register 4 q + e = (A X)[32 ib + l32][32 kb + 8 q + 4 G + e]
        int yo[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) yo[q] = base32 + (((kb * 4 + q) ^ key32) << 4) + 8 * G;
        u32x2_t ypk[NB][4];
#pragma unroll
        for (int ib = 0; ib < NB; ++ib)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x2_t xv = *reinterpret_cast<const u32x2_t*>(xs + yo[q] + ib * 32 * geo.row);
            const float y0 = fmaf(alpha, lo_bf16(xv[0]), beta * c[ib][4 * q + 0]);
            const float y1 = fmaf(alpha, hi_bf16(xv[0]), beta * c[ib][4 * q + 1]);
            const float y2 = fmaf(alpha, lo_bf16(xv[1]), beta * c[ib][4 * q + 2]);
            const float y3 = fmaf(alpha, hi_bf16(xv[1]), beta * c[ib][4 * q + 3]);
            ypk[ib][q] = u32x2_t{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
          }
        wave_lds_sync();  // this wave's reads of block kb before its writes
#pragma unroll
        for (int ib = 0; ib < NB; ++ib)
#pragma unroll
          for (int q = 0; q < 4; ++q) *reinterpret_cast<u32x2_t*>(xs + yo[q] + ib * 32 * geo.row) = ypk[ib][q];
      }
      __syncthreads();  // Y complete before the next Gram or the store
    }

    for (int q0 = threadIdx.x; q0 < chunks; q0 += 4 * NT) {
      u32x4_t v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int q = q0 + e * NT;
        if (q < chunks) {
          const int r = q / geo.cpr, c = q - r * geo.cpr;
          v[e] = *reinterpret_cast<const u32x4_t*>(xs + geo.chunk_off(r, c));
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int q = q0 + e * NT;
        if (q < chunks) {
          const int r = q / geo.cpr, c = q - r * geo.cpr;
          u32x4_t o = v[e];
          if (P.steps == 0) {
#pragma unroll
            for (int t = 0; t < 4; ++t) o[t] = pack_bf16x2(lo_bf16(o[t]) * inv, hi_bf16(o[t]) * inv);
          }
          __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(dst + static_cast<long long>(r) * P.ld_out + c * 8));
        }
      }
    }
    __syncthreads();  // the next matrix overwrites X and the reduction slots
  }
}

// ---- bf16, one matrix per workgroup, rows split over the waves ----
// The variant of ns_small_bf16_wg_kernel that keeps only X in LDS, so that two
// workgroups share a CU where X alone fits twice (128 x 256: 64 KB).  Wave w
// accumulates column block w of the Gram, A[32 b + ..][32 w + ..], which by
// symmetry holds, lane by lane, the combine's operand fragments for output
// rows 32 w .. 32 w + 31 (as in ns_small_bf16_kernel, with one row block per
// wave instead of all of them); the wave then forms those rows of Y for every
// 32-column block, reading X's operand for the block with transposing reads.
// A workgroup barrier per column block separates every wave's reads of the
// block from the writes of Y into it.
template <int S>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
ns_small_bf16_wgr_kernel(NsSmallLaunch P) {
  extern __shared__ __attribute__((aligned(16))) char lds_dyn[];
  __shared__ float red[8];
  constexpr int NB = S / 32, NJ = S / 16, NT = NB * 64;
  const int L = P.l;
  const RtGeo geo(L);
  const int nk = L / 32, chunks = S * geo.cpr;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  char* xs = lds_dyn;
  const int G = lane >> 5, l32 = lane & 31;
  const int key32 = l32 & geo.swm1, base32 = l32 * geo.row;
  const int g4 = lane >> 4, rr = (lane >> 2) & 3, u = lane & 3;
  int trow[2], tkey[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 8 * h + 4 * (g4 >> 1) + rr;
    trow[h] = r * geo.row + 8 * (u & 1);
    tkey[h] = r & geo.swm1;
  }
  const int tchunk = 2 * (g4 & 1) + (u >> 1);
  const int ybase = base32 + w * 32 * geo.row;  // this wave's output rows

  for (long long mat = blockIdx.x; mat < P.count; mat += gridDim.x) {
    const bf16_t* src = static_cast<const bf16_t*>(P.X) + mat * P.in_stride;
    bf16_t* dst = static_cast<bf16_t*>(P.Y) + mat * P.out_stride;
    float ss = 0.0f;
    for (int q0 = threadIdx.x; q0 < chunks; q0 += 8 * NT) {
      u32x4_t v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int q = q0 + e * NT;
        if (q < chunks) {
          const int r = q / geo.cpr, c = q - r * geo.cpr;
          v[e] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4_t*>(src + static_cast<long long>(r) * P.ld_in + c * 8));
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int q = q0 + e * NT;
        if (q < chunks) {
          const int r = q / geo.cpr, c = q - r * geo.cpr;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float x0 = lo_bf16(v[e][t]), x1 = hi_bf16(v[e][t]);
            ss = fmaf(x0, x0, ss);
            ss = fmaf(x1, x1, ss);
          }
          *reinterpret_cast<u32x4_t*>(xs + geo.chunk_off(r, c)) = v[e];
        }
      }
    }
    float tot;
    if (P.partials != nullptr) {
      float s2 = 0.0f;
      for (int i = threadIdx.x; i < P.P; i += NT) s2 += P.partials[mat * P.P + i];
      tot = block_sum(s2, red);
    } else {
      tot = block_sum(ss, red);
    }
    const float inv = 1.0f / (sqrtf(tot) + P.eps);

    for (int step = 0; step < P.steps; ++step) {
      const float sc = step == 0 ? inv : 1.0f;
      f32x16_t g[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) g[b][r] = 0.0f;
#pragma unroll 2
      for (int ks = 0; ks < L / 16; ++ks) {
        const int co = ((ks * 2 + G) ^ key32) << 4;
        bf16x8_t f[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) f[b] = *reinterpret_cast<const bf16x8_t*>(xs + base32 + b * 32 * geo.row + co);
        bf16x8_t fw = f[0];
#pragma unroll
        for (int b = 1; b < NB; ++b)
          if (b == w) fw = f[b];
#pragma unroll
        for (int b = 0; b < NB; ++b) g[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[b], fw, g[b], 0, 0, 0);
      }
      // g[bm] lane (G, l32), register 4 q + e = A[32 bm + 8 q + 4 G + e][32 w + l32]:
      // the B operand of the combine for output row 32 w + l32 and contraction
      // j = 16 js + 8 h + 4 G + e (js = 2 bm + kap, q = 2 kap + h)
      const float gs = sc * sc;
      u32x4_t af[NJ];
#pragma unroll
      for (int js = 0; js < NJ; ++js) {
        const int bm = js >> 1, kap = js & 1;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int gp = 2 * kap + h;
          af[js][2 * h] = pack_bf16x2(g[bm][4 * gp + 0] * gs, g[bm][4 * gp + 1] * gs);
          af[js][2 * h + 1] = pack_bf16x2(g[bm][4 * gp + 2] * gs, g[bm][4 * gp + 3] * gs);
        }
      }
      const float alpha = P.a[step] * sc, beta = P.b[step] * sc;
#pragma unroll 1
      for (int kb = 0; kb < nk; ++kb) {
        f32x16_t c;
#pragma unroll
        for (int r = 0; r < 16; ++r) c[r] = 0.0f;
        int xo[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) xo[h] = trow[h] + (((kb * 4 + tchunk) ^ tkey[h]) << 4);
#pragma unroll
        for (int js = 0; js < NJ; ++js) {
          const u32x2_t p0 = tr_read(xs + xo[0] + js * 16 * geo.row);
          const u32x2_t p1 = tr_read(xs + xo[1] + js * 16 * geo.row);
          const bf16x8_t xf = __builtin_bit_cast(bf16x8_t, u32x4_t{p0[0], p0[1], p1[0], p1[1]});
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf, __builtin_bit_cast(bf16x8_t, af[js]), c, 0, 0, 0);
        }
        // c lane (G, l32), register 4 q + e = (A X)[32 w + l32][32 kb + 8 q + 4 G + e]
        int yo[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) yo[q] = ybase + (((kb * 4 + q) ^ key32) << 4) + 8 * G;
        u32x2_t ypk[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x2_t xv = *reinterpret_cast<const u32x2_t*>(xs + yo[q]);
          const float y0 = fmaf(alpha, lo_bf16(xv[0]), beta * c[4 * q + 0]);
          const float y1 = fmaf(alpha, hi_bf16(xv[0]), beta * c[4 * q + 1]);
          const float y2 = fmaf(alpha, lo_bf16(xv[1]), beta * c[4 * q + 2]);
          const float y3 = fmaf(alpha, hi_bf16(xv[1]), beta * c[4 * q + 3]);
          ypk[q] = u32x2_t{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
        }
        __syncthreads();  // every wave has read column block kb
#pragma unroll
        for (int q = 0; q < 4; ++q) *reinterpret_cast<u32x2_t*>(xs + yo[q]) = ypk[q];
      }
      __syncthreads();  // Y complete before the next Gram or the store
    }

    for (int q0 = threadIdx.x; q0 < chunks; q0 += 4 * NT) {
      u32x4_t v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int q = q0 + e * NT;
        if (q < chunks) {
          const int r = q / geo.cpr, c = q - r * geo.cpr;
          v[e] = *reinterpret_cast<const u32x4_t*>(xs + geo.chunk_off(r, c));
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int q = q0 + e * NT;
        if (q < chunks) {
          const int r = q / geo.cpr, c = q - r * geo.cpr;
          u32x4_t o = v[e];
          if (P.steps == 0) {
#pragma unroll
            for (int t = 0; t < 4; ++t) o[t] = pack_bf16x2(lo_bf16(o[t]) * inv, hi_bf16(o[t]) * inv);
          }
          __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(dst + static_cast<long long>(r) * P.ld_out + c * 8));
        }
      }
    }
    __syncthreads();  // the next matrix overwrites X
  }
}

constexpr int kRtMaxL = 512;
constexpr int kMaxLds = 160 * 1024;

// ---- float32: one workgroup per matrix --------------------------------------
// fp32: one workgroup of sixteen waves per matrix on the fp32 matrix cores
// (v_mfma_f32_16x16x4f32: fp32 products, fp32 accumulation).  X (s x l,
// s <= 64, l <= LMAX) sits in LDS zero-padded to multiples of 32 on both
// sides.  Operands are one float per lane per MFMA: A[i][k] from lane
// 16 (k % 4) + i, B[k][j] from lane 16 (k % 4) + j; the result's lane l holds
// column l % 16, rows 4 (l / 16) + e.  Per step:
//  * the Gram A = X X^T on its upper 16 x 16 blocks (ti <= tj; ten for s = 64),
//    dealt to the waves, each stored with its mirror (A exactly symmetric);
//  * the combine Y = a X + b A X on 16 x 16 blocks (32 for 64 x 128), dealt
//    to the waves.
// Within each 16 contraction indices, MFMA t takes index 4 kq + t from lane
// group kq (a fixed permutation of the summation order), so the row-wise
// operands (both of the Gram's, A's in the combine) arrive as one 16-byte
// read per four MFMAs.
// A single matrix runs on one CU, so its step time is the dependent chain of
// each wave's products: sixteen waves on 16 x 16 blocks and the Gram's
// symmetry cut it to a quarter of four waves on 32 x 32 blocks.
template <int LMAX>
__global__ void __launch_bounds__(1024) ns_small_f32_kernel(NsSmallLaunch P) {
  // Row strides keep 16-byte row reads aligned and put the four rows of a
  // column read 16 (X) or 4 (A) banks apart.
  constexpr int SMAX = 64, XS = LMAX + 16, AS = SMAX + 4, NT = 1024, NW = NT / 64;
  __shared__ __attribute__((aligned(16))) float xa[SMAX][XS];
  __shared__ __attribute__((aligned(16))) float xb[SMAX][XS];
  __shared__ __attribute__((aligned(16))) float am[SMAX][AS];
  __shared__ float red[NW];
  const int S = P.s, Lw = P.l, tid = threadIdx.x;
  const int Sp = (S + 31) & ~31, Lp = (Lw + 31) & ~31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  for (long long mat = blockIdx.x; mat < P.count; mat += gridDim.x) {
    const float* src = static_cast<const float*>(P.X) + mat * P.in_stride;
    float* dst = static_cast<float*>(P.Y) + mat * P.out_stride;
    // stage X, zero padded to Sp x Lp (the padding stays zero through every step)
    float ss = 0.0f;
    for (int e = tid; e < Sp * Lp; e += NT) {
      int i, k;
      if (P.transposed) {  // stored as l x s: consecutive threads read consecutive i
        i = e % Sp; k = e / Sp;
      } else {
        i = e / Lp; k = e % Lp;
      }
      float v = 0.0f;
      if (i < S && k < Lw)
        v = P.transposed ? src[static_cast<long long>(k) * P.ld_in + i] : src[static_cast<long long>(i) * P.ld_in + k];
      xa[i][k] = v;
      ss = fmaf(v, v, ss);
    }
    float inv;
    if (P.partials != nullptr) {
      float s2 = 0.0f;
      for (int i = tid; i < P.P; i += NT) s2 += P.partials[mat * P.P + i];
      inv = 1.0f / (sqrtf(block_sum(s2, red)) + P.eps);
    } else {
      inv = 1.0f / (sqrtf(block_sum(ss, red)) + P.eps);
    }
    __syncthreads();
    for (int e = tid; e < Sp * Lp; e += NT) xa[e / Lp][e % Lp] *= inv;
    __syncthreads();
    float (*cur)[XS] = xa;
    float (*nxt)[XS] = xb;
    const int n16 = Sp / 16, nu = n16 * (n16 + 1) / 2;
    for (int step = 0; step < P.steps; ++step) {
      // Gram: upper 16 x 16 block u (row-major over ti <= tj) per wave
      for (int u = w; u < nu; u += NW) {
        int ti = 0, rem = u;
        while (rem >= n16 - ti) {
          rem -= n16 - ti;
          ++ti;
        }
        const int tj = ti + rem;
        f32x4_t g = {0.0f, 0.0f, 0.0f, 0.0f};
        // contraction order within 16 columns: MFMA t takes column 4 kq + t
        // from lane group kq, so one 16-byte read serves four MFMAs
#pragma unroll 2
        for (int k = 0; k < Lp; k += 16) {
          const f32x4_t av = *reinterpret_cast<const f32x4_t*>(&cur[ti * 16 + r16][k + 4 * kq]);
          const f32x4_t bv = *reinterpret_cast<const f32x4_t*>(&cur[tj * 16 + r16][k + 4 * kq]);
#pragma unroll
          for (int t = 0; t < 4; ++t) g = __builtin_amdgcn_mfma_f32_16x16x4f32(av[t], bv[t], g, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = ti * 16 + 4 * kq + e, j = tj * 16 + r16;
          am[i][j] = g[e];
          if (ti != tj) am[j][i] = g[e];
        }
      }
      __syncthreads();
      // combine Y = a X + b A X: 16 x 16 block (ti, tk) per wave
      const float a = P.a[step], b = P.b[step];
      const int n16l = Lp / 16;
      for (int blk = w; blk < n16 * n16l; blk += NW) {
        const int ti = blk % n16, tk = blk / n16;
        f32x4_t y = {0.0f, 0.0f, 0.0f, 0.0f};
        // the same order: MFMA t contracts over row 4 kq + t of X
#pragma unroll 2
        for (int j = 0; j < Sp; j += 16) {
          const f32x4_t av = *reinterpret_cast<const f32x4_t*>(&am[ti * 16 + r16][j + 4 * kq]);
#pragma unroll
          for (int t = 0; t < 4; ++t)
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(av[t], cur[j + 4 * kq + t][tk * 16 + r16], y, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = ti * 16 + 4 * kq + e, k = tk * 16 + r16;
          nxt[i][k] = fmaf(a, cur[i][k], b * y[e]);
        }
      }
      __syncthreads();
      float (*t)[XS] = cur;
      cur = nxt;
      nxt = t;
    }
    for (int e = tid; e < S * Lw; e += NT) {
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
  // bf16: the kernels take s in {32, 64, 96, 128} and l a multiple of 32;
  // muon_step pads other sides with zeros up to those
  if (bf16) return s >= 1 && s <= 128 && l >= s && l <= kRtMaxL;
  return s >= 1 && s <= 64 && l >= s && l <= 256;
}

hipError_t launch_ns_small(const NsSmallLaunch& P, bool bf16, hipStream_t st) {
  if (bf16 && (P.s % 32 != 0 || P.l % 32 != 0 || P.s > 128 || P.l < P.s || P.l > kRtMaxL))
    return hipErrorInvalidValue;
  // one matrix per workgroup of s / 32 waves, X and A in dynamic LDS: short
  // sides above 64, long sides above 256, and 64 x 160 .. 64 x 256, where one
  // wave per matrix holds too many accumulators for two waves per SIMD.  Rows
  // split over the waves (X alone in LDS) wherever X fits a CU twice: the
  // same results bit for bit, 1.1-2x faster (more workgroups per CU, no A
  // round trip); columns split (X and A) for the larger shapes, where one
  // workgroup per CU is all either can have and the row split reads more LDS.
  if (bf16 && (P.s > 64 || P.l > 256 || (P.s == 64 && P.l >= 160))) {
    const size_t xbytes = static_cast<size_t>(P.s) * P.l * 2;
    const size_t lds = xbytes + static_cast<size_t>(P.s) * P.s * 2;
    if (lds > static_cast<size_t>(kMaxLds)) return hipErrorInvalidValue;
    const long long blocks = small_grid(P.count, 1LL << 16);
    const dim3 grid(static_cast<unsigned>(blocks)), block(P.s * 2);
    const bool rows = kMaxLds / xbytes >= 2;
#define MUON_SMALL_WGR(SS)                                                                               \
  if (P.s == SS) {                                                                                       \
    const void* fn = reinterpret_cast<const void*>(ns_small_bf16_wgr_kernel<SS>);                        \
    if (xbytes > 65536 && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,          \
                                              static_cast<int>(xbytes)) != hipSuccess)                   \
      return hipErrorInvalidValue;                                                                       \
    hipLaunchKernelGGL((ns_small_bf16_wgr_kernel<SS>), grid, block, xbytes, st, P);                      \
    return hipGetLastError();                                                                            \
  }
    if (rows) {
      MUON_SMALL_WGR(32) MUON_SMALL_WGR(64) MUON_SMALL_WGR(96) MUON_SMALL_WGR(128)
      return hipErrorInvalidValue;
    }
#undef MUON_SMALL_WGR
#define MUON_SMALL_WG(SS)                                                                                \
  if (P.s == SS) {                                                                                       \
    const void* fn = reinterpret_cast<const void*>(ns_small_bf16_wg_kernel<SS>);                         \
    if (lds > 65536 && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,             \
                                           static_cast<int>(lds)) != hipSuccess)                         \
      return hipErrorInvalidValue;                                                                       \
    hipLaunchKernelGGL((ns_small_bf16_wg_kernel<SS>), grid, block, lds, st, P);                          \
    return hipGetLastError();                                                                            \
  }
    MUON_SMALL_WG(32) MUON_SMALL_WG(64) MUON_SMALL_WG(96) MUON_SMALL_WG(128)
#undef MUON_SMALL_WG
    return hipErrorInvalidValue;
  }
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
    MUON_SMALL(64, 64) MUON_SMALL(64, 96) MUON_SMALL(64, 128)
#undef MUON_SMALL
    return hipErrorInvalidValue;
  }
  const long long blocks = small_grid(P.count, 1LL << 16);
  if (P.l <= 128)
    hipLaunchKernelGGL((ns_small_f32_kernel<128>), dim3(static_cast<unsigned>(blocks)), dim3(1024), 0, st, P);
  else
    hipLaunchKernelGGL((ns_small_f32_kernel<256>), dim3(static_cast<unsigned>(blocks)), dim3(1024), 0, st, P);
  return hipGetLastError();
}

}  // namespace muon
