// Spectral diagnostics of a stack of matrices.  The "Muon Meets Mamba"
// practitioner article (sections on the training checkpoints and on
// long-term engineering) asks for the largest singular value of each weight
// or state matrix every few steps, checked against a safety threshold, and
// for singular values in the training log; the orthogonality error measures
// how far a Newton-Schulz update is from orthogonal.  For A (m x n) with X its
// short-side orientation (s x l) and H = X X^T:
//   orth_err  = ||H - I_s||_F / sqrt(s)
//   sigma_max, sigma_min = sqrt of the extreme Ritz values after k Lanczos
//               steps on H with full reorthogonalisation (exact once k = s).
// Three passes per chunk of matrices:
//   diag_pack_kernel     orient X (transposing tall inputs through LDS) into
//                        bf16 operand rows for the symmetric-product kernel;
//                        float32 inputs are split exactly into three bf16
//                        pieces x = h + d + e, stored once side by side; the
//                        Gram contracts over six segments that pair them as the
//                        six products that matter, hh + hd + dh + dd + he + eh
//                        (L segments h h d d h e, R segments h d h d e h)
//   symprod (float32 output) H = L R^T on the matrix cores
//   diag_lanczos_kernel  one workgroup per matrix: ||H - I|| in float64, then
//                        the Lanczos run in float32 with its vectors in LDS and
//                        the basis in global memory, and the extreme eigenvalues
//                        of the tridiagonal matrix by float64 multisection.
//   diag_lanczos_split_kernel  the same run when few matrices would leave most
//                        CUs idle: P co-resident workgroups per matrix (one
//                        cooperative launch) each own a 256 x 256 block of the
//                        upper block triangle of H (or a range of its rows)
//                        and contribute its column sums and, off the diagonal,
//                        its row sums to H q; the contributions meet through
//                        global memory as tagged words that the readers wait
//                        on, and every workgroup then repeats the vector work
//                        on its own copy of the basis in LDS (identical
//                        arithmetic, so the copies stay equal).
// Every reduction runs in a fixed order: results are deterministic.
#include <cstdlib>
#include <mutex>

#include "common.cuh"
#include "launch.h"

namespace muon {
namespace {

constexpr int kPackT = 64;  // pack tile: 64 rows of X x 64 columns

__device__ __forceinline__ float load_elem(const void* a, long long i, bool f32) {
  return f32 ? static_cast<const float*>(a)[i] : bf16_to_f32(static_cast<const bf16_t*>(a)[i]);
}

__global__ void __launch_bounds__(256) diag_pack_kernel(DiagPackLaunch P) {
  __shared__ float t[kPackT][kPackT + 1];
  const long long tiles_k = P.kdim / kPackT, tiles_r = P.s_pad / kPackT;
  const long long b = blockIdx.x;
  const long long z = b / (tiles_k * tiles_r);
  const int tr = static_cast<int>((b / tiles_k) % tiles_r), tk = static_cast<int>(b % tiles_k);
  const int r0 = tr * kPackT, k0 = tk * kPackT;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const long long abase = z * P.astride;
  if (P.clr != nullptr) {  // zero the split run's scratch: this block's share of it
    const long long nblk = tiles_k * tiles_r, me = static_cast<long long>(tr) * tiles_k + tk;
    for (long long i = me * 256 + threadIdx.x; i < P.clr_words; i += nblk * 256) P.clr[z * P.cstride + i] = 0u;
  }
  // t[row of X][column of X]
  for (int yy = ty; yy < kPackT; yy += 4) {
    if (!P.tall) {  // X[r][k] = A[r][k]: rows r0 + yy, columns k0 + tx
      const int r = r0 + yy, k = k0 + tx;
      t[yy][tx] = (r < P.s && k < P.l) ? load_elem(P.A, abase + static_cast<long long>(r) * P.n + k, P.f32) : 0.0f;
    } else {        // X[r][k] = A[k][r]: read A row k0 + yy, columns r0 + tx
      const int k = k0 + yy, r = r0 + tx;
      t[tx][yy] = (r < P.s && k < P.l) ? load_elem(P.A, abase + static_cast<long long>(k) * P.n + r, P.f32) : 0.0f;
    }
  }
  __syncthreads();
  const long long obase = z * P.ostride;
  for (int yy = ty; yy < kPackT; yy += 4) {
    const float x = t[yy][tx];
    const long long o = obase + static_cast<long long>(r0 + yy) * P.ld + k0 + tx;
    if (!P.f32) {
      P.L[o] = f32_to_bf16(x);  // exact: x came from bf16
    } else {
      const bf16_t h = f32_to_bf16(x);
      const float xd = x - bf16_to_f32(h);          // exact
      const bf16_t d = f32_to_bf16(xd);
      const bf16_t e = f32_to_bf16(xd - bf16_to_f32(d));
      const long long K = P.kdim;
      P.L[o] = h;
      P.L[o + K] = d;
      P.L[o + 2 * K] = e;
    }
  }
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ double block_sum_d(double v, double* red) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave, nw = blockDim.x / kWave;
  v = wave_sum_d(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// Deterministic block maximum of non-negative values (or NaN); every thread
// gets the result.  `red` holds blockDim.x / 64 floats of LDS.
__device__ __forceinline__ float block_max(float v, float* red) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave, nw = blockDim.x / kWave;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float o = __shfl_xor(v, off, kWave);
    v = (v != v || o != o) ? NAN : fmaxf(v, o);
  }
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float t = red[0];
  for (int i = 1; i < nw; ++i) t = (t != t || red[i] != red[i]) ? NAN : fmaxf(t, red[i]);
  return t;
}

// ||v|| over v[0..n) in LDS, scaled by max |v_i| so that tiny entries do not
// underflow when squared (NaN if any entry is NaN).  Every thread gets it.
__device__ float scaled_norm(const float* v, int n, float* red) {
  float mx = 0.0f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) mx = (v[i] != v[i] || mx != mx) ? NAN : fmaxf(mx, fabsf(v[i]));
  mx = block_max(mx, red);
  if (!(mx > 0.0f) || mx == INFINITY) return mx;  // 0, NaN or Inf
  const float inv = 1.0f / mx;
  float part = 0.0f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const float x = v[i] * inv;
    part = fmaf(x, x, part);
  }
  return mx * sqrtf(block_sum(part, red));
}

constexpr float kBreakdown = 0x1p-20f;  // relative size of a residual taken as zero

// Number of eigenvalues of T below x (Sturm sequence of the LDL^T pivots).
__device__ int sturm_count(const float* al, const float* be, int k, double x, double pivmin) {
  int c = 0;
  double d = static_cast<double>(al[0]) - x;
  if (fabs(d) < pivmin) d = -pivmin;
  c += d < 0.0;
  for (int i = 1; i < k; ++i) {
    const double b = be[i];
    d = static_cast<double>(al[i]) - x - b * b / d;
    if (fabs(d) < pivmin) d = -pivmin;
    c += d < 0.0;
  }
  return c;
}

// Wave 0: smallest x with count(x) >= need on [lo, hi], by 64-point
// multisection (each round shrinks the bracket 65-fold).
__device__ double multisect(const float* al, const float* be, int k, double lo, double hi, int need,
                            double pivmin) {
  const int lane = threadIdx.x & 63;
  for (int round = 0; round < 12; ++round) {
    const double x = lo + (hi - lo) * static_cast<double>(lane + 1) / 65.0;
    const bool p = sturm_count(al, be, k, x, pivmin) >= need;
    const unsigned long long m = __ballot(p);
    if (m == 0) {
      lo = __shfl(x, 63, kWave);
    } else {
      const int f = __ffsll(static_cast<long long>(m)) - 1;  // first point where it holds (wave-uniform)
      const double xf = __shfl(x, f, kWave);
      const double xp = __shfl(x, f > 0 ? f - 1 : 0, kWave);
      lo = f > 0 ? xp : lo;
      hi = xf;
    }
  }
  return 0.5 * (lo + hi);
}

// Wave 0: sqrt of the extreme eigenvalues of the k x k tridiagonal matrix
// (alphas al[0..k), couplings be[1..k)) by multisection inside the
// Gershgorin bounds; NaN if any alpha is not finite.
__device__ void tridiag_extremes(const float* al, const float* be, int kk, long long z, const DiagLaunch& D) {
  const int lane = threadIdx.x & 63;
  bool finite = true;
  double lo = INFINITY, hi = -INFINITY, bmax = 0.0;
  for (int i = 0; i < kk; ++i) {
    const double a = al[i];
    const double bl = i > 0 ? fabs(static_cast<double>(be[i])) : 0.0;
    const double br = i + 1 < kk ? fabs(static_cast<double>(be[i + 1])) : 0.0;
    finite = finite && isfinite(a);
    lo = fmin(lo, a - bl - br);
    hi = fmax(hi, a + bl + br);
    bmax = fmax(bmax, bl);
  }
  float smin = NAN, smax = NAN;
  if (finite) {
    const double span = fmax(fabs(lo), fabs(hi));
    const double pad = 1e-12 * span + 1e-300;
    lo -= pad;
    hi += pad;
    const double pivmin = fmax(1e-290, 1e-290 * bmax * bmax);
    const double lmin = multisect(al, be, kk, lo, hi, 1, pivmin);
    const double lmax = multisect(al, be, kk, lo, hi, kk, pivmin);
    smin = static_cast<float>(sqrt(fmax(lmin, 0.0)));
    smax = static_cast<float>(sqrt(fmax(lmax, 0.0)));
  }
  if (lane == 0) {
    if (D.smin != nullptr) D.smin[z] = smin;
    if (D.smax != nullptr) D.smax[z] = smax;
  }
}

__device__ __forceinline__ float weyl_start(int i) {
  const uint32_t h = static_cast<uint32_t>(i) * 2654435769u;  // mod 2^32
  return static_cast<float>(h >> 8) * (1.0f / 16777216.0f) - 0.5f;
}

// w = H q for symmetric H, column-parallel: w_c = sum_r H[r][c] q[r].  Work
// items (128-column chunk, range of rows) are dealt to the waves; a lane owns
// two adjacent columns and accumulates over its rows (rows read whole and
// coalesced, kMvRows in flight, q[r] an LDS broadcast, no cross-lane
// reduction); the row ranges' partials are added in a fixed order.
constexpr int kMvRows = 16;
__device__ void sym_matvec(const float* H, int s, int sp, const float* q, float* w, float* part) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int nchunk = sp / 128;
  const int nsplit = (2 * nw + nchunk - 1) / nchunk;
  const int rows_per = (s + nsplit - 1) / nsplit;
  for (int it = wv; it < nchunk * nsplit; it += nw) {
    const int cc = it % nchunk, rr = it / nchunk;
    const int c = cc * 128 + lane * 2;
    const int r0 = rr * rows_per, r1 = r0 + rows_per < s ? r0 + rows_per : s;
    const float* hc = H + c;
    float a0 = 0.0f, a1 = 0.0f;
    int r = r0;
    for (; r + kMvRows <= r1; r += kMvRows) {
      f32x2_t h[kMvRows];
#pragma unroll
      for (int u = 0; u < kMvRows; ++u)
        h[u] = *reinterpret_cast<const f32x2_t*>(hc + static_cast<long long>(r + u) * sp);
#pragma unroll
      for (int u = 0; u < kMvRows; ++u) {
        const float qr = q[r + u];
        a0 = fmaf(h[u][0], qr, a0);
        a1 = fmaf(h[u][1], qr, a1);
      }
    }
    for (; r < r1; ++r) {
      const f32x2_t h = *reinterpret_cast<const f32x2_t*>(hc + static_cast<long long>(r) * sp);
      a0 = fmaf(h[0], q[r], a0);
      a1 = fmaf(h[1], q[r], a1);
    }
    part[rr * sp + c] = a0;
    part[rr * sp + c + 1] = a1;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < sp; i += blockDim.x) {
    float x = 0.0f;
    for (int rr = 0; rr < nsplit; ++rr) x += part[rr * sp + i];
    w[i] = x;
  }
  __syncthreads();
}

int sym_matvec_splits(int sp, int nw) {
  const int nchunk = sp / 128;
  return (2 * nw + nchunk - 1) / nchunk;
}

__global__ void __launch_bounds__(1024) diag_lanczos_kernel(DiagLaunch D) {
  extern __shared__ __attribute__((aligned(16))) float sh[];  // 16-byte LDS accesses need the base aligned
  const int sp = D.s_pad, s = D.s;
  float* q = sh;                 // [sp]
  float* w = q + sp;             // [sp]
  float* qp = w + sp;            // [sp] previous vector
  float* al = qp + sp;           // [kmax] alphas
  float* be = al + D.kmax;       // [kmax] betas (be[j] couples j-1, j)
  float* cf = be + D.kmax;       // [kmax] reorthogonalisation coefficients
  float* mvp = cf + D.kmax;      // [splits][sp] matrix-vector partials
  __shared__ float red[16];
  __shared__ double redd[16];
  const long long z = blockIdx.x;
  const float* H = D.H + z * D.hstride;
  float* Q = D.Q + z * D.qstride;
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, wv = tid >> 6, nw = nthr >> 6;
  const int k = D.iters < s ? D.iters : s;

  // ||H - I||_F^2 over the s x s block (rows by wave, 4 columns per lane)
  if (D.orth != nullptr) {
    double acc = 0.0;
    for (int r = wv; r < s; r += nw) {
      const float* row = H + static_cast<long long>(r) * sp;
      for (int c = lane * 4; c < sp; c += 256) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(row + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (c + e < s) {
            const double d = static_cast<double>(v[e]) - (c + e == r ? 1.0 : 0.0);
            acc += d * d;
          }
        }
      }
    }
    const double tot = block_sum_d(acc, redd);
    if (tid == 0) D.orth[z] = static_cast<float>(sqrt(tot / s));
  }
  if (D.smax == nullptr && D.smin == nullptr) return;

  // start vector
  float part = 0.0f;
  for (int i = tid; i < sp; i += nthr) {
    const float v = i < s ? weyl_start(i) : 0.0f;
    q[i] = v;
    qp[i] = 0.0f;
    part += v * v;
  }
  const float qn = sqrtf(block_sum(part, red));
  for (int i = tid; i < sp; i += nthr) {
    q[i] /= qn;
    Q[i] = q[i];
  }
  __syncthreads();

  float beta = 0.0f;
  int kk = k;
  for (int j = 0; j < k; ++j) {
    sym_matvec(H, s, sp, q, w, mvp);
    const float hq = scaled_norm(w, sp, red);  // ||H q||: the scale of a residual taken as zero
    part = 0.0f;
    for (int i = tid; i < sp; i += nthr) part = fmaf(q[i], w[i], part);
    const float alpha = block_sum(part, red);
    for (int i = tid; i < sp; i += nthr) w[i] = w[i] - alpha * q[i] - beta * qp[i];
    __syncthreads();
    // two passes of classical Gram-Schmidt against q_0 .. q_j
    for (int pass = 0; pass < 2; ++pass) {
      for (int t = wv; t <= j; t += nw) {
        const float* qt = Q + static_cast<long long>(t) * sp;
        float d = 0.0f;
        for (int c = lane * 4; c < sp; c += 256) {
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(qt + c);
          d = fmaf(v[0], w[c], fmaf(v[1], w[c + 1], fmaf(v[2], w[c + 2], fmaf(v[3], w[c + 3], d))));
        }
        d = wave_sum(d);
        if (lane == 0) cf[t] = d;
      }
      __syncthreads();
      // the j + 1 loads of an element are issued eight at a time ahead of
      // their FMAs (same order of FMAs: the result does not change)
      for (int i = tid; i < sp; i += nthr) {
        float x = w[i];
        int t = 0;
        for (; t + 8 <= j + 1; t += 8) {
          float qv[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) qv[u] = Q[static_cast<long long>(t + u) * sp + i];
#pragma unroll
          for (int u = 0; u < 8; ++u) x = fmaf(-cf[t + u], qv[u], x);
        }
        for (; t <= j; ++t) x = fmaf(-cf[t], Q[static_cast<long long>(t) * sp + i], x);
        w[i] = x;
      }
      __syncthreads();
    }
    // the run ends when the residual is rounding noise (beta <= 2^-20 ||H q||:
    // the Krylov space is invariant to working accuracy, and a basis grown
    // from noise would not stay orthogonal) or is not finite
    const float bn = scaled_norm(w, sp, red);
    if (tid == 0) al[j] = alpha;
    if (j + 1 == k || !(bn > kBreakdown * hq && bn < INFINITY)) {
      kk = j + 1;
      break;
    }
    if (tid == 0) be[j + 1] = bn;
    float* qn1 = Q + static_cast<long long>(j + 1) * sp;
    for (int i = tid; i < sp; i += nthr) {
      const float v = w[i] / bn;
      qp[i] = q[i];
      q[i] = v;
      qn1[i] = v;
    }
    beta = bn;
    __syncthreads();
  }
  __syncthreads();

  if (wv == 0) tridiag_extremes(al, be, kk, z, D);
}

// ---- split run: several workgroups per matrix ----------------------------------
constexpr int kSplitThreads = 512;
constexpr int kSplitWaves = kSplitThreads / 64;
constexpr int kSplitBlock = 256;           // H is cut into 256 x 256 blocks (4 columns per lane)
constexpr int kSplitMaxR = 16;             // row ranges per block
constexpr unsigned kSpinLimit = 1u << 20;  // polls before a wait is given up (unless a test shortens it)

// A matrix's split scratch, in floats from the start of its basis region
// (unused by this kernel: the basis lives in LDS): [0] a barrier counter,
// [64, 64 + 2P) the per-workgroup float64 partials of ||H - I||^2, then the
// tagged partial products, two buffers (steps alternate) of
// [nb][nb][R][256] 64-bit words.  The whole range is zeroed before launch.
__host__ __device__ constexpr long long split_tag_off(int p) { return 64 + (2LL * p + 63) / 64 * 64; }
__host__ __device__ constexpr long long split_scratch_floats(int p, int r, int nb) {
  return split_tag_off(p) + 2LL * 2 * kSplitBlock * nb * nb * r;
}

// Barrier of the P workgroups of one matrix (used once, to hand over the
// float64 partials).  Only lane 0 of wave 0 has stored what the other
// workgroups read (they may sit on another XCD): it releases those stores
// at agent scope with its arrival, waits for `target` arrivals and
// acquires; the workgroup barrier then orders every wave's later loads.
// The wait is bounded: a workgroup that gives up marks itself dead.
__device__ bool split_barrier(unsigned* cnt, unsigned target, int* dead, unsigned limit) {
  if (threadIdx.x == 0 && *dead == 0) {
    __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    unsigned polls = 0;
    while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (++polls > limit) {
        *dead = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  return *dead == 0;
}

// Partial products travel as one 64-bit atomic word {step tag, float value}:
// the reader waits on the word itself, so no fence and no separate flag is
// needed.  Tags are the step number + 1 (the zeroed buffer matches none).
__device__ __forceinline__ void put_tagged(unsigned long long* a, float v, unsigned tag) {
  __hip_atomic_store(a, (static_cast<unsigned long long>(tag) << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded wait for a tagged word (out of line: the common case finds the
// word ready on the first read); after a timeout, or once another wave of
// the workgroup has timed out, returns NaN and leaves *dead set.
__device__ __noinline__ float wait_tagged(unsigned long long* a, unsigned tag, int* dead, unsigned limit) {
  for (unsigned polls = 0;; ++polls) {
    const unsigned long long x = __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (static_cast<unsigned>(x >> 32) == tag) return __uint_as_float(static_cast<unsigned>(x));
    if (polls > limit || __hip_atomic_load(dead, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0) {
      __hip_atomic_store(dead, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      return NAN;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

__device__ __forceinline__ double wave_total_d(double v) {
  v += dpp_d<kDppShr1>(v);
  v += dpp_d<kDppShr2>(v);
  v += dpp_d<kDppShr4>(v);
  v += dpp_d<kDppShr8>(v);
  {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b), kDppBcast15, 0xa, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), kDppBcast15, 0xa, 0xf, false);
    v += __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
  }
  {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b), kDppBcast31, 0xc, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), kDppBcast31, 0xc, 0xf, false);
    v += __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
  }
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), 63);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), 63);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}

// Block sums for the split kernel (DPP wave totals; `red` holds 2 x waves
// doubles of LDS); every thread gets the result.
__device__ __forceinline__ double split_sum_d(double a, double* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  a = wave_total_d(a);
  __syncthreads();
  if (lane == 0) red[wid] = a;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}
__device__ __forceinline__ void split_sum2_d(double& a, double& b, double* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  a = wave_total_d(a);
  b = wave_total_d(b);
  __syncthreads();
  if (lane == 0) { red[2 * wid] = a; red[2 * wid + 1] = b; }
  __syncthreads();
  a = 0.0;
  b = 0.0;
  for (int i = 0; i < nw; ++i) { a += red[2 * i]; b += red[2 * i + 1]; }
}

// One halving exchange of the row reduce-scatter over lane bit M: each pair
// (row u, row u + H) becomes row u in lanes with bit M clear and row u + H
// where it is set, summed with the partner lane's copy.  Bits 5 and 4 use
// the permlane swaps, bits 3 and 2 the DPP row rotations/shifts.
template <int M, int H, int NR>
__device__ __forceinline__ void rs_halve(float (&v)[NR], int lane) {
#pragma unroll
  for (int u = 0; u < H; ++u) {
    const float a = v[u], b = v[u + H];
    if constexpr (M == 32 || M == 16) {
      const auto r = M == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false)
                             : __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
      v[u] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else if constexpr (M == 8) {
      const float sa = a + dpp_f<kDppRor8>(a), sb = b + dpp_f<kDppRor8>(b);
      v[u] = (lane & 8) ? sb : sa;
    } else {
      static_assert(M == 4, "halving over lane bits 5..2");
      const float sa = a + dpp_f<kDppShl4>(a), sb = b + dpp_f<kDppShr4>(b);
      v[u] = (lane & 4) ? sb : sa;
    }
  }
}

// Sums NR values per lane (row u of a batch, NR = 8 or 16) over the 64
// lanes: log2(NR) halving exchanges, then a butterfly over the remaining
// lane bits.  Lane L ends with the total of row L >> (6 - log2 NR).  Fixed
// order; no LDS.
template <int NR>
__device__ __forceinline__ float reduce_scatter_rows(float (&v)[NR], int lane) {
  static_assert(NR == 8 || NR == 16, "8 or 16 rows per batch");
  rs_halve<32, NR / 2>(v, lane);
  rs_halve<16, NR / 4>(v, lane);
  rs_halve<8, NR / 8>(v, lane);
  if constexpr (NR == 16) rs_halve<4, 1>(v, lane);
  float x = v[0];
  if constexpr (NR == 8) {
    // both moves by every lane: a DPP read from a lane switched off by a
    // branch returns nothing, so neither may sit inside the selection
    const float from_below = dpp_f<kDppShr4>(x), from_above = dpp_f<kDppShl4>(x);
    x += (lane & 4) ? from_below : from_above;
  }
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppXor1>(x);
  return x;
}

// This workgroup's share of w = H q from one block of the upper block
// triangle: rows [ra0, rb0) of block row bi (consecutive runs per wave, NR
// 16-byte loads in flight), the 256 columns from cb (four per lane).  The
// column sums (H^T q over these rows) are left per wave in part[wave][256];
// an off-diagonal block also stands for its mirror image, so the row sums
// H q over these columns are stored, tagged, to rowslot[r - row0].  With
// ORTH also returns this thread's share of sum (H_rc - delta_rc)^2 over
// r, c < s (off-diagonal blocks counted twice).
template <bool ORTH, int NR = ORTH ? kMvRows / 2 : kMvRows>
__device__ double tri_matvec(const float* H, int s, int sp, int ra0, int rb0, int row0, int cb, bool offdiag,
                             const float* q, float* part, unsigned long long* rowslot, unsigned tag) {
  constexpr int kLog = NR == 16 ? 4 : NR == 8 ? 3 : NR == 4 ? 2 : NR == 2 ? 1 : 0;
  static_assert((1 << kLog) == NR, "NR: a power of two up to 16");
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c = cb + lane * 4;
  const bool on = c < sp;
  const int per = (rb0 - ra0 + kSplitWaves - 1) / kSplitWaves;
  const int ra = ra0 + wv * per, rb = ra + per < rb0 ? ra + per : rb0;
  const float* hc = H + (on ? c : 0);
  const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const f32x4_t qc = on ? *reinterpret_cast<const f32x4_t*>(q + c) : zero;
  f32x4_t acc = zero;
  double oa = 0.0;
  const double ow = offdiag ? 2.0 : 1.0;
  for (int r = ra; r < rb; r += NR) {
    f32x4_t h[NR];
#pragma unroll
    for (int u = 0; u < NR; ++u)
      h[u] = (on && r + u < rb) ? *reinterpret_cast<const f32x4_t*>(hc + static_cast<long long>(r + u) * sp) : zero;
    float rs[NR];
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const float qr = r + u < rb ? q[r + u] : 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(h[u][e], qr, acc[e]);
      rs[u] = fmaf(h[u][3], qc[3], fmaf(h[u][2], qc[2], fmaf(h[u][1], qc[1], h[u][0] * qc[0])));
      if constexpr (ORTH) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (r + u < rb && c + e < s) {
            const double d = static_cast<double>(h[u][e]) - (c + e == r + u ? 1.0 : 0.0);
            oa += ow * d * d;
          }
        }
      }
    }
    if (offdiag) {
      const float x = reduce_scatter_rows<NR>(rs, lane);
      const int rr = r + (lane >> (6 - kLog));
      if ((lane & ((1 << (6 - kLog)) - 1)) == 0 && rr < rb) put_tagged(rowslot + (rr - row0), x, tag);
    }
  }
  *reinterpret_cast<f32x4_t*>(part + wv * kSplitBlock + lane * 4) = acc;
  return oa;
}

__global__ void __launch_bounds__(kSplitThreads) diag_lanczos_split_kernel(DiagLaunch D) {
  extern __shared__ __attribute__((aligned(16))) float sh[];  // 16-byte LDS accesses need the base aligned
  const int sp = D.s_pad, s = D.s, P = D.split_p, R = D.split_r, nb = D.split_nb;
  float* Qs = sh;                          // [kmax][sp] basis
  float* w = Qs + static_cast<long long>(D.kmax) * sp;  // [sp]
  float* part = w + sp;                    // [waves][256] column sums of the block
  const int kpad = (D.kmax + 3) & ~3;
  float* cf = part + kSplitWaves * kSplitBlock;  // [kpad] reorthogonalisation coefficients (16-byte aligned)
  float* al = cf + kpad;                   // [kpad] alphas
  float* be = al + kpad;                   // [kpad] betas
  float* gat = be + kpad;                  // [nb][nb][R][256] gathered partial products
  __shared__ double redd[2 * kSplitWaves];
  __shared__ int dead;
  __shared__ int rpb[16];  // rows per range in each block row
  const long long z = blockIdx.x / P;
  const int p = static_cast<int>(blockIdx.x % P);
  // block (bi, bj), bi <= bj, of the upper block triangle; row range rsub of its rows
  int u = p / R, bi = 0;
  while (u >= nb - bi) {
    u -= nb - bi;
    ++bi;
  }
  const int bj = bi + u, rsub = p % R;
  auto rows_per = [&](int b) {  // rows per range in block row b
    const int nr = s - b * kSplitBlock < kSplitBlock ? s - b * kSplitBlock : kSplitBlock;
    return (nr + R - 1) / R;
  };
  if (threadIdx.x < nb) rpb[threadIdx.x] = rows_per(threadIdx.x);
  const int row0 = bi * kSplitBlock;
  const int nrow = s - row0 < kSplitBlock ? s - row0 : kSplitBlock;
  const int ra0 = row0 + (rsub * rows_per(bi) < nrow ? rsub * rows_per(bi) : nrow);
  const int rb0 = row0 + ((rsub + 1) * rows_per(bi) < nrow ? (rsub + 1) * rows_per(bi) : nrow);
  const float* H = D.H + z * D.hstride;
  float* scr = D.Q + z * D.qstride;
  unsigned* cnt = reinterpret_cast<unsigned*>(scr);
  double* gorth = reinterpret_cast<double*>(scr + 64);
  unsigned long long* tags = reinterpret_cast<unsigned long long*>(scr + split_tag_off(P));
  auto slot = [&](int buf, int b, int o, int rs) {  // contribution of block column/row o to block b of w
    return tags + ((static_cast<long long>(buf * nb + b) * nb + o) * R + rs) * kSplitBlock;
  };
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, wv = tid >> 6;
  const int k = D.iters < s ? D.iters : s;
  const bool want_sigma = D.smax != nullptr || D.smin != nullptr;
  if (tid == 0) dead = 0;

  // start vector (the same in every workgroup)
  float part0 = 0.0f;
  for (int i = tid; i < sp; i += nthr) {
    const float v = i < s ? weyl_start(i) : 0.0f;
    Qs[i] = v;
    part0 += v * v;
  }
  const float qn = sqrtf(block_sum(part0, reinterpret_cast<float*>(redd)));
  for (int i = tid; i < sp; i += nthr) Qs[i] /= qn;
  __syncthreads();

  float beta = 0.0f;
  int kk = k;
  for (int j = 0; j < k; ++j) {
    const float* q = Qs + static_cast<long long>(j) * sp;
    const unsigned tag = static_cast<unsigned>(j + 1);
    const int buf = j & 1;
    unsigned long long* rowslot = slot(buf, bi, bj, rsub);
    if (j == 0) {
      double oa = tri_matvec<true>(H, s, sp, ra0, rb0, row0, bj * kSplitBlock, bi != bj, q, part, rowslot, tag);
      oa = split_sum_d(oa, redd);  // its barriers also publish `part`
      if (tid == 0) gorth[p] = oa;
    } else {
      tri_matvec<false>(H, s, sp, ra0, rb0, row0, bj * kSplitBlock, bi != bj, q, part, rowslot, tag);
      __syncthreads();
    }
    // wave 0 adds the waves' column sums (in order) and publishes them
    if (wv == 0 && bj * kSplitBlock + lane * 4 < sp) {
      f32x4_t x = *reinterpret_cast<const f32x4_t*>(part + lane * 4);
      for (int v = 1; v < kSplitWaves; ++v) x += *reinterpret_cast<const f32x4_t*>(part + v * kSplitBlock + lane * 4);
      unsigned long long* cs = slot(buf, bj, bi, rsub) + lane * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) put_tagged(cs + e, x[e], tag);
    }
    if (j == 0) {
      const bool alive = split_barrier(cnt, static_cast<unsigned>(P), &dead, D.spin_limit);
      if (alive && p == 0 && tid == 0 && D.orth != nullptr) {
        double tot = 0.0;
        for (int i = 0; i < P; ++i) tot += gorth[i];
        D.orth[z] = static_cast<float>(sqrt(tot / s));
      }
      if (!alive || !want_sigma) {
        if (!alive && p == 0 && tid == 0) {
          if (D.orth != nullptr) D.orth[z] = NAN;
          if (D.smax != nullptr) D.smax[z] = NAN;
          if (D.smin != nullptr) D.smin[z] = NAN;
        }
        return;
      }
    }
    // w = H q: block b of w gathers the column sums of blocks (o, b), o <= b,
    // and the row sums of blocks (b, o), o > b.  First every word needed is
    // read into LDS (eight loads in flight per lane; a word whose tag is not
    // there yet is waited for), then each element adds its words in order of o.
    {
      // lane `pos` of each 256-thread group reads slots si = group, group +
      // groups, ... (b, o, rs advanced incrementally)
      unsigned long long* base = slot(buf, 0, 0, 0);
      const int pos = tid % kSplitBlock, step = nthr / kSplitBlock, nslot = nb * nb * R;
      int si = tid / kSplitBlock;
      int b = si / (nb * R), o = (si / R) % nb, rs = si % R;
      while (si < nslot) {
        unsigned long long v[8];
        int at[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int e = b * kSplitBlock + pos;
          const bool need = si < nslot && e < sp && (o <= b || (e < s && rs == pos / rpb[b]));
          at[t] = need ? si * kSplitBlock + pos : -1;
          v[t] = need ? __hip_atomic_load(base + at[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
          si += step;
          for (rs += step; rs >= R; rs -= R) {
            if (++o == nb) {
              o = 0;
              ++b;
            }
          }
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          if (at[t] >= 0)
            gat[at[t]] = static_cast<unsigned>(v[t] >> 32) == tag ? __uint_as_float(static_cast<unsigned>(v[t]))
                                                                  : wait_tagged(base + at[t], tag, &dead, D.spin_limit);
        }
      }
      __syncthreads();
    }
    // ... and, on the way, ||H q|| (the scale of a residual taken as zero)
    // and alpha = q . H q
    double hq2 = 0.0, qw = 0.0;
    for (int i = tid; i < sp; i += nthr) {
      const int b = i / kSplitBlock, pos = i % kSplitBlock;
      float x = 0.0f;
      for (int o = 0; o < nb; ++o) {
        const float* g = gat + static_cast<long long>(b * nb + o) * R * kSplitBlock + pos;
        if (o <= b) {
          for (int rs = 0; rs < R; ++rs) x += g[rs * kSplitBlock];
        } else if (i < s) {
          x += g[(pos / rpb[b]) * kSplitBlock];
        }
      }
      w[i] = x;
      hq2 += static_cast<double>(x) * x;
      qw += static_cast<double>(q[i]) * x;
    }
    if (dead != 0) {
      if (p == 0 && tid == 0) {
        if (D.smax != nullptr) D.smax[z] = NAN;
        if (D.smin != nullptr) D.smin[z] = NAN;
      }
      return;
    }
    split_sum2_d(hq2, qw, redd);  // its barriers also publish w
    const float hq = static_cast<float>(sqrt(hq2));
    const float alpha = static_cast<float>(qw);
    const float* qp = Qs + static_cast<long long>(j > 0 ? j - 1 : 0) * sp;
    // vector work four elements per lane (16-byte LDS accesses)
    const int n4 = sp / 4;
    for (int i4 = tid; i4 < n4; i4 += nthr) {
      f32x4_t v = *reinterpret_cast<const f32x4_t*>(w + 4 * i4);
      const f32x4_t qv = *reinterpret_cast<const f32x4_t*>(q + 4 * i4);
      const f32x4_t pv = *reinterpret_cast<const f32x4_t*>(qp + 4 * i4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = v[e] - alpha * qv[e];
        if (j > 0) v[e] -= beta * pv[e];
      }
      *reinterpret_cast<f32x4_t*>(w + 4 * i4) = v;
    }
    __syncthreads();
    // two passes of classical Gram-Schmidt against q_0 .. q_j
    double bn2 = 0.0;
    for (int pass = 0; pass < 2; ++pass) {
      for (int t = wv; t <= j; t += kSplitWaves) {
        const float* qt = Qs + static_cast<long long>(t) * sp;
        float d = 0.0f;
        for (int c = lane * 4; c < sp; c += 256) {
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(qt + c);
          const f32x4_t x = *reinterpret_cast<const f32x4_t*>(w + c);
          d = fmaf(v[0], x[0], fmaf(v[1], x[1], fmaf(v[2], x[2], fmaf(v[3], x[3], d))));
        }
        d = wave_total(d);
        if (lane == 0) cf[t] = d;
      }
      __syncthreads();
      // w -= sum_t cf[t] q_t, t ascending; four basis rows read together
      for (int i4 = tid; i4 < n4; i4 += nthr) {
        f32x4_t x = *reinterpret_cast<const f32x4_t*>(w + 4 * i4);
        const float* qb = Qs + 4 * i4;
        int t = 0;
        for (; t + 4 <= j + 1; t += 4) {
          const f32x4_t c = *reinterpret_cast<const f32x4_t*>(cf + t);
          f32x4_t qv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) qv[u] = *reinterpret_cast<const f32x4_t*>(qb + static_cast<long long>(t + u) * sp);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = fmaf(-c[u], qv[u][e], x[e]);
          }
        }
        for (; t <= j; ++t) {
          const float c = cf[t];
          const f32x4_t qv = *reinterpret_cast<const f32x4_t*>(qb + static_cast<long long>(t) * sp);
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = fmaf(-c, qv[e], x[e]);
        }
        *reinterpret_cast<f32x4_t*>(w + 4 * i4) = x;
        if (pass == 1) {
#pragma unroll
          for (int e = 0; e < 4; ++e) bn2 += static_cast<double>(x[e]) * x[e];
        }
      }
      if (pass == 0) __syncthreads();
    }
    bn2 = split_sum_d(bn2, redd);
    const float bn = static_cast<float>(sqrt(bn2));
    if (tid == 0) al[j] = alpha;
    // the run ends when the residual is rounding noise or not finite
    if (j + 1 == k || !(bn > kBreakdown * hq && bn < INFINITY)) {
      kk = j + 1;
      break;
    }
    if (tid == 0) be[j + 1] = bn;
    float* qn1 = Qs + static_cast<long long>(j + 1) * sp;
    for (int i4 = tid; i4 < n4; i4 += nthr) {
      const f32x4_t x = *reinterpret_cast<const f32x4_t*>(w + 4 * i4);
      f32x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = x[e] / bn;
      *reinterpret_cast<f32x4_t*>(qn1 + 4 * i4) = v;
    }
    beta = bn;
    __syncthreads();
  }
  __syncthreads();
  if (p == 0 && wv == 0) tridiag_extremes(al, be, kk, z, D);
}

}  // namespace

hipError_t launch_diag_pack(const DiagPackLaunch& P, hipStream_t st) {
  const long long blocks = P.count * (P.s_pad / kPackT) * (P.kdim / kPackT);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(diag_pack_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, P);
  return hipGetLastError();
}

namespace {
int lanczos_threads(int s_pad) { return s_pad <= 256 ? 256 : 1024; }
}  // namespace

size_t diag_lanczos_lds(int s_pad, int kmax) {
  const int splits = sym_matvec_splits(s_pad, lanczos_threads(s_pad) / 64);
  return ((3 + static_cast<size_t>(splits)) * s_pad + 3 * static_cast<size_t>(kmax)) * sizeof(float);
}

namespace {
size_t split_lds(int s_pad, int kmax, int nb, int r) {
  return (static_cast<size_t>(kmax + 1) * s_pad + kSplitWaves * kSplitBlock + 3 * static_cast<size_t>((kmax + 3) & ~3) +
          static_cast<size_t>(nb) * nb * r * kSplitBlock) *
         sizeof(float);
}

struct SplitDevice {
  int cus = 0, coop = 0, max_lds = 0;
  bool ok = false;
};

// Workgroups per matrix for the split run (0: run one workgroup per matrix).
// Only when the whole grid fits on the device at once (the cooperative launch
// guarantees residency), the basis fits in LDS, and the scratch fits in the
// matrix's basis region.
int plan_split(DiagLaunch& D, size_t* lds) {
  static SplitDevice devs[64];
  static std::mutex devs_mu;
  D.split_p = D.split_r = D.split_nb = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  SplitDevice sd;
  {
    std::lock_guard<std::mutex> lock(devs_mu);
    SplitDevice& cached = devs[dev];
    if (!cached.ok) {
      if (hipDeviceGetAttribute(&cached.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
          hipDeviceGetAttribute(&cached.coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess ||
          hipDeviceGetAttribute(&cached.max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
        return 0;
      cached.ok = true;
    }
    sd = cached;
  }
  const int k = D.iters < D.s ? D.iters : D.s;
  if (D.count <= 0 || !sd.coop || sd.cus <= 0 || k < 2) return 0;
  const int nb = (D.s_pad + kSplitBlock - 1) / kSplitBlock;
  const int units = nb * (nb + 1) / 2;
  const int rows0 = D.s < kSplitBlock ? D.s : kSplitBlock;
  long long r = (rows0 + 15) / 16;  // at least 16 rows per workgroup
  r = r < kSplitMaxR ? r : kSplitMaxR;
  // the most row ranges whose scratch fits the basis region, whose LDS fits,
  // and whose grid is resident at once
  for (; r >= 1; --r) {
    if (units * r < 2) return 0;
    if (split_scratch_floats(static_cast<int>(units * r), static_cast<int>(r), nb) >
        static_cast<long long>(D.kmax) * D.s_pad)
      continue;
    *lds = split_lds(D.s_pad, D.kmax, nb, static_cast<int>(r));
    if (*lds > static_cast<size_t>(sd.max_lds)) continue;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(diag_lanczos_split_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(*lds)) != hipSuccess)
      return 0;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(diag_lanczos_split_kernel), kSplitThreads, *lds) != hipSuccess)
      return 0;
    if (D.count * units * r <= static_cast<long long>(per_cu) * sd.cus) break;
  }
  if (r < 1) return 0;
  D.split_nb = nb;
  D.split_r = static_cast<int>(r);
  D.split_p = static_cast<int>(units * r);
  return D.split_p;
}

}  // namespace

long long diag_split_clear_words(DiagLaunch& D) {
  size_t lds = 0;
  if (plan_split(D, &lds) == 0) return 0;
  return split_scratch_floats(D.split_p, D.split_r, D.split_nb);
}

hipError_t launch_diag_lanczos(const DiagLaunch& D0, hipStream_t st) {
  if (D0.count == 0) return hipSuccess;
  DiagLaunch D = D0;
  // debug hook for tests only: MUON_DEBUG_DIAG_SPIN_LIMIT shortens the split
  // run's bounded waits so that their give-up path (NaN outputs, every wave
  // ends) can be exercised; it can only lower the bound
  D.spin_limit = kSpinLimit;
  if (const char* e = std::getenv("MUON_DEBUG_DIAG_SPIN_LIMIT")) {
    char* end = nullptr;
    const unsigned long v = std::strtoul(e, &end, 10);
    if (end != e && v < kSpinLimit) D.spin_limit = static_cast<unsigned>(v);
  }
  size_t lds = 0;
  if (plan_split(D, &lds) > 0) {
    void* args[] = {&D};
    if (hipLaunchCooperativeKernel(reinterpret_cast<const void*>(diag_lanczos_split_kernel),
                                   dim3(static_cast<unsigned>(D.count * D.split_p)), dim3(kSplitThreads), args,
                                   static_cast<unsigned>(lds), st) == hipSuccess)
      return hipSuccess;
    (void)hipGetLastError();  // refused (e.g. the grid cannot be resident now): one workgroup per matrix
  }
  hipLaunchKernelGGL(diag_lanczos_kernel, dim3(static_cast<unsigned>(D.count)), dim3(lanczos_threads(D.s_pad)),
                     diag_lanczos_lds(D.s_pad, D.kmax), st, D);
  return hipGetLastError();
}

}  // namespace muon
