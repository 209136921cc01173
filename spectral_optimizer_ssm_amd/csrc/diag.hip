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
//                        pieces x = h + d + e and the operand rows carry the six
//                        products that matter, h h + h d + d h + d d + h e + e h,
//                        as L = [h h d d h e], R = [h d h d e h]
//   symprod (float32 output) H = L R^T on the matrix cores
//   diag_lanczos_kernel  one workgroup per matrix: ||H - I|| in float64, then
//                        the Lanczos run in float32 with its vectors in LDS and
//                        the basis in global memory, and the extreme eigenvalues
//                        of the tridiagonal matrix by float64 multisection.
// Every reduction runs in a fixed order: results are deterministic.
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
      P.L[o] = h;         P.R[o] = h;
      P.L[o + K] = h;     P.R[o + K] = d;
      P.L[o + 2 * K] = d; P.R[o + 2 * K] = h;
      P.L[o + 3 * K] = d; P.R[o + 3 * K] = d;
      P.L[o + 4 * K] = h; P.R[o + 4 * K] = e;
      P.L[o + 5 * K] = e; P.R[o + 5 * K] = h;
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
  extern __shared__ float sh[];
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
      for (int i = tid; i < sp; i += nthr) {
        float x = w[i];
        for (int t = 0; t <= j; ++t) x = fmaf(-cf[t], Q[static_cast<long long>(t) * sp + i], x);
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

  if (wv == 0) {
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

hipError_t launch_diag_lanczos(const DiagLaunch& D, hipStream_t st) {
  if (D.count == 0) return hipSuccess;
  hipLaunchKernelGGL(diag_lanczos_kernel, dim3(static_cast<unsigned>(D.count)), dim3(lanczos_threads(D.s_pad)),
                     diag_lanczos_lds(D.s_pad, D.kmax), st, D);
  return hipGetLastError();
}

}  // namespace muon
