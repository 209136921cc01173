// Spectral cap of the Muon update ("An Isotropy-Preserving Spectral Cap for
// Muon"): the update loses the component that would grow the weight's top
// singular value to first order, and the top singular pair is tracked from
// step to step by one power step on the new weight.
//
// With the current estimates u (m), v (n) of W's top singular vectors and
// sigma of its top singular value, and W' = W - lr * scale * O:
//   c = u^T O v;   gamma = c if sigma >= cap and c < 0, else 0;
//   W' = W - lr * scale * (O - gamma u v^T)        (in the apply pass);
//   u <- W' v / ||W' v||,  v <- W'^T u / ||W'^T u||,  sigma <- ||W' v||.
// All passes are deterministic (fixed-order partial sums, no atomics):
//   cap_coef_kernel         per-block partials of u^T O v over the oriented
//                           final iterate X (O = X, or X^T for tall matrices);
//   power_partials_kernel   one read of W': W' v complete per 32-row block
//                           (lane shares kept in registers, one wave sum per
//                           row), partials of W'^T u over those rows, norm
//                           partials;
//   power_zsum_kernel       W'^T u from its partials;
//   power_normalize_kernel  writes u, v, sigma.
#include "common.cuh"
#include "launch.h"

namespace muon {
namespace {

template <typename XT> __device__ __forceinline__ float ldx(const XT* p);
template <> __device__ __forceinline__ float ldx<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ldx<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

// c partial over rows [16 chunk, 16 chunk + 16) of X (s x l, row stride ld):
// sum_r a_r sum_k X[r][k] b_k with (a, b) = (u, v) for wide, (v, u) for tall.
// One wave per row at a time, 8 elements per lane per load when the row and b
// allow it.
template <typename XT>
__global__ void __launch_bounds__(256) cap_coef_kernel(CapCoefLaunch L) {
  __shared__ float red[8];
  const int z = blockIdx.y;
  const XT* x = static_cast<const XT*>(L.X) + z * L.xstride;
  const float* a = static_cast<const float*>(L.tall ? L.v.p[z] : L.u.p[z]);
  const float* b = static_cast<const float*>(L.tall ? L.u.p[z] : L.v.p[z]);
  const int r0 = blockIdx.x * 16;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool vec = (L.l % 8) == 0 && (L.ld % 8) == 0 && ((reinterpret_cast<uintptr_t>(b) & 15u) == 0);
  float acc = 0.0f;
  for (int rr = 0; rr < 4; ++rr) {
    const int r = r0 + wave * 4 + rr;
    if (r >= L.s) break;
    const XT* row = x + static_cast<long long>(r) * L.ld;
    float d = 0.0f;
    if (vec) {
      for (int k = lane * 8; k < L.l; k += 64 * 8) {
        float xv[8];
        if constexpr (sizeof(XT) == 2) {
          const u32x4_t w = *reinterpret_cast<const u32x4_t*>(row + k);
#pragma unroll
          for (int h = 0; h < 4; ++h) { xv[2 * h] = lo_bf16(w[h]); xv[2 * h + 1] = hi_bf16(w[h]); }
        } else {
          const f32x4_t p = *reinterpret_cast<const f32x4_t*>(row + k);
          const f32x4_t q = *reinterpret_cast<const f32x4_t*>(row + k + 4);
#pragma unroll
          for (int h = 0; h < 4; ++h) { xv[h] = p[h]; xv[4 + h] = q[h]; }
        }
        const f32x4_t b0 = *reinterpret_cast<const f32x4_t*>(b + k);
        const f32x4_t b1 = *reinterpret_cast<const f32x4_t*>(b + k + 4);
#pragma unroll
        for (int h = 0; h < 4; ++h) d = fmaf(xv[h], b0[h], fmaf(xv[4 + h], b1[h], d));
      }
    } else {
      for (int k = lane; k < L.l; k += 64) d = fmaf(ldx<XT>(row + k), b[k], d);
    }
    acc = fmaf(a[r], d, acc);
  }
  acc = block_sum(acc, red);
  if (threadIdx.x == 0) L.part[static_cast<long long>(z) * L.P + blockIdx.x] = acc;
}

// One read of W (m x n fp32) for both products of the power step.  A block
// owns 32 full rows: each lane keeps its share of y_r = (W v)_r for the 32
// rows in registers across the columns it reads, and each row is summed over
// the wave once at the end (DPP), the four waves in order; y_r is written with
// its square to the per-block norm partial.  (W^T u)_j gets a partial over the
// 32 rows.
constexpr int kPowRows = 32;
__global__ void __launch_bounds__(256) power_partials_kernel(PowerLaunch L) {
  __shared__ float yw[4][kPowRows];
  const int z = blockIdx.y;
  const float* w = static_cast<const float*>(L.W.p[z]);
  const float* u = static_cast<const float*>(L.u.p[z]);
  const float* v = static_cast<const float*>(L.v.p[z]);
  const int r0 = blockIdx.x * kPowRows;
  const int rows = L.m - r0 < kPowRows ? L.m - r0 : kPowRows;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool vec = (L.n % 4) == 0 && ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(v)) & 15u) == 0;
  float* zp = L.zpart + (static_cast<long long>(z) * L.nrc + blockIdx.x) * L.n;
  float yacc[kPowRows];
#pragma unroll
  for (int i = 0; i < kPowRows; ++i) yacc[i] = 0.0f;
  if (vec) {
    const int groups = L.n / 4;
    for (int g = threadIdx.x; g < groups; g += 256) {  // four columns per thread and pass
      const f32x4_t vg = *reinterpret_cast<const f32x4_t*>(v + 4 * g);
      f32x4_t zg = {0, 0, 0, 0};
#pragma unroll 8
      for (int i = 0; i < kPowRows; ++i) {
        if (i < rows) {
          const float ur = u[r0 + i];
          const f32x4_t x = *reinterpret_cast<const f32x4_t*>(w + static_cast<long long>(r0 + i) * L.n + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            zg[e] = fmaf(x[e], ur, zg[e]);
            yacc[i] = fmaf(x[e], vg[e], yacc[i]);
          }
        }
      }
      *reinterpret_cast<f32x4_t*>(zp + 4 * g) = zg;
    }
  } else {
    for (int c = threadIdx.x; c < L.n; c += 256) {
      const float vc = v[c];
      float zc = 0.0f;
#pragma unroll 8
      for (int i = 0; i < kPowRows; ++i) {
        if (i < rows) {
          const float x = w[static_cast<long long>(r0 + i) * L.n + c];
          zc = fmaf(x, u[r0 + i], zc);
          yacc[i] = fmaf(x, vc, yacc[i]);
        }
      }
      zp[c] = zc;
    }
  }
#pragma unroll
  for (int i = 0; i < kPowRows; ++i) {
    const float y = wave_total(yacc[i]);
    if (lane == 0) yw[wave][i] = y;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int i = threadIdx.x;
    float y = 0.0f;
    if (i < rows) {
      y = ((yw[0][i] + yw[1][i]) + yw[2][i]) + yw[3][i];
      L.ybuf[static_cast<long long>(z) * L.m + r0 + i] = y;
    }
    const float yy = wave_sum(y * y);
    if (threadIdx.x == 0) L.ynorm[static_cast<long long>(z) * L.nrc + blockIdx.x] = yy;
  }
}

// z_j = sum over the row blocks of the partials: each of the four waves adds
// a quarter of the row blocks for the block's 64 columns, and the quarters
// are added in order (fixed order throughout); per-block partial sums of z_j^2.
constexpr int kZCols = 64;
__global__ void __launch_bounds__(256) power_zsum_kernel(PowerLaunch L) {
  __shared__ float part[4][kZCols];
  __shared__ float red[8];
  const int z = blockIdx.y;
  const int cl = threadIdx.x & (kZCols - 1), q = threadIdx.x >> 6;
  const int j = blockIdx.x * kZCols + cl;
  const int per = (L.nrc + 3) / 4;
  const int k0 = q * per, k1 = k0 + per < L.nrc ? k0 + per : L.nrc;
  float t = 0.0f;
  if (j < L.n) {
    const float* zp = L.zpart + static_cast<long long>(z) * L.nrc * L.n + j;
    for (int k = k0; k < k1; ++k) t += zp[static_cast<long long>(k) * L.n];
  }
  part[q][cl] = t;
  __syncthreads();
  float tt = 0.0f;
  if (q == 0 && j < L.n) {
    const float zj = ((part[0][cl] + part[1][cl]) + part[2][cl]) + part[3][cl];
    L.zbuf[static_cast<long long>(z) * L.n + j] = zj;
    tt = zj * zj;
  }
  tt = block_sum(tt, red);
  if (threadIdx.x == 0) L.znorm[static_cast<long long>(z) * L.ncb + blockIdx.x] = tt;
}

// u = y / ||y||, v = z / ||z||, sigma = ||y|| (a zero vector keeps u or v);
// every block re-reduces the small norm partials in the same order.
__global__ void __launch_bounds__(256) power_normalize_kernel(PowerLaunch L) {
  __shared__ float red[8];
  const int z = blockIdx.y;
  float a = 0.0f, b = 0.0f;
  for (int k = threadIdx.x; k < L.nrc; k += 256) a += L.ynorm[static_cast<long long>(z) * L.nrc + k];
  for (int k = threadIdx.x; k < L.ncb; k += 256) b += L.znorm[static_cast<long long>(z) * L.ncb + k];
  const float ny = sqrtf(block_sum(a, red));
  const float nz = sqrtf(block_sum(b, red));
  float* u = static_cast<float*>(L.u.p[z]);
  float* v = static_cast<float*>(L.v.p[z]);
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (ny > 0.0f && t < L.m) u[t] = L.ybuf[static_cast<long long>(z) * L.m + t] / ny;
  if (nz > 0.0f && t < L.n) v[t] = L.zbuf[static_cast<long long>(z) * L.n + t] / nz;
  if (blockIdx.x == 0 && threadIdx.x == 0) L.sigma[z] = ny;
}

}  // namespace

int cap_coef_blocks(int s) { return (s + 15) / 16; }
int power_row_blocks(int m) { return (m + kPowRows - 1) / kPowRows; }
int power_col_blocks(int n) { return (n + kZCols - 1) / kZCols; }

hipError_t launch_cap_coef(const CapCoefLaunch& L, bool x_bf16, hipStream_t st) {
  const dim3 grid(cap_coef_blocks(L.s), L.count);
  if (x_bf16) hipLaunchKernelGGL(cap_coef_kernel<bf16_t>, grid, dim3(256), 0, st, L);
  else hipLaunchKernelGGL(cap_coef_kernel<float>, grid, dim3(256), 0, st, L);
  return hipGetLastError();
}

hipError_t launch_power_step(const PowerLaunch& L, hipStream_t st) {
  hipLaunchKernelGGL(power_partials_kernel, dim3(L.nrc, L.count), dim3(256), 0, st, L);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(power_zsum_kernel, dim3(L.ncb, L.count), dim3(256), 0, st, L);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int span = L.m > L.n ? L.m : L.n;
  hipLaunchKernelGGL(power_normalize_kernel, dim3((span + 255) / 256, L.count), dim3(256), 0, st, L);
  return hipGetLastError();
}

}  // namespace muon
