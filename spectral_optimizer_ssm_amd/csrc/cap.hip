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
//   power_partials_kernel   one read of W': W' v complete per 32-row block,
//                           partials of W'^T u over those rows, norm partials;
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
// owns 32 full rows: y_r = (W v)_r is complete within it (lane partials, wave
// butterflies, the four waves summed in order), written with its square to
// the per-block norm partial; (W^T u)_j gets a partial over the 32 rows.
constexpr int kPowRows = 32;
__global__ void __launch_bounds__(256) power_partials_kernel(PowerLaunch L) {
  __shared__ float yw[4][kPowRows];
  const int z = blockIdx.y;
  const float* w = static_cast<const float*>(L.W.p[z]);
  const float* u = static_cast<const float*>(L.u.p[z]);
  const float* v = static_cast<const float*>(L.v.p[z]);
  const int r0 = blockIdx.x * kPowRows;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool vec = (L.n % 4) == 0 && ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(v)) & 15u) == 0;
  float* zp = L.zpart + (static_cast<long long>(z) * L.nrc + blockIdx.x) * L.n;
  if (vec) {
    const int groups = L.n / 4;
    // column groups of this thread: g = threadIdx.x + 256 k (at most 8: n <= 8192)
    for (int g0 = 0; g0 < groups; g0 += 256 * 2) {
      const int ga = g0 + threadIdx.x, gb = ga + 256;
      const bool ina = ga < groups, inb = gb < groups;
      const f32x4_t va = ina ? *reinterpret_cast<const f32x4_t*>(v + 4 * ga) : f32x4_t{0, 0, 0, 0};
      const f32x4_t vb = inb ? *reinterpret_cast<const f32x4_t*>(v + 4 * gb) : f32x4_t{0, 0, 0, 0};
      f32x4_t za = {0, 0, 0, 0}, zb = {0, 0, 0, 0};
      for (int i = 0; i < kPowRows; ++i) {
        const int r = r0 + i;
        float yp = 0.0f;
        if (r < L.m) {
          const float ur = u[r];
          const float* row = w + static_cast<long long>(r) * L.n;
          if (ina) {
            const f32x4_t x = *reinterpret_cast<const f32x4_t*>(row + 4 * ga);
#pragma unroll
            for (int e = 0; e < 4; ++e) { za[e] = fmaf(x[e], ur, za[e]); yp = fmaf(x[e], va[e], yp); }
          }
          if (inb) {
            const f32x4_t x = *reinterpret_cast<const f32x4_t*>(row + 4 * gb);
#pragma unroll
            for (int e = 0; e < 4; ++e) { zb[e] = fmaf(x[e], ur, zb[e]); yp = fmaf(x[e], vb[e], yp); }
          }
        }
        yp = wave_sum(yp);
        if (lane == 0) yw[wave][i] = (g0 == 0 ? 0.0f : yw[wave][i]) + yp;
      }
      if (ina) *reinterpret_cast<f32x4_t*>(zp + 4 * ga) = za;
      if (inb) *reinterpret_cast<f32x4_t*>(zp + 4 * gb) = zb;
    }
  } else {
    for (int c0 = 0; c0 < L.n; c0 += 256) {
      const int c = c0 + threadIdx.x;
      const bool in = c < L.n;
      const float vc = in ? v[c] : 0.0f;
      float zc = 0.0f;
      for (int i = 0; i < kPowRows; ++i) {
        const int r = r0 + i;
        float yp = 0.0f;
        if (r < L.m && in) {
          const float x = w[static_cast<long long>(r) * L.n + c];
          zc = fmaf(x, u[r], zc);
          yp = x * vc;
        }
        yp = wave_sum(yp);
        if (lane == 0) yw[wave][i] = (c0 == 0 ? 0.0f : yw[wave][i]) + yp;
      }
      if (in) zp[c] = zc;
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int i = threadIdx.x;
    float y = 0.0f;
    if (i < kPowRows) {
      y = ((yw[0][i] + yw[1][i]) + yw[2][i]) + yw[3][i];
      if (r0 + i < L.m) L.ybuf[static_cast<long long>(z) * L.m + r0 + i] = y;
      else y = 0.0f;
    }
    const float yy = wave_sum(y * y);
    if (threadIdx.x == 0) L.ynorm[static_cast<long long>(z) * L.nrc + blockIdx.x] = yy;
  }
}

// z_j = sum over the row blocks of the partials (fixed order), and per-block
// partial sums of z_j^2.
__global__ void __launch_bounds__(256) power_zsum_kernel(PowerLaunch L) {
  __shared__ float red[8];
  const int z = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  float t = 0.0f;
  if (j < L.n) {
    const float* zp = L.zpart + static_cast<long long>(z) * L.nrc * L.n + j;
    for (int k = 0; k < L.nrc; ++k) t += zp[static_cast<long long>(k) * L.n];
    L.zbuf[static_cast<long long>(z) * L.n + j] = t;
  }
  const float tt = block_sum(t * t, red);
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
int power_col_blocks(int n) { return (n + 255) / 256; }

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
