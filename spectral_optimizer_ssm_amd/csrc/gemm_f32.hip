// Newton-Schulz products in float32 (the MUON_F32 precision for matrices too
// large for the on-chip kernel).  Same step as the bf16 path ("Muon Meets
// Mamba", abstract; cubic step A = X X^T, X' = a X + b A X) with the same
// padded layout (X [count][s_pad][ld], A [count][s_pad][s_pad], s_pad and ld
// multiples of 64) and the same step-1 normalisation folded into the
// epilogues.  Classic LDS-tiled FMA kernels: 64 x 64 tiles, BK = 16, 256
// threads each owning a 4 x 4 block of outputs.
#include "common.cuh"
#include "launch.h"

namespace muon {
namespace {

constexpr int T = 64, BKF = 16;

__device__ __forceinline__ float f32_inv(const NsGemmLaunch& L, int z, float* red) {
  if (L.partials == nullptr) return 1.0f;
  return inv_norm_from_partials(L.partials + static_cast<long long>(z) * L.P, L.P, L.eps, red, nullptr);
}

// A = X X^T (all tiles).
__global__ void __launch_bounds__(256) gram_f32_kernel(NsGemmLaunch L) {
  __shared__ float sa[BKF][T + 4], sb[BKF][T + 4];
  __shared__ float red[4];
  const int z = blockIdx.z;
  const float* X = static_cast<const float*>(L.X) + z * L.xstride;
  float* A = static_cast<float*>(L.A) + z * L.astride;
  const float inv = f32_inv(L, z, red);
  const int i0 = blockIdx.y * T, j0 = blockIdx.x * T;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4] = {};
  // loader: 64 rows x 16 k = 1024 values per operand, 4 per thread
  const int lr = threadIdx.x / 4, lk = (threadIdx.x % 4) * 4;
  for (int k0 = 0; k0 < L.ld; k0 += BKF) {
    const f32x4_t va = *reinterpret_cast<const f32x4_t*>(X + static_cast<long long>(i0 + lr) * L.ld + k0 + lk);
    const f32x4_t vb = *reinterpret_cast<const f32x4_t*>(X + static_cast<long long>(j0 + lr) * L.ld + k0 + lk);
#pragma unroll
    for (int q = 0; q < 4; ++q) { sa[lk + q][lr] = va[q]; sb[lk + q][lr] = vb[q]; }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BKF; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) { a[q] = sa[k][ty * 4 + q]; b[q] = sb[k][tx * 4 + q]; }
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[p][q] = fmaf(a[p], b[q], acc[p][q]);
    }
    __syncthreads();
  }
  const float sc = inv * inv;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    f32x4_t v = {acc[p][0] * sc, acc[p][1] * sc, acc[p][2] * sc, acc[p][3] * sc};
    *reinterpret_cast<f32x4_t*>(A + static_cast<long long>(i0 + ty * 4 + p) * L.s_pad + j0 + tx * 4) = v;
  }
}

// Y = alpha X + beta A X.
__global__ void __launch_bounds__(256) combine_f32_kernel(NsGemmLaunch L) {
  __shared__ float sa[BKF][T + 4], sx[BKF][T + 4];
  __shared__ float red[4];
  const int z = blockIdx.z;
  const float* X = static_cast<const float*>(L.X) + z * L.xstride;
  float* Y = static_cast<float*>(L.Y) + z * L.xstride;
  const float* A = static_cast<const float*>(L.A) + z * L.astride;
  const float inv = f32_inv(L, z, red);
  const float alpha = L.alpha * inv, beta = L.beta * inv;
  const int i0 = blockIdx.y * T, k0 = blockIdx.x * T;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4] = {};
  const int lr = threadIdx.x / 4, lc = (threadIdx.x % 4) * 4;   // A rows i, 4 j's
  const int xr = threadIdx.x / 16, xc = (threadIdx.x % 16) * 4;  // X rows j, 4 k's
  for (int j0 = 0; j0 < L.s_pad; j0 += BKF) {
    const f32x4_t va = *reinterpret_cast<const f32x4_t*>(A + static_cast<long long>(i0 + lr) * L.s_pad + j0 + lc);
#pragma unroll
    for (int q = 0; q < 4; ++q) sa[lc + q][lr] = va[q];
    const f32x4_t vx = *reinterpret_cast<const f32x4_t*>(X + static_cast<long long>(j0 + xr) * L.ld + k0 + xc);
#pragma unroll
    for (int q = 0; q < 4; ++q) sx[xr][xc + q] = vx[q];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < BKF; ++j) {
      float a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) { a[q] = sa[j][ty * 4 + q]; b[q] = sx[j][tx * 4 + q]; }
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[p][q] = fmaf(a[p], b[q], acc[p][q]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const long long off = static_cast<long long>(i0 + ty * 4 + p) * L.ld + k0 + tx * 4;
    const f32x4_t xv = *reinterpret_cast<const f32x4_t*>(X + off);
    f32x4_t v;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = fmaf(alpha, xv[q], beta * acc[p][q]);
    *reinterpret_cast<f32x4_t*>(Y + off) = v;
  }
}

}  // namespace

hipError_t launch_gram_f32(const NsGemmLaunch& L, hipStream_t st) {
  const dim3 grid(L.s_pad / T, L.s_pad / T, L.count);
  hipLaunchKernelGGL(gram_f32_kernel, grid, dim3(256), 0, st, L);
  return hipGetLastError();
}

hipError_t launch_combine_f32(const NsGemmLaunch& L, hipStream_t st) {
  const dim3 grid(L.ld / T, L.s_pad / T, L.count);
  hipLaunchKernelGGL(combine_f32_kernel, grid, dim3(256), 0, st, L);
  return hipGetLastError();
}

}  // namespace muon
