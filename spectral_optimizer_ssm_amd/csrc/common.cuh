// Device helpers shared by the libmuon kernels (gfx950 / CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace muon {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kMaxTable = 64;      // matrices per launch in a pointer table

typedef uint16_t bf16_t;           // bfloat16 storage (raw bits)
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

// Per-launch tables of user pointers (kernel arguments, no device copies).
struct PtrTable {
  const void* p[kMaxTable];
};
struct MutPtrTable {
  void* p[kMaxTable];
};

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Two floats -> two bfloat16 packed in one dword (hardware RNE convert).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ bf16_t f32_to_bf16(float x) {
  return static_cast<bf16_t>(pack_bf16x2(x, 0.0f) & 0xFFFFu);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Deterministic wavefront sum (butterfly over 64 lanes).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Cross-lane moves on the DPP path (no LDS round trip).  Lanes whose source
// falls outside the row read 0.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned>(lo));
}
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118, kDppShl4 = 0x104;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143, kDppRor8 = 0x128, kDppXor1 = 0xB1, kDppXor2 = 0x4E;

// Wave totals: inclusive scans within each 16-lane row, then the rows are
// carried into lane 63, whose value every lane reads (fixed order).
__device__ __forceinline__ float wave_total(float v) {
  v += dpp_f<kDppShr1>(v);
  v += dpp_f<kDppShr2>(v);
  v += dpp_f<kDppShr4>(v);
  v += dpp_f<kDppShr8>(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppBcast15, 0xa, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppBcast31, 0xc, 0xf, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// Deterministic block sum; every thread gets the result.  `red` holds at
// least blockDim.x / 64 floats of LDS.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int nw = (blockDim.x + kWave - 1) / kWave;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float t = 0.0f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// 1 / (||U||_F + eps) from the per-block partial sums of squares written by
// the momentum pass; optionally returns nu = ||U||_F.
__device__ __forceinline__ float inv_norm_from_partials(const float* part, int nparts, float eps,
                                                        float* red, float* nu_out) {
  float s = 0.0f;
  for (int i = threadIdx.x; i < nparts; i += blockDim.x) s += part[i];
  s = block_sum(s, red);
  const float nu = sqrtf(s);
  if (nu_out) *nu_out = nu;
  return 1.0f / (nu + eps);
}

// Compute units of the current device, cached per device (relaxed atomics:
// concurrent first calls store the same value); 256 if the query fails.
inline int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

}  // namespace muon
