// lh_device.h - device-side helpers shared by the HIP kernels of liblh.
//
// NVFP4 format facts ("Local-Hessian weight-scale guide", xxmr.cn/news/266017,
// "What is Local-Hessian"): 16 weights share one FP8 E4M3 block scale; the
// elements are FP4 E2M1 values in [-6, 6].  The sweep tries the 126 positive
// finite E4M3 values ("Algorithm principle").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lh {

// Workgroup size of every kernel here: 4 wave64s.
constexpr int kThreads = 256;

// One 16-element NVFP4 block.
constexpr int kBlock = 16;

// Positive finite OCP E4M3FN values: codes 0x01..0x7E, candidate k <-> code k+1.
constexpr int kCandidates = 126;

// fp32 IEEE divisor of the global amax: S_g = g / (E2M1 max * E4M3 max).
constexpr float kAmaxDivisor = 2688.0f;  // 6 * 448

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}

// E4M3 value of candidate k (code k+1): exponent field E = code >> 3,
// mantissa m = code & 7; E == 0 is subnormal m * 2^-9, else (8+m) * 2^(E-10).
// Exact in fp32.
__host__ __device__ __forceinline__ float e4m3_candidate(int k) {
  const int code = k + 1;
  const int E = code >> 3, m = code & 7;
  return E == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), E - 10);
}

// Round a non-negative fp32 quotient x to the E2M1 magnitude grid
// {0, .5, 1, 1.5, 2, 3, 4, 6}: nearest value, ties to the even code, values
// beyond 6 saturate.  Clamp to 6, then add and subtract 1.5 * 2^(22+e) whose
// ulp equals the grid step at x (0.5 below 2, 1 below 4, 2 from 4), so the
// fp32 round-to-nearest-even of the sum lands on the nearest grid point and
// resolves ties to the even multiple of the step, which is the even code.
__device__ __forceinline__ float e2m1_round_mag(float x) {
  const float xc = fminf(x, 6.0f);
  uint32_t e = __float_as_uint(xc) >> 23;  // biased exponent (sign is 0)
  e = e < 127u ? 127u : e;                 // step 0.5 below 1 as well
  const float magic = __uint_as_float((e << 23) + 0x0B400000u);  // 1.5 * 2^(e-127+22)
  return (xc + magic) - magic;
}

}  // namespace lh
