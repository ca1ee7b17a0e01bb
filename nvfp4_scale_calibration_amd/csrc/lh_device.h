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

// p[0] + p[stride] + ... + p[(n-1) stride], added in slice order; eight
// loads are issued ahead of their adds.
__device__ __forceinline__ float sum_slices(const float* __restrict__ p, int64_t stride, int64_t n) {
  float v = p[0];
  int64_t s = 1;
  for (; s + 8 <= n; s += 8) {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = p[(s + i) * stride];
#pragma unroll
    for (int i = 0; i < 8; ++i) v += t[i];
  }
  for (; s < n; ++s) v += p[s * stride];
  return v;
}

// Largest |w| bit pattern among the 16 bytes u (eight bf16 or four fp32):
// |w| as fp32 bits is monotone in |w|, so the maximum is an unsigned max.
__device__ __forceinline__ uint32_t absbits_max(uint32_t m, const uint4 u, bool bf16) {
  const uint32_t v[4] = {u.x, u.y, u.z, u.w};
  if (bf16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, max((v[i] << 16) & 0x7FFF0000u, v[i] & 0x7FFF0000u));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, v[i] & 0x7FFFFFFFu);
  }
  return m;
}

// Workgroup share `chunk` of `per_group` of a flat array of n16 16-byte
// vectors: the largest |w| bits it holds (grid-stride, four loads in
// flight per thread), reduced over the kT-thread workgroup; valid in thread 0.
template <bool kBf16, int kT = kThreads>
__device__ __forceinline__ uint32_t absmax_flat_share(const uint4* __restrict__ v, int64_t n16, int64_t chunk,
                                                      int64_t per_group) {
  __shared__ uint32_t part[kT / 64];
  uint32_t m = 0;
  const int64_t stride = per_group * kT;
  int64_t i = chunk * kT + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = v[i], b = v[i + stride], c = v[i + 2 * stride], d = v[i + 3 * stride];
    m = absbits_max(m, a, kBf16);
    m = absbits_max(m, b, kBf16);
    m = absbits_max(m, c, kBf16);
    m = absbits_max(m, d, kBf16);
  }
  for (; i < n16; i += stride) m = absbits_max(m, v[i], kBf16);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t t = part[0];
#pragma unroll
  for (int k = 1; k < kT / 64; ++k) t = max(t, part[k]);
  return t;
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// NVFP4 cast of one 16-weight block with block scale s ("Algorithm
// principle": Q(W, s) = Cast(W / s) * s).  x = fl32(w / s) by IEEE division
// (0 when s == 0); v_cvt_scalef32_pk_fp4_f32 with scale 1 rounds pairs of x
// to signed E2M1 nibbles (nearest, ties to even, saturating at 6), packed
// low nibble first into the bytes of pk[0] (weights 0-7) and pk[1] (8-15);
// a sign on a zero magnitude is cleared, so -0 is written as +0.
__device__ __forceinline__ void nvfp4_cast_block(const float (&w)[16], float s, uint32_t (&pk)[2]) {
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = (s == 0.0f) ? 0.0f : w[i] / s;  // IEEE division
  pk[0] = pk[1] = 0u;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    pk[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[h], x[8 * h + 0], x[8 * h + 1], 1.0f, 0);
    pk[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[h], x[8 * h + 2], x[8 * h + 3], 1.0f, 1);
    pk[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[h], x[8 * h + 4], x[8 * h + 5], 1.0f, 2);
    pk[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[h], x[8 * h + 6], x[8 * h + 7], 1.0f, 3);
    // keep the sign bit (bit 3 of a nibble) only where the magnitude is non-zero
    const uint32_t nz = (pk[h] | (pk[h] >> 1) | (pk[h] >> 2)) & 0x11111111u;
    pk[h] &= 0x77777777u | (nz << 3);
  }
}

// Dequantised block: v_cvt_scalef32_pk_f32_fp4 (scale 1) decodes the signed
// grid values r and Q = fl32(r * s).
__device__ __forceinline__ void nvfp4_decode_block(const uint32_t (&pk)[2], float s, float (&q)[16]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const f32x2_t r0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], 1.0f, 0);
    const f32x2_t r1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], 1.0f, 1);
    const f32x2_t r2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], 1.0f, 2);
    const f32x2_t r3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], 1.0f, 3);
    q[8 * h + 0] = r0.x * s; q[8 * h + 1] = r0.y * s; q[8 * h + 2] = r1.x * s; q[8 * h + 3] = r1.y * s;
    q[8 * h + 4] = r2.x * s; q[8 * h + 5] = r2.y * s; q[8 * h + 6] = r3.x * s; q[8 * h + 7] = r3.y * s;
  }
}

// The per-block outputs of the fake-quant for the block with index o in a
// dense [rows][nb] layout (o = row * nb + b) from its nibbles, each optional:
// 16 fp32 Q = fl32(r * s) values, 8 bytes of nibbles, the E4M3 code k + 1.
// kAll: every output pointer is known to be non-null.
template <bool kAll = false>
__device__ __forceinline__ void nvfp4_emit_at(const uint32_t (&pk)[2], float s, int k, int64_t o,
                                              float* __restrict__ wq, uint8_t* __restrict__ packed,
                                              uint8_t* __restrict__ codes) {
  if (kAll || wq) {
    float q[16];
    nvfp4_decode_block(pk, s, q);
    float4* d = reinterpret_cast<float4*>(wq + 16 * o);
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) d[qd] = make_float4(q[4 * qd], q[4 * qd + 1], q[4 * qd + 2], q[4 * qd + 3]);
  }
  if (kAll || packed) *reinterpret_cast<uint2*>(packed + 8 * o) = make_uint2(pk[0], pk[1]);
  if (kAll || codes) codes[o] = (uint8_t)(k + 1);
}

// Same, for block (row rg, input block b).
__device__ __forceinline__ void nvfp4_emit_block(const uint32_t (&pk)[2], float s, int k, int64_t rg, int64_t b,
                                                 int64_t nb, float* __restrict__ wq, uint8_t* __restrict__ packed,
                                                 uint8_t* __restrict__ codes) {
  nvfp4_emit_at(pk, s, k, rg * nb + b, wq, packed, codes);
}

}  // namespace lh
