// lh_sweep.hip - Local-Hessian 126-candidate FP8 block-scale sweep.
//
// "Local-Hessian weight-scale guide" (xxmr.cn/news/266017):
//   "What is Local-Hessian": every 16 weights share one FP8 E4M3 block
//     scale; the sweep covers all 126 positive non-zero FP8 values.
//   "Algorithm principle": Q(W, s) = Cast(W / s) * s, dw = Q - w, block error
//     E_b(s) = dw^T (X_b X_b^T) dw; blocks are independent, so one kernel
//     sweeps a whole layer; inputs are the weight blocks in (cout, cin//16)
//     order, the global FP32 amax and the per-block Hessians [cin//16,16,16];
//     output is the per-block best amax; candidate generation matches the
//     fake-quant path bit for bit.
//
// Mapping (MI355X): one lane owns one (group, input block b) pair and walks
// output rows r, r + K, r + 2K, ...  Its H_b stays in VGPRs for the whole walk
// (16 diagonal values + 120 symmetrised H_ij + H_ji), so the inner loop
// touches no memory; consecutive lanes own consecutive b, so the weight rows
// they read are contiguous.  For each row the lane evaluates the 126
// candidates in registers and keeps (best error, lowest index).
//
// Candidate structure: every E4M3 value is c = mu * 2^j with mu one of the
// eight mantissas 1, 1.125, ..., 1.875 (subnormal codes included: e.g.
// 3 * 2^-9 = 1.5 * 2^-8).  With sigma_mu = fl32(mu * S_g) the candidate scale
// is s = fl32(c * S_g) = 2^j * sigma_mu exactly, and fl32(w / s) =
// 2^-j * fl32(w / sigma_mu) exactly (power-of-two scaling commutes with
// rounding away from the subnormal/overflow range).  So one IEEE division per
// (weight, mantissa) serves the 14-18 candidates of that mantissa.
//
// Cast: gfx950's scaled FP4 conversions do the E2M1 rounding.
// v_cvt_scalef32_pk_fp4_f32 divides two fp32 values by the power-of-two part
// of its scale operand and rounds them to E2M1 (round to nearest, ties to
// even, saturating at +-6), which with scale 2^j is exactly the cast of
// 2^-j * p = fl32(w / s); v_cvt_scalef32_pk_f32_fp4 with scale 1 returns the
// signed grid values.  Then Q = fl32(r * s) and dw = Q - w.  Three VALU
// instructions per weight and candidate.
//
// Units: the lane works in units of 2^e with e = ilogb(S_g): w' = w 2^-e and
// sigma' = sigma 2^-e are exact, so every Q', dw' = dw 2^-e and the error
// E' = E 2^-2e are the same fp32 numbers scaled by a power of two (identical
// argmin) while staying far from fp32 underflow for tiny amax.  The reported
// error is ldexp(E', 2e).
//
// When S_g < 2^-117 some candidate scales are subnormal and the identities
// above can fail, so the kernel divides per candidate and rounds in software
// instead, which is the definition itself (then rescales dw exactly).
#include <math.h>

#include "lh_device.h"
#include "lh_internal.h"

namespace lh {
namespace {

// Index of (i, j), i < j, in the packed strict upper triangle (row-major).
__host__ __device__ constexpr int tri(int i, int j) { return i * 15 - (i * (i - 1)) / 2 + (j - i - 1); }

struct Best {
  float err;
  int k;
};

__device__ __forceinline__ void keep_best(Best& b, float e, int k) {
  // lowest index on equal errors (bitwise ops: no branches)
  const bool take = (e < b.err) | ((e == b.err) & (k < b.k));
  b.err = take ? e : b.err;
  b.k = take ? k : b.k;
}

// E = dw^T H dw = sum_i dw_i (H_ii dw_i + sum_{j>i} (H_ij + H_ji) dw_j)
__device__ __forceinline__ float quad_form(const float (&diag)[16], const float (&sym)[120],
                                           const float (&dw)[16]) {
  float e = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float y = diag[i] * dw[i];
#pragma unroll
    for (int j = i + 1; j < 16; ++j) y = __builtin_fmaf(sym[tri(i, j)], dw[j], y);
    e = __builtin_fmaf(dw[i], y, e);
  }
  return e;
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Candidate k with scale s = 2^j * sigma, from the per-mantissa quotients
// p_i = fl32(w_i / sigma) (signed).  The eight FP4 pairs are packed into the
// four bytes of two dwords (byte select 0..3); `pk` carries them from one
// candidate to the next so no register has to be cleared first.
__device__ __forceinline__ void eval_scaled(Best& best, int k, int j, float sigma, const float (&p)[16],
                                            const float (&w)[16], const float (&diag)[16],
                                            const float (&sym)[120], uint32_t (&pk)[2]) {
  const float s = ldexpf(sigma, j);
  const float pow2j = __uint_as_float((uint32_t)(127 + j) << 23);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    pk[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[h], p[8 * h + 0], p[8 * h + 1], pow2j, 0);
    pk[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[h], p[8 * h + 2], p[8 * h + 3], pow2j, 1);
    pk[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[h], p[8 * h + 4], p[8 * h + 5], pow2j, 2);
    pk[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[h], p[8 * h + 6], p[8 * h + 7], pow2j, 3);
  }
  float r[16];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const f32x2_t r0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], 1.0f, 0);
    const f32x2_t r1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], 1.0f, 1);
    const f32x2_t r2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], 1.0f, 2);
    const f32x2_t r3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], 1.0f, 3);
    r[8 * h + 0] = r0.x; r[8 * h + 1] = r0.y; r[8 * h + 2] = r1.x; r[8 * h + 3] = r1.y;
    r[8 * h + 4] = r2.x; r[8 * h + 5] = r2.y; r[8 * h + 6] = r3.x; r[8 * h + 7] = r3.y;
  }
  float dw[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) dw[i] = r[i] * s - w[i];  // Q = fl32(r * s), then Q - w
  keep_best(best, quad_form(diag, sym, dw), k);
}

// Candidate k straight from the definition: x = fl32(|w| / s), software
// rounding to the grid, Q = fl32(sign(w) r s), dw = Q - w, then dw 2^-e.
__device__ __forceinline__ void eval_direct(Best& best, int k, float Sg, int e, const float (&w)[16],
                                            const float (&diag)[16], const float (&sym)[120]) {
  const float s = e4m3_candidate(k) * Sg;
  float dw[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float x = (s == 0.0f) ? 0.0f : fabsf(w[i]) / s;
    const float q = copysignf(e2m1_round_mag(x) * s, w[i]);
    dw[i] = ldexpf(q - w[i], -e);
  }
  keep_best(best, quad_form(diag, sym, dw), k);
}

// All candidates of mantissa class m (mu = 1 + m/8), in increasing index.
template <int m>
__device__ __forceinline__ void sweep_mantissa(Best& best, float Sg, const float (&w)[16],
                                               const float (&diag)[16], const float (&sym)[120],
                                               uint32_t (&pk)[2]) {
  const float sigma = (1.0f + 0.125f * (float)m) * Sg;  // fl32(mu * S_g)
  float p[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) p[i] = w[i] / sigma;  // IEEE division
  // subnormal E4M3 codes that share this mantissa: code = 1..7 -> k = code-1
  if constexpr (m == 0) {
    eval_scaled(best, 0, -9, sigma, p, w, diag, sym, pk);   // 1 * 2^-9
    eval_scaled(best, 1, -8, sigma, p, w, diag, sym, pk);   // 2 * 2^-9
    eval_scaled(best, 3, -7, sigma, p, w, diag, sym, pk);   // 4 * 2^-9
  } else if constexpr (m == 2) {
    eval_scaled(best, 4, -7, sigma, p, w, diag, sym, pk);   // 5 * 2^-9
  } else if constexpr (m == 4) {
    eval_scaled(best, 2, -8, sigma, p, w, diag, sym, pk);   // 3 * 2^-9
    eval_scaled(best, 5, -7, sigma, p, w, diag, sym, pk);   // 6 * 2^-9
  } else if constexpr (m == 6) {
    eval_scaled(best, 6, -7, sigma, p, w, diag, sym, pk);   // 7 * 2^-9
  }
  // normal codes 8E + m (E = 1..15; code 0x7F is NaN): value mu * 2^(E-7)
  constexpr int emax = (m == 7) ? 14 : 15;
  for (int E = 1; E <= emax; ++E) eval_scaled(best, 8 * E + m - 1, E - 7, sigma, p, w, diag, sym, pk);
}

template <typename T, bool kVec>
__device__ __forceinline__ void load_block(const T* p, float (&w)[16]) {
  if constexpr (sizeof(T) == 2) {
    if (kVec) {
      const uint4 u0 = reinterpret_cast<const uint4*>(p)[0];
      const uint4 u1 = reinterpret_cast<const uint4*>(p)[1];
      const uint32_t v[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        w[2 * i] = __uint_as_float(v[i] << 16);
        w[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i] = bf16_bits_to_f32(p[i]);
    }
  } else {
    if (kVec) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 f = reinterpret_cast<const float4*>(p)[q];
        w[4 * q] = f.x;
        w[4 * q + 1] = f.y;
        w[4 * q + 2] = f.z;
        w[4 * q + 3] = f.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i] = p[i];
    }
  }
}

template <typename T, bool kVec>
__global__ __launch_bounds__(kThreads) void sweep_kernel(const T* __restrict__ wt, int64_t c_out,
                                                         int64_t ld_w, int64_t gstride_w, int64_t nb,
                                                         int64_t rows_step, int64_t lanes,
                                                         const float* __restrict__ h, int64_t gstride_h,
                                                         const float* __restrict__ amax,
                                                         uint8_t* __restrict__ idx_out,
                                                         float* __restrict__ err_out,
                                                         float* __restrict__ amax_out) {
  const int64_t L = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (L >= lanes) return;
  const int64_t per_group = nb * rows_step;
  const int64_t grp = L / per_group;
  const int64_t rem = L - grp * per_group;
  const int64_t row0 = rem / nb;
  const int64_t b = rem - row0 * nb;

  float diag[16], sym[120];
  {
    const float* hb = h + grp * gstride_h + b * 256;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float r[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 f = reinterpret_cast<const float4*>(hb + 16 * i)[q];
        r[4 * q] = f.x;
        r[4 * q + 1] = f.y;
        r[4 * q + 2] = f.z;
        r[4 * q + 3] = f.w;
      }
      diag[i] = r[i];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j > i) sym[tri(i, j)] = r[j];
        if (j < i) sym[tri(j, i)] += r[j];
      }
    }
  }

  const float g = amax[grp];
  const float Sg = g / kAmaxDivisor;
  const bool fast = (Sg >= 0x1p-117f) && (Sg <= 0x1p127f);
  const int e = (Sg > 0.0f && Sg <= 0x1p127f) ? ilogbf(Sg) : 0;
  const float Su = ldexpf(Sg, -e);  // S_g in units of 2^e: [1, 2)

  for (int64_t row = row0; row < c_out; row += rows_step) {
    float w[16];
    load_block<T, kVec>(wt + grp * gstride_w + row * ld_w + 16 * b, w);
    Best best{INFINITY, kCandidates};
    uint32_t pk[2] = {0u, 0u};
    if (fast) {
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i] = ldexpf(w[i], -e);
      sweep_mantissa<0>(best, Su, w, diag, sym, pk);
      sweep_mantissa<1>(best, Su, w, diag, sym, pk);
      sweep_mantissa<2>(best, Su, w, diag, sym, pk);
      sweep_mantissa<3>(best, Su, w, diag, sym, pk);
      sweep_mantissa<4>(best, Su, w, diag, sym, pk);
      sweep_mantissa<5>(best, Su, w, diag, sym, pk);
      sweep_mantissa<6>(best, Su, w, diag, sym, pk);
      sweep_mantissa<7>(best, Su, w, diag, sym, pk);
    } else {
      for (int k = 0; k < kCandidates; ++k) eval_direct(best, k, Sg, e, w, diag, sym);
    }
    const int k = best.k < kCandidates ? best.k : 0;  // NaN errors only
    const int64_t o = (grp * c_out + row) * nb + b;
    idx_out[o] = (uint8_t)k;
    if (err_out) err_out[o] = ldexpf(best.err, 2 * e);
    if (amax_out) amax_out[o] = 6.0f * (e4m3_candidate(k) * Sg);
  }
}

template <typename T, bool kVec>
hipError_t launch_sweep_typed(const SweepArgs& a, hipStream_t stream) {
  const int64_t nb = a.c_in / 16;
  const int64_t per_k = a.n_groups * nb;
  // Enough lanes to fill 256 CUs x 4 SIMDs x 2 waves; rows split evenly.
  const int64_t target = 256LL * 4 * 2 * 64;
  int64_t k = (target + per_k - 1) / per_k;
  if (k > a.c_out) k = a.c_out;
  if (k < 1) k = 1;
  const int64_t rows_per_lane = (a.c_out + k - 1) / k;
  k = (a.c_out + rows_per_lane - 1) / rows_per_lane;
  const int64_t lanes = per_k * k;
  const int64_t grid = (lanes + kThreads - 1) / kThreads;
  sweep_kernel<T, kVec><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
      static_cast<const T*>(a.w), a.c_out, a.ld_w, a.gstride_w, nb, k, lanes, a.h, a.gstride_h, a.amax,
      a.idx, a.err, a.best_amax);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sweep(const SweepArgs& a, hipStream_t stream) {
  if (a.n_groups == 0 || a.c_out == 0 || a.c_in == 0) return hipSuccess;
  const int64_t esz = a.dtype == 1 ? 2 : 4;
  const int64_t epv = 16 / esz;
  const bool aligned = (reinterpret_cast<uintptr_t>(a.w) % 16 == 0) && (a.ld_w % epv == 0) &&
                       (a.gstride_w % epv == 0);
  const bool h_aligned = (reinterpret_cast<uintptr_t>(a.h) % 16 == 0) && (a.gstride_h % 4 == 0);
  if (!h_aligned) return hipErrorInvalidValue;  // rejected earlier by the front end
  if (a.dtype == 1)
    return aligned ? launch_sweep_typed<uint16_t, true>(a, stream) : launch_sweep_typed<uint16_t, false>(a, stream);
  return aligned ? launch_sweep_typed<float, true>(a, stream) : launch_sweep_typed<float, false>(a, stream);
}

}  // namespace lh
