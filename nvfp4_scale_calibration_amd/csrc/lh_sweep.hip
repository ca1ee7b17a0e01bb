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
// 2^-j * p = fl32(w / s); v_cvt_scalef32_pk_f32_fp4 with the same scale
// returns the signed grid values times 2^j, exactly.  Then
// Q = fl32((r 2^j) sigma) = fl32(r s) and dw = Q - w.  Three VALU
// instructions per weight and candidate.
//
// Skipping (exact): for a symmetric H with positive diagonal and
// C = D^-1/2 H D^-1/2 (D = diag H), any tau <= lambda_min(C) gives
// E_k >= tau * sum_i H_ii dw_i^2 >= tau * sum_{e in T} H_ee dw_e^2 for every
// candidate and any subset T.  tau comes from a pre-pass that certifies
// C - tau I positive definite with an fp32 Cholesky factorisation (when the
// caller passes a workspace), else from Gershgorin in-kernel.  Level 1: each
// lane keeps T = its four elements with the largest H_ii w_i^2 and bounds
// every candidate with ~20 VALU operations before casting all 16 weights
// (~207 for a full evaluation).  Level 2: after the cast, the full diagonal
// bound reuses the products H_ii dw_i that start the rows of the quadratic
// form.  A candidate (or the rest of its form) is skipped only when every
// lane of the wave proves lb > best * (1 + 2^-10); the skipped candidate then
// cannot be the minimum or tie with it, so indices and errors are
// bit-identical to the exhaustive loop.  The margin covers the fp32 rounding
// of the bound and of E, which the certificate keeps below 2^-11 relative;
// lanes without a certificate never vote to skip.  Each row first evaluates
// the lane's max-scaling candidate with the same arithmetic as the loop, so
// the bound has a good incumbent from the start.
//
// Units: each row works in units of 2^e with e = ilogb(S_g): w' = w 2^-e and
// sigma' = sigma 2^-e are exact, so every Q', dw' = dw 2^-e and the error
// E' = E 2^-2e are the same fp32 numbers scaled by a power of two (identical
// argmin) while staying far from fp32 underflow for tiny amax.  When a row's
// weights lie far from the amax (beyond 2^+-20 S_g), e follows the weights
// instead, so that dw' and E' stay far from overflow and underflow.  The
// reported error is ldexp(E', 2e).
//
// When S_g < 2^-117 some candidate scales are subnormal and the identities
// above can fail, so the kernel divides per candidate and rounds in software
// instead, which is the definition itself (then rescales dw exactly).
#include <math.h>

#include "lh_device.h"
#include "lh_internal.h"

namespace lh {
hipError_t launch_certificate(const float* h, int64_t gstride_h, int64_t c_in, int64_t n_groups, float* cert,
                              hipStream_t stream);
namespace {

// Index of (i, j), i < j, in the packed strict upper triangle (row-major).
__host__ __device__ constexpr int tri(int i, int j) { return i * 15 - (i * (i - 1)) / 2 + (j - i - 1); }

// Workgroup size of the sweep kernel: one wave, so that a finished wave's
// slot is refilled at once (lanes do unequal work: a workgroup of several
// waves holds its slots until its slowest wave ends).
constexpr int kSweepThreads = 64;

struct Best {
  float err;
  int k;
};

__device__ __forceinline__ void keep_best(Best& b, float e, int k, bool has = true) {
  // lowest index on equal errors (bitwise ops: no branches); has == false:
  // the lane evaluated no candidate of its own and keeps its best
  const bool take = has & ((e < b.err) | ((e == b.err) & (k < b.k)));
  b.err = take ? e : b.err;
  b.k = take ? k : b.k;
}

constexpr float kSkipMargin = 1.0f + 0x1p-10f;

// True when p holds on some active lane of the wave (the lane mask of a
// comparison goes straight to the ballot, without a round trip through a
// 0/1 register).
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Per-row state of the skip test: the four bound elements (prescaled weights,
// gamma * H_ee) and their packed FP4 codes.
struct SkipSet {
  float w[4];
  float dg[4];
  float p[4];      // w[e] / sigma of the current mantissa class (same bits as p[idx])
  uint32_t pk;
  float gamma;     // certificate (0 when off)
  float margin;    // kSkipMargin, or NaN when the lane has no certificate
                   // (then best * margin is NaN, no bound exceeds it and
                   // nothing is skipped, whatever the sign of best)
};

// E = dw^T H dw = sum_i dw_i (H_ii dw_i + sum_{j>i} (H_ij + H_ji) dw_j), or
// the plain weight error sum_i dw_i^2 (H = I) when kMse.
template <bool kMse>
__device__ __forceinline__ float quad_form(const float (&diag)[16], const float (&sym)[120],
                                           const float (&dw)[16]) {
  float e = 0.0f;
  if constexpr (kMse) {
    e = dw[0] * dw[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) e = __builtin_fmaf(dw[i], dw[i], e);
    return e;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float y = diag[i] * dw[i];
#pragma unroll
    for (int j = i + 1; j < 16; ++j) y = __builtin_fmaf(sym[tri(i, j)], dw[j], y);
    e = __builtin_fmaf(dw[i], y, e);
  }
  return e;
}

// Same sum with the row starts y_i = H_ii dw_i already formed.
__device__ __forceinline__ float quad_form_from(const float (&yd)[16], const float (&sym)[120],
                                                const float (&dw)[16]) {
  float e = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float y = yd[i];
#pragma unroll
    for (int j = i + 1; j < 16; ++j) y = __builtin_fmaf(sym[tri(i, j)], dw[j], y);
    e = __builtin_fmaf(dw[i], y, e);
  }
  return e;
}

// RN(a / b) given rb = RN(1 / b): q = RN(a rb), r = a - b q (exact by fma),
// q' = RN(q + r rb).  Markstein's theorem makes q' the correctly rounded
// quotient when no step overflows and the quotient is normal; the fast path
// guarantees the range (row working exponent), and a subnormal quotient
// rounds to E2M1 zero either way.  Checked against IEEE division on the host
// over every divisor significand.  Three instructions instead of the ~10 of
// a full IEEE division sequence.
__device__ __forceinline__ float div_rn(float a, float b, float rb) {
  const float q = a * rb;
  const float r = __builtin_fmaf(-q, b, a);
  return __builtin_fmaf(r, rb, q);
}

// Candidate k with scale s = 2^j * sigma, from the per-mantissa quotients
// p_i = fl32(w_i / sigma) (signed).  The eight FP4 pairs are packed into the
// four bytes of two dwords (byte select 0..3); `pk` carries them from one
// candidate to the next so no register has to be cleared first.
template <bool kMse>
__device__ __forceinline__ void eval_scaled(Best& best, int k, int j, float sigma, const float (&p)[16],
                                            const float (&w)[16], const float (&diag)[16],
                                            const float (&sym)[120], uint32_t (&pk)[2], bool has = true) {
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
    const f32x2_t r0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], pow2j, 0);
    const f32x2_t r1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], pow2j, 1);
    const f32x2_t r2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], pow2j, 2);
    const f32x2_t r3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], pow2j, 3);
    r[8 * h + 0] = r0.x; r[8 * h + 1] = r0.y; r[8 * h + 2] = r1.x; r[8 * h + 3] = r1.y;
    r[8 * h + 4] = r2.x; r[8 * h + 5] = r2.y; r[8 * h + 6] = r3.x; r[8 * h + 7] = r3.y;
  }
  float dw[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) dw[i] = r[i] * sigma - w[i];  // Q = fl32(r 2^j sigma) = fl32(r s), then Q - w
  keep_best(best, quad_form<kMse>(diag, sym, dw), k, has);
}

// eval_scaled with a second skip test after the cast: E >= gamma *
// sum_i H_ii dw_i^2 over all 16 weights, which reuses the products H_ii dw_i
// that start the rows of the quadratic form; the rest of the form runs only
// if some lane of the wave with a candidate (has) still needs it.
// Bit-identical E when it runs.  Every lane executes it, so that the wave
// runs no divergent branch; lanes without a candidate compute on a dummy
// power and change nothing.
template <bool kMse>
__device__ __forceinline__ void eval_scaled_skip(Best& best, const SkipSet& t, bool has, int k, int j,
                                                 float sigma, const float (&p)[16], const float (&w)[16],
                                                 const float (&diag)[16], const float (&sym)[120],
                                                 uint32_t (&pk)[2]) {
  if constexpr (kMse) {  // the diagonal bound is the whole error here
    eval_scaled<true>(best, k, j, sigma, p, w, diag, sym, pk, has);
    return;
  }
  const float pow2j = __uint_as_float((uint32_t)(127 + j) << 23);
  (void)pk;
  uint32_t pkl[2] = {0u, 0u};  // every byte is written below
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    pkl[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pkl[h], p[8 * h + 0], p[8 * h + 1], pow2j, 0);
    pkl[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pkl[h], p[8 * h + 2], p[8 * h + 3], pow2j, 1);
    pkl[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pkl[h], p[8 * h + 4], p[8 * h + 5], pow2j, 2);
    pkl[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pkl[h], p[8 * h + 6], p[8 * h + 7], pow2j, 3);
  }
  float r[16];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const f32x2_t r0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pkl[h], pow2j, 0);
    const f32x2_t r1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pkl[h], pow2j, 1);
    const f32x2_t r2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pkl[h], pow2j, 2);
    const f32x2_t r3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pkl[h], pow2j, 3);
    r[8 * h + 0] = r0.x; r[8 * h + 1] = r0.y; r[8 * h + 2] = r1.x; r[8 * h + 3] = r1.y;
    r[8 * h + 4] = r2.x; r[8 * h + 5] = r2.y; r[8 * h + 6] = r3.x; r[8 * h + 7] = r3.y;
  }
  float dw[16], yd[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    dw[i] = r[i] * sigma - w[i];  // Q = fl32(r 2^j sigma) = fl32(r s), then Q - w
    yd[i] = diag[i] * dw[i];
  }
  float d2 = yd[0] * dw[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) d2 = __builtin_fmaf(yd[i], dw[i], d2);
  if (!wave_any(has && !(t.gamma * d2 > best.err * t.margin))) return;
  keep_best(best, quad_form_from(yd, sym, dw), k, has);
}

// Candidate k straight from the definition: x = fl32(|w| / s), software
// rounding to the grid, Q = fl32(sign(w) r s), dw = Q - w, then dw 2^-e.
template <bool kMse>
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
  keep_best(best, quad_form<kMse>(diag, sym, dw), k);
}

// True when this lane cannot prove the candidate worse than its incumbent.
// The bound over the two largest elements comes first; the other two are
// added only when some lane of the wave survives it.  Terms are added in the
// same order either way and adding a non-negative term never lowers a
// rounded sum, so a lane stopped by the two-element bound would also be
// stopped by the four-element one: the outcome is that of the four-element
// test alone.
__device__ __forceinline__ bool needs_eval(SkipSet& t, const Best& best, int j, float sigma, uint64_t& live2) {
  const float pow2j = __uint_as_float((uint32_t)(127 + j) << 23);
  const float thr = best.err * t.margin;
  t.pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(t.pk, t.p[0], t.p[1], pow2j, 0);
  const f32x2_t r01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(t.pk, pow2j, 0);
  const float d0 = r01.x * sigma - t.w[0], d1 = r01.y * sigma - t.w[1];
  float lb = (t.dg[0] * d0) * d0;
  lb = __builtin_fmaf(t.dg[1] * d1, d1, lb);
  live2 = __builtin_amdgcn_ballot_w64(!(lb > thr));  // lanes the two-element bound leaves in
  if (live2 != 0) {
    t.pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(t.pk, t.p[2], t.p[3], pow2j, 1);
    const f32x2_t r23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(t.pk, pow2j, 1);
    const float d2 = r23.x * sigma - t.w[2], d3 = r23.y * sigma - t.w[3];
    lb = __builtin_fmaf(t.dg[2] * d2, d2, lb);
    lb = __builtin_fmaf(t.dg[3] * d3, d3, lb);
  }
  return !(lb > thr);
}

// E4M3 code of mantissa class m at power j (value (1 + m/8) 2^j): normal
// codes 8 (j + 7) + m for j >= -6, subnormal codes (8 + m) 2^(j + 9) / 8
// below (e.g. 3 * 2^-9 = 1.5 * 2^-8).
__device__ __forceinline__ int class_code(int m, int j) {
  return j >= -6 ? 8 * (j + 7) + m : ((8 + m) << (j + 9)) >> 3;
}

// All candidates of mantissa class m (mu = 1 + m/8): powers j in
// [jmin, jmax] (codes 1..126 only; 0x7F is NaN).  First every lane runs the
// level-1 test on the class's candidates against its incumbent at the class
// start and keeps a mask of the candidates it cannot rule out; then
// each lane evaluates its own candidates in increasing index while any lane
// of the wave has one left.  A wave therefore costs the largest per-lane
// count rather than the union over its lanes, and every candidate a lane
// skips is still certified worse than that lane's incumbent.  The level-1
// tests run from the highest power down and stop where the saturation
// argument below rules out all the lower ones at once, so the masks are
// those of testing every power.
// Powers of two of mantissa class m that are E4M3 candidates (codes 1..126;
// 0x7F is NaN): j in [jmin, jmax].
template <int m>
struct ClassRange {
  static constexpr int jmin = (m == 0) ? -9 : (m == 4) ? -8 : (m == 2 || m == 6) ? -7 : -6;
  static constexpr int jmax = (m == 7) ? 7 : 8;
};

// Level-1 tests of class m (quotients t.p of the bound elements already
// formed) against the lane's incumbent: returns the mask of the powers
// (bit c = power jmin + c) this lane cannot rule out.  The tests run from the
// highest power down and stop where the saturation argument below rules out
// all the lower ones at once, so the mask is that of testing every power.
template <int m>
__device__ __forceinline__ uint32_t level1_scan(const Best& best, SkipSet& t, float sigma) {
  constexpr int jmin = ClassRange<m>::jmin, jmax = ClassRange<m>::jmax;
  uint32_t need = 0;
  // Powers from the top down.  Below js2 the two leading bound elements
  // both saturate (|p| >= 6 * 2^j: E2M1 gives 6, Q = 6 * 2^j * sigma), so
  // their |dw| only grows as j falls and so does the two-element bound
  // (rounded products and sums of non-negative terms are monotone): once
  // every lane of the wave is at or below its js2 and the two-element
  // bound rules the candidate out on every lane, it rules out every lower
  // power too, and the scan stops.
  const uint32_t a0 = __float_as_uint(t.p[0]) & 0x7FFFFFFFu, a1 = __float_as_uint(t.p[1]) & 0x7FFFFFFFu;
  const uint32_t amin2 = min(a0, a1);  // a NaN (above every finite value) only counts when both are
  const int js2 = (int)(amin2 >> 23) - 130 + (int)((amin2 & 0x7FFFFFu) >= 0x400000u);
#pragma unroll
  for (int c = jmax - jmin; c >= 0; --c) {
    const int j = jmin + c;
    uint64_t live2;
    if (needs_eval(t, best, j, sigma, live2)) need |= 1u << c;
    if ((__builtin_amdgcn_ballot_w64(j > js2) | live2) == 0) break;
  }
  return need;
}

// All candidates of mantissa class m (mu = 1 + m/8) for the lanes-on-blocks
// sweep: first the level-1 scan gives each lane a mask of the candidates it
// cannot rule out; then each lane evaluates its own candidates in increasing
// index while any lane of the wave has one left.  A wave therefore costs the
// largest per-lane count rather than the union over its lanes, and every
// candidate a lane skips is still certified worse than that lane's
// incumbent.
template <int m, bool kMse>
__device__ __forceinline__ void sweep_mantissa(Best& best, SkipSet& t, float Sg, const float (&w)[16],
                                               const float (&diag)[16], const float (&sym)[120],
                                               uint32_t (&pk)[2]) {
  const float sigma = (1.0f + 0.125f * (float)m) * Sg;  // fl32(mu * S_g)
  const float rs = 1.0f / sigma;                        // IEEE division, once per class
  float p[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) p[i] = div_rn(w[i], sigma, rs);  // = fl32(w / sigma)
#pragma unroll
  for (int e = 0; e < 4; ++e) t.p[e] = div_rn(t.w[e], sigma, rs);  // same operation on the same bits as p[idx]
  uint32_t need = level1_scan<m>(best, t, sigma);
  while (wave_any(need != 0)) {
    const bool has = need != 0;
    const int j = ClassRange<m>::jmin + __builtin_ctz(need | 0x80000000u);  // a dummy power when !has
    need &= need - 1;
    eval_scaled_skip<kMse>(best, t, has, class_code(m, j) - 1, j, sigma, p, w, diag, sym, pk);
  }
}

// Mantissa class and power of two of candidate k: c_k = (1 + m/8) 2^j.
__device__ __forceinline__ void candidate_class(int k, int& m, int& j) {
  const int code = k + 1;
  if (code >= 8) {
    m = code & 7;
    j = (code >> 3) - 7;
    return;
  }
  // subnormal codes c * 2^-9, c = 1..7: with f = floor(log2 c),
  // c = (c 2^(3-f) / 8) 2^f, so m = c 2^(3-f) - 8 and j = f - 9 (computed,
  // not looked up: a table in memory would be a load, and waiting for it
  // would also wait for the stores issued before it)
  const int f = 31 - __builtin_clz((unsigned)code);
  m = (code << (3 - f)) - 8;
  j = f - 9;
}

// The lane's max-scaling candidate: smallest c_k >= max|w| / (6 S_g), i.e. the
// block scale that keeps every weight on the grid without saturating.
__device__ __forceinline__ int max_scaling_candidate(const float (&w)[16], float Su) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(w[i]));
  float t = a / (6.0f * Su);
  t = fminf(fmaxf(t, 0x1p-9f), 448.0f);
  int code;
  if (t <= 0x1p-6f) {
    code = (int)ceilf(t * 512.0f);  // subnormal codes 1..8 (8 is 2^-6)
  } else {
    int e2 = ilogbf(t);
    int mm = (int)ceilf((ldexpf(t, -e2) - 1.0f) * 8.0f);
    if (mm == 8) {
      mm = 0;
      ++e2;
    }
    code = (e2 + 7) * 8 + mm;
  }
  code = code < 1 ? 1 : (code > kCandidates ? kCandidates : code);
  return code - 1;
}

// Working exponent of one row (see "Units"): that of S_g (e_g) while the
// row's largest |w| is within 2^+-20 of S_g, else that of the largest |w|
// itself, kept within e_g +- 100 so that S_g 2^-e times every candidate stays
// a normal fp32 number.
__device__ __forceinline__ int row_exponent(int e_g, const float (&w)[16]) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(w[i]));
  if (!(a > 0.0f)) return e_g;
  const int d = ilogbf(a) - e_g;
  if (d >= -20 && d <= 20) return e_g;
  return e_g + (d > 100 ? 100 : (d < -100 ? -100 : d));
}

// Nibbles of candidate k for a row in its working units (w and Su prescaled
// by 2^-e), computed with the sweep's own arithmetic: p = fl32(w / sigma)
// (div_rn) and the scaled FP4 conversion with scale 2^j.  When e is S_g's
// own exponent every quantity involved is a normal fp32 number except
// quotients that round to a zero nibble either way, so these are exactly
// the nibbles of nvfp4_cast_block(w 2^e, s_k) (IEEE quotient fl32(w / s_k),
// then the E2M1 rounding).  Signs on zero magnitudes are cleared as there.
__device__ __forceinline__ void candidate_nibbles(int k, float Su, const float (&w)[16], uint32_t (&pk)[2]) {
  int m, j;
  candidate_class(k, m, j);
  const float sigma = (1.0f + 0.125f * (float)m) * Su;
  const float rs = 1.0f / sigma;
  const float pow2j = __uint_as_float((uint32_t)(127 + j) << 23);
  float p[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) p[i] = div_rn(w[i], sigma, rs);
  pk[0] = pk[1] = 0u;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    pk[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[h], p[8 * h + 0], p[8 * h + 1], pow2j, 0);
    pk[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[h], p[8 * h + 2], p[8 * h + 3], pow2j, 1);
    pk[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[h], p[8 * h + 4], p[8 * h + 5], pow2j, 2);
    pk[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[h], p[8 * h + 6], p[8 * h + 7], pow2j, 3);
    const uint32_t nz = (pk[h] | (pk[h] >> 1) | (pk[h] >> 2)) & 0x11111111u;
    pk[h] &= 0x77777777u | (nz << 3);
  }
}

// The block's raw weights read again with relaxed atomic loads, which the
// compiler does not merge with the row's first load (that would keep the raw
// values live across the candidate loop); used only for rows whose working
// exponent is not S_g's.
template <typename T>
__device__ __forceinline__ void reload_block(const T* p, float (&w)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if constexpr (sizeof(T) == 2) w[i] = bf16_bits_to_f32(__atomic_load_n(p + i, __ATOMIC_RELAXED));
    else w[i] = __uint_as_float(__atomic_load_n(reinterpret_cast<const uint32_t*>(p) + i, __ATOMIC_RELAXED));
  }
}

// H_b (16x16 row-major, 16-byte aligned) as its diagonal and the symmetrised
// strict upper triangle H_ij + H_ji.
__device__ __forceinline__ void load_hessian(const float* hb, float (&diag)[16], float (&sym)[120]) {
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

// Makes the compiler treat the 16 words as used at this point.
__device__ __forceinline__ void wait_raw(uint32_t (&r)[16]) {
  asm volatile("" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]),
               "+v"(r[7]), "+v"(r[8]), "+v"(r[9]), "+v"(r[10]), "+v"(r[11]), "+v"(r[12]), "+v"(r[13]),
               "+v"(r[14]), "+v"(r[15]));
}

// A weight row's 16 values as loaded (bf16 pairs or fp32 bits), and their
// fp32 values: split so that a load can be issued long before its use.
template <typename T, bool kVec>
__device__ __forceinline__ void load_raw(const T* p, uint32_t (&r)[16]) {
  if constexpr (sizeof(T) == 2) {
    if (kVec) {
      const uint4 u0 = reinterpret_cast<const uint4*>(p)[0];
      const uint4 u1 = reinterpret_cast<const uint4*>(p)[1];
      r[0] = u0.x; r[1] = u0.y; r[2] = u0.z; r[3] = u0.w;
      r[4] = u1.x; r[5] = u1.y; r[6] = u1.z; r[7] = u1.w;
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) r[i] = p[i];
    }
  } else {
    if (kVec) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 u = reinterpret_cast<const uint4*>(p)[q];
        r[4 * q] = u.x; r[4 * q + 1] = u.y; r[4 * q + 2] = u.z; r[4 * q + 3] = u.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) r[i] = __float_as_uint(p[i]);
    }
  }
}

template <typename T, bool kVec>
__device__ __forceinline__ void raw_to_float(const uint32_t (&r)[16], float (&w)[16]) {
  if constexpr (sizeof(T) == 2) {
    if (kVec) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        w[2 * i] = __uint_as_float(r[i] << 16);
        w[2 * i + 1] = __uint_as_float(r[i] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i] = bf16_bits_to_f32(r[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = __uint_as_float(r[i]);
  }
}

// Scaled Gershgorin certificate gamma = 1 - max_i sum_{j != i} |S_ij| /
// (2 sqrt(H_ii H_jj)), less 1e-3 for the rounding of this estimate, used
// only when >= 0.1 (then the fp32 error of E is below 35u * 19); 0 when the
// diagonal is not positive and finite.
__device__ __forceinline__ float gershgorin_gamma(const float (&diag)[16], const float (&sym)[120]) {
  bool pos = true;
  float rs[16], rho[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    pos = pos && (diag[i] > 0.0f) && (diag[i] < INFINITY);
    rs[i] = diag[i] > 0.0f ? 1.0f / sqrtf(diag[i]) : 0.0f;
    rho[i] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int j = i + 1; j < 16; ++j) {
      const float c = fabsf(sym[tri(i, j)]) * 0.5f * rs[i] * rs[j];
      rho[i] += c;
      rho[j] += c;
    }
  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = fmaxf(mx, rho[i]);
  const float gamma = 1.0f - mx - 1e-3f;
  return (!pos || !(gamma >= 0.1f)) ? 0.0f : gamma;
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

// ---------------------------------------------------------------------------
// Skip certificate pre-pass.  With S = (H + H^T)/2, D = diag S and
// C = D^-1/2 S D^-1/2 (unit diagonal), it finds a large tau with C - tau I
// positive definite, testing each tau with an fp32 Cholesky factorisation
// (operations accurate to a few ulps): if every pivot is positive, the
// computed factor is the exact factor of C - tau I + dA with
// |dA| <= 20u |L||L^T| (Cholesky backward error), and |L||L^T| <= 1
// entrywise, so lambda_min(C) >= tau - 16*20u.  The certificate stored is
// tau - 2e-3, which also covers the rounding of C itself.  It is zeroed (no
// skipping) when the diagonal is not positive and finite, when it falls
// below 0.02, or when the fp32 error bound of the quadratic form,
// 35u (1 + rho) / tau with rho the largest off-diagonal row sum of |C| (so
// lambda_max(|C|) <= 1 + rho), would exceed 2^-11.
// ---------------------------------------------------------------------------

// Up to this many blocks the team kernel (short dependency chains, 16 lanes
// per factorisation) is faster; beyond it the lane kernel (one
// factorisation per lane, 16x fewer instructions in total) is.
constexpr int64_t kCertTeamMaxBlocks = 2048;

// Value of lane k of this lane's 16-lane team.  A team is one DPP row, and
// row_newbcast copies the row's lane k to all sixteen (a VALU move, no LDS
// round trip; every lane of the team is active here).
template <int k>
__device__ __forceinline__ float team_lane(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + k, 0xF, 0xF, false));
}

// A_ik -= l_ij l_kj for k = k0..15, l_kj from lane k of the team.
template <int k0>
__device__ __forceinline__ void team_column_update(float (&a)[16], float l) {
  if constexpr (k0 < 16) {
    a[k0] = __builtin_fmaf(-l, team_lane<k0>(l), a[k0]);
    team_column_update<k0 + 1>(a, l);
  }
}

// Columns j..15 of a right-looking Cholesky factorisation held one row per
// lane (a = row i of the matrix): the pivot d = A_jj comes from lane j,
// l_ij = A_ij / sqrt(d), then the trailing entries are updated.  Entries
// above a lane's diagonal are updated too but never read by a valid step.
// ok stays true while every pivot is positive.
template <int j>
__device__ __forceinline__ void team_cholesky(float (&a)[16], bool& ok) {
  if constexpr (j < 16) {
    const float d = team_lane<j>(a[j]);
    ok = ok && (d > 0.0f);
    const float l = a[j] * __builtin_amdgcn_rsqf(fmaxf(d, 0x1p-126f));
    team_column_update<j + 1>(a, l);
    team_cholesky<j + 1>(a, ok);
  }
}

// For few blocks (latency-bound): one workgroup per block, team q (16
// lanes) tests tau = q/16, team 0 the
// Gershgorin bound (no factorisation); the block keeps the largest tau that
// passes.  Lane i of a team holds row i of C - tau I and the team factorises
// it column by column (right-looking: the pivot and then each entry of the
// new column are broadcast within the team), so each lane does 16 steps of
// a few operations instead of a whole factorisation.
// The certificate of one block whose H sits in hs (row q, column i), by the
// 256 threads of the workgroup (team q = threadIdx.x / 16); the result is
// valid in thread 0.
__device__ float certify_team(const float (*hs)[17], float* taus) {
  const int q = threadIdx.x >> 4, i = threadIdx.x & 15;
  bool pos = true;
  float rs[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float d = hs[j][j];
    pos = pos && (d > 0.0f) && (d < INFINITY);
    rs[j] = d > 0.0f ? __builtin_amdgcn_rsqf(d) : 0.0f;
  }
  // row i of C and its off-diagonal absolute sum
  const float hii = hs[i][i];
  const float ri = hii > 0.0f ? __builtin_amdgcn_rsqf(hii) : 0.0f;
  float a[16];
  float r = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    a[j] = (j == i) ? hii * ri * ri : 0.5f * (hs[i][j] + hs[j][i]) * ri * rs[j];
    if (j != i) r += fabsf(a[j]);
  }
  float rho = pos ? r : 0.0f;
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) rho = fmaxf(rho, __shfl_xor(rho, off, 16));
  float tau = 0.0f;
  if (q == 0) {
    tau = fmaxf(1.0f - rho - 1e-3f, 0.0f);
  } else {
    const float tq = (float)q * 0.0625f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j == i) a[j] -= tq;
    bool ok = true;
    team_cholesky<0>(a, ok);
    tau = ok ? tq - 2e-3f : 0.0f;
  }
  if (i == 0) taus[q] = tau;
  __syncthreads();
  float best = taus[0];
#pragma unroll
  for (int k = 1; k < 16; ++k) best = fmaxf(best, taus[k]);
  const float err = 35.0f * 0x1p-24f * (1.0f + rho) / best;
  if (!pos || !(best >= 0.02f) || !(err <= 0x1p-11f)) best = 0.0f;
  return best;
}

__global__ __launch_bounds__(kThreads) void sweep_certificate_team_kernel(const float* __restrict__ h, int64_t gstride_h,
                                                                     int64_t nb, float* __restrict__ cert) {
  __shared__ float hs[16][17];
  __shared__ float taus[16];
  const int64_t t = blockIdx.x;
  const int64_t grp = t / nb, b = t - grp * nb;
  hs[threadIdx.x >> 4][threadIdx.x & 15] = h[grp * gstride_h + b * 256 + threadIdx.x];  // row q, column i
  __syncthreads();
  const float c = certify_team(hs, taus);
  if (threadIdx.x == 0) cert[t] = c;
}

// The calibration prologue's second launch, one workgroup per block: H_b =
// alpha * (sum of the token slices, in slice order), its skip certificate
// from the same registers (when cert is given), and for the first n_groups
// workgroups the global amax of group blockIdx.x from its partial maxima.
__global__ __launch_bounds__(kThreads) void finalize_certify_kernel(const float* __restrict__ part, int64_t nsplit,
                                                                    int64_t n_groups, int64_t nb, float alpha,
                                                                    float* __restrict__ h, int64_t h_gstride,
                                                                    float* __restrict__ cert,
                                                                    const uint32_t* __restrict__ abs_part,
                                                                    int64_t abs_per_group, float* __restrict__ amax) {
  __shared__ float hs[16][17];
  __shared__ float taus[16];
  __shared__ uint32_t wmax[kThreads / 64];
  const int64_t blk = blockIdx.x;
  const int64_t grp = blk / nb, b = blk - grp * nb;
  const int e = threadIdx.x;
  if (blk < n_groups) {  // the whole workgroup folds group blk's partial maxima
    uint32_t m = 0;
    for (int64_t k = e; k < abs_per_group; k += kThreads) m = max(m, abs_part[blk * abs_per_group + k]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    if ((e & 63) == 0) wmax[e >> 6] = m;
  }
  const float v = alpha * sum_slices(part + blk * 256 + e, n_groups * nb * 256, nsplit);
  h[grp * h_gstride + b * 256 + e] = v;
  hs[e >> 4][e & 15] = v;
  __syncthreads();
  const float c = cert ? certify_team(hs, taus) : 0.0f;  // cert is uniform across the launch
  if (e == 0) {
    if (cert) cert[blk] = c;
    if (blk < n_groups) {
      uint32_t m = wmax[0];
#pragma unroll
      for (int k = 1; k < kThreads / 64; ++k) m = max(m, wmax[k]);
      amax[blk] = __uint_as_float(m);
    }
  }
}

// In-place Cholesky of the packed lower triangle a (a[i (i + 1) / 2 + j],
// j <= i); true when every pivot is positive.
__device__ bool cholesky_ok(float (&a)[136]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float d = a[j * (j + 1) / 2 + j];
#pragma unroll
    for (int m = 0; m < j; ++m) d = __builtin_fmaf(-a[j * (j + 1) / 2 + m], a[j * (j + 1) / 2 + m], d);
    if (!(d > 0.0f)) return false;
    const float ljj = sqrtf(d);
    a[j * (j + 1) / 2 + j] = ljj;
    const float inv = 1.0f / ljj;
#pragma unroll
    for (int i = j + 1; i < 16; ++i) {
      float v = a[i * (i + 1) / 2 + j];
#pragma unroll
      for (int m = 0; m < j; ++m) v = __builtin_fmaf(-a[i * (i + 1) / 2 + m], a[j * (j + 1) / 2 + m], v);
      a[i * (i + 1) / 2 + j] = v * inv;
    }
  }
  return true;
}

// For many blocks: sixteen lanes per block, lane q tests tau = q/16 (lane 0
// the Gershgorin bound, which needs no factorisation) with a whole
// factorisation of its own; the block keeps the largest tau that passes.  The 16 lanes stage the block's H in LDS (one
// row each), then replace it by C (lane q computes row q and its
// off-diagonal sum), so each lane only reads C's lower triangle before its
// factorisation.
__global__ __launch_bounds__(kThreads) void sweep_certificate_lane_kernel(const float* __restrict__ h, int64_t gstride_h,
                                                                     int64_t nb, int64_t total,
                                                                     float* __restrict__ cert) {
  constexpr int kPitch = 260;  // 16-byte aligned rows; the four teams of a wave start 4 banks apart
  __shared__ __align__(16) float hs[kThreads / 16][kPitch];
  const int slot = threadIdx.x >> 4;
  const int64_t t = (int64_t)blockIdx.x * (kThreads / 16) + slot;
  const int q = threadIdx.x & 15;
  const bool live = t < total;  // all 16 lanes of a block share t
  const int64_t tc = live ? t : 0;
  const int64_t grp = tc / nb, b = tc - grp * nb;
  float* hb = hs[slot];
  {
    const float4* src = reinterpret_cast<const float4*>(h + grp * gstride_h + b * 256 + q * 16);
#pragma unroll
    for (int c = 0; c < 4; ++c) reinterpret_cast<float4*>(hb + q * 16)[c] = src[c];
  }
  __syncthreads();
  float rs[16];
  bool pos = true;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float d = hb[i * 17];
    pos = pos && (d > 0.0f) && (d < INFINITY);
    rs[i] = d > 0.0f ? 1.0f / sqrtf(d) : 0.0f;
  }
  // row q of C = D^-1/2 S D^-1/2 (the same operations for entry (q, j) as
  // for the lower-triangle entry the factorisation reads) and its
  // off-diagonal absolute sum
  const float hqq = hb[q * 17];
  const float rq = hqq > 0.0f ? 1.0f / sqrtf(hqq) : 0.0f;
  float crow[16];
  float r = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    crow[j] = (j == q) ? hqq * rq * rq : 0.5f * (hb[q * 16 + j] + hb[j * 16 + q]) * rq * rs[j];
    if (j != q) r += fabsf(crow[j]);
  }
  __syncthreads();  // every lane has read H
#pragma unroll
  for (int c = 0; c < 4; ++c)
    reinterpret_cast<float4*>(hb + q * 16)[c] = make_float4(crow[4 * c], crow[4 * c + 1], crow[4 * c + 2], crow[4 * c + 3]);
  float rho = pos ? r : 0.0f;
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) rho = fmaxf(rho, __shfl_xor(rho, off, 16));
  __syncthreads();
  float tau = 0.0f;
  if (pos && live) {
    if (q == 0) {
      tau = fmaxf(1.0f - rho - 1e-3f, 0.0f);
    } else {
      const float tq = (float)q * 0.0625f;
      float a[136];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float row[16];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (4 * c <= i) {
            const float4 v = reinterpret_cast<const float4*>(hb + i * 16)[c];
            row[4 * c] = v.x;
            row[4 * c + 1] = v.y;
            row[4 * c + 2] = v.z;
            row[4 * c + 3] = v.w;
          }
        }
#pragma unroll
        for (int j = 0; j <= i; ++j) a[i * (i + 1) / 2 + j] = row[j] - (i == j ? tq : 0.0f);
      }
      tau = cholesky_ok(a) ? tq - 2e-3f : 0.0f;
    }
  }
  // max over the 16 lanes of this block
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) tau = fmaxf(tau, __shfl_xor(tau, off, 16));
  const float err = 35.0f * 0x1p-24f * (1.0f + rho) / tau;
  if (!(tau >= 0.02f) || !(err <= 0x1p-11f)) tau = 0.0f;
  if (live && q == 0) cert[t] = tau;
}

// Fake-quant outputs written by the fused sweep (each optional).
// Rows of a sweep launch split over lanes in two phases.  The first waves_a
// waves hold lanes_a lanes that walk rows [0, rows_a) with stride step_a
// (several rows each); the waves after them hold lanes_b lanes that walk rows
// [rows_a, c_out) with stride step_b.  Phases start on a wave boundary, so
// each wave's walk (stride, end) is uniform.  The dispatcher starts
// workgroups roughly in index order, so the second phase's short lanes fill
// the end of the launch, where long ones would leave SIMDs idle while the
// last waves finish.
struct LanePlan {
  int64_t waves;
  int64_t waves_a;
  int64_t lanes_a;
  int64_t lanes_b;
  int64_t rows_a;
  int64_t step_a;
  int64_t step_b;
};

struct QuantOut {
  float* wq;
  uint8_t* packed;
  uint8_t* codes;
  float* gscale;
  int64_t n_groups;
};

// Two waves per SIMD: the allocator then spills ~15 row-setup values to
// scratch (none inside the candidate loop), which costs far less than the
// latency a single wave per SIMD leaves exposed.  With kQuant each row also
// writes the fake-quant of its block with the index just chosen: the
// nibbles come from candidate_nibbles on the row's working values (or
// nvfp4_cast_block on the raw weights for the rare rows that need them),
// the stores from nvfp4_emit_at, the standalone fake-quant's code.  kAll:
// every optional per-block output pointer is non-null.
template <typename T, bool kVec, bool kMse, bool kQuant, bool kAll = false>
__global__ __launch_bounds__(kSweepThreads, 2) void sweep_kernel(const T* __restrict__ wt, int64_t c_out,
                                                         int64_t ld_w, int64_t gstride_w, int64_t nb,
                                                         LanePlan lp,
                                                         const float* __restrict__ h, int64_t gstride_h,
                                                         const float* __restrict__ amax,
                                                         uint8_t* __restrict__ idx_out,
                                                         float* __restrict__ err_out,
                                                         float* __restrict__ amax_out,
                                                         const float* __restrict__ cert, QuantOut qo) {
  const int64_t L = (int64_t)blockIdx.x * kSweepThreads + threadIdx.x;
  const bool tail = (int64_t)blockIdx.x >= lp.waves_a;  // uniform over the wave
  const int64_t Lp = tail ? L - lp.waves_a * kSweepThreads : L;
  if (Lp >= (tail ? lp.lanes_b : lp.lanes_a)) return;
  const int64_t rows_step = tail ? lp.step_b : lp.step_a;
  const int64_t row_end = tail ? c_out : lp.rows_a;
  const int64_t per_group = nb * rows_step;
  const int64_t grp = Lp / per_group;
  const int64_t rem = Lp - grp * per_group;
  const int64_t r0 = rem / nb;
  const int64_t b = rem - r0 * nb;
  const int64_t row0 = (tail ? lp.rows_a : 0) + r0;

  float diag[16], sym[120];
  if constexpr (kMse) {
#pragma unroll
    for (int i = 0; i < 16; ++i) diag[i] = 1.0f;
  } else {
    load_hessian(h + grp * gstride_h + b * 256, diag, sym);
  }

  // Skip certificate: from the pre-pass when given, else scaled Gershgorin
  // gamma = 1 - max_i sum_{j != i} |S_ij| / (2 sqrt(H_ii H_jj)), less 1e-3 for
  // the rounding of this estimate, used only when >= 0.1 (then the fp32 error
  // of E is below 35u * 19).
  // H = I: C = I and tau = 1 exactly; E = sum dw^2 is accurate to 16u.
  float gamma = 1.0f;
  if constexpr (!kMse) {
    gamma = cert ? cert[grp * nb + b] : gershgorin_gamma(diag, sym);
  }
  // Per-lane scratch in LDS, element-major so that 64 lanes hit 64 consecutive
  // words: the diagonal (fixed) and the current row's prescaled weights.
  __shared__ float lds_diag[16][kSweepThreads];
  __shared__ float lds_w[16][kSweepThreads];
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 16; ++i) lds_diag[i][tid] = diag[i];

  const float g = amax[grp];
  const float Sg = g / kAmaxDivisor;
  const bool fast = (Sg >= 0x1p-117f) && (Sg <= 0x1p127f);
  const int e_g = (Sg > 0.0f && Sg <= 0x1p127f) ? ilogbf(Sg) : 0;

  // Vector-memory loads and stores share one completion counter that
  // retires in issue order, so a wait for a load also waits for every store
  // issued before it.  Hence the next row's weights are loaded before this
  // row's stores and awaited after them (wait_raw: with the same stores on
  // every path in between, the wait leaves them in flight), and the row's
  // position and output base live in LDS rather than in registers, where
  // they would be spilled across the candidate loops and reloaded from
  // scratch (a load) after the stores.  The empty asm with a memory clobber
  // at each row start makes the compiler read them back from LDS.
  uint32_t raw[16];
  __shared__ int64_t lds_row[kSweepThreads];
  __shared__ int64_t lds_obase[kSweepThreads];  // output index of the lane's block in row 0
  __shared__ int64_t lds_wofs[kSweepThreads];   // element offset of the lane's block in row 0
  lds_row[tid] = row0;
  lds_obase[tid] = grp * c_out * nb + b;
  lds_wofs[tid] = grp * gstride_w + 16 * b;
  load_raw<T, kVec>(wt + (grp * gstride_w + 16 * b) + row0 * ld_w, raw);
  wait_raw(raw);
  float w[16];
  raw_to_float<T, kVec>(raw, w);
  for (;;) {  // row0 < row_end: every lane has a first row
    asm volatile("" ::: "memory");
    const int e = row_exponent(e_g, w);
    const float Su = ldexpf(Sg, -e);  // S_g in units of 2^e: [1, 2) unless the weights moved e
    Best best{INFINITY, kCandidates};
    uint32_t pk[2] = {0u, 0u};
    if (fast) {
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i] = ldexpf(w[i], -e);
      // bound set: the four largest H_ii w_i^2 (insertion network on indices)
      SkipSet t;
      {
        float kv[4] = {-1.0f, -1.0f, -1.0f, -1.0f};
        int ki[4] = {0, 1, 2, 3};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          lds_w[i][tid] = w[i];
          const float key = diag[i] * w[i] * w[i];
          const bool c0 = key > kv[0], c1 = key > kv[1], c2 = key > kv[2], c3 = key > kv[3];
          kv[3] = c2 ? kv[2] : (c3 ? key : kv[3]);
          ki[3] = c2 ? ki[2] : (c3 ? i : ki[3]);
          kv[2] = c1 ? kv[1] : (c2 ? key : kv[2]);
          ki[2] = c1 ? ki[1] : (c2 ? i : ki[2]);
          kv[1] = c0 ? kv[0] : (c1 ? key : kv[1]);
          ki[1] = c0 ? ki[0] : (c1 ? i : ki[1]);
          kv[0] = c0 ? key : kv[0];
          ki[0] = c0 ? i : ki[0];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          t.w[q] = lds_w[ki[q]][tid];
          t.dg[q] = gamma * lds_diag[ki[q]][tid];
        }
        t.pk = 0u;
        t.gamma = gamma;
        t.margin = gamma > 0.0f ? kSkipMargin : __int_as_float(0x7FC00000);
      }
      // incumbent: the max-scaling candidate, evaluated exactly as in the loop
      {
        const int k0 = max_scaling_candidate(w, Su);
        int m0, j0;
        candidate_class(k0, m0, j0);
        const float sigma0 = (1.0f + 0.125f * (float)m0) * Su;
        const float rs0 = 1.0f / sigma0;
        float p0[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) p0[i] = div_rn(w[i], sigma0, rs0);
        eval_scaled<kMse>(best, k0, j0, sigma0, p0, w, diag, sym, pk);
      }
      sweep_mantissa<0, kMse>(best, t, Su, w, diag, sym, pk);
      sweep_mantissa<1, kMse>(best, t, Su, w, diag, sym, pk);
      sweep_mantissa<2, kMse>(best, t, Su, w, diag, sym, pk);
      sweep_mantissa<3, kMse>(best, t, Su, w, diag, sym, pk);
      sweep_mantissa<4, kMse>(best, t, Su, w, diag, sym, pk);
      sweep_mantissa<5, kMse>(best, t, Su, w, diag, sym, pk);
      sweep_mantissa<6, kMse>(best, t, Su, w, diag, sym, pk);
      sweep_mantissa<7, kMse>(best, t, Su, w, diag, sym, pk);
    } else {
      for (int k = 0; k < kCandidates; ++k) eval_direct<kMse>(best, k, Sg, e, w, diag, sym);
    }
    const int64_t row = lds_row[tid];
    const T* const wrow = wt + lds_wofs[tid] + row * ld_w;
    // (the last row loads itself again: the load count per row stays fixed)
    load_raw<T, kVec>(row + rows_step < row_end ? wrow + rows_step * ld_w : wrow, raw);
    const int k = best.k < kCandidates ? best.k : 0;  // NaN errors only
    const int64_t o = lds_obase[tid] + row * nb;
    idx_out[o] = (uint8_t)k;
    if (kAll || err_out) err_out[o] = ldexpf(best.err, 2 * e);
    if (kAll || amax_out) amax_out[o] = 6.0f * (e4m3_candidate(k) * Sg);
    if constexpr (kQuant) {
      const float s = e4m3_candidate(k) * Sg;
      uint32_t pk[2];
      if (fast && e == e_g) {
        candidate_nibbles(k, Su, w, pk);
      } else {
        if (fast) reload_block(wrow, w);  // w was prescaled
        nvfp4_cast_block(w, s, pk);
      }
      nvfp4_emit_at<kAll>(pk, s, k, o, qo.wq, qo.packed, qo.codes);
    }
    lds_row[tid] = row + rows_step;
    if (row + rows_step >= row_end) break;
    // The next row's weights are awaited here, after this row's stores (an
    // empty asm that takes them as operands): on every path to this point
    // the same stores follow the loads, so the wait need not cover them.
    wait_raw(raw);
    raw_to_float<T, kVec>(raw, w);
  }
  if constexpr (kQuant) {
    if (qo.gscale && L < qo.n_groups) qo.gscale[L] = amax[L] / kAmaxDivisor;  // S_g, once per group
  }
}


// ---------------------------------------------------------------------------
// The sweep with one input block per wave: lane i of a wave takes row
// chunk * 64 + i of the wave's (group, block b), and the wave walks chunks
// c0, c0 + cstep, ...  H_b, its certificate and gamma are then the same on
// every lane, and so are most of the skip decisions: rows of one block
// under one Hessian need similar candidates, so a wave pays less for its
// busiest lane than when its lanes hold 64 different blocks.  The H_b load
// is a broadcast (every lane reads the same 1 KiB).  Each lane does the work
// of sweep_kernel on its row with the same arithmetic, so the results are
// the same bits.  Lanes past the last row work on the last row and store
// nothing.
// ---------------------------------------------------------------------------
struct RowPlan {
  int64_t n_chunks;  // chunks of 64 rows
  int64_t cstep;     // waves per (group, block); cstep == n_chunks: one chunk per wave
  int64_t blocks;    // (group, block) pairs
};

// Workgroups go to the 8 XCDs in turn (workgroup id % 8), each XCD with its
// own L2.  The four input blocks 4q .. 4q+3 share each 128-byte line of a
// row of W, so the four waves on one chunk offset c0 of those blocks (a
// "unit", q * cstep + c0) read the same lines.  Spread over the XCDs, each
// line is read from HBM by up to four of them.  wave_unit keeps a unit's
// waves next to each other on one XCD and deals the units to the XCDs in
// turn; it returns false for the ids past the last block (the grid is whole
// units, a multiple of 8 of them).  wave_block is the plain order, the
// chunks of one block on consecutive ids.
constexpr int kXcds = 8;

__device__ __forceinline__ bool wave_unit(int64_t id, const RowPlan& rp, int64_t& gb, int64_t& c0) {
  const int64_t s = id / kXcds;
  const int64_t u = (id - s * kXcds) + kXcds * (s >> 2);
  const int64_t q = u / rp.cstep;
  c0 = u - q * rp.cstep;
  gb = 4 * q + (s & 3);
  return gb < rp.blocks;
}

int64_t unit_grid(const RowPlan& rp) {
  const int64_t units = (rp.blocks + 3) / 4 * rp.cstep;
  return (units + kXcds - 1) / kXcds * kXcds * 4;
}

__device__ __forceinline__ void wave_block(int64_t id, const RowPlan& rp, int64_t& gb, int64_t& c0) {
  gb = id / rp.cstep;
  c0 = id - gb * rp.cstep;
}

// Orders this wave's LDS accesses at this point: a workgroup here is one
// wave, whose LDS instructions execute in issue order, so only the compiler
// has to be kept from moving accesses across.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
// Pooled candidate rounds.  After a class's level-1 scan each lane holds the
// mask of candidates its row still needs, and the counts differ a lot between
// the rows of a wave (the busiest row needs about three times the mean).  So
// rather than each lane working through its own list, the wave lists every
// pending (row, power) item in LDS and evaluates them 64 at a time, each lane
// on any row: the rows of a wave share H_b and the skip certificate, and
// what else an item needs (the row's quotients for the class, its working
// weights, sigma and incumbent) is in LDS.  Items are listed by rank (every
// row's first pending power, then every row's second, ...), so a row's
// candidates still go in increasing index and later ones see the errors
// found before them.  Each row's best (error, index) is a 64-bit key in LDS
// that orders by the error's value, then by the index, and is lowered with an
// atomic min, so ties keep the lowest index.  Which candidates get evaluated
// depends on the incumbents at the time, but a candidate is only skipped when
// certified worse than an evaluated one, so the result is the exact minimum,
// the same bits as evaluating every candidate.
// ---------------------------------------------------------------------------
constexpr int kRowStride = 20;                   // floats per row in LDS (16 + 4 spreads rows over the banks)
constexpr int kMaxItems = kSweepThreads * 18;    // a class has at most 18 powers

struct __align__(16) PoolLds {
  float w[kSweepThreads * kRowStride];    // each lane's working weights
  float p[kSweepThreads * kRowStride];    // each row's quotients fl32(w / sigma) for the current class
  float sig[kSweepThreads];               // each row's sigma for the class (rows differ in working exponent)
  unsigned long long key[kSweepThreads];  // each row's best, as best_key()
  uint16_t items[kMaxItems];              // pending items: (row << 5) | power index
};

// An fp32 error's bits mapped to an unsigned order (negative values below
// positive ones), above the candidate index.
__device__ __forceinline__ unsigned long long best_key(float e, int k) {
  const uint32_t u = __float_as_uint(e);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (uint32_t)k;
}

__device__ __forceinline__ Best key_best(unsigned long long key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return Best{__uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o), (int)(uint32_t)key};
}

__device__ __forceinline__ void store_row(float* dst, const float (&v)[16]) {
  float4* d = reinterpret_cast<float4*>(dst);
#pragma unroll
  for (int q = 0; q < 4; ++q) d[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
}

__device__ __forceinline__ void load_row(const float* src, float (&v)[16]) {
  const float4* s = reinterpret_cast<const float4*>(src);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 f = s[q];
    v[4 * q] = f.x;
    v[4 * q + 1] = f.y;
    v[4 * q + 2] = f.z;
    v[4 * q + 3] = f.w;
  }
}

// The symmetrised strict upper triangle of H_b in LDS (shared by every lane
// of the wave, read as broadcasts), in the order of tri(): 30 float4.
// Same sum as quad_form_from, term for term: y_i starts at yd_i and takes
// S_ij dw_j for j = i+1 .. 15 in order, then E = sum_i dw_i y_i in order of
// i, so the result has the same bits.
__device__ __forceinline__ float quad_form_lds(const float (&yd)[16], const float4* __restrict__ S,
                                               const float (&dw)[16]) {
  float y[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = yd[i];
#pragma unroll
  for (int q = 0; q < 30; ++q) {
    const float4 f = S[q];
    const float v[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int k = 4 * q + c;
      // (i, j) of packed index k, resolved at compile time
      int i = 0;
      while (tri(i, 15) < k) ++i;
      const int j = k - tri(i, i + 1) + i + 1;
      y[i] = __builtin_fmaf(v[c], dw[j], y[i]);
    }
  }
  float e = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) e = __builtin_fmaf(dw[i], y[i], e);
  return e;
}

// Class m of the lane's row (working weights w, bound set t, units Su; its
// best in `best` and in L.key[tid] on entry and on return).  `live` is false
// for lanes past the last row: they list nothing.
template <int m>
__device__ __forceinline__ void sweep_class_pooled(PoolLds& L, int tid, bool live, Best& best, SkipSet& t,
                                                   float Su, const float (&w)[16], const float (&diag)[16],
                                                   const float4* __restrict__ S) {
  constexpr int jmin = ClassRange<m>::jmin;
  const float sigma = (1.0f + 0.125f * (float)m) * Su;  // fl32(mu * S_g) in the row's units
  const float rs = 1.0f / sigma;                        // IEEE division, once per class
  {
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = div_rn(w[i], sigma, rs);  // = fl32(w / sigma)
    store_row(&L.p[tid * kRowStride], p);
  }
  L.sig[tid] = sigma;
#pragma unroll
  for (int e = 0; e < 4; ++e) t.p[e] = div_rn(t.w[e], sigma, rs);  // same operation on the same bits as p[idx]
  uint32_t need = level1_scan<m>(best, t, sigma);
  if (!live) need = 0;
  // List the pending items by rank.
  int total = 0;
  for (uint32_t rem = need;;) {
    const uint64_t mask = __builtin_amdgcn_ballot_w64(rem != 0);
    if (mask == 0) break;
    if (rem != 0) {
      const int pos = total + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
      L.items[pos] = (uint16_t)((tid << 5) | __builtin_ctz(rem));
      rem &= rem - 1;
    }
    total += (int)__builtin_popcountll(mask);
  }
  // Rounds of 64 items; lanes past the end redo the last item and change
  // nothing.  Each round's row data is loaded during the round before (the
  // registers of the quotients and weights are free once the residual is
  // formed), so the LDS latency hides behind the quadratic form; the
  // incumbent is read at the top of its own round, after every earlier
  // round's atomic (a wave's LDS accesses complete in issue order).
  if (total == 0) return;
  wave_sync();  // the list and the rows are in place
  const int last = total - 1;
  uint32_t item = L.items[tid < total ? tid : last];
  uint32_t next = L.items[kSweepThreads + tid < total ? kSweepThreads + tid : last];
  float p[16], wo[16];
  load_row(&L.p[(item >> 5) * kRowStride], p);
  load_row(&L.w[(item >> 5) * kRowStride], wo);
  float sg = L.sig[item >> 5];
  for (int base = 0; base < total; base += kSweepThreads) {
    const bool has = base + tid < total;
    const int owner = (int)(item >> 5);
    const int j = jmin + (int)(item & 31u);
    // issued first: the incumbent (after every earlier round's atomic) and
    // the item two rounds ahead
    const unsigned long long okey = L.key[owner];
    const int nn = base + 2 * kSweepThreads + tid;
    const uint32_t after = L.items[nn < total ? nn : last];
    __builtin_amdgcn_sched_barrier(0);
    const float pow2j = __uint_as_float((uint32_t)(127 + j) << 23);
    uint32_t pk[2] = {0u, 0u};  // every byte is written below
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      pk[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[h], p[8 * h + 0], p[8 * h + 1], pow2j, 0);
      pk[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[h], p[8 * h + 2], p[8 * h + 3], pow2j, 1);
      pk[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[h], p[8 * h + 4], p[8 * h + 5], pow2j, 2);
      pk[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[h], p[8 * h + 6], p[8 * h + 7], pow2j, 3);
    }
    float dw[16];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x2_t r0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], pow2j, 0);
      const f32x2_t r1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], pow2j, 1);
      const f32x2_t r2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], pow2j, 2);
      const f32x2_t r3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[h], pow2j, 3);
      const float r[8] = {r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
#pragma unroll
      for (int i = 0; i < 8; ++i) dw[8 * h + i] = r[i] * sg - wo[8 * h + i];  // Q = fl32(r s), then Q - w
    }
    // the next round's rows, into the registers just freed
    item = next;
    next = after;
    load_row(&L.p[(item >> 5) * kRowStride], p);
    load_row(&L.w[(item >> 5) * kRowStride], wo);
    sg = L.sig[item >> 5];
    float yd[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) yd[i] = diag[i] * dw[i];
    float d2 = yd[0] * dw[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) d2 = __builtin_fmaf(yd[i], dw[i], d2);
    // level 2: the rest of the form only if some lane's item survives (a lane
    // without an item compares against -inf and never asks for it)
    const float thr = has ? key_best(okey).err * t.margin : -INFINITY;
    if (!wave_any(!(t.gamma * d2 > thr))) continue;
    const float e = quad_form_lds(yd, S, dw);
    // only a key below the one read at the top can lower the row's minimum
    const unsigned long long key = best_key(e, class_code(m, j) - 1);
    if (!(t.gamma * d2 > thr) && !isnan(e) && key < okey) atomicMin(&L.key[owner], key);
  }
  wave_sync();
  best = key_best(L.key[tid]);
}

template <typename T, bool kVec, bool kQuant, bool kAll>
__global__ __launch_bounds__(kSweepThreads, 3) void sweep_rows_kernel(const T* __restrict__ wt, int64_t c_out,
                                                              int64_t ld_w, int64_t gstride_w, int64_t nb,
                                                              RowPlan rp, const float* __restrict__ h,
                                                              int64_t gstride_h, const float* __restrict__ amax,
                                                              uint8_t* __restrict__ idx_out,
                                                              float* __restrict__ err_out,
                                                              float* __restrict__ amax_out,
                                                              const float* __restrict__ cert, QuantOut qo) {
  const int tid = threadIdx.x;
  if constexpr (kQuant) {
    const int64_t gl = (int64_t)blockIdx.x * kSweepThreads + tid;
    if (qo.gscale && gl < qo.n_groups) qo.gscale[gl] = amax[gl] / kAmaxDivisor;  // S_g, once per group
  }
  int64_t gb, c0;
  // block order: measured 1% faster here than wave_unit on a 5120 x 17408
  // layer, although wave_unit reads 43% fewer bytes on a 12288 x 4096 one
  wave_block((int64_t)blockIdx.x, rp, gb, c0);
  const int64_t grp = gb / nb;
  const int64_t b = gb - grp * nb;
  __shared__ PoolLds lds;  // rows, quotients, keys and items of the pooled rounds
  __shared__ float lds_diag[16];
  __shared__ float4 lds_sym[30];  // H_ij + H_ji, i < j, in the order of tri()
  const float* const hb = h + grp * gstride_h + b * 256;
  float diag[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) diag[i] = hb[17 * i];
  if (tid < 16) lds_diag[tid] = hb[17 * tid];
  for (int k = tid; k < 120; k += kSweepThreads) {
    int i = 0;
    while (tri(i, 15) < k) ++i;
    const int j = k - tri(i, i + 1) + i + 1;
    reinterpret_cast<float*>(lds_sym)[k] = hb[16 * i + j] + hb[16 * j + i];
  }
  wave_sync();
  float gamma;
  if (cert) {
    gamma = cert[gb];
  } else {
    float sym[120];
#pragma unroll
    for (int k = 0; k < 120; ++k) sym[k] = reinterpret_cast<const float*>(lds_sym)[k];
    gamma = gershgorin_gamma(diag, sym);
  }
  const float g = amax[grp];
  const float Sg = g / kAmaxDivisor;
  const bool fast = (Sg >= 0x1p-117f) && (Sg <= 0x1p127f);
  const int e_g = (Sg > 0.0f && Sg <= 0x1p127f) ? ilogbf(Sg) : 0;
  wave_sync();
  const T* const wblk = wt + grp * gstride_w + 16 * b;
  uint32_t raw[16];
  load_raw<T, kVec>(wblk + (c0 * kSweepThreads + tid < c_out ? c0 * kSweepThreads + tid : c_out - 1) * ld_w, raw);
  wait_raw(raw);
  float w[16];
  raw_to_float<T, kVec>(raw, w);
  for (int64_t chunk = c0;;) {
    const int64_t row = chunk * kSweepThreads + tid;
    const bool valid = row < c_out;
    const int64_t rr = valid ? row : c_out - 1;
    const T* const wrow = wblk + rr * ld_w;
    const int e = row_exponent(e_g, w);
    const float Su = ldexpf(Sg, -e);
    Best best{INFINITY, kCandidates};
    uint32_t pk[2] = {0u, 0u};
    if (fast) {
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i] = ldexpf(w[i], -e);
      SkipSet t;
      {
        float kv[4] = {-1.0f, -1.0f, -1.0f, -1.0f};
        int ki[4] = {0, 1, 2, 3};
        wave_sync();  // the previous chunk's readers of the rows are done
        store_row(&lds.w[tid * kRowStride], w);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float key = diag[i] * w[i] * w[i];
          const bool q0 = key > kv[0], q1 = key > kv[1], q2 = key > kv[2], q3 = key > kv[3];
          kv[3] = q2 ? kv[2] : (q3 ? key : kv[3]);
          ki[3] = q2 ? ki[2] : (q3 ? i : ki[3]);
          kv[2] = q1 ? kv[1] : (q2 ? key : kv[2]);
          ki[2] = q1 ? ki[1] : (q2 ? i : ki[2]);
          kv[1] = q0 ? kv[0] : (q1 ? key : kv[1]);
          ki[1] = q0 ? ki[0] : (q1 ? i : ki[1]);
          kv[0] = q0 ? key : kv[0];
          ki[0] = q0 ? i : ki[0];
        }
        wave_sync();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          t.w[q] = lds.w[tid * kRowStride + ki[q]];
          t.dg[q] = gamma * lds_diag[ki[q]];
        }
        t.pk = 0u;
        t.gamma = gamma;
        t.margin = gamma > 0.0f ? kSkipMargin : __int_as_float(0x7FC00000);
      }
      {
        const int k0 = max_scaling_candidate(w, Su);
        int m0, j0;
        candidate_class(k0, m0, j0);
        const float sigma0 = (1.0f + 0.125f * (float)m0) * Su;
        const float rs0 = 1.0f / sigma0;
        float p0[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) p0[i] = div_rn(w[i], sigma0, rs0);
        // the incumbent: the max-scaling candidate, with the arithmetic of the rounds
        const float pow2j = __uint_as_float((uint32_t)(127 + j0) << 23);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          pk[hh] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[hh], p0[8 * hh + 0], p0[8 * hh + 1], pow2j, 0);
          pk[hh] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[hh], p0[8 * hh + 2], p0[8 * hh + 3], pow2j, 1);
          pk[hh] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[hh], p0[8 * hh + 4], p0[8 * hh + 5], pow2j, 2);
          pk[hh] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[hh], p0[8 * hh + 6], p0[8 * hh + 7], pow2j, 3);
        }
        float dw0[16], yd0[16];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const f32x2_t r0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[hh], pow2j, 0);
          const f32x2_t r1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[hh], pow2j, 1);
          const f32x2_t r2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[hh], pow2j, 2);
          const f32x2_t r3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pk[hh], pow2j, 3);
          const float r[8] = {r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
#pragma unroll
          for (int i = 0; i < 8; ++i) dw0[8 * hh + i] = r[i] * sigma0 - w[8 * hh + i];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) yd0[i] = diag[i] * dw0[i];
        keep_best(best, quad_form_lds(yd0, lds_sym, dw0), k0);
      }
      lds.key[tid] = best_key(best.err, best.k);
      sweep_class_pooled<0>(lds, tid, valid, best, t, Su, w, diag, lds_sym);
      sweep_class_pooled<1>(lds, tid, valid, best, t, Su, w, diag, lds_sym);
      sweep_class_pooled<2>(lds, tid, valid, best, t, Su, w, diag, lds_sym);
      sweep_class_pooled<3>(lds, tid, valid, best, t, Su, w, diag, lds_sym);
      sweep_class_pooled<4>(lds, tid, valid, best, t, Su, w, diag, lds_sym);
      sweep_class_pooled<5>(lds, tid, valid, best, t, Su, w, diag, lds_sym);
      sweep_class_pooled<6>(lds, tid, valid, best, t, Su, w, diag, lds_sym);
      sweep_class_pooled<7>(lds, tid, valid, best, t, Su, w, diag, lds_sym);
    } else {
      // subnormal candidate scales: the definition, per candidate (see eval_direct)
      for (int k = 0; k < kCandidates; ++k) {
        const float sk = e4m3_candidate(k) * Sg;
        float dw[16], yd[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = (sk == 0.0f) ? 0.0f : fabsf(w[i]) / sk;
          const float q = copysignf(e2m1_round_mag(x) * sk, w[i]);
          dw[i] = ldexpf(q - w[i], -e);
          yd[i] = diag[i] * dw[i];
        }
        keep_best(best, quad_form_lds(yd, lds_sym, dw), k);
      }
    }
    // Past the last chunk: stores for the valid lanes, done.  Otherwise the
    // next chunk's weights are loaded before this chunk's stores and awaited
    // after them (wait_raw): a wait for a load also waits for every store
    // issued before it, and with the same stores on every path in between
    // the compiler's wait leaves them in flight.  Only the last chunk of a
    // block can hold lanes past the last row, so the stores of the other
    // chunks are unconditional.
    const int64_t next = chunk + rp.cstep;
    const bool last = next >= rp.n_chunks;  // uniform over the wave
    auto emit = [&]() {
      const int k = best.k < kCandidates ? best.k : 0;  // NaN errors only
      const int64_t o = (grp * c_out + rr) * nb + b;
      idx_out[o] = (uint8_t)k;
      if (kAll || err_out) err_out[o] = ldexpf(best.err, 2 * e);
      if (kAll || amax_out) amax_out[o] = 6.0f * (e4m3_candidate(k) * Sg);
      if constexpr (kQuant) {
        const float s = e4m3_candidate(k) * Sg;
        uint32_t qk[2];
        if (fast && e == e_g) {
          candidate_nibbles(k, Su, w, qk);
        } else {
          if (fast) reload_block(wrow, w);  // w was prescaled
          nvfp4_cast_block(w, s, qk);
        }
        nvfp4_emit_at<kAll>(qk, s, k, o, qo.wq, qo.packed, qo.codes);
      }
    };
    if (last) {
      if (valid) emit();
      break;
    }
    const int64_t nrow = next * kSweepThreads + tid;
    load_raw<T, kVec>(wblk + (nrow < c_out ? nrow : c_out - 1) * ld_w, raw);
    emit();
    chunk = next;
    wait_raw(raw);
    raw_to_float<T, kVec>(raw, w);
  }
}

// The same sweep with each lane working through its own row's candidates
// (sweep_mantissa) and H_b in registers, two waves per SIMD: for layers
// whose waves walk several chunks of rows (fewer than 32 chunks per input
// block), where the rows of a wave need similar numbers of candidates and
// most evaluations run the full form, it measured faster than the pooled
// rounds (which read H_b from LDS in every full form).  Same results, bit
// for bit.  Waves in unit order: on 64 experts of 1024 x 2048 it reads 1.14x
// the bytes of W and H instead of 2.1x, in the same time.
template <typename T, bool kVec, bool kQuant, bool kAll>
__global__ __launch_bounds__(kSweepThreads, 2) void sweep_rows_own_kernel(const T* __restrict__ wt, int64_t c_out,
                                                              int64_t ld_w, int64_t gstride_w, int64_t nb,
                                                              RowPlan rp, const float* __restrict__ h,
                                                              int64_t gstride_h, const float* __restrict__ amax,
                                                              uint8_t* __restrict__ idx_out,
                                                              float* __restrict__ err_out,
                                                              float* __restrict__ amax_out,
                                                              const float* __restrict__ cert, QuantOut qo) {
  const int tid = threadIdx.x;
  if constexpr (kQuant) {
    const int64_t gl = (int64_t)blockIdx.x * kSweepThreads + tid;
    if (qo.gscale && gl < qo.n_groups) qo.gscale[gl] = amax[gl] / kAmaxDivisor;  // S_g, once per group
  }
  int64_t gb, c0;
  if (!wave_unit((int64_t)blockIdx.x, rp, gb, c0)) return;  // the whole (one-wave) workgroup
  const int64_t grp = gb / nb;
  const int64_t b = gb - grp * nb;
  __shared__ float lds_w[16][kSweepThreads];  // the lanes' working weights (bound-set gather)
  __shared__ float lds_diag[16];
  float diag[16], sym[120];
  // The same address on every lane; a zero the compiler cannot see as
  // uniform keeps the 136 values in vector registers (scalar registers
  // cannot hold them, and spilled ones would cost a read-lane per use).
  int zero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
  load_hessian(h + grp * gstride_h + b * 256 + zero, diag, sym);
  if (tid < 16) lds_diag[tid] = h[grp * gstride_h + b * 256 + tid * 17];
  const float gamma = cert ? cert[gb] : gershgorin_gamma(diag, sym);
  const float g = amax[grp];
  const float Sg = g / kAmaxDivisor;
  const bool fast = (Sg >= 0x1p-117f) && (Sg <= 0x1p127f);
  const int e_g = (Sg > 0.0f && Sg <= 0x1p127f) ? ilogbf(Sg) : 0;
  wave_sync();
  const T* const wblk = wt + grp * gstride_w + 16 * b;
  uint32_t raw[16];
  load_raw<T, kVec>(wblk + (c0 * kSweepThreads + tid < c_out ? c0 * kSweepThreads + tid : c_out - 1) * ld_w, raw);
  wait_raw(raw);
  float w[16];
  raw_to_float<T, kVec>(raw, w);
  for (int64_t chunk = c0;;) {
    const int64_t row = chunk * kSweepThreads + tid;
    const bool valid = row < c_out;
    const int64_t rr = valid ? row : c_out - 1;
    const T* const wrow = wblk + rr * ld_w;
    const int e = row_exponent(e_g, w);
    const float Su = ldexpf(Sg, -e);
    Best best{INFINITY, kCandidates};
    uint32_t pk[2] = {0u, 0u};
    if (fast) {
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i] = ldexpf(w[i], -e);
      SkipSet t;
      {
        float kv[4] = {-1.0f, -1.0f, -1.0f, -1.0f};
        int ki[4] = {0, 1, 2, 3};
        wave_sync();  // the previous chunk's readers of lds_w are done
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          lds_w[i][tid] = w[i];
          const float key = diag[i] * w[i] * w[i];
          const bool q0 = key > kv[0], q1 = key > kv[1], q2 = key > kv[2], q3 = key > kv[3];
          kv[3] = q2 ? kv[2] : (q3 ? key : kv[3]);
          ki[3] = q2 ? ki[2] : (q3 ? i : ki[3]);
          kv[2] = q1 ? kv[1] : (q2 ? key : kv[2]);
          ki[2] = q1 ? ki[1] : (q2 ? i : ki[2]);
          kv[1] = q0 ? kv[0] : (q1 ? key : kv[1]);
          ki[1] = q0 ? ki[0] : (q1 ? i : ki[1]);
          kv[0] = q0 ? key : kv[0];
          ki[0] = q0 ? i : ki[0];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          t.w[q] = lds_w[ki[q]][tid];
          t.dg[q] = gamma * lds_diag[ki[q]];
        }
        t.pk = 0u;
        t.gamma = gamma;
        t.margin = gamma > 0.0f ? kSkipMargin : __int_as_float(0x7FC00000);
      }
      {
        const int k0 = max_scaling_candidate(w, Su);
        int m0, j0;
        candidate_class(k0, m0, j0);
        const float sigma0 = (1.0f + 0.125f * (float)m0) * Su;
        const float rs0 = 1.0f / sigma0;
        float p0[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) p0[i] = div_rn(w[i], sigma0, rs0);
        eval_scaled<false>(best, k0, j0, sigma0, p0, w, diag, sym, pk);
      }
      sweep_mantissa<0, false>(best, t, Su, w, diag, sym, pk);
      sweep_mantissa<1, false>(best, t, Su, w, diag, sym, pk);
      sweep_mantissa<2, false>(best, t, Su, w, diag, sym, pk);
      sweep_mantissa<3, false>(best, t, Su, w, diag, sym, pk);
      sweep_mantissa<4, false>(best, t, Su, w, diag, sym, pk);
      sweep_mantissa<5, false>(best, t, Su, w, diag, sym, pk);
      sweep_mantissa<6, false>(best, t, Su, w, diag, sym, pk);
      sweep_mantissa<7, false>(best, t, Su, w, diag, sym, pk);
    } else {
      for (int k = 0; k < kCandidates; ++k) eval_direct<false>(best, k, Sg, e, w, diag, sym);
    }
    // Past the last chunk: stores for the valid lanes, done.  Otherwise the
    // next chunk's weights are loaded before this chunk's stores and awaited
    // after them (wait_raw): a wait for a load also waits for every store
    // issued before it, and with the same stores on every path in between
    // the compiler's wait leaves them in flight.  Only the last chunk of a
    // block can hold lanes past the last row, so the stores of the other
    // chunks are unconditional.
    const int64_t next = chunk + rp.cstep;
    const bool last = next >= rp.n_chunks;  // uniform over the wave
    auto emit = [&]() {
      const int k = best.k < kCandidates ? best.k : 0;  // NaN errors only
      const int64_t o = (grp * c_out + rr) * nb + b;
      idx_out[o] = (uint8_t)k;
      if (kAll || err_out) err_out[o] = ldexpf(best.err, 2 * e);
      if (kAll || amax_out) amax_out[o] = 6.0f * (e4m3_candidate(k) * Sg);
      if constexpr (kQuant) {
        const float s = e4m3_candidate(k) * Sg;
        uint32_t qk[2];
        if (fast && e == e_g) {
          candidate_nibbles(k, Su, w, qk);
        } else {
          if (fast) reload_block(wrow, w);  // w was prescaled
          nvfp4_cast_block(w, s, qk);
        }
        nvfp4_emit_at<kAll>(qk, s, k, o, qo.wq, qo.packed, qo.codes);
      }
    };
    if (last) {
      if (valid) emit();
      break;
    }
    const int64_t nrow = next * kSweepThreads + tid;
    load_raw<T, kVec>(wblk + (nrow < c_out ? nrow : c_out - 1) * ld_w, raw);
    emit();
    chunk = next;
    wait_raw(raw);
    raw_to_float<T, kVec>(raw, w);
  }
}

// ---------------------------------------------------------------------------
// Scale rules other than the 126-value sweep ("Local-Hessian weight-scale
// guide", "What is Local-Hessian": max scaling from the block's largest |w|,
// Four-Over-Six choosing between two candidate scales by the in-block error;
// "Entry API and calibration flow": the amax search from multiplier 0.25 to
// 4.0 in steps of 0.1).  A wanted block scale t (in units of S_g) is stored
// as the nearest positive finite E4M3 value, ties to the even code,
// saturating at 448 and never zero.  Candidates: max t = fl32(fl32(a/6)/S_g)
// with a = max|w|; Four-Over-Six adds t = fl32(fl32(a/4)/S_g); the amax
// search takes a_i = fl32(m_i a), m_i = fl32((25 + 10 i) / 100), i < 38.
// The objective is dw^T H dw, or sum dw^2 without a Hessian.  S_g = 0
// selects candidate 0 (every Q is 0).
// ---------------------------------------------------------------------------

// E4M3 byte (1..126) stored for a wanted positive scale value t.
__device__ __forceinline__ int e4m3_store_code(float t) {
  if (!(t > 0.0f)) return 1;
  if (t >= 448.0f) return 126;
  int code;
  if (t < 0x1p-6f) {
    code = (int)rintf(t * 512.0f);  // subnormal step 2^-9; ties to the even code
  } else {
    const int E = ilogbf(t);                  // -6 .. 8
    const float mfrac = ldexpf(t, -E) - 1.0f;  // [0, 1), exact
    code = (E + 7) * 8 + (int)rintf(mfrac * 8.0f);  // a rounded-up 8 carries into the next binade
  }
  return code < 1 ? 1 : (code > kCandidates ? kCandidates : code);
}

// Candidate set of one block as a 128-bit mask (bit k = candidate k).
__device__ __forceinline__ void rule_mask(int rule, float a, float Sg, uint64_t (&mask)[2]) {
  mask[0] = mask[1] = 0;
  auto add = [&](int k) {
    if (k < 64) mask[0] |= 1ull << k;
    else mask[1] |= 1ull << (k - 64);
  };
  if (!(Sg > 0.0f)) {
    add(0);
    return;
  }
  if (rule == 3) {
    for (int i = 0; i < 38; ++i) {
      const float m = (float)((double)(25 + 10 * i) / 100.0);
      add(e4m3_store_code((m * a / 6.0f) / Sg) - 1);
    }
    return;
  }
  add(e4m3_store_code((a / 6.0f) / Sg) - 1);
  if (rule == 2) add(e4m3_store_code((a / 4.0f) / Sg) - 1);
}

template <typename T, bool kVec, bool kMse>
__global__ __launch_bounds__(kThreads) void select_kernel(int rule, const T* __restrict__ wt, int64_t c_out,
                                                          int64_t ld_w, int64_t gstride_w, int64_t nb,
                                                          int64_t rows_step, int64_t lanes,
                                                          const float* __restrict__ h, int64_t gstride_h,
                                                          const float* __restrict__ amax,
                                                          uint8_t* __restrict__ idx_out,
                                                          float* __restrict__ err_out,
                                                          float* __restrict__ amax_out) {
  const int64_t L = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (L >= lanes) return;
  // With H, rows fastest: the lanes of a wave share their block (rows_step
  // >= 64), so its Hessian load is one broadcast per wave instead of 64
  // blocks' (dense-4096: max 61 -> 46 us, Four-Over-Six 76 -> 62 us).
  // Without H, blocks fastest: a wave's weight loads are then contiguous
  // (the plain-MSE forms were 7-32% slower with rows fastest).
  const int64_t per_group = nb * rows_step;
  const int64_t grp = L / per_group;
  const int64_t rem = L - grp * per_group;
  const int64_t b = kMse ? rem % nb : rem / rows_step;
  const int64_t row0 = kMse ? rem / nb : rem - b * rows_step;

  float diag[16], sym[120];
  if constexpr (kMse) {
#pragma unroll
    for (int i = 0; i < 16; ++i) diag[i] = 1.0f;
  } else {
    load_hessian(h + grp * gstride_h + b * 256, diag, sym);
  }
  const float g = amax[grp];
  const float Sg = g / kAmaxDivisor;
  const int e_g = (Sg > 0.0f && Sg <= 0x1p127f) ? ilogbf(Sg) : 0;
  const bool fast = (Sg >= 0x1p-117f) && (Sg <= 0x1p127f);

  // each row's weights are loaded while the previous row is evaluated
  // (row0 < rows_step <= c_out; past the last row the last row is loaded again)
  const T* const wcol = wt + grp * gstride_w + 16 * b;
  uint32_t raw[16];
  load_raw<T, kVec>(wcol + row0 * ld_w, raw);
  for (int64_t row = row0; row < c_out; row += rows_step) {
    wait_raw(raw);
    float w[16];
    raw_to_float<T, kVec>(raw, w);
    load_raw<T, kVec>(wcol + (row + rows_step < c_out ? row + rows_step : row) * ld_w, raw);
    const int e = row_exponent(e_g, w);
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(w[i]));
    uint64_t mask[2];
    rule_mask(rule, a, Sg, mask);
    Best best{INFINITY, kCandidates};
    // In the sweep's fast range (normal candidate scales) each candidate is
    // evaluated with the sweep's own arithmetic: weights in units of 2^e, the
    // quotient by sigma = mu S_g of its mantissa class (reciprocal and two
    // fma), the scaled hardware cast at 2^j; these give the definition's
    // bits, as the sweep does (eval_direct: an IEEE division and a software
    // rounding per weight, kept for subnormal candidate scales).
    float ws[16];
    const float Su = ldexpf(Sg, -e);
    if (fast) {
#pragma unroll
      for (int i = 0; i < 16; ++i) ws[i] = ldexpf(w[i], -e);
    }
    uint32_t pk[2] = {0u, 0u};
    // ascending candidate order; lanes leave the loop when their mask is empty
    while ((mask[0] | mask[1]) != 0) {
      int k;
      if (mask[0] != 0) {
        k = __builtin_ctzll(mask[0]);
        mask[0] &= mask[0] - 1;
      } else {
        k = 64 + __builtin_ctzll(mask[1]);
        mask[1] &= mask[1] - 1;
      }
      if (fast) {
        int m, j;
        candidate_class(k, m, j);
        const float sigma = (1.0f + 0.125f * (float)m) * Su;
        const float rs = 1.0f / sigma;
        float p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) p[i] = div_rn(ws[i], sigma, rs);
        eval_scaled<kMse>(best, k, j, sigma, p, ws, diag, sym, pk);
      } else {
        eval_direct<kMse>(best, k, Sg, e, w, diag, sym);
      }
    }
    const int k = best.k < kCandidates ? best.k : 0;  // NaN errors only
    const int64_t o = (grp * c_out + row) * nb + b;
    idx_out[o] = (uint8_t)k;
    if (err_out) err_out[o] = ldexpf(best.err, 2 * e);
    if (amax_out) amax_out[o] = 6.0f * (e4m3_candidate(k) * Sg);
  }
}

// The 126-value sweep's lanes: about sixteen rounds of lanes at two waves per
// SIMD on 256 CUs, so that waves of unequal work pack well, with at least
// three rows per lane (its Hessian load and certificate are paid once per
// walk); the last rows, up to four rounds' worth and at most a quarter of
// them, go to lanes of one row each (measured: 1-3% faster on the larger
// layers, no change on 4096 x 4096).
LanePlan sweep_lane_plan(int64_t c_out, int64_t per_k) {
  const int64_t round = 256LL * 4 * 2 * 64;
  int64_t p = (c_out * per_k + 16 * round - 1) / (16 * round);
  p = (p < 2 ? 2 : p) + 1;
  int64_t rows_b = 4 * round / per_k;
  if (rows_b > c_out / 4) rows_b = c_out / 4;
  const int64_t rows_a = c_out - rows_b;  // >= 1 when c_out >= 1
  if (p > rows_a) p = rows_a > 0 ? rows_a : 1;
  LanePlan lp;
  lp.rows_a = rows_a;
  lp.step_a = rows_a > 0 ? (rows_a + p - 1) / p : 1;
  lp.lanes_a = rows_a > 0 ? per_k * lp.step_a : 0;
  lp.waves_a = (lp.lanes_a + kSweepThreads - 1) / kSweepThreads;
  lp.step_b = rows_b > 0 ? rows_b : 1;
  lp.lanes_b = rows_b > 0 ? per_k * rows_b : 0;
  lp.waves = lp.waves_a + (lp.lanes_b + kSweepThreads - 1) / kSweepThreads;
  return lp;
}

// The row-per-lane sweep's waves.  With at least 32 chunks of rows per
// block, one chunk per wave (measured best on 4096 and 5120 rows); with
// fewer, about sixteen rounds of waves at two waves per SIMD on 256 CUs,
// each walking every cstep-th chunk of its block, so that its Hessian load
// serves several chunks (measured best on 1024 rows).
RowPlan row_plan(int64_t c_out, int64_t per_k) {
  RowPlan rp;
  rp.blocks = per_k;
  rp.n_chunks = (c_out + kSweepThreads - 1) / kSweepThreads;
  const int64_t target = 256LL * 4 * 2 * 16;
  int64_t cs = (target + per_k - 1) / per_k;
  if (cs > rp.n_chunks || rp.n_chunks >= 32) cs = rp.n_chunks;
  rp.cstep = cs < 1 ? 1 : cs;
  return rp;
}

template <typename T, bool kVec, bool kQuant, bool kAll>
void launch_rows(bool pooled, dim3 grid, hipStream_t stream, const T* wp, const SweepArgs& a, int64_t nb,
                 const RowPlan& rp, const float* cert, const QuantOut& qo) {
  if (pooled)
    sweep_rows_kernel<T, kVec, kQuant, kAll><<<grid, dim3(kSweepThreads), 0, stream>>>(
        wp, a.c_out, a.ld_w, a.gstride_w, nb, rp, a.h, a.gstride_h, a.amax, a.idx, a.err, a.best_amax, cert, qo);
  else
    sweep_rows_own_kernel<T, kVec, kQuant, kAll><<<grid, dim3(kSweepThreads), 0, stream>>>(
        wp, a.c_out, a.ld_w, a.gstride_w, nb, rp, a.h, a.gstride_h, a.amax, a.idx, a.err, a.best_amax, cert, qo);
}

template <typename T, bool kVec>
hipError_t launch_sweep_typed(const SweepArgs& a, hipStream_t stream) {
  const int64_t nb = a.c_in / 16;
  const int64_t per_k = a.n_groups * nb;
  const bool mse = a.h == nullptr;
  if (a.rule != 0) {
    // Few candidates per row: two rounds of lanes at two waves per SIMD, so
    // that each lane's Hessian load serves as many rows as possible.
    const int64_t target = 256LL * 4 * 2 * 64 * 2;
    int64_t k = (target + per_k - 1) / per_k;
    if (k > a.c_out) k = a.c_out;
    const int64_t rows_per_lane = (a.c_out + k - 1) / k;
    k = (a.c_out + rows_per_lane - 1) / rows_per_lane;
    const int64_t lanes = per_k * k;
    const int64_t grid = (lanes + kThreads - 1) / kThreads;
    if (mse)
      select_kernel<T, kVec, true><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
          a.rule, static_cast<const T*>(a.w), a.c_out, a.ld_w, a.gstride_w, nb, k, lanes, nullptr, 0, a.amax,
          a.idx, a.err, a.best_amax);
    else
      select_kernel<T, kVec, false><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
          a.rule, static_cast<const T*>(a.w), a.c_out, a.ld_w, a.gstride_w, nb, k, lanes, a.h, a.gstride_h,
          a.amax, a.idx, a.err, a.best_amax);
    return hipGetLastError();
  }
  const LanePlan lp = sweep_lane_plan(a.c_out, per_k);
  const int64_t sgrid = lp.waves;
  const QuantOut qo{a.wq, a.packed, a.codes, a.gscale, a.n_groups};
  const bool quant = a.wq || a.packed || a.codes || a.gscale;
  if (mse) {
    if (quant)
      sweep_kernel<T, kVec, true, true><<<dim3((unsigned)sgrid), dim3(kSweepThreads), 0, stream>>>(
          static_cast<const T*>(a.w), a.c_out, a.ld_w, a.gstride_w, nb, lp, nullptr, 0, a.amax, a.idx,
          a.err, a.best_amax, nullptr, qo);
    else
      sweep_kernel<T, kVec, true, false><<<dim3((unsigned)sgrid), dim3(kSweepThreads), 0, stream>>>(
          static_cast<const T*>(a.w), a.c_out, a.ld_w, a.gstride_w, nb, lp, nullptr, 0, a.amax, a.idx,
          a.err, a.best_amax, nullptr, qo);
    return hipGetLastError();
  }
  float* cert = nullptr;
  if (a.cert_ready) {
    cert = static_cast<float*>(a.ws);  // certificates already written (finalize_certify_kernel)
  } else if (a.ws != nullptr && a.ws_bytes >= sweep_ws_bytes(a.c_in, a.n_groups)) {
    cert = static_cast<float*>(a.ws);
    hipError_t e = launch_certificate(a.h, a.gstride_h, a.c_in, a.n_groups, cert, stream);
    if (e != hipSuccess) return e;
  }
  // With a Hessian, the row-per-lane kernel; kAll: every optional per-block
  // output requested (the fake-quant's too, with them), no null checks.
  const bool all = a.err && a.best_amax && a.wq && a.packed && a.codes;
  const RowPlan rp = row_plan(a.c_out, per_k);
  const T* wp = static_cast<const T*>(a.w);
  // One chunk of rows per wave: the pooled rounds; several (small c_out):
  // each lane through its own candidates (measured faster there).
  const bool pooled = rp.cstep == rp.n_chunks;
  const dim3 rgrid((unsigned)(pooled ? per_k * rp.cstep : unit_grid(rp)));
  if (quant && all)
    launch_rows<T, kVec, true, true>(pooled, rgrid, stream, wp, a, nb, rp, cert, qo);
  else if (quant)
    launch_rows<T, kVec, true, false>(pooled, rgrid, stream, wp, a, nb, rp, cert, qo);
  else if (a.err && a.best_amax)
    launch_rows<T, kVec, false, true>(pooled, rgrid, stream, wp, a, nb, rp, cert, qo);
  else
    launch_rows<T, kVec, false, false>(pooled, rgrid, stream, wp, a, nb, rp, cert, qo);
  return hipGetLastError();
}

}  // namespace

size_t sweep_ws_bytes(int64_t c_in, int64_t n_groups) {
  return (size_t)n_groups * (size_t)(c_in / 16) * sizeof(float);
}

bool finalize_certifies(int64_t blocks) { return blocks <= kCertTeamMaxBlocks; }

hipError_t launch_certificate(const float* h, int64_t gstride_h, int64_t c_in, int64_t n_groups, float* cert,
                              hipStream_t stream) {
  const int64_t nb = c_in / 16, per_k = n_groups * nb;
  if (per_k == 0) return hipSuccess;
  if (per_k <= kCertTeamMaxBlocks)
    sweep_certificate_team_kernel<<<dim3((unsigned)per_k), dim3(kThreads), 0, stream>>>(h, gstride_h, nb, cert);
  else
    sweep_certificate_lane_kernel<<<dim3((unsigned)((per_k + kThreads / 16 - 1) / (kThreads / 16))), dim3(kThreads), 0,
                                    stream>>>(h, gstride_h, nb, per_k, cert);
  return hipGetLastError();
}

hipError_t launch_finalize_certify(const FinalizeCertifyArgs& a, hipStream_t stream) {
  const int64_t nb = a.c_in / 16;
  const int64_t blocks = a.n_groups * nb;
  // beyond kCertTeamMaxBlocks the sweep's own lane pre-pass is the faster certificate
  float* cert = finalize_certifies(blocks) ? a.cert : nullptr;
  finalize_certify_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(
      a.h_part, a.nsplit, a.n_groups, nb, a.alpha, a.h, a.h_gstride, cert, a.abs_part, a.abs_per_group, a.amax);
  return hipGetLastError();
}

hipError_t launch_sweep(const SweepArgs& a, hipStream_t stream) {
  if (a.n_groups == 0 || a.c_out == 0 || a.c_in == 0) return hipSuccess;
  const int64_t esz = a.dtype == 1 ? 2 : 4;
  const int64_t epv = 16 / esz;
  const bool aligned = (reinterpret_cast<uintptr_t>(a.w) % 16 == 0) && (a.ld_w % epv == 0) &&
                       (a.gstride_w % epv == 0);
  const bool h_aligned = a.h == nullptr || ((reinterpret_cast<uintptr_t>(a.h) % 16 == 0) && (a.gstride_h % 4 == 0));
  if (!h_aligned) return hipErrorInvalidValue;  // rejected earlier by the front end
  if (a.dtype == 1)
    return aligned ? launch_sweep_typed<uint16_t, true>(a, stream) : launch_sweep_typed<uint16_t, false>(a, stream);
  return aligned ? launch_sweep_typed<float, true>(a, stream) : launch_sweep_typed<float, false>(a, stream);
}

}  // namespace lh
