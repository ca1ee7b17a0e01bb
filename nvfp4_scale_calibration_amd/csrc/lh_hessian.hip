// lh_hessian.hip - local Hessian accumulation on CDNA4 matrix cores.
//
// "Local-Hessian weight-scale guide" (xxmr.cn/news/266017), "Algorithm
// principle": for input block b the local Hessian is X_b X_b^T (16 x 16),
// X_b = the 16 rows of X [C_in x N] that multiply weight block b; "Entry API
// and calibration flow", phase 2: H accumulates the sum of X^T X over the
// calibration tokens and is normalised before the search.
//
//   h[g][b] = beta * h[g][b] + alpha * X_b X_b^T
//
// Design: one 256-thread workgroup (4 wave64s) per (group, block, token
// slice).  The contraction over tokens runs on MFMA with fp32 accumulation:
// v_mfma_f32_16x16x32_bf16 for bf16 X, v_mfma_f32_16x16x4_f32 for fp32 X.
// For H = X_b X_b^T the A operand (16 channels x K tokens) and the B operand
// (its transpose) hold the same values in each lane (lane l: channel l%16,
// K-slot group l/16), so one register set feeds both.  The token order inside
// a K step is free (a sum), which lets each lane read 16 contiguous tokens
// (channel-major) or a bank-conflict-free LDS column (token-major).
// The four waves of a workgroup reduce in LDS in a fixed order; token slices
// of one block reduce in a second kernel in a fixed order: results do not
// depend on timing.
#include "lh_device.h"
#include "lh_internal.h"

namespace lh {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int kSlab = 64;                 // tokens per wave per step
constexpr int kRound = kSlab * 4;         // tokens per workgroup per step

// Sixteen token values of one channel, in the lane's register layout.
template <typename T>
struct Vals16;
template <>
struct Vals16<uint16_t> {
  uint4 u[2];  // 16 bf16
};
template <>
struct Vals16<float> {
  float f[16];
};

__device__ __forceinline__ f32x4_t mfma_accumulate(const Vals16<uint16_t>& v, f32x4_t acc) {
  const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, v.u[0]);
  const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, v.u[1]);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, a0, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, a1, acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ f32x4_t mfma_accumulate(const Vals16<float>& v, f32x4_t acc) {
#pragma unroll
  for (int i = 0; i < 16; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v.f[i], v.f[i], acc, 0, 0, 0);
  return acc;
}

// Channel-major: lane reads tokens [tb, tb+16) of its channel row.  With
// kInRange the caller guarantees tb + 16 <= t1.
template <bool kVec, bool kInRange = false>
__device__ __forceinline__ void load_cm(const uint16_t* row, int64_t tb, int64_t t1, Vals16<uint16_t>& v) {
  if (kVec && (kInRange || tb + 16 <= t1)) {
    v.u[0] = *reinterpret_cast<const uint4*>(row + tb);
    v.u[1] = *reinterpret_cast<const uint4*>(row + tb + 8);
  } else {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t lo = (tb + 2 * i < t1) ? row[tb + 2 * i] : 0u;
      const uint32_t hi = (tb + 2 * i + 1 < t1) ? row[tb + 2 * i + 1] : 0u;
      w[i] = lo | (hi << 16);
    }
    v.u[0] = make_uint4(w[0], w[1], w[2], w[3]);
    v.u[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

template <bool kVec, bool kInRange = false>
__device__ __forceinline__ void load_cm(const float* row, int64_t tb, int64_t t1, Vals16<float>& v) {
  if (kVec && (kInRange || tb + 16 <= t1)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = *reinterpret_cast<const float4*>(row + tb + 4 * q);
      v.f[4 * q + 0] = f.x;
      v.f[4 * q + 1] = f.y;
      v.f[4 * q + 2] = f.z;
      v.f[4 * q + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v.f[i] = (tb + i < t1) ? row[tb + i] : 0.0f;
  }
}

// ---------------------------------------------------------------------------
// Channel-major kernel: x[(16b + c) * ld + t].
// ---------------------------------------------------------------------------
template <typename T, bool kVec>
__global__ __launch_bounds__(kThreads) void hessian_cm_kernel(const T* __restrict__ x, int64_t n_tok,
                                                              int64_t ld, int64_t gstride, int64_t nb,
                                                              int64_t n_groups, int64_t nsplit,
                                                              int64_t chunk, float alpha, float beta,
                                                              float* __restrict__ h, int64_t h_gstride,
                                                              float* __restrict__ ws) {
  __shared__ float red[4][256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ch = lane & 15, kg = lane >> 4;
  int64_t id = blockIdx.x;
  const int64_t s = id % nsplit;
  id /= nsplit;
  const int64_t b = id % nb, grp = id / nb;
  const int64_t t0 = s * chunk;
  const int64_t t1 = min(n_tok, t0 + chunk);
  const T* row = x + grp * gstride + (16 * b + ch) * ld;

  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  int64_t t = t0 + wave * kSlab;
  // Two slabs per trip keep four 16-byte loads per lane in flight; while both
  // slabs lie inside the slice no load needs a bounds check.
  if (kVec) {
    for (; t + kRound + kSlab <= t1; t += 2 * kRound) {
      Vals16<T> v0, v1;
      load_cm<true, true>(row, t + 16 * kg, t1, v0);
      load_cm<true, true>(row, t + kRound + 16 * kg, t1, v1);
      acc = mfma_accumulate(v0, acc);
      acc = mfma_accumulate(v1, acc);
    }
  }
  for (; t < t1; t += kRound) {
    Vals16<T> v0;
    load_cm<kVec>(row, t + 16 * kg, t1, v0);
    acc = mfma_accumulate(v0, acc);
  }

  // C layout: lane holds rows 4*kg .. 4*kg+3 of column ch.
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][(4 * kg + i) * 16 + ch] = acc[i];
  __syncthreads();
  const int e = threadIdx.x;
  const float v = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
  if (nsplit == 1) {
    float* hp = h + grp * h_gstride + b * 256 + e;
    *hp = (beta == 0.0f) ? alpha * v : beta * (*hp) + alpha * v;
  } else {
    ws[((s * n_groups + grp) * nb + b) * 256 + e] = v;
  }
}

// ---------------------------------------------------------------------------
// Token-major accumulation: x[t * ld + 16b + c] for tokens [t0, t1).  Each
// wave stages a 64-token x 16-channel tile in LDS (row = one token, 16
// values, no padding) and lane (ch, kg) reads tokens kg, kg+4, ..., kg+60 of
// column ch: for bf16 the 64 lanes touch 32 distinct words in 32 distinct
// banks, for fp32 every bank serves exactly two lanes (the minimum for 64
// four-byte reads).  The trip count is uniform over the workgroup (slabs
// past the end load zeros), so the barriers are reached by every wave.
// `base` points at channel 16b of token 0.
// ---------------------------------------------------------------------------
template <typename T, bool kVec>
__device__ __forceinline__ f32x4_t tm_accumulate(const T* __restrict__ base, int64_t ld, int64_t t0, int64_t t1,
                                                 T* my, int wave, int lane) {
  constexpr int kElemsPer16B = 16 / sizeof(T);          // 8 bf16 or 4 fp32
  constexpr int kLanesPerTok = 16 / kElemsPer16B;       // 2 or 4
  constexpr int kToksPerLoad = 64 / kLanesPerTok;       // 32 or 16
  constexpr int kLoads = kSlab / kToksPerLoad;          // 2 or 4
  const int ch = lane & 15, kg = lane >> 4;
  const int ltok = lane / kLanesPerTok;                 // token within a load
  const int lcol = (lane % kLanesPerTok) * kElemsPer16B;  // first channel

  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const int64_t rounds = t1 > t0 ? (t1 - t0 + kRound - 1) / kRound : 0;
  for (int64_t r = 0; r < rounds; ++r) {
    const int64_t t = t0 + r * kRound + wave * kSlab;
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
      const int trow = q * kToksPerLoad + ltok;
      const int64_t tok = t + trow;
      T* dst = my + trow * 16 + lcol;
      if (kVec && tok < t1) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(base + tok * ld + lcol);
      } else {
#pragma unroll
        for (int c = 0; c < kElemsPer16B; ++c) dst[c] = (tok < t1) ? base[tok * ld + lcol + c] : T(0);
      }
    }
    __syncthreads();
    Vals16<T> v;
    if constexpr (sizeof(T) == 2) {
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t lo = my[(kg + 4 * (2 * i)) * 16 + ch];
        const uint32_t hi = my[(kg + 4 * (2 * i + 1)) * 16 + ch];
        w[i] = lo | (hi << 16);
      }
      v.u[0] = make_uint4(w[0], w[1], w[2], w[3]);
      v.u[1] = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v.f[i] = my[(kg + 4 * i) * 16 + ch];
    }
    __syncthreads();
    acc = mfma_accumulate(v, acc);
  }
  return acc;
}

// Fixed-order sum of the four waves' 16x16 results; thread e gets entry e.
__device__ __forceinline__ float reduce_waves(f32x4_t acc, float (&red)[4][256], int wave, int lane) {
  const int ch = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][(4 * kg + i) * 16 + ch] = acc[i];
  __syncthreads();
  const int e = threadIdx.x;
  return ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
}

template <typename T, bool kVec>
__global__ __launch_bounds__(kThreads) void hessian_tm_kernel(const T* __restrict__ x, int64_t n_tok,
                                                              int64_t ld, int64_t gstride, int64_t nb,
                                                              int64_t n_groups, int64_t nsplit,
                                                              int64_t chunk, float alpha, float beta,
                                                              float* __restrict__ h, int64_t h_gstride,
                                                              float* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) T tile[4][kSlab * 16];
  __shared__ float red[4][256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int64_t id = blockIdx.x;
  const int64_t s = id % nsplit;
  id /= nsplit;
  const int64_t b = id % nb, grp = id / nb;
  const int64_t t0 = s * chunk;
  const int64_t t1 = min(n_tok, t0 + chunk);
  const f32x4_t acc = tm_accumulate<T, kVec>(x + grp * gstride + 16 * b, ld, t0, t1, tile[wave], wave, lane);
  const float v = reduce_waves(acc, red, wave, lane);
  const int e = threadIdx.x;
  if (nsplit == 1) {
    float* hp = h + grp * h_gstride + b * 256 + e;
    *hp = (beta == 0.0f) ? alpha * v : beta * (*hp) + alpha * v;
  } else {
    ws[((s * n_groups + grp) * nb + b) * 256 + e] = v;
  }
}

// ---------------------------------------------------------------------------
// Ragged groups ("Entry API and calibration flow", phase 2: hooks capture
// token-major inputs per batch; MoE experts receive different, possibly
// zero, numbers of tokens).  Group g owns rows offsets[g] .. offsets[g+1]-1
// of x (clamped to [0, n_rows], so no offset can move a read outside the
// buffer).  Without counts: H_g = S_g / n_g.  With counts (running mean over
// batches): H_g = (n_old H_g + S_g) / (n_old + n_g).  A group whose token
// total is still zero keeps its H (the caller's fallback).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void ragged_range(const int64_t* __restrict__ offsets, int64_t grp, int64_t n_rows,
                                             int64_t& r0, int64_t& r1) {
  int64_t a = offsets[grp], z = offsets[grp + 1];
  a = a < 0 ? 0 : (a > n_rows ? n_rows : a);
  z = z < a ? a : (z > n_rows ? n_rows : z);
  r0 = a;
  r1 = z;
}

__device__ __forceinline__ void ragged_store(float* hp, float v, int64_t n_g, const int64_t* __restrict__ counts,
                                             int64_t grp) {
  if (n_g == 0) return;  // no new tokens: H stays as it is
  if (counts) {
    const int64_t n_old = counts[grp];
    *hp = ((float)n_old * (*hp) + v) / (float)(n_old + n_g);
  } else {
    *hp = v / (float)n_g;
  }
}

template <typename T, bool kVec>
__global__ __launch_bounds__(kThreads) void hessian_ragged_kernel(const T* __restrict__ x, int64_t ld,
                                                                  int64_t n_rows,
                                                                  const int64_t* __restrict__ offsets,
                                                                  int64_t nb, int64_t n_groups, int64_t nsplit,
                                                                  float* __restrict__ h, int64_t h_gstride,
                                                                  const int64_t* __restrict__ counts,
                                                                  float* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) T tile[4][kSlab * 16];
  __shared__ float red[4][256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int64_t id = blockIdx.x;
  const int64_t s = id % nsplit;
  id /= nsplit;
  const int64_t b = id % nb, grp = id / nb;
  int64_t r0, r1;
  ragged_range(offsets, grp, n_rows, r0, r1);
  // slice s of the group's rows: equal whole rounds of 256 tokens
  const int64_t per = ((r1 - r0 + nsplit - 1) / nsplit + kRound - 1) / kRound * kRound;
  const int64_t t0 = min(r1, r0 + s * per);
  const int64_t t1 = min(r1, t0 + per);
  const f32x4_t acc = tm_accumulate<T, kVec>(x + 16 * b, ld, t0, t1, tile[wave], wave, lane);
  const float v = reduce_waves(acc, red, wave, lane);
  const int e = threadIdx.x;
  if (nsplit == 1)
    ragged_store(h + grp * h_gstride + b * 256 + e, v, r1 - r0, counts, grp);
  else
    ws[((s * n_groups + grp) * nb + b) * 256 + e] = v;
}

__global__ __launch_bounds__(kThreads) void hessian_ragged_finalize_kernel(
    const float* __restrict__ ws, int64_t nsplit, int64_t n_groups, int64_t nb, int64_t n_rows,
    const int64_t* __restrict__ offsets, const int64_t* __restrict__ counts, float* __restrict__ h,
    int64_t h_gstride) {
  const int64_t blk = blockIdx.x;  // grp * nb + b
  const int64_t grp = blk / nb, b = blk % nb;
  const int e = threadIdx.x;
  const int64_t per_split = n_groups * nb * 256;
  float v = ws[blk * 256 + e];
  for (int64_t s = 1; s < nsplit; ++s) v += ws[s * per_split + blk * 256 + e];
  int64_t r0, r1;
  ragged_range(offsets, grp, n_rows, r0, r1);
  ragged_store(h + grp * h_gstride + b * 256 + e, v, r1 - r0, counts, grp);
}

// counts[g] += n_g, after every block of the group has read the old count.
__global__ __launch_bounds__(kThreads) void hessian_ragged_counts_kernel(const int64_t* __restrict__ offsets,
                                                                         int64_t n_groups, int64_t n_rows,
                                                                         int64_t* __restrict__ counts) {
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (g >= n_groups) return;
  int64_t r0, r1;
  ragged_range(offsets, g, n_rows, r0, r1);
  counts[g] += r1 - r0;
}

// Sum of the token slices in slice order, then h = beta * h + alpha * sum.
__global__ __launch_bounds__(kThreads) void hessian_finalize_kernel(const float* __restrict__ ws,
                                                                    int64_t nsplit, int64_t n_groups,
                                                                    int64_t nb, float alpha, float beta,
                                                                    float* __restrict__ h,
                                                                    int64_t h_gstride) {
  const int64_t blk = blockIdx.x;  // grp * nb + b
  const int64_t grp = blk / nb, b = blk % nb;
  const int e = threadIdx.x;
  const int64_t per_split = n_groups * nb * 256;
  float v = ws[blk * 256 + e];
  for (int64_t s = 1; s < nsplit; ++s) v += ws[s * per_split + blk * 256 + e];
  float* hp = h + grp * h_gstride + b * 256 + e;
  *hp = (beta == 0.0f) ? alpha * v : beta * (*hp) + alpha * v;
}

// n_tok == 0: h = beta * h (the sum is empty).
__global__ __launch_bounds__(kThreads) void hessian_scale_kernel(float beta, float* __restrict__ h,
                                                                 int64_t h_gstride, int64_t nb) {
  const int64_t blk = blockIdx.x;
  const int64_t grp = blk / nb, b = blk % nb;
  float* hp = h + grp * h_gstride + b * 256 + threadIdx.x;
  *hp = (beta == 0.0f) ? 0.0f : beta * (*hp);
}

template <typename T, bool kVec>
hipError_t launch_typed(const HessianArgs& a, const HessianPlan& p, hipStream_t stream) {
  const int64_t nb = a.c_in / 16;
  const int64_t grid = a.n_groups * nb * p.nsplit;
  float* ws = p.nsplit > 1 ? static_cast<float*>(a.ws) : nullptr;
  const T* x = static_cast<const T*>(a.x);
  if (a.layout == 0)
    hessian_cm_kernel<T, kVec><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
        x, a.n_tok, a.ld, a.gstride, nb, a.n_groups, p.nsplit, p.chunk, a.alpha, a.beta, a.h,
        a.h_gstride, ws);
  else
    hessian_tm_kernel<T, kVec><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
        x, a.n_tok, a.ld, a.gstride, nb, a.n_groups, p.nsplit, p.chunk, a.alpha, a.beta, a.h,
        a.h_gstride, ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.nsplit == 1) return err;
  hessian_finalize_kernel<<<dim3((unsigned)(a.n_groups * nb)), dim3(kThreads), 0, stream>>>(
      ws, p.nsplit, a.n_groups, nb, a.alpha, a.beta, a.h, a.h_gstride);
  return hipGetLastError();
}

template <typename T, bool kVec>
hipError_t launch_ragged_typed(const HessianRaggedArgs& a, int64_t nsplit, hipStream_t stream) {
  const int64_t nb = a.c_in / 16;
  const int64_t grid = a.n_groups * nb * nsplit;
  float* ws = nsplit > 1 ? static_cast<float*>(a.ws) : nullptr;
  hessian_ragged_kernel<T, kVec><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
      static_cast<const T*>(a.x), a.ld, a.n_rows, a.offsets, nb, a.n_groups, nsplit, a.h, a.h_gstride, a.counts, ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (nsplit > 1) {
    hessian_ragged_finalize_kernel<<<dim3((unsigned)(a.n_groups * nb)), dim3(kThreads), 0, stream>>>(
        ws, nsplit, a.n_groups, nb, a.n_rows, a.offsets, a.counts, a.h, a.h_gstride);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (a.counts) {
    hessian_ragged_counts_kernel<<<dim3((unsigned)((a.n_groups + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                                   stream>>>(a.offsets, a.n_groups, a.n_rows, a.counts);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace

// Ragged slices per group: planned from the average rows per group (the
// per-group counts live on the device), ~1024 rows per slice, at most 16.
int64_t hessian_ragged_nsplit(int64_t c_in, int64_t n_rows, int64_t n_groups, bool have_ws) {
  if (!have_ws || n_groups <= 0 || c_in < 16) return 1;
  const int64_t avg = n_rows / n_groups;
  if (avg < 2048) return 1;
  const int64_t ns = avg / 1024;
  return ns > 16 ? 16 : ns;
}

size_t hessian_ragged_ws_bytes(int64_t c_in, int64_t n_rows, int64_t n_groups) {
  const int64_t ns = hessian_ragged_nsplit(c_in, n_rows, n_groups, true);
  if (ns <= 1) return 0;
  return (size_t)ns * (size_t)n_groups * (size_t)(c_in / 16) * 256u * sizeof(float);
}

hipError_t launch_hessian_ragged(const HessianRaggedArgs& a, hipStream_t stream) {
  const int64_t nb = a.c_in / 16;
  if (a.n_groups == 0 || nb == 0) return hipSuccess;
  const size_t need = hessian_ragged_ws_bytes(a.c_in, a.n_rows, a.n_groups);
  const bool have_ws = a.ws != nullptr && need > 0 && a.ws_bytes >= need;
  const int64_t nsplit = hessian_ragged_nsplit(a.c_in, a.n_rows, a.n_groups, have_ws);
  const int64_t epv = a.dtype == 1 ? 8 : 4;
  const bool aligned = (reinterpret_cast<uintptr_t>(a.x) % 16 == 0) && (a.ld % epv == 0);
  if (a.dtype == 1)
    return aligned ? launch_ragged_typed<uint16_t, true>(a, nsplit, stream)
                   : launch_ragged_typed<uint16_t, false>(a, nsplit, stream);
  return aligned ? launch_ragged_typed<float, true>(a, nsplit, stream) : launch_ragged_typed<float, false>(a, nsplit, stream);
}

// Token slices per block.  Measured on MI355X (17408 x 16384 bf16 X): the
// pass streams best with ~1024-token slices (16 slices: 5.7 TB/s, vs 4.7 TB/s
// for 2 slices, whose 2176 workgroups leave a nearly empty second wave of
// workgroups), so slices are ~1024 tokens, at most 16 of them.
HessianPlan hessian_plan(int64_t c_in, int64_t n_tok, int64_t n_groups, bool have_ws) {
  HessianPlan p{1, ((n_tok + kRound - 1) / kRound) * kRound};
  const int64_t blocks = n_groups * (c_in / 16);
  if (!have_ws || blocks <= 0 || n_tok < 2048) return p;
  int64_t ns = n_tok / 1024;
  if (ns > 16) ns = 16;
  int64_t chunk = (n_tok + ns - 1) / ns;
  chunk = ((chunk + kRound - 1) / kRound) * kRound;
  p.chunk = chunk;
  p.nsplit = (n_tok + chunk - 1) / chunk;
  if (p.nsplit <= 1) p = HessianPlan{1, ((n_tok + kRound - 1) / kRound) * kRound};
  return p;
}

size_t hessian_ws_bytes(int64_t c_in, int64_t n_tok, int64_t n_groups) {
  const HessianPlan p = hessian_plan(c_in, n_tok, n_groups, true);
  if (p.nsplit <= 1) return 0;
  return (size_t)p.nsplit * (size_t)n_groups * (size_t)(c_in / 16) * 256u * sizeof(float);
}

hipError_t launch_hessian(const HessianArgs& a, hipStream_t stream) {
  const int64_t nb = a.c_in / 16;
  if (a.n_groups == 0 || nb == 0) return hipSuccess;
  if (a.n_tok == 0) {
    if (a.beta == 1.0f) return hipSuccess;
    hessian_scale_kernel<<<dim3((unsigned)(a.n_groups * nb)), dim3(kThreads), 0, stream>>>(
        a.beta, a.h, a.h_gstride, nb);
    return hipGetLastError();
  }
  const size_t need = hessian_ws_bytes(a.c_in, a.n_tok, a.n_groups);
  const bool have_ws = a.ws != nullptr && need > 0 && a.ws_bytes >= need;
  const HessianPlan p = hessian_plan(a.c_in, a.n_tok, a.n_groups, have_ws);
  const size_t esz = a.dtype == 1 ? 2 : 4;
  const int64_t epv = 16 / (int64_t)esz;  // elements per 16-byte vector
  const bool aligned = (reinterpret_cast<uintptr_t>(a.x) % 16 == 0) && (a.ld % epv == 0) &&
                       (a.gstride % epv == 0);
  if (a.dtype == 1)
    return aligned ? launch_typed<uint16_t, true>(a, p, stream) : launch_typed<uint16_t, false>(a, p, stream);
  return aligned ? launch_typed<float, true>(a, p, stream) : launch_typed<float, false>(a, p, stream);
}

}  // namespace lh
