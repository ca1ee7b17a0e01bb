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
// Design: one workgroup per (group, block, token slice): 4, 8 or 16 wave64s
// channel-major (the plan's choice), 4 token-major.  The contraction over
// tokens runs on MFMA with fp32 accumulation:
// v_mfma_f32_16x16x32_bf16 for bf16 X, v_mfma_f32_16x16x4_f32 for fp32 X.
// For H = X_b X_b^T the A operand (16 channels x K tokens) and the B operand
// (its transpose) hold the same values in each lane (lane l: channel l%16,
// K-slot group l/16), so one register set feeds both.  The token order inside
// a K step is free (a sum), which lets each lane read 16 contiguous tokens
// (channel-major) or a bank-conflict-free LDS column (token-major).
// The waves of a workgroup reduce in LDS in a fixed order; token slices
// of one block reduce in a second kernel in a fixed order: results do not
// depend on timing.
#include "lh_device.h"
#include "lh_internal.h"

namespace lh {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int kSlab = 64;                 // tokens per wave per step
constexpr int kRound = kSlab * 4;         // tokens per 4-wave workgroup per step
constexpr int64_t kRaggedSlice = 1024;    // rows per ragged slice when the largest group is known

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
// Workgroup `id` = (group, block, token slice): the slice's X_b X_b^T,
// written as h = beta h + alpha S without a workspace, else as the slice's
// partial sum in ws[slice][group][block].
// kNW waves: at each step the waves take kNW consecutive 64-token slabs
// (mod the slice's full steps), so together they read 128 kNW contiguous
// bytes of each bf16 row at a time.
template <typename T, bool kVec, int kNW>
__device__ __forceinline__ void hessian_cm_block(int64_t id, const T* __restrict__ x, int64_t n_tok, int64_t ld,
                                                 int64_t gstride, int64_t nb, int64_t n_groups, int64_t nsplit,
                                                 int64_t chunk, float alpha, float beta, float* __restrict__ h,
                                                 int64_t h_gstride, float* __restrict__ ws) {
  constexpr int kR = kSlab * kNW;  // tokens per workgroup per step
  __shared__ float red[kNW][256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ch = lane & 15, kg = lane >> 4;
  // the grid's workgroup ids, slices and blocks fit 32 bits: 32-bit division
  const uint32_t wg = (uint32_t)id;
  const uint32_t s = wg % (uint32_t)nsplit;
  const uint32_t gbk = wg / (uint32_t)nsplit;
  const int64_t b = gbk % (uint32_t)nb, grp = gbk / (uint32_t)nb;
  const int64_t t0 = (int64_t)s * chunk;
  const int64_t t1 = min(n_tok, t0 + chunk);
  const T* row = x + grp * gstride + (16 * b + ch) * ld;

  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  // The slice's full steps hold S = K kNW slabs of 64 tokens.  Wave w takes
  // slabs r + w, r + w + kNW, ... (mod S) from a start r that moves 17 slabs
  // per workgroup, so workgroups running side by side read different
  // offsets of their rows: with rows and blocks a power of two bytes long,
  // a common start put them all on the same HBM channels at once (4096 x
  // 8192 bf16, cache-cold: 20.0 -> 15.8 us).  Two slabs per trip keep four
  // 16-byte loads per lane in flight; no full-step load needs a bounds check.
  const int64_t K = (t1 - t0) / kR;
  if (K > 0) {
    const int64_t S = K * kNW;
    int64_t q = wave;
    if (S < (1 << 27)) {  // 17 (wg mod S) fits 32 bits
      const uint32_t S32 = (uint32_t)S;
      q += ((wg % S32) * 17u) % S32;
    } else {
      q += (int64_t)(((uint64_t)wg * 17u) % (uint64_t)S);
    }
    if (q >= S) q -= S;
    const T* base = row + t0 + 16 * kg;
    const int64_t rel = t1 - t0 - 16 * kg;  // the slice's end, relative to base
    int64_t k = 0;
    for (; k + 1 < K; k += 2) {
      int64_t q1 = q + kNW;
      if (q1 >= S) q1 -= S;
      Vals16<T> v0, v1;
      load_cm<kVec, true>(base, q * kSlab, rel, v0);
      load_cm<kVec, true>(base, q1 * kSlab, rel, v1);
      acc = mfma_accumulate(v0, acc);
      acc = mfma_accumulate(v1, acc);
      q = q1 + kNW;
      if (q >= S) q -= S;
    }
    if (k < K) {
      Vals16<T> v0;
      load_cm<kVec, true>(base, q * kSlab, rel, v0);
      acc = mfma_accumulate(v0, acc);
    }
  }
  // the rest of the slice (less than a step), with bounds checks
  for (int64_t t = t0 + K * kR + wave * kSlab; t < t1; t += kR) {
    Vals16<T> v0;
    load_cm<kVec>(row, t + 16 * kg, t1, v0);
    acc = mfma_accumulate(v0, acc);
  }

  // C layout: lane holds rows 4*kg .. 4*kg+3 of column ch.
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][(4 * kg + i) * 16 + ch] = acc[i];
  __syncthreads();
  const int e = threadIdx.x;
  if (e >= 256) return;
  float v = red[0][e];
#pragma unroll
  for (int k = 1; k < kNW; ++k) v += red[k][e];  // waves in order
  if (ws == nullptr) {
    float* hp = h + grp * h_gstride + b * 256 + e;
    *hp = (beta == 0.0f) ? alpha * v : beta * (*hp) + alpha * v;
  } else {
    ws[((s * n_groups + grp) * nb + b) * 256 + e] = v;
  }
}

template <typename T, bool kVec, int kNW>
__global__ __launch_bounds__(64 * kNW) void hessian_cm_kernel(const T* __restrict__ x, int64_t n_tok,
                                                              int64_t ld, int64_t gstride, int64_t nb,
                                                              int64_t n_groups, int64_t nsplit,
                                                              int64_t chunk, float alpha, float beta,
                                                              float* __restrict__ h, int64_t h_gstride,
                                                              float* __restrict__ ws) {
  hessian_cm_block<T, kVec, kNW>(blockIdx.x, x, n_tok, ld, gstride, nb, n_groups, nsplit, chunk, alpha, beta, h,
                            h_gstride, ws);
}

// The calibration prologue in one launch: the first workgroups fold W's
// |w| bits into one partial maximum each (W flat, 16-byte aligned), the
// others compute the token-slice partial sums of the channel-major Hessian
// (X 16-byte aligned); no atomics, so no output has to be zeroed first.  The
// finalize kernel completes both.
template <typename T, typename TW, int kNW>
__global__ __launch_bounds__(64 * kNW) void prologue_cm_kernel(const T* __restrict__ x, int64_t n_tok, int64_t ld,
                                                               int64_t gstride, int64_t nb, int64_t n_groups,
                                                               int64_t nsplit, int64_t chunk, float* __restrict__ ws,
                                                               const TW* __restrict__ w,
                                                               int64_t w_n16, int64_t w_gstride, int64_t per_group,
                                                               uint32_t* __restrict__ abs_part) {
  // the amax shares (long, few) come first in the grid, the Hessian slices fill in behind them
  const int64_t n_abs = n_groups * per_group;
  if ((int64_t)blockIdx.x >= n_abs) {
    hessian_cm_block<T, true, kNW>((int64_t)blockIdx.x - n_abs, x, n_tok, ld, gstride, nb, n_groups, nsplit, chunk, 1.0f,
                              0.0f, nullptr, 0, ws);
    return;
  }
  const int64_t id = blockIdx.x;
  const int64_t grp = id / per_group, share = id - grp * per_group;
  const uint32_t m = absmax_flat_share<sizeof(TW) == 2, 64 * kNW>(reinterpret_cast<const uint4*>(w + grp * w_gstride),
                                                                  w_n16, share, per_group);
  if (threadIdx.x == 0) abs_part[id] = m;
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

// Rows per slice of a group of n_g rows split nsplit ways: an even split, or
// fixed slices of slice_rows where those cover the group (the plan sizes
// nsplit for the largest group); whole multiples of 256 rows.  Slice s holds
// rows [s per, (s + 1) per); the group uses ceil(n_g / per) slices.
__device__ __forceinline__ int64_t ragged_per(int64_t n_g, int64_t nsplit, int64_t slice_rows) {
  int64_t per = (n_g + nsplit - 1) / nsplit;
  if (slice_rows > per) per = slice_rows;
  return (per + kRound - 1) / kRound * kRound;
}

// ---------------------------------------------------------------------------
// Token-major kernel: x[t * ld + c].  A workgroup owns four consecutive
// blocks (64 channels: one 128-byte bf16 row segment per token) and a slice
// of tokens; wave w accumulates block 4q + w over the whole slice, so no
// cross-wave reduction is needed.  Each round the 256 threads copy a
// kTok-token x 64-channel tile into LDS (16-byte loads, rows padded to 80
// elements) and every wave reads its 16-channel column in the MFMA operand
// layout: lane (ch, kg) takes tokens kg, kg+4, ...  With the 80-element
// pitch the four kg rows of one read fall on disjoint banks (bf16: 8 banks
// apart; fp32: two lanes per bank, the minimum for 64 four-byte reads).
// The tile is double-buffered and the next round's global loads are in
// flight while the current round is multiplied: one barrier per round.
// The trip count is uniform over the workgroup (rows past the slice load
// zeros), so every wave reaches every barrier.
// ---------------------------------------------------------------------------
constexpr int kPitch = 80;  // LDS row pitch in elements (64 channels + 16 pad)

template <typename T>
struct TmShape {
  static constexpr int kEP = 16 / sizeof(T);                // elements per 16-byte chunk
  static constexpr int kCPR = 64 / kEP;                     // chunks per 64-channel row
  static constexpr int kRowsPerPass = kThreads / kCPR;      // rows one pass of loads covers
  static constexpr int kTok = sizeof(T) == 2 ? 128 : 64;    // tokens per round
  static constexpr int kPasses = kTok / kRowsPerPass;       // 16-byte loads per thread per round
  static constexpr int kVecs = kTok / 64;                   // Vals16 per lane per round
};

template <typename T, bool kVec>
struct TmLoader {
  using S = TmShape<T>;
  uint4 r[S::kPasses];
  // Rows [t, t + kTok) of the 64-channel segment at `seg` (row stride ld),
  // rows at or past t1 and chunks at or past the last channel read as zero.
  __device__ __forceinline__ void load(const T* __restrict__ seg, int64_t ld, int64_t t, int64_t t1, int crow,
                                       int ccol, bool col_ok) {
#pragma unroll
    for (int p = 0; p < S::kPasses; ++p) {
      const int64_t tok = t + p * S::kRowsPerPass + crow;
      const bool ok = col_ok && tok < t1;
      if (kVec) {
        r[p] = ok ? *reinterpret_cast<const uint4*>(seg + tok * ld + ccol) : make_uint4(0u, 0u, 0u, 0u);
      } else {
        T v[S::kEP];
#pragma unroll
        for (int c = 0; c < S::kEP; ++c) v[c] = ok ? seg[tok * ld + ccol + c] : T(0);
        r[p] = __builtin_bit_cast(uint4, v);
      }
    }
  }
  __device__ __forceinline__ void store(T* buf, int crow, int ccol) const {
#pragma unroll
    for (int p = 0; p < S::kPasses; ++p)
      *reinterpret_cast<uint4*>(buf + (p * S::kRowsPerPass + crow) * kPitch + ccol) = r[p];
  }
};

// Channel column 16 w + ch of an LDS tile, tokens kg + 4 i, as MFMA operands.
template <typename T>
__device__ __forceinline__ f32x4_t tile_mfma(const T* buf, int wave, int lane, f32x4_t acc) {
  const int ch = lane & 15, kg = lane >> 4;
  const T* col = buf + 16 * wave + ch;
#pragma unroll
  for (int q = 0; q < TmShape<T>::kVecs; ++q) {
    Vals16<T> v;
    const int tb = 64 * q + kg;
    if constexpr (sizeof(T) == 2) {
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t lo = col[(tb + 4 * (2 * i)) * kPitch];
        const uint32_t hi = col[(tb + 4 * (2 * i + 1)) * kPitch];
        w[i] = lo | (hi << 16);
      }
      v.u[0] = make_uint4(w[0], w[1], w[2], w[3]);
      v.u[1] = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v.f[i] = col[(tb + 4 * i) * kPitch];
    }
    acc = mfma_accumulate(v, acc);
  }
  return acc;
}

template <typename T, bool kVec, bool kRagged>
__global__ __launch_bounds__(kThreads) void hessian_tm_kernel(const T* __restrict__ x, int64_t ld, int64_t gstride,
                                                              int64_t n_tok, int64_t n_rows,
                                                              const int64_t* __restrict__ offsets, int64_t c_in,
                                                              int64_t nb, int64_t n_groups, int64_t nsplit,
                                                              int64_t chunk, int64_t slice_rows, float alpha,
                                                              float beta,
                                                              float* __restrict__ h, int64_t h_gstride,
                                                              const int64_t* __restrict__ counts,
                                                              float* __restrict__ ws, uint32_t* __restrict__ snap) {
  using S = TmShape<T>;
  __shared__ __attribute__((aligned(16))) T tile[2][S::kTok * kPitch];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t quads = (nb + 3) / 4;
  int64_t id = blockIdx.x;
  const int64_t s = id % nsplit;
  id /= nsplit;
  const int64_t q = id % quads, grp = id / quads;

  int64_t t0, t1, r0 = 0, r1 = 0;
  const T* seg;
  if constexpr (kRagged) {
    // the group's token count before this call, for the slice-sum kernel
    // (which also updates it); halves of the int64 at 4-byte alignment
    if (snap != nullptr && s == 0 && q == 0 && threadIdx.x == 0) {
      const uint64_t n_old = (uint64_t)counts[grp];
      snap[2 * grp] = (uint32_t)n_old;
      snap[2 * grp + 1] = (uint32_t)(n_old >> 32);
    }
    ragged_range(offsets, grp, n_rows, r0, r1);
    const int64_t per = ragged_per(r1 - r0, nsplit, slice_rows);
    t0 = r0 + s * per;
    if (nsplit > 1 && t0 >= r1) return;  // unused slice: the finalize kernel skips it (whole workgroup)
    t0 = min(r1, t0);
    t1 = min(r1, t0 + per);
    seg = x + 64 * q;
  } else {
    t0 = s * chunk;
    t1 = min(n_tok, t0 + chunk);
    seg = x + grp * gstride + 64 * q;
  }
  const int crow = threadIdx.x / S::kCPR;
  const int ccol = (threadIdx.x % S::kCPR) * S::kEP;
  const bool col_ok = 64 * q + ccol < c_in;  // chunks never straddle c_in (c_in % 16 == 0)

  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const int64_t rounds = t1 > t0 ? (t1 - t0 + S::kTok - 1) / S::kTok : 0;
  // Two register sets keep the loads of the next two rounds in flight while a
  // round is multiplied (twice the bytes in flight of one set, no more LDS).
  TmLoader<T, kVec> ra, rb;
  if (rounds > 0) {
    ra.load(seg, ld, t0, t1, crow, ccol, col_ok);
    ra.store(tile[0], crow, ccol);
  }
  if (rounds > 1) ra.load(seg, ld, t0 + S::kTok, t1, crow, ccol, col_ok);
  if (rounds > 2) rb.load(seg, ld, t0 + 2 * S::kTok, t1, crow, ccol, col_ok);
  __syncthreads();
  for (int64_t r = 0; r < rounds; r += 2) {
    // even round r: tile[0]; ra holds round r+1, rb round r+2
    acc = tile_mfma<T>(tile[0], wave, lane, acc);
    if (r + 1 < rounds) ra.store(tile[1], crow, ccol);
    if (r + 3 < rounds) ra.load(seg, ld, t0 + (r + 3) * S::kTok, t1, crow, ccol, col_ok);
    __syncthreads();
    if (r + 1 >= rounds) break;
    // odd round r+1: tile[1]; rb holds round r+2, ra round r+3
    acc = tile_mfma<T>(tile[1], wave, lane, acc);
    if (r + 2 < rounds) rb.store(tile[0], crow, ccol);
    if (r + 4 < rounds) rb.load(seg, ld, t0 + (r + 4) * S::kTok, t1, crow, ccol, col_ok);
    __syncthreads();
  }

  const int64_t b = 4 * q + wave;
  if (b >= nb) return;
  const int ch = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = (4 * kg + i) * 16 + ch;
    const float v = acc[i];
    if (nsplit > 1) {
      ws[((s * n_groups + grp) * nb + b) * 256 + e] = v;
    } else if constexpr (kRagged) {
      ragged_store(h + grp * h_gstride + b * 256 + e, v, r1 - r0, counts, grp);
    } else {
      float* hp = h + grp * h_gstride + b * 256 + e;
      *hp = (beta == 0.0f) ? alpha * v : beta * (*hp) + alpha * v;
    }
  }
}

// One workgroup per (group, kFinBlocks consecutive blocks): each thread sums
// entry e of its blocks over the group's slices in slice order (the loads
// of all its blocks for one slice in flight together), stores h, and the
// group's first workgroup then sets the count from the snapshot the main
// kernel took (every workgroup of the group reads the snapshot, never the
// count it updates).
constexpr int kFinBlocks = 8;

__global__ __launch_bounds__(kThreads) void hessian_ragged_finalize_kernel(
    const float* __restrict__ ws, int64_t nsplit, int64_t slice_rows, int64_t n_groups, int64_t nb, int64_t n_rows,
    const int64_t* __restrict__ offsets, const uint32_t* __restrict__ snap, int64_t* __restrict__ counts,
    float* __restrict__ h, int64_t h_gstride) {
  const int64_t chunks = (nb + kFinBlocks - 1) / kFinBlocks;
  const int64_t grp = blockIdx.x / chunks, c = blockIdx.x % chunks;
  const int e = threadIdx.x;
  int64_t r0, r1;
  ragged_range(offsets, grp, n_rows, r0, r1);
  const int64_t n_g = r1 - r0;
  if (n_g == 0) return;  // h and the count stay as they are
  const int64_t per = ragged_per(n_g, nsplit, slice_rows);
  const int64_t used = (n_g + per - 1) / per;  // slices the group wrote, in order
  const int64_t b0 = c * kFinBlocks;
  const int nblk = (int)min((int64_t)kFinBlocks, nb - b0);
  const int64_t sstride = n_groups * nb * 256;
  const float* p = ws + (grp * nb + b0) * 256 + e;
  float* hp = h + grp * h_gstride + b0 * 256 + e;
  // the running mean's inputs (old count and old H) are loaded with the
  // first slice, not after the sum
  int64_t n_old = 0;
  float hold[kFinBlocks];
  if (counts != nullptr) {
    n_old = (int64_t)(((uint64_t)snap[2 * grp + 1] << 32) | snap[2 * grp]);
#pragma unroll
    for (int i = 0; i < kFinBlocks; ++i) hold[i] = i < nblk ? hp[i * 256] : 0.0f;
  }
  float v[kFinBlocks];
#pragma unroll
  for (int i = 0; i < kFinBlocks; ++i) v[i] = i < nblk ? p[i * 256] : 0.0f;
  for (int64_t sl = 1; sl < used; ++sl) {
    float t[kFinBlocks];
#pragma unroll
    for (int i = 0; i < kFinBlocks; ++i) t[i] = i < nblk ? p[sl * sstride + i * 256] : 0.0f;
#pragma unroll
    for (int i = 0; i < kFinBlocks; ++i) v[i] += t[i];
  }
#pragma unroll
  for (int i = 0; i < kFinBlocks; ++i) {
    if (i >= nblk) break;
    hp[i * 256] = counts != nullptr ? ((float)n_old * hold[i] + v[i]) / (float)(n_old + n_g)
                                    : v[i] / (float)n_g;
  }
  if (counts != nullptr && c == 0 && e == 0) counts[grp] = n_old + n_g;
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
  const float v = sum_slices(ws + blk * 256 + e, n_groups * nb * 256, nsplit);
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
  float* ws = p.nsplit > 1 ? static_cast<float*>(a.ws) : nullptr;
  const T* x = static_cast<const T*>(a.x);
  if (a.layout == 0) {
    const dim3 grid((unsigned)(a.n_groups * nb * p.nsplit));
    if (p.nw == 16)
      hessian_cm_kernel<T, kVec, 16><<<grid, dim3(64 * 16), 0, stream>>>(
          x, a.n_tok, a.ld, a.gstride, nb, a.n_groups, p.nsplit, p.chunk, a.alpha, a.beta, a.h, a.h_gstride, ws);
    else if (p.nw == 8)
      hessian_cm_kernel<T, kVec, 8><<<grid, dim3(64 * 8), 0, stream>>>(
          x, a.n_tok, a.ld, a.gstride, nb, a.n_groups, p.nsplit, p.chunk, a.alpha, a.beta, a.h, a.h_gstride, ws);
    else
      hessian_cm_kernel<T, kVec, 4><<<grid, dim3(64 * 4), 0, stream>>>(
          x, a.n_tok, a.ld, a.gstride, nb, a.n_groups, p.nsplit, p.chunk, a.alpha, a.beta, a.h, a.h_gstride, ws);
  } else {
    const int64_t grid = a.n_groups * ((nb + 3) / 4) * p.nsplit;
    hessian_tm_kernel<T, kVec, false><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
        x, a.ld, a.gstride, a.n_tok, 0, nullptr, a.c_in, nb, a.n_groups, p.nsplit, p.chunk, 0, a.alpha, a.beta,
        a.h, a.h_gstride, nullptr, ws, nullptr);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.nsplit == 1) return err;
  hessian_finalize_kernel<<<dim3((unsigned)(a.n_groups * nb)), dim3(kThreads), 0, stream>>>(
      ws, p.nsplit, a.n_groups, nb, a.alpha, a.beta, a.h, a.h_gstride);
  return hipGetLastError();
}

template <typename T, bool kVec>
hipError_t launch_ragged_typed(const HessianRaggedArgs& a, const RaggedPlan& p, hipStream_t stream) {
  const int64_t nb = a.c_in / 16;
  const int64_t nsplit = p.nsplit;
  const int64_t grid = a.n_groups * ((nb + 3) / 4) * nsplit;
  float* ws = nsplit > 1 ? static_cast<float*>(a.ws) : nullptr;
  // after the slice partials: the groups' counts before this call
  uint32_t* snap = (ws != nullptr && a.counts != nullptr)
                       ? reinterpret_cast<uint32_t*>(ws + nsplit * a.n_groups * nb * 256)
                       : nullptr;
  hessian_tm_kernel<T, kVec, true><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
      static_cast<const T*>(a.x), a.ld, 0, 0, a.n_rows, a.offsets, a.c_in, nb, a.n_groups, nsplit, 0, p.slice_rows,
      1.0f, 0.0f, a.h, a.h_gstride, a.counts, ws, snap);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (nsplit > 1) {  // the slice sums also update the counts
    const int64_t chunks = (nb + kFinBlocks - 1) / kFinBlocks;
    hessian_ragged_finalize_kernel<<<dim3((unsigned)(a.n_groups * chunks)), dim3(kThreads), 0, stream>>>(
        ws, nsplit, p.slice_rows, a.n_groups, nb, a.n_rows, a.offsets, snap, a.counts, a.h, a.h_gstride);
    return hipGetLastError();
  }
  if (a.counts) {
    hessian_ragged_counts_kernel<<<dim3((unsigned)((a.n_groups + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                                   stream>>>(a.offsets, a.n_groups, a.n_rows, a.counts);
    err = hipGetLastError();
  }
  return err;
}

// Token-major slices: enough workgroups of four blocks to keep ~16 per CU
// busy (4096), slices of at least 512 tokens, at most 64 slices.
int64_t tm_nsplit(int64_t c_in, int64_t tokens_per_group, int64_t n_groups) {
  const int64_t wgs = n_groups * ((c_in / 16 + 3) / 4);
  if (wgs <= 0) return 1;
  int64_t ns = (4096 + wgs - 1) / wgs;
  int64_t cap = tokens_per_group / 512;
  if (cap > 64) cap = 64;
  if (ns > cap) ns = cap;
  return ns < 1 ? 1 : ns;
}

}  // namespace

// Ragged slices.  The per-group counts live on the device, so the plan uses
// what the host knows: with a bound on the largest group, fixed 1024-row
// slices (the largest group gets all the workgroups it can use and unused
// slices of smaller groups exit at once); otherwise an even split planned
// from the average rows per group.
RaggedPlan hessian_ragged_plan(int64_t c_in, int64_t n_rows, int64_t n_groups, int64_t max_group_rows,
                               bool have_ws) {
  RaggedPlan p{1, 0};
  if (!have_ws || n_groups <= 0 || c_in < 16) return p;
  if (max_group_rows > 0) {
    int64_t ns = (max_group_rows + kRaggedSlice - 1) / kRaggedSlice;
    if (ns > 64) ns = 64;
    if (ns > 1) {
      p.nsplit = ns;
      p.slice_rows = kRaggedSlice;
    }
    return p;
  }
  p.nsplit = tm_nsplit(c_in, n_rows / n_groups, n_groups);
  return p;
}

size_t hessian_ragged_ws_bytes(int64_t c_in, int64_t n_rows, int64_t n_groups, int64_t max_group_rows) {
  const RaggedPlan p = hessian_ragged_plan(c_in, n_rows, n_groups, max_group_rows, true);
  if (p.nsplit <= 1) return 0;
  // slice partials, then each group's token count before the call (two
  // 32-bit halves, for the running mean)
  return (size_t)p.nsplit * (size_t)n_groups * (size_t)(c_in / 16) * 256u * sizeof(float) +
         (size_t)n_groups * 2u * sizeof(uint32_t);
}

hipError_t launch_hessian_ragged(const HessianRaggedArgs& a, hipStream_t stream) {
  const int64_t nb = a.c_in / 16;
  if (a.n_groups == 0 || nb == 0) return hipSuccess;
  const size_t need = hessian_ragged_ws_bytes(a.c_in, a.n_rows, a.n_groups, a.max_group_rows);
  const bool have_ws = a.ws != nullptr && need > 0 && a.ws_bytes >= need;
  const RaggedPlan p = hessian_ragged_plan(a.c_in, a.n_rows, a.n_groups, a.max_group_rows, have_ws);
  const int64_t epv = a.dtype == 1 ? 8 : 4;
  const bool aligned = (reinterpret_cast<uintptr_t>(a.x) % 16 == 0) && (a.ld % epv == 0);
  if (a.dtype == 1)
    return aligned ? launch_ragged_typed<uint16_t, true>(a, p, stream)
                   : launch_ragged_typed<uint16_t, false>(a, p, stream);
  return aligned ? launch_ragged_typed<float, true>(a, p, stream) : launch_ragged_typed<float, false>(a, p, stream);
}

// Channel-major plan: waves per workgroup and token slices per block,
// measured on MI355X with the caches flushed by a 1 GiB read (bf16, kernel
// plus the slice sum):
//   X 17408 x 16384: 16 waves, 4 slices 100-102 us; 2, 3, 5, 6, 8 slices
//   103-108 us; 1 slice 104 us (1088 workgroups of 16 waves: two rounds and
//   a thin third); 4 waves, 8 slices 112 us;
//   X 4096 x 4096: 16 waves, 1 slice 10.2 us; 4 waves, 4 slices 12.4 us;
//   64 x 2048 x 512: 8 waves 26.0 us, 4 waves 26.5 us, 16 waves 34.8 us
//   (half of them without a slab).
// So: the most waves (up to 16) that each still get a 64-token slab; one
// slice while the chip holds every workgroup at once (no sum kernel) or
// there are 8 rounds of them anyway; in between, slices until there are
// 8 rounds (at most 16 slices, each at least one step of the workgroup).
// Token-major workgroups cover four blocks: see tm_nsplit.  Chunks are whole
// multiples of 256 tokens.
HessianPlan hessian_plan(int64_t c_in, int64_t n_tok, int64_t n_groups, int layout, bool have_ws) {
  HessianPlan p{1, ((n_tok + kRound - 1) / kRound) * kRound, 4};
  if (layout == 0)
    while (p.nw < 16 && (int64_t)kSlab * 2 * p.nw <= n_tok) p.nw *= 2;
  const int64_t blocks = n_groups * (c_in / 16);
  if (!have_ws || blocks <= 0) return p;
  int64_t ns = 1;
  if (layout == 0) {
    const int64_t resident = 256 * 32 / p.nw;  // 256 CUs x 32 waves
    const int64_t cap = n_tok / ((int64_t)kSlab * p.nw);
    if (blocks > resident)
      while (ns < 16 && 2 * ns <= cap && blocks * ns < 8 * resident) ns *= 2;
  } else {
    ns = tm_nsplit(c_in, n_tok, n_groups);
  }
  if (ns <= 1) return p;
  int64_t chunk = (n_tok + ns - 1) / ns;
  chunk = ((chunk + kRound - 1) / kRound) * kRound;
  p.chunk = chunk;
  p.nsplit = (n_tok + chunk - 1) / chunk;
  if (p.nsplit <= 1) {
    p.nsplit = 1;
    p.chunk = ((n_tok + kRound - 1) / kRound) * kRound;
  }
  return p;
}

// Enough for either layout's plan.
size_t hessian_ws_bytes(int64_t c_in, int64_t n_tok, int64_t n_groups) {
  int64_t ns = 1;
  for (int layout = 0; layout < 2; ++layout) {
    const HessianPlan p = hessian_plan(c_in, n_tok, n_groups, layout, true);
    if (p.nsplit > ns) ns = p.nsplit;
  }
  if (ns <= 1) return 0;
  return (size_t)ns * (size_t)n_groups * (size_t)(c_in / 16) * 256u * sizeof(float);
}

ProloguePlan prologue_plan(int64_t c_in, int64_t n_tok, int64_t n_groups, int64_t w_elems) {
  ProloguePlan q;
  q.hess = hessian_plan(c_in, n_tok, n_groups, 0, true);
  const int64_t threads = 64 * q.hess.nw;  // the launch's workgroup size
  const int64_t n16 = w_elems / 8;  // at least this many 16-byte vectors (bf16); fp32 has twice as many
  int64_t per = (4096 / q.hess.nw + n_groups - 1) / n_groups;  // ~256 K threads over W
  // When the Hessian's workgroups take several rounds of the chip, half as
  // many shares leave more room to them (cache-cold, W + X read once: MoE
  // 64 x 1024 x 2048 85 -> 72 us, 5120 x 17408 with 16384 tokens 129 -> 124
  // us); when both kinds fit in one round (256 Hessian workgroups), halving
  // makes that round uneven (12288 x 4096: 32 -> 36 us).
  const int64_t resident = 256 * 32 / q.hess.nw;  // 256 CUs x 32 waves
  if (n_groups * (c_in / 16) * q.hess.nsplit > resident) per = (per + 1) / 2;
  const int64_t need = (n16 + 4 * threads - 1) / (4 * threads);
  if (per > need) per = need;
  q.abs_per_group = per < 1 ? 1 : per;
  return q;
}

size_t prologue_ws_bytes(int64_t c_in, int64_t n_tok, int64_t n_groups, int64_t w_elems) {
  const ProloguePlan q = prologue_plan(c_in, n_tok, n_groups, w_elems);
  return (size_t)q.hess.nsplit * n_groups * (c_in / 16) * 256 * sizeof(float) +
         (size_t)n_groups * q.abs_per_group * sizeof(uint32_t);
}

template <typename T, typename TW, int kNW>
void launch_prologue_nw(const PrologueArgs& a, const ProloguePlan& q, hipStream_t stream) {
  const int64_t nb = a.c_in / 16;
  const int64_t n_hess = a.n_groups * nb * q.hess.nsplit;
  const int64_t w_n16 = a.c_out * a.c_in * (int64_t)sizeof(TW) / 16;
  const int64_t grid = n_hess + a.n_groups * q.abs_per_group;
  prologue_cm_kernel<T, TW, kNW><<<dim3((unsigned)grid), dim3(64 * kNW), 0, stream>>>(
      static_cast<const T*>(a.x), a.n_tok, a.ld_x, a.gstride_x, nb, a.n_groups, q.hess.nsplit, q.hess.chunk, a.h_part,
      static_cast<const TW*>(a.w), w_n16, a.gstride_w, q.abs_per_group, a.abs_part);
}

template <typename T, typename TW>
hipError_t launch_prologue_typed(const PrologueArgs& a, const ProloguePlan& q, hipStream_t stream) {
  if (q.hess.nw == 16)
    launch_prologue_nw<T, TW, 16>(a, q, stream);
  else if (q.hess.nw == 8)
    launch_prologue_nw<T, TW, 8>(a, q, stream);
  else
    launch_prologue_nw<T, TW, 4>(a, q, stream);
  return hipGetLastError();
}

hipError_t launch_prologue(const PrologueArgs& a, const ProloguePlan& q, hipStream_t stream) {
  if (a.x_dtype == 1)
    return a.w_dtype == 1 ? launch_prologue_typed<uint16_t, uint16_t>(a, q, stream)
                          : launch_prologue_typed<uint16_t, float>(a, q, stream);
  return a.w_dtype == 1 ? launch_prologue_typed<float, uint16_t>(a, q, stream)
                        : launch_prologue_typed<float, float>(a, q, stream);
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
  const HessianPlan p = hessian_plan(a.c_in, a.n_tok, a.n_groups, a.layout, have_ws);
  const size_t esz = a.dtype == 1 ? 2 : 4;
  const int64_t epv = 16 / (int64_t)esz;  // elements per 16-byte vector
  const bool aligned = (reinterpret_cast<uintptr_t>(a.x) % 16 == 0) && (a.ld % epv == 0) &&
                       (a.gstride % epv == 0);
  if (a.dtype == 1)
    return aligned ? launch_typed<uint16_t, true>(a, p, stream) : launch_typed<uint16_t, false>(a, p, stream);
  return aligned ? launch_typed<float, true>(a, p, stream) : launch_typed<float, false>(a, p, stream);
}

}  // namespace lh
