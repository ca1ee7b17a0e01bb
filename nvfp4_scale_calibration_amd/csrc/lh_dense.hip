// lh_dense.hip - dense C_in x C_in work on CDNA4 matrix cores: the full
// Hessian X X^T, the layer output error (q - w) H (q - w)^T, and the W/s
// histogram.
//
// "Local-Hessian weight-scale guide" (xxmr.cn/news/266017), "Algorithm
// principle": the layer's output error is ||Delta X||_F^2 =
// tr(Delta X X^T Delta^T); Local-Hessian keeps only the 16 x 16 diagonal
// blocks of X X^T.  These kernels measure what that approximation leaves
// out, on the same inputs.  "How scaling reshapes the weight distribution":
// the histogram of W/s, the values the E2M1 rounding receives.
//
// GEMM design: C[m][n] = sum_k A[m][k] B[n][k] ("NT": both operands
// K-contiguous, which is how X [C_in][N] feeds X X^T and how the symmetric
// H feeds D H).  A 256-thread workgroup owns a 64 x 64 tile of C; its four
// waves own 32 x 32 quadrants as 2 x 2 MFMA tiles (v_mfma_f32_16x16x32_bf16
// for bf16 operands, v_mfma_f32_16x16x4_f32 for fp32), fp32 accumulation.
// K advances in 128-byte chunks staged through LDS (rows padded by 16 bytes)
// with the next chunk's global loads in flight during the MFMAs.  Operand
// loaders are plug-ins (plain, or q - w formed on the fly); epilogues are a
// scaled store or a fixed-order row dot with D (for the output error).  The
// full Hessian of a wide bf16 layer (at least 128 tiles of 256 x 256) runs
// on xxt_big_kernel below instead.
#include "lh_device.h"
#include "lh_internal.h"

namespace lh {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

namespace {

constexpr int kTile = 64;

// Operand element type on the MFMA side and the K chunk (128 bytes per row).
template <typename T>
struct Mfma;
template <>
struct Mfma<uint16_t> {
  static constexpr int kKc = 64;   // bf16 elements per chunk
  static constexpr int kEP = 8;    // elements per 16 bytes
};
template <>
struct Mfma<float> {
  static constexpr int kKc = 32;
  static constexpr int kEP = 4;
};

// Plain operand: rows of T with leading dimension ld.  The 16-byte chunk at
// (row, k) with k % kEP == 0; rows >= rows_end or k >= k_end read as zero.
template <typename T, bool kVec>
struct PlainLoader {
  const T* p;
  int64_t ld;
  int64_t gs;  // group stride (elements)
  __device__ __forceinline__ void group(int64_t g) { p += g * gs; }
  __device__ __forceinline__ uint4 chunk(int64_t row, int64_t k, int64_t rows_end, int64_t k_end) const {
    constexpr int EP = Mfma<T>::kEP;
    if (row >= rows_end || k >= k_end) return make_uint4(0u, 0u, 0u, 0u);
    if (kVec && k + EP <= k_end) return *reinterpret_cast<const uint4*>(p + row * ld + k);
    T v[EP];
#pragma unroll
    for (int i = 0; i < EP; ++i) v[i] = (k + i < k_end) ? p[row * ld + k + i] : T(0);
    return __builtin_bit_cast(uint4, v);
  }
};

// Four consecutive w as fp32 from one vector load (kVec: 16-byte aligned
// fp32 or 8-byte aligned bf16).
__device__ __forceinline__ float4 load4_as_f32(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4_as_f32(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}

// fp32 operand D = q - w (q fp32, w of type TW), formed while loading; kVec:
// q rows 16-byte aligned and w rows aligned to four elements, so a whole
// chunk is one vector load of each.
template <typename TW, bool kVec>
struct DiffLoader {
  const float* q;
  int64_t ldq;
  const TW* w;
  int64_t ldw;
  int64_t gsq, gsw;  // group strides (elements)
  __device__ __forceinline__ void group(int64_t g) {
    q += g * gsq;
    w += g * gsw;
  }
  __device__ __forceinline__ float value(int64_t row, int64_t k) const {
    return q[row * ldq + k] - load_as_f32<TW>(w, row * ldw + k);
  }
  __device__ __forceinline__ uint4 chunk(int64_t row, int64_t k, int64_t rows_end, int64_t k_end) const {
    float v[4];
    if (kVec && row < rows_end && k + 4 <= k_end) {
      const float4 a = *reinterpret_cast<const float4*>(q + row * ldq + k);
      const float4 b = load4_as_f32(w + row * ldw + k);
      v[0] = a.x - b.x;
      v[1] = a.y - b.y;
      v[2] = a.z - b.z;
      v[3] = a.w - b.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (row < rows_end && k + i < k_end) ? value(row, k + i) : 0.0f;
    }
    return __builtin_bit_cast(uint4, v);
  }
};

template <typename T>
__device__ __forceinline__ f32x4_t mfma_step(const T* a, const T* b, f32x4_t acc);
template <>
__device__ __forceinline__ f32x4_t mfma_step<uint16_t>(const uint16_t* a, const uint16_t* b, f32x4_t acc) {
  const bf16x8_t av = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(a));
  const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(b));
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4_t mfma_step<float>(const float* a, const float* b, f32x4_t acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(*a, *b, acc, 0, 0, 0);
}

enum Epi { kEpiStore = 0, kEpiRowDot = 1 };

struct GemmArgs {
  int64_t M, N, K;
  float alpha, beta;
  int lower_only;            // skip tiles strictly above the diagonal (square M == N)         // kEpiStore: C = alpha * acc + beta * C (beta == 0: C not read)
  float* c;                  // kEpiStore output
  int64_t ldc, sc;
  float* part;               // kEpiRowDot: partial[g][m][n-tile]
};

// One workgroup: C tile (blockIdx.y, blockIdx.x) of group blockIdx.z.
template <typename T, typename LA, typename LB, int kEpi>
__global__ __launch_bounds__(kThreads) void gemm_nt_kernel(LA la, LB lb, GemmArgs g) {
  constexpr int kKc = Mfma<T>::kKc;
  constexpr int kEP = Mfma<T>::kEP;
  constexpr int kPitch = kKc + kEP;            // +16 bytes per row
  constexpr int kCPR = kKc / kEP;              // 16-byte chunks per row (8)
  constexpr int kLoads = kTile * kCPR / kThreads;  // per operand per thread (2)
  __shared__ __attribute__((aligned(16))) T as[2][kTile * kPitch];
  __shared__ __attribute__((aligned(16))) T bs[2][kTile * kPitch];

  if (g.lower_only && blockIdx.x > blockIdx.y) return;  // whole workgroup: no barrier is skipped
  const int64_t grp = blockIdx.z;
  la.group(grp);
  lb.group(grp);
  const int64_t m0 = (int64_t)blockIdx.y * kTile, n0 = (int64_t)blockIdx.x * kTile;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;

  uint4 ra[kLoads], rb[kLoads];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / kCPR, col = (c % kCPR) * kEP;
      ra[i] = la.chunk(m0 + row, k0 + col, g.M, g.K);
      rb[i] = lb.chunk(n0 + row, k0 + col, g.N, g.K);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / kCPR, col = (c % kCPR) * kEP;
      *reinterpret_cast<uint4*>(&as[buf][row * kPitch + col]) = ra[i];
      *reinterpret_cast<uint4*>(&bs[buf][row * kPitch + col]) = rb[i];
    }
  };

  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t chunks = (g.K + kKc - 1) / kKc;
  if (chunks > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  const int r16 = lane & 15, kg = lane >> 4;
  for (int64_t ck = 0; ck < chunks; ++ck) {
    const int buf = (int)(ck & 1);
    const bool more = ck + 1 < chunks;
    if (more) gload((ck + 1) * kKc);
    const T* A = as[buf];
    const T* B = bs[buf];
    // bf16: K step 32, lane takes 8 consecutive k at 8 * kg; fp32: K step 4, lane takes k = kg
    constexpr int kStep = sizeof(T) == 2 ? 32 : 4;
    constexpr int kLaneK = sizeof(T) == 2 ? 8 : 1;
#pragma unroll
    for (int ks = 0; ks < kKc; ks += kStep) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const T* arow = A + (32 * wm + 16 * i + r16) * kPitch + ks + kLaneK * kg;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const T* brow = B + (32 * wn + 16 * j + r16) * kPitch + ks + kLaneK * kg;
          acc[i][j] = mfma_step<T>(arow, brow, acc[i][j]);
        }
      }
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
  }

  // lane holds C[32 wm + 16 i + 4 kg + r][32 wn + 16 j + r16]
  if constexpr (kEpi == kEpiStore) {
    float* C = g.c + grp * g.sc;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t m = m0 + 32 * wm + 16 * i + 4 * kg + r;
          const int64_t n = n0 + 32 * wn + 16 * j + r16;
          if (m < g.M && n < g.N) {
            float* cp = C + m * g.ldc + n;
            *cp = (g.beta == 0.0f) ? g.alpha * acc[i][j][r] : g.alpha * acc[i][j][r] + g.beta * (*cp);
          }
        }
  } else {
    // row dot with D = A-source over this tile's 64 columns (K == N here):
    // lane sums its two columns, then the 16 lanes of a row group (xor
    // shuffles), then the two column waves in LDS, all in a fixed order.
    __shared__ float rowsum[2][kTile];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + 32 * wm + 16 * i + 4 * kg + r;
        float v = 0.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t n = n0 + 32 * wn + 16 * j + r16;
          const float d = (m < g.M && n < g.N) ? la.value(m, n) : 0.0f;
          v = __builtin_fmaf(acc[i][j][r], d, v);
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) v += __shfl_xor(v, off, 16);
        if (r16 == 0) rowsum[wn][32 * wm + 16 * i + 4 * kg + r] = v;
      }
    __syncthreads();
    if (tid < kTile) {
      const int64_t m = m0 + tid;
      if (m < g.M) g.part[(grp * g.M + m) * gridDim.x + blockIdx.x] = rowsum[0][tid] + rowsum[1][tid];
    }
  }
}

// Large-tile X X^T for bf16 X (the full Hessian of a wide layer), rows of
// X 16-byte aligned.  A 256-thread workgroup owns a 256 x 256 (or 192 x 192)
// tile of C and its four waves 128 x 128 (96 x 96) quadrants, each a 4 x 4
// (3 x 3) grid of 32 x 32 MFMA tiles (v_mfma_f32_32x32x16_bf16: measured on
// MI355X at 2.2 PFLOP/s with independent accumulators, against 1.4 for the
// 16 x 16 x 32 form; up to 256 fp32 accumulators per lane in the
// accumulation registers, one wave per SIMD).  Per 32-token sub-step a wave
// of the 256 tile reads 16 KiB of operands from LDS for 32 MFMAs, 64 flop
// per LDS byte (48 for the 192 tile; the 64 x 64 tile above gets 16).
//
// The operands come in 64-token steps: per row one whole 128-byte line, so
// each L2 request carries a full line (with 32-token steps every request
// was half a line, and the L2 request rate held the kernel back).  LDS
// holds three buffers of operand A and two of B, 256 (192) rows of 128
// bytes each (160 KiB, or 120), filled straight from global memory (no
// staging registers); the 16-byte chunk c of row r sits at slot c ^ f(r),
// f(r) = ((r & 7) ^ (r >> 3)) & 7 over r mod 32, so the 8 (or 16) lanes
// that LDS serves together read 8 (16) rows' chunk c from distinct banks.
// The step loop below gives the schedule.  Tokens past the last whole step
// go through one more step with checked register loads.  Rows past c_in
// read row c_in - 1 (those outputs are not stored).
constexpr int kBigKc = 64;                  // tokens per step (one 128-byte line of a bf16 row)

__device__ __forceinline__ int big_slot(int row, int chunk) { return chunk ^ (((row & 7) ^ (row >> 3)) & 7); }

// 16 bytes of a row at token kk (past k_len: zeros; the chunk that straddles
// k_len is read whole, which stays inside the 16-byte aligned row, and its
// elements past k_len are cleared).
__device__ __forceinline__ uint4 big_tail_chunk(const uint16_t* p, int64_t kk, int64_t k_len) {
  if (kk >= k_len) return make_uint4(0u, 0u, 0u, 0u);
  uint4 v = *reinterpret_cast<const uint4*>(p);
  const int64_t n = k_len - kk;  // valid elements, 1..
  if (n < 8) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t keep = (2 * e + 1 < n) ? 0xffffffffu : (2 * e < n ? 0x0000ffffu : 0u);
      w[e] &= keep;
    }
    v = make_uint4(w[0], w[1], w[2], w[3]);
  }
  return v;
}

// 16 bytes per lane from global memory straight into LDS: lane l writes
// LDS bytes lds + 16 l .. lds + 16 l + 15 (lds wave-uniform).  Written in
// asm so that the compiler, which would otherwise wait for every such load
// before any LDS read, leaves the waits to the kernel: the kernel waits with
// s_waitcnt vmcnt before the barrier that publishes the data.  No register
// is written; M0 carries the LDS address (nothing else in the kernel uses it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}
#pragma clang diagnostic pop
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Tile (ty, tx) of the lower triangle ty >= tx numbered row by row:
// t = ty (ty + 1) / 2 + tx.
__device__ __forceinline__ void tri_tile(int64_t t, int64_t& ty, int64_t& tx) {
  int64_t y = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
  while ((y + 1) * (y + 2) / 2 <= t) ++y;
  while (y * (y + 1) / 2 > t) --y;
  ty = y;
  tx = t - y * (y + 1) / 2;
}

// The grid walks the lower triangle of tiles (blockIdx.x = t above, one
// group per blockIdx.z); an off-diagonal tile also writes its transpose (H is
// symmetric), staged through LDS so that the transposed rows go out as whole
// 128-byte lines.  kWT MFMA tiles per wave and side: 256 x 256 workgroup
// tiles (kWT = 4) or 192 x 192 (kWT = 3).  vec_h: H rows are 16-byte aligned
// (ldh, gstride_h multiples of 4).
template <int kWT>
__global__ __launch_bounds__(kThreads, 1) void xxt_big_kernel(const uint16_t* __restrict__ x, int64_t ld,
                                                              int64_t gstride, int64_t c, int64_t k_len,
                                                              float alpha, float* __restrict__ h, int64_t ldh,
                                                              int64_t gstride_h, bool vec_h) {
  constexpr int kTile = 64 * kWT;    // workgroup tile (256 or 192)
  constexpr int kWTile = 32 * kWT;   // wave tile
  constexpr int kLoads = kTile * (kBigKc / 8) / kThreads;  // direct loads per operand per wave and step (2 kWT)
  __shared__ __attribute__((aligned(16))) uint16_t as[3][kTile * kBigKc];  // 3 x 32 (24) KiB
  __shared__ __attribute__((aligned(16))) uint16_t bs[2][kTile * kBigKc];  // 2 x 32 (24) KiB
  const int64_t grp = blockIdx.z;
  int64_t ty, tx;
  tri_tile(blockIdx.x, ty, tx);
  const int64_t m0 = ty * kTile, n0 = tx * kTile;
  const bool mirror = ty != tx;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const uint16_t* xg = x + grp * gstride;

  // Direct loads: one wave instruction fills a 1 KiB block of LDS (8 rows
  // of 128 bytes), lane l writing bytes 16 l .. 16 l + 15, i.e. row l >> 3,
  // slot l & 7.  So lane l fetches chunk (l & 7) ^ f(row) of its row, and
  // the 8 lanes of a row together fetch its whole line.  Wave w fills row
  // blocks w + 4 i (i < 2 kWT) of both operand tiles; f depends on the row mod
  // 32 = 8 w + (l >> 3) alone.
  const int drow = lane >> 3;
  const int dcol = big_slot(8 * wave + drow, lane & 7) * 8;
  const uint16_t* ga[kLoads];
  const uint16_t* gb[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int64_t r = 8 * (wave + 4 * i) + drow;
    ga[i] = xg + min(m0 + r, c - 1) * ld + dcol;
    gb[i] = xg + min(n0 + r, c - 1) * ld + dcol;
  }
  // LDS byte address of row block w of buffer 0 (wave-uniform); block w + 4 i
  // is i KiB x 4 further on
  const uint32_t la0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(as[0] + 8 * wave * kBigKc));
  const uint32_t lb0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(bs[0] + 8 * wave * kBigKc));
  constexpr uint32_t kBufBytes = kTile * kBigKc * 2;
  constexpr uint32_t kBlkStride = 32 * kBigKc * 2;  // row blocks w and w + 4
  // the direct loads of operand A (B) for step st into A buffer abuf (B buffer bbuf)
  auto dload_a = [&](int st, int abuf, int i) {
    lds_dma16(ga[i] + (int64_t)st * kBigKc, la0 + abuf * kBufBytes + i * kBlkStride);
  };
  auto dload_b = [&](int st, int bbuf, int i) {
    lds_dma16(gb[i] + (int64_t)st * kBigKc, lb0 + bbuf * kBufBytes + i * kBlkStride);
  };

  // fragment (tile t, half q of sub-step u) of lane l: row 32 t + (l & 31)
  // (+ 32 kWT w), 16-byte chunk 4 (u & 1) + 2 q + (l >> 5) of the buffers that
  // hold step u >> 1; f(row) depends on l & 31 alone
  const int l32 = lane & 31, lh = lane >> 5;
  bf16x8_t fa[2][2][kWT], fb[2][2][kWT];
  // read k (< 4 kWT) of sub-step u from A buffer abuf and B buffer bbuf
  // (those of step u >> 1): half q = k / (2 kWT), tile t = (k / 2) % kWT,
  // operand B for even k, A for odd k
  auto fread1 = [&](int p, int u, int abuf, int bbuf, int k) {
    const int q = k / (2 * kWT), t = (k >> 1) % kWT;
    const int slot = big_slot(l32, 4 * (u & 1) + 2 * q + lh) * 8;
    if (k & 1)
      fa[p][q][t] = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const uint4*>(as[abuf] + (kWTile * wm + 32 * t + l32) * kBigKc + slot));
    else
      fb[p][q][t] = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const uint4*>(bs[bbuf] + (kWTile * wn + 32 * t + l32) * kBigKc + slot));
  };
  auto fread = [&](int p, int u, int abuf, int bbuf) {
#pragma unroll
    for (int k = 0; k < 4 * kWT; ++k) fread1(p, u, abuf, bbuf, k);
  };

  f32x16_t acc[kWT][kWT];
#pragma unroll
  for (int i = 0; i < kWT; ++i)
#pragma unroll
    for (int j = 0; j < kWT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  auto mfma = [&](int p, int q, int i, int j) {
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[p][q][i], fb[p][q][j], acc[i][j], 0, 0, 0);
  };
  auto mfmas = [&](int p) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < kWT; ++i)
#pragma unroll
        for (int j = 0; j < kWT; ++j) mfma(p, q, i, j);
  };

  // Step S in two sub-steps of 2 kWT^2 MFMAs (fragments in set 0, then set 1);
  // step S's operands are in A buffer S % 3 and B buffer S % 2.
  // * First sub-step: A's loads of step S + 2 go into A buffer (S + 2) % 3
  //   (step S - 1's, last read before the barrier that ended step S - 1's
  //   first sub-step), one per kWT MFMAs; the second sub-step's fragments
  //   are read, one per MFMA over the first 4 kWT.  Then the wave waits for all
  //   but those eight loads (step S + 1's A and B have landed) and the
  //   barrier publishes them.
  // * Second sub-step: B's loads of step S + 2 go into B buffer S % 2 (its
  //   last fragments were read before that barrier), one per kWT MFMAs; the
  //   next step's first fragments are read, one per MFMA over the first 4 kWT.
  //   No barrier.
  // A step's 64 KiB of direct loads thus spread over both sub-steps: the
  // load path takes 64 bytes per clock per CU, half of what the MFMAs leave
  // it per sub-step.  The last steps load the last slice again (never
  // read): with no branch around the loads the compiler waits for exactly
  // the loads each step needs.  sched_barrier keeps every group where it is
  // written.
  auto sub_step = [&](int p, bool first, int ld_st, int ld_buf, int u, int abuf, int bbuf) {
#pragma unroll
    for (int n = 0; n < 2 * kWT * kWT; ++n) {
      if (n % kWT == 0) {
        if (first)
          dload_a(ld_st, ld_buf, n / kWT);
        else
          dload_b(ld_st, ld_buf, n / kWT);
      }
      if (n < 4 * kWT) fread1(p ^ 1, u, abuf, bbuf, n);
      mfma(p, n / (kWT * kWT), (n % (kWT * kWT)) / kWT, n % kWT);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // step counts in 32 bits (the launcher keeps K below 2^31)
  const int full = (int)(k_len / kBigKc);
  if (full > 0) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) dload_a(0, 0, i);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) dload_b(0, 0, i);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) dload_a(min(1, full - 1), 1, i);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) dload_b(min(1, full - 1), 1, i);
    wait_vmcnt<2 * kLoads>();  // step 0 has landed
    __syncthreads();
    fread(0, 0, 0, 0);
  }
  int a_cur = 0, a_nxt = 1, a_ld = 2;  // S % 3, (S + 1) % 3, (S + 2) % 3
  for (int S = 0; S < full; ++S) {
    const int ld = min(S + 2, full - 1);
    sub_step(0, true, ld, a_ld, 2 * S + 1, a_cur, S & 1);
    wait_vmcnt<kLoads>();  // all but this sub-step's loads: step S + 1 has landed
    __syncthreads();
    sub_step(1, false, ld, S & 1, 2 * S + 2, a_nxt, (S + 1) & 1);
    const int t3 = a_cur;
    a_cur = a_nxt;
    a_nxt = a_ld;
    a_ld = t3;
  }
  if ((int64_t)full * kBigKc < k_len) {  // the partial last step, through registers
    wait_vmcnt<0>();  // no direct load still lands
    __syncthreads();
    const int64_t k0 = (int64_t)full * kBigKc;
    const int lrow = tid >> 3, lchunk = tid & 7;
    const int lslot = big_slot(lrow, lchunk) * 8;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int64_t ra = min(m0 + lrow + 32 * i, c - 1), rb = min(n0 + lrow + 32 * i, c - 1);
      const uint4 va = big_tail_chunk(xg + ra * ld + 8 * lchunk + k0, k0 + 8 * lchunk, k_len);
      const uint4 vb = big_tail_chunk(xg + rb * ld + 8 * lchunk + k0, k0 + 8 * lchunk, k_len);
      *reinterpret_cast<uint4*>(&as[0][(lrow + 32 * i) * kBigKc + lslot]) = va;
      *reinterpret_cast<uint4*>(&bs[0][(lrow + 32 * i) * kBigKc + lslot]) = vb;
    }
    __syncthreads();
    fread(0, 0, 0, 0);
    mfmas(0);
    if (k_len - k0 > kBigKc / 2) {  // the second half holds tokens too
      fread(0, 1, 0, 0);
      mfmas(0);
    }
  }

  // lane holds C[m0 + 32 kWT wm + 32 i + 8 (e / 4) + 4 (l >> 5) + e % 4][n0 + 32 kWT wn + 32 j + (l & 31)]
  float* C = h + grp * gstride_h;
  if (mirror) {
    // C^T for the tile: n < c always holds here (tx < ty, so tx is not the
    // last tile column); m may pass c in the last tile row.  Per 32-row
    // slab i a wave writes its 32 kWT x 32 block transposed into its own LDS
    // region (32 kWT rows of kMirPitch floats, at most 18 KiB: waves 0, 1 at
    // the start of as, waves 2, 3 at the start of bs), then stores row n of
    // it, 32 consecutive m, as 8 lanes x 16 bytes.
    wait_vmcnt<0>();  // the last steps' direct loads have landed in LDS
    __syncthreads();  // and every wave has finished reading its fragments
    constexpr int kMirPitch = 36;
    float* T = reinterpret_cast<float*>(wave < 2 ? &as[0][0] : &bs[0][0]) + (wave & 1) * (kWTile * kMirPitch);
    const int rr = lane >> 3, cc = 4 * (lane & 7);
#pragma unroll
    for (int i = 0; i < kWT; ++i) {
#pragma unroll
      for (int j = 0; j < kWT; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4*>(&T[(32 * j + l32) * kMirPitch + 8 * q + 4 * lh]) =
              make_float4(alpha * acc[i][j][4 * q], alpha * acc[i][j][4 * q + 1], alpha * acc[i][j][4 * q + 2],
                          alpha * acc[i][j][4 * q + 3]);
      __syncthreads();
      const int64_t m = m0 + kWTile * wm + 32 * i + cc;
#pragma unroll
      for (int s = 0; s < 4 * kWT; ++s) {
        const int r = 8 * s + rr;
        const float4 v = *reinterpret_cast<const float4*>(&T[r * kMirPitch + cc]);
        float* dst = C + (n0 + kWTile * wn + r) * ldh + m;
        if (vec_h && m + 3 < c) {
          *reinterpret_cast<float4*>(dst) = v;
        } else {
          if (m < c) dst[0] = v.x;
          if (m + 1 < c) dst[1] = v.y;
          if (m + 2 < c) dst[2] = v.z;
          if (m + 3 < c) dst[3] = v.w;
        }
      }
      __syncthreads();  // the slab is read before the next one overwrites it
    }
  }
#pragma unroll
  for (int i = 0; i < kWT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t m = m0 + kWTile * wm + 32 * i + 8 * (e >> 2) + 4 * lh + (e & 3);
      if (m >= c) continue;
#pragma unroll
      for (int j = 0; j < kWT; ++j) {
        const int64_t n = n0 + kWTile * wn + 32 * j + l32;
        if (n < c) C[m * ldh + n] = alpha * acc[i][j][e];
      }
    }
}

// e[g][m] = sum over n-tiles of part, in tile order.
__global__ __launch_bounds__(kThreads) void rowdot_reduce_kernel(const float* __restrict__ part, int64_t rows,
                                                                 int64_t tiles, float* __restrict__ e) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= rows) return;
  float v = 0.0f;
  for (int64_t t = 0; t < tiles; ++t) v += part[i * tiles + t];
  e[i] = v;
}

// ---------------------------------------------------------------------------
// W/s histogram: x = fl32(|w| / s_k) with the block's chosen k (the cast's
// own quotient); bin = floor(fl32(x * bins_per_unit)), values at or past
// n_bins count in the overflow bin n_bins.  Per-workgroup LDS counts, then
// one 64-bit atomic add per non-empty bin: integer sums, so the result does
// not depend on the order.
// ---------------------------------------------------------------------------
constexpr int kMaxBins = 4096;

__global__ __launch_bounds__(kThreads) void zero_counts_kernel(unsigned long long* __restrict__ c, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) c[i] = 0ull;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void histogram_kernel(const T* __restrict__ w, int64_t c_out, int64_t c_in,
                                                             int64_t ld_w, int64_t gstride_w,
                                                             const uint8_t* __restrict__ idx,
                                                             const float* __restrict__ amax, int n_bins,
                                                             float bins_per_unit,
                                                             unsigned long long* __restrict__ counts) {
  // A thread takes a 16-weight block at a time (one index and one scale
  // per block, no index division per weight), and each wave
  // counts into its own copy of the bins when four copies fit: the weights
  // of a layer crowd into a few bins, so one shared copy serialised the LDS
  // atomics.  Counts are integers: the result does not depend on the order.
  __shared__ unsigned int local[kMaxBins + 1];
  const int nb1 = n_bins + 1;
  const int copies = (4 * nb1 <= kMaxBins + 1) ? 4 : 1;
  for (int i = threadIdx.x; i < copies * nb1; i += kThreads) local[i] = 0u;
  __syncthreads();
  unsigned int* const mine = local + (copies == 4 ? (threadIdx.x >> 6) * nb1 : 0);
  const int64_t grp = blockIdx.y;
  const float Sg = amax[grp] / kAmaxDivisor;
  const int64_t nb = c_in / 16;
  const int64_t nblk = c_out * nb;
  for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < nblk; q += (int64_t)gridDim.x * kThreads) {
    const int64_t r = q / nb, bb = q - r * nb;
    const int k = idx[grp * nblk + q];
    const float s = e4m3_candidate(k) * Sg;
    const int64_t base = grp * gstride_w + r * ld_w + 16 * bb;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float a = fabsf(load_as_f32<T>(w, base + i));
      const float x = (s == 0.0f) ? 0.0f : a / s;
      const float y = x * bins_per_unit;
      const int bin = (y >= (float)n_bins) ? n_bins : (int)floorf(y);
      atomicAdd(&mine[bin], 1u);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nb1; i += kThreads) {
    unsigned int v = local[i];
    for (int c = 1; c < copies; ++c) v += local[c * nb1 + i];
    if (v) atomicAdd(&counts[grp * nb1 + i], (unsigned long long)v);
  }
}


// ---------------------------------------------------------------------------
// GPTQ rounding with fixed Local-Hessian scales ("Combining with GPTQ":
// Local-Hessian chooses the block scales, GPTQ then replaces the
// round-to-nearest step).  The steps follow the published GPTQ method
// (Frantar et al., ICLR 2023):
//   H' = H + damp * mean(diag H) * I  (I when the diagonal is all zero),
//   U  = the upper Cholesky factor of H'^-1 (H'^-1 = U^T U),
//   per row, for i = 0 .. C_in-1:  q_i = Q(w_i, s_block);
//     e = (w_i - q_i) / U_ii;  w_j = fma(-e, U_ij, w_j) for j > i.
// Every w_j receives its updates in increasing i, one fused multiply-add
// each, whichever kernel applies them: the panel kernel for j inside the
// current 128-column block, the trailing kernel for the columns after it.
// So the result does not depend on the blocking.
//
// U without forming H'^-1: with P the index reversal, A = P H' P = L L^T
// (lower Cholesky, blocked by 64: one wave factorises the diagonal block in
// registers and inverts it; the panel L_r = A_r L_kk^-T and the trailing
// update A -= L_r L_r^T run on the matrix-core GEMM), then H' = R R^T with
// R = P L P upper, and U = R^-1 = P L^-1 P.  L^-1 is formed by block rows,
// X_i = L_ii^-1 (E_i - L_i,<i X_<i), both products on the GEMM (X stored
// transposed so that every operand is K-contiguous).
// ---------------------------------------------------------------------------
constexpr int kCb = 64;     // Cholesky / inverse block
constexpr int kGb = 128;    // GPTQ column block

// ws layout (floats): A/L [n][n] | X = L^-1 [n][n] | Y = X^T [n][n] |
// T [n^2 / 4] | scalars
__global__ __launch_bounds__(kThreads) void gptq_damp_kernel(const float* __restrict__ h, int64_t n, int64_t ld_h,
                                                             float damp, float* __restrict__ out) {
  __shared__ float part[kThreads];
  float v = 0.0f;
  for (int64_t i = threadIdx.x; i < n; i += kThreads) v += h[i * ld_h + i];
  part[threadIdx.x] = v;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (threadIdx.x < off) part[threadIdx.x] += part[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float mean = part[0] / (float)n;
    out[0] = mean;                // 0: no signal, use the identity
    out[1] = damp * mean;
  }
}

// A[i][j] = H'[n-1-i][n-1-j]; X = Y = 0.
__global__ __launch_bounds__(kThreads) void gptq_reverse_kernel(const float* __restrict__ h, int64_t n, int64_t ld_h,
                                                                const float* __restrict__ dm, float* __restrict__ A,
                                                                float* __restrict__ X, float* __restrict__ Y) {
  const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (e >= n * n) return;
  const int64_t i = e / n, j = e - i * n;
  const float mean = dm[0], add = dm[1];
  float v;
  if (mean == 0.0f) v = (i == j) ? 1.0f : 0.0f;
  else v = h[(n - 1 - i) * ld_h + (n - 1 - j)] + (i == j ? add : 0.0f);
  A[e] = v;
  X[e] = 0.0f;
  Y[e] = 0.0f;
}

// In-place lower Cholesky of the bs x bs diagonal block at (k0, k0) of A,
// by one wave, and the inverse of the factor into the same block of X (and
// transposed into Y): lane i keeps
// row i in registers (padded with the identity beyond bs); the pivot comes
// from lane j by v_readlane and column j's entries reach the other lanes
// through LDS.  Lane i's lower entries only ever combine lower entries
// (a[c] -= a[j] l_cj with j < c <= i), so whatever the upper part holds is
// never used; it is written back as zeros.
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__global__ __launch_bounds__(64) void chol_diag_kernel(float* __restrict__ A, int64_t n, int64_t k0, int bs,
                                                       float* __restrict__ X, float* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) float col[kCb];
  __shared__ __attribute__((aligned(16))) float l[kCb][kCb + 4];
  const int i = threadIdx.x;
  float a[kCb];
#pragma unroll
  for (int c4 = 0; c4 < kCb; c4 += 4) {  // bs is a multiple of 16
    float4 v = make_float4(c4 == i, c4 + 1 == i, c4 + 2 == i, c4 + 3 == i);
    if (i < bs && c4 < bs) v = *reinterpret_cast<const float4*>(A + (k0 + i) * n + k0 + c4);
    a[c4] = v.x;
    a[c4 + 1] = v.y;
    a[c4 + 2] = v.z;
    a[c4 + 3] = v.w;
  }
  // right-looking: column j's entries l_cj reach every lane through LDS,
  // four at a time
#pragma unroll
  for (int j = 0; j < kCb; ++j) {
    const float d = lane_value(a[j], j);
    const float inv = __builtin_amdgcn_rsqf(d);  // 1/sqrt(d) to about an ulp
    a[j] = (i == j) ? d * inv : a[j] * inv;
    if (j + 1 < kCb) {
      col[i] = a[j];
      __syncthreads();
#pragma unroll
      for (int c4 = ((j + 1) & ~3); c4 < kCb; c4 += 4) {
        const float4 v = *reinterpret_cast<const float4*>(&col[c4]);
        const float vc[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (c4 + t > j) a[c4 + t] = __builtin_fmaf(-a[j], vc[t], a[c4 + t]);
      }
      __syncthreads();  // col is rewritten for the next column
    }
  }
#pragma unroll
  for (int c = 0; c < kCb; ++c) l[i][c] = c <= i ? a[c] : 0.0f;
  if (i < bs) {
#pragma unroll
    for (int c = 0; c < kCb; ++c)
      if (c < bs) A[(k0 + i) * n + k0 + c] = c <= i ? a[c] : 0.0f;
  }
  __syncthreads();
  // L^-1 (lower; the identity padding inverts to itself): lane j solves
  // L x = e_j by forward substitution (four partial sums per row) and
  // writes column j of the block into X and row j into Y = X^T.
  float x[kCb];
#pragma unroll
  for (int r = 0; r < kCb; ++r) {
    float p[4] = {(r == i) ? 1.0f : 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c4 = 0; c4 < r; c4 += 4) {
      const float4 v = *reinterpret_cast<const float4*>(&l[r][c4]);
      const float vc[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (c4 + t < r) p[t] = __builtin_fmaf(-vc[t], x[c4 + t], p[t]);
    }
    x[r] = ((p[0] + p[1]) + (p[2] + p[3])) * (1.0f / l[r][r]);  // the reciprocal is off the chain
  }
  __syncthreads();  // every lane is done reading l
#pragma unroll
  for (int r = 0; r < kCb; ++r) l[r][i] = x[r];
  __syncthreads();
  if (i < bs) {
    float* xp = X + k0 * n + k0 + i;  // X[k0 + r][k0 + i] = L^-1[r][i]
    float* yp = Y + k0 * n + k0 + i;  // Y[k0 + r][k0 + i] = L^-1[i][r]
    for (int r = 0; r < bs; ++r) {
      xp[r * n] = l[r][i];
      yp[r * n] = l[i][r];
    }
  }
}

// U[i][j] = X[n-1-i][n-1-j] (upper; zero below).
__global__ __launch_bounds__(kThreads) void gptq_u_kernel(const float* __restrict__ X, int64_t n, float* __restrict__ U,
                                                          int64_t ld_u) {
  const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (e >= n * n) return;
  const int64_t i = e / n, j = e - i * n;
  U[i * ld_u + j] = (j >= i) ? X[(n - 1 - i) * n + (n - 1 - j)] : 0.0f;
}

// X21 = Y12^T for each pair of one level of the triangular inverse: pair z
// has Y12 at Y[o][o + b] and X21 at X[o + b][o], o = o0 + z * 2b (b x s2
// and s2 x b), through 32 x 32 LDS tiles.
__global__ __launch_bounds__(kThreads) void gptq_transpose_kernel(const float* __restrict__ Y, float* __restrict__ X,
                                                                  int64_t n, int64_t o0, int64_t b, int64_t s2) {
  __shared__ float t[32][33];
  const int64_t o = o0 + (int64_t)blockIdx.z * 2 * b;
  const int64_t m0 = (int64_t)blockIdx.y * 32, c0 = (int64_t)blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int r = ty; r < 32; r += 8) {
    const int64_t m = m0 + r, c = c0 + tx;
    t[r][tx] = (m < b && c < s2) ? Y[(o + m) * n + o + b + c] : 0.0f;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int64_t c = c0 + r, m = m0 + tx;
    if (m < b && c < s2) X[(o + b + c) * n + o + m] = t[tx][r];
  }
}

// Running fp32 weights.
template <typename T>
__global__ __launch_bounds__(kThreads) void gptq_copy_kernel(const T* __restrict__ w, int64_t c_out, int64_t c_in,
                                                             int64_t ld_w, float* __restrict__ wf) {
  const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (e >= c_out * c_in) return;
  const int64_t r = e / c_in, c = e - r * c_in;
  wf[e] = load_as_f32<T>(w, r * ld_w + c);
}

// Q(x, s) of the cast: x' = fl32(|x| / s) (IEEE), nearest E2M1 value (ties
// to the even code, saturating), q = fl32(sign(x) r s), -0 -> +0.
__device__ __forceinline__ float cast_q(float x, float s) {
  const float r = (s == 0.0f) ? 0.0f : e2m1_round_mag(fabsf(x) / s);
  return copysignf(r * s, x) + 0.0f;
}

// Value held by lane o of this lane's group of eight (ds_swizzle bit mode
// within 32-lane halves: new lane = (lane & 24) | o).
template <int o>
__device__ __forceinline__ float group8_lane(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x18 | (o << 5)));
}

constexpr int kPanelChunk = 20;  // LDS floats per 16-column chunk: 8 chunks start on 8 disjoint bank quads

// Steps for the columns owned by lanes o .. 7 of each group (see
// gptq_panel_kernel): for each of owner o's sixteen columns, the owner
// quantises, the error is broadcast, and every lane updates its columns.
template <int o>
__device__ __forceinline__ void panel_steps(float (&w)[16], float (&qv)[16], float (&ev)[16], float s, int g,
                                            int width, const float (*u)[8 * kPanelChunk]) {
  if constexpr (o < 8) {
    if (16 * o >= width) return;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const int i = 16 * o + c;
      float e = 0.0f;
      if (g == o) {
        const float x = w[c];
        const float qi = cast_q(x, s);
        qv[c] = qi;
        e = (x - qi) / u[i][o * kPanelChunk + c];
        ev[c] = e;
      }
      e = group8_lane<o>(e);
      const float4* ur = reinterpret_cast<const float4*>(&u[i][g * kPanelChunk]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 v = ur[k];
        w[4 * k] = __builtin_fmaf(-e, v.x, w[4 * k]);
        w[4 * k + 1] = __builtin_fmaf(-e, v.y, w[4 * k + 1]);
        w[4 * k + 2] = __builtin_fmaf(-e, v.z, w[4 * k + 2]);
        w[4 * k + 3] = __builtin_fmaf(-e, v.w, w[4 * k + 3]);
      }
    }
    panel_steps<o + 1>(w, qv, ev, s, g, width, u);
  }
}

// Panel: eight lanes per output row, lane g owning the block's columns
// 16g .. 16g+15 (one NVFP4 block, so one block scale per lane).  Column i is
// quantised by its owner; the error e_i = (w_i - q_i) / U_ii reaches the
// row's other lanes by a broadcast within the group of eight, and every lane
// applies w_j -= e_i U_ij (one fused multiply-add) to its sixteen columns.
// U_ij = 0 for j < i, so the columns already quantised (never read again)
// are the only ones an update may touch besides j > i, and each w_j with
// j > i receives exactly the sequential chain of updates in increasing i.
// Writes Q and the errors, transposed: E[i][row].
__global__ __launch_bounds__(kThreads) void gptq_panel_kernel(float* __restrict__ wf, int64_t c_out, int64_t c_in,
                                                              int64_t b0, int width, const float* __restrict__ U,
                                                              int64_t ld_u, const uint8_t* __restrict__ idx,
                                                              const float* __restrict__ amax, float* __restrict__ q,
                                                              int64_t ld_q, float* __restrict__ E) {
  __shared__ __attribute__((aligned(16))) float u[kGb][8 * kPanelChunk];
  // staging: sixteen loads in flight per thread before their LDS writes
  for (int base = 0; base < kGb * kGb / kThreads; base += 16) {
    float v[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int e = (base + t) * kThreads + threadIdx.x;
      const int i = e / kGb, j = e % kGb;
      v[t] = (i < width && j < width) ? U[(b0 + i) * ld_u + b0 + j] : 0.0f;
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int e = (base + t) * kThreads + threadIdx.x;
      const int i = e / kGb, j = e % kGb;
      u[i][(j >> 4) * kPanelChunk + (j & 15)] = v[t];
    }
  }
  __syncthreads();
  const int g = threadIdx.x & 7;
  const int64_t r = (int64_t)blockIdx.x * (kThreads / 8) + (threadIdx.x >> 3);
  if (r >= c_out) return;  // whole groups of eight leave together
  const bool mine = 16 * g < width;
  float w[16];
  if (mine) {
    const float4* src = reinterpret_cast<const float4*>(wf + r * c_in + b0 + 16 * g);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 v = src[k];
      w[4 * k] = v.x;
      w[4 * k + 1] = v.y;
      w[4 * k + 2] = v.z;
      w[4 * k + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) w[k] = 0.0f;
  }
  const float Sg = amax[0] / kAmaxDivisor;
  const float s = mine ? e4m3_candidate(idx[r * (c_in / 16) + (b0 >> 4) + g]) * Sg : 0.0f;
  float qv[16], ev[16];
  panel_steps<0>(w, qv, ev, s, g, width, u);
  if (mine) {
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      q[r * ld_q + b0 + 16 * g + c] = qv[c];
      E[(int64_t)(16 * g + c) * c_out + r] = ev[c];
    }
  }
}

// Trailing columns j >= b0 + width: wf[r][j] receives the block's updates
// -E[i][r] U[b0+i][j] as fused multiply-adds in increasing i (the sequential
// chain).  128 x 128 tile per workgroup, 8 x 8 per thread; E^T and the U
// rows go through LDS 64 values of i at a time (67 KB, two workgroups per
// CU).
constexpr int kTrail = 128;
constexpr int kTrailI = 64;
__global__ __launch_bounds__(kThreads) void gptq_trailing_kernel(float* __restrict__ wf, int64_t c_out, int64_t c_in,
                                                                 int64_t b0, int width, const float* __restrict__ U,
                                                                 int64_t ld_u, const float* __restrict__ E) {
  constexpr int kP = kTrail + 4;
  __shared__ __attribute__((aligned(16))) float es[kTrailI][kP];
  __shared__ __attribute__((aligned(16))) float us[kTrailI][kP];
  const int64_t j0 = b0 + width + (int64_t)blockIdx.x * kTrail;
  const int64_t r0 = (int64_t)blockIdx.y * kTrail;
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
  const int64_t jc = j0 + 8 * tc;
  const bool cols = jc < c_in;  // c_in is a multiple of 16: all eight columns or none
  float acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int64_t r = r0 + 8 * tr + a;
    if (r < c_out && cols) {
      const float4* src = reinterpret_cast<const float4*>(wf + r * c_in + jc);
      const float4 v0 = src[0], v1 = src[1];
      acc[a][0] = v0.x; acc[a][1] = v0.y; acc[a][2] = v0.z; acc[a][3] = v0.w;
      acc[a][4] = v1.x; acc[a][5] = v1.y; acc[a][6] = v1.z; acc[a][7] = v1.w;
    } else {
#pragma unroll
      for (int b = 0; b < 8; ++b) acc[a][b] = 0.0f;
    }
  }
  for (int i0 = 0; i0 < width; i0 += kTrailI) {
    if (i0 > 0) __syncthreads();  // every thread is done with the previous chunk
    // staging: sixteen loads of each array in flight per thread before their
    // LDS writes
    for (int base = 0; base < kTrailI * kTrail / kThreads; base += 16) {
      float ve[16], vu[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int e = (base + t) * kThreads + threadIdx.x;
        const int i = i0 + e / kTrail, x = e % kTrail;
        ve[t] = (i < width && r0 + x < c_out) ? E[(int64_t)i * c_out + r0 + x] : 0.0f;
        vu[t] = (i < width && j0 + x < c_in) ? U[(b0 + i) * ld_u + j0 + x] : 0.0f;
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int e = (base + t) * kThreads + threadIdx.x;
        es[e / kTrail][e % kTrail] = ve[t];
        us[e / kTrail][e % kTrail] = vu[t];
      }
    }
    __syncthreads();
    const int n = width - i0 < kTrailI ? width - i0 : kTrailI;
#pragma unroll 2
    for (int i = 0; i < n; ++i) {
      const float4 e0 = *reinterpret_cast<const float4*>(&es[i][8 * tr]);
      const float4 e1 = *reinterpret_cast<const float4*>(&es[i][8 * tr + 4]);
      const float4 v0 = *reinterpret_cast<const float4*>(&us[i][8 * tc]);
      const float4 v1 = *reinterpret_cast<const float4*>(&us[i][8 * tc + 4]);
      const float ev[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
      const float uv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = __builtin_fmaf(-ev[a], uv[b], acc[a][b]);
    }
  }
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int64_t r = r0 + 8 * tr + a;
    if (r < c_out && cols) {
      float4* dst = reinterpret_cast<float4*>(wf + r * c_in + jc);
      dst[0] = make_float4(acc[a][0], acc[a][1], acc[a][2], acc[a][3]);
      dst[1] = make_float4(acc[a][4], acc[a][5], acc[a][6], acc[a][7]);
    }
  }
}

template <typename T, bool kVec>
hipError_t launch_full_hessian_typed(const FullHessianArgs& a, hipStream_t stream) {
  if constexpr (sizeof(T) == 2 && kVec) {
    // Wide layers (at least 128 tiles of 256 x 256 in the square) on the
    // large-tile kernel: the lower triangle of 256 x 256 tiles, or of
    // 192 x 192 where its rounds of the 256 CUs (one workgroup each) cost
    // less, a 192 tile's work counted at 0.5625 x 1.15 of a 256 tile's (its
    // smaller MFMA grid reads more LDS per MFMA; measured 1.16-1.23).
    const int64_t n4 = (a.c_in + 255) / 256, n3 = (a.c_in + 191) / 192;
    if (n4 * n4 * a.n_groups >= 128 && a.n_tok < ((int64_t)1 << 31) && n3 * (n3 + 1) / 2 < ((int64_t)1 << 31)) {
      const bool vec_h = reinterpret_cast<uintptr_t>(a.h) % 16 == 0 && a.ld_h % 4 == 0 && a.gstride_h % 4 == 0;
      const uint16_t* xx = static_cast<const uint16_t*>(a.x);
      const int64_t t4 = n4 * (n4 + 1) / 2, t3 = n3 * (n3 + 1) / 2;
      const int64_t r4 = (t4 * a.n_groups + 255) / 256, r3 = (t3 * a.n_groups + 255) / 256;
      if ((double)r3 * 0.5625 * 1.15 < (double)r4)
        xxt_big_kernel<3><<<dim3((unsigned)t3, 1, (unsigned)a.n_groups), dim3(kThreads), 0, stream>>>(
            xx, a.ld_x, a.gstride_x, a.c_in, a.n_tok, a.alpha, a.h, a.ld_h, a.gstride_h, vec_h);
      else
        xxt_big_kernel<4><<<dim3((unsigned)t4, 1, (unsigned)a.n_groups), dim3(kThreads), 0, stream>>>(
            xx, a.ld_x, a.gstride_x, a.c_in, a.n_tok, a.alpha, a.h, a.ld_h, a.gstride_h, vec_h);
      return hipGetLastError();
    }
  }
  PlainLoader<T, kVec> L{static_cast<const T*>(a.x), a.ld_x, a.gstride_x};
  GemmArgs g{a.c_in, a.c_in, a.n_tok, a.alpha, 0.0f, 0, a.h, a.ld_h, a.gstride_h, nullptr};
  const dim3 grid((unsigned)((a.c_in + kTile - 1) / kTile), (unsigned)((a.c_in + kTile - 1) / kTile),
                  (unsigned)a.n_groups);
  gemm_nt_kernel<T, PlainLoader<T, kVec>, PlainLoader<T, kVec>, kEpiStore><<<grid, dim3(kThreads), 0, stream>>>(L, L, g);
  return hipGetLastError();
}

template <typename TW, bool kVecH, bool kVecD>
hipError_t launch_output_error_typed(const OutputErrorArgs& a, hipStream_t stream) {
  DiffLoader<TW, kVecD> D{a.q, a.ld_q, static_cast<const TW*>(a.w), a.ld_w, a.gstride_q, a.gstride_w};
  PlainLoader<float, kVecH> H{a.h, a.ld_h, a.gstride_h};
  const int64_t tiles = (a.c_in + kTile - 1) / kTile;
  float* part = static_cast<float*>(a.ws);
  GemmArgs g{a.c_out, a.c_in, a.c_in, 1.0f, 0.0f, 0, nullptr, 0, 0, part};
  const dim3 grid((unsigned)tiles, (unsigned)((a.c_out + kTile - 1) / kTile), (unsigned)a.n_groups);
  gemm_nt_kernel<float, DiffLoader<TW, kVecD>, PlainLoader<float, kVecH>, kEpiRowDot>
      <<<grid, dim3(kThreads), 0, stream>>>(D, H, g);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t rows = a.n_groups * a.c_out;
  rowdot_reduce_kernel<<<dim3((unsigned)((rows + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream>>>(
      part, rows, tiles, a.err);
  return hipGetLastError();
}

}  // namespace


size_t gptq_prepare_ws_bytes(int64_t n) {
  // A, X, Y (n x n each), T (the products of one inverse level: at most n^2 / 4)
  return ((size_t)3 * n * n + (size_t)n * n / 4 + 64) * sizeof(float);
}

size_t gptq_quantize_ws_bytes(int64_t c_out, int64_t c_in) {
  return ((size_t)c_out * c_in + (size_t)c_out * kGb) * sizeof(float);
}

hipError_t launch_gptq_prepare(const GptqPrepareArgs& a, hipStream_t stream) {
  const int64_t n = a.n;
  if (n == 0) return hipSuccess;
  float* ws = static_cast<float*>(a.ws);
  float* A = ws;                   // A, then L
  float* X = A + n * n;            // L^-1
  float* Y = X + n * n;            // (L^-1)^T
  float* T = Y + n * n;            // products of one inverse level
  float* dm = T + n * n / 4;
  gptq_damp_kernel<<<dim3(1), dim3(kThreads), 0, stream>>>(a.h, n, a.ld_h, a.damp, dm);
  gptq_reverse_kernel<<<dim3((unsigned)((n * n + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream>>>(
      a.h, n, a.ld_h, dm, A, X, Y);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // blocked lower Cholesky of A: diagonal block (and its inverse, into X and
  // Y), panel L_r = A_r L_kk^-T in place on the GEMM, trailing A -= L_r L_r^T
  for (int64_t k0 = 0; k0 < n; k0 += kCb) {
    const int bs = (int)(n - k0 < kCb ? n - k0 : kCb);
    chol_diag_kernel<<<dim3(1), dim3(64), 0, stream>>>(A, n, k0, bs, X, Y);
    const int64_t rest = n - k0 - bs;
    if (rest > 0) {
      const unsigned tiles = (unsigned)((rest + kTile - 1) / kTile);
      {
        // each workgroup reads its rows of the panel before writing them
        PlainLoader<float, true> P{A + (k0 + bs) * n + k0, n, 0};
        PlainLoader<float, true> Lb{X + k0 * n + k0, n, 0};
        GemmArgs g{rest, bs, bs, 1.0f, 0.0f, 0, A + (k0 + bs) * n + k0, n, 0, nullptr};
        gemm_nt_kernel<float, PlainLoader<float, true>, PlainLoader<float, true>, kEpiStore>
            <<<dim3(1, tiles, 1), dim3(kThreads), 0, stream>>>(P, Lb, g);
      }
      PlainLoader<float, true> P{A + (k0 + bs) * n + k0, n, 0};
      GemmArgs g{rest, rest, bs, -1.0f, 1.0f, 1, A + (k0 + bs) * n + k0 + bs, n, 0, nullptr};
      gemm_nt_kernel<float, PlainLoader<float, true>, PlainLoader<float, true>, kEpiStore>
          <<<dim3(tiles, tiles, 1), dim3(kThreads), 0, stream>>>(P, P, g);
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // X = L^-1 from the diagonal blocks' inverses by doubling: for each pair
  // of neighbouring blocks [L11 0; L21 L22] of size b (the second possibly
  // shorter, s2), X21 = -X22 L21 X11, computed as its transpose
  // Y12 = -(Y11 L21^T) Y22 = -R X22^T with R = Y11 L21^T (both products on
  // the GEMM with K-contiguous operands), then X21 = Y12^T.  All full pairs
  // of a level go in one batched launch.
  for (int64_t b = kCb; b < n; b *= 2) {
    const int64_t full = n / (2 * b);                 // pairs of two full blocks
    const int64_t tail_o = full * 2 * b;              // a last pair with a shorter second block
    const int64_t tail_s2 = n - tail_o - b;           // > 0 when that pair exists
    for (int part = 0; part < 2; ++part) {
      const int64_t o0 = part == 0 ? 0 : tail_o;
      const int64_t s2 = part == 0 ? b : tail_s2;
      const int64_t groups = part == 0 ? full : (tail_s2 > 0 ? 1 : 0);
      if (groups == 0 || s2 <= 0) continue;
      const int64_t gs = 2 * b * (n + 1);             // one pair to the next along the diagonal
      const unsigned tb = (unsigned)((b + kTile - 1) / kTile), ts = (unsigned)((s2 + kTile - 1) / kTile);
      {
        PlainLoader<float, true> Ya{Y + o0 * n + o0, n, gs};
        PlainLoader<float, true> Lb{A + (o0 + b) * n + o0, n, gs};
        GemmArgs g{b, s2, b, 1.0f, 0.0f, 0, T, s2, b * s2, nullptr};  // R: b x s2 per pair (<= n^2 / 4 in all)
        gemm_nt_kernel<float, PlainLoader<float, true>, PlainLoader<float, true>, kEpiStore>
            <<<dim3(ts, tb, (unsigned)groups), dim3(kThreads), 0, stream>>>(Ya, Lb, g);
      }
      {
        PlainLoader<float, true> Ra{T, s2, b * s2};
        PlainLoader<float, true> Xb{X + (o0 + b) * n + o0 + b, n, gs};
        GemmArgs g{b, s2, s2, -1.0f, 0.0f, 0, Y + o0 * n + o0 + b, n, gs, nullptr};
        gemm_nt_kernel<float, PlainLoader<float, true>, PlainLoader<float, true>, kEpiStore>
            <<<dim3(ts, tb, (unsigned)groups), dim3(kThreads), 0, stream>>>(Ra, Xb, g);
      }
      gptq_transpose_kernel<<<dim3((unsigned)((s2 + 31) / 32), (unsigned)((b + 31) / 32), (unsigned)groups),
                              dim3(kThreads), 0, stream>>>(Y, X, n, o0, b, s2);
      err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
  }
  gptq_u_kernel<<<dim3((unsigned)((n * n + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream>>>(X, n, a.u, a.ld_u);
  return hipGetLastError();
}

hipError_t launch_gptq_quantize(const GptqQuantizeArgs& a, hipStream_t stream) {
  if (a.c_out == 0 || a.c_in == 0) return hipSuccess;
  float* wf = static_cast<float*>(a.ws);
  float* E = wf + a.c_out * a.c_in;
  const unsigned ge = (unsigned)((a.c_out * a.c_in + kThreads - 1) / kThreads);
  if (a.dtype == 1)
    gptq_copy_kernel<uint16_t><<<dim3(ge), dim3(kThreads), 0, stream>>>(static_cast<const uint16_t*>(a.w), a.c_out,
                                                                        a.c_in, a.ld_w, wf);
  else
    gptq_copy_kernel<float><<<dim3(ge), dim3(kThreads), 0, stream>>>(static_cast<const float*>(a.w), a.c_out, a.c_in,
                                                                     a.ld_w, wf);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  for (int64_t b0 = 0; b0 < a.c_in; b0 += kGb) {
    const int width = (int)(a.c_in - b0 < kGb ? a.c_in - b0 : kGb);
    const int64_t rows_per_wg = kThreads / 8;  // eight lanes per row
    gptq_panel_kernel<<<dim3((unsigned)((a.c_out + rows_per_wg - 1) / rows_per_wg)), dim3(kThreads), 0, stream>>>(
        wf, a.c_out, a.c_in, b0, width, a.u, a.ld_u, a.idx, a.amax, a.q, a.ld_q, E);
    const int64_t rest = a.c_in - b0 - width;
    if (rest > 0)
      gptq_trailing_kernel<<<dim3((unsigned)((rest + kTrail - 1) / kTrail),
                                  (unsigned)((a.c_out + kTrail - 1) / kTrail)),
                             dim3(kThreads), 0, stream>>>(wf, a.c_out, a.c_in, b0, width, a.u, a.ld_u, E);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

size_t output_error_ws_bytes(int64_t c_out, int64_t c_in, int64_t n_groups) {
  return (size_t)n_groups * (size_t)c_out * (size_t)((c_in + kTile - 1) / kTile) * sizeof(float);
}

int histogram_max_bins() { return kMaxBins; }

hipError_t launch_full_hessian(const FullHessianArgs& a, hipStream_t stream) {
  if (a.n_groups == 0 || a.c_in == 0) return hipSuccess;
  const int64_t ep = a.dtype == 1 ? 8 : 4;
  const bool vec = reinterpret_cast<uintptr_t>(a.x) % 16 == 0 && a.ld_x % ep == 0 && a.gstride_x % ep == 0;
  if (a.dtype == 1)
    return vec ? launch_full_hessian_typed<uint16_t, true>(a, stream) : launch_full_hessian_typed<uint16_t, false>(a, stream);
  return vec ? launch_full_hessian_typed<float, true>(a, stream) : launch_full_hessian_typed<float, false>(a, stream);
}

hipError_t launch_output_error(const OutputErrorArgs& a, hipStream_t stream) {
  if (a.n_groups == 0 || a.c_out == 0) return hipSuccess;
  const bool vh = reinterpret_cast<uintptr_t>(a.h) % 16 == 0 && a.ld_h % 4 == 0 && a.gstride_h % 4 == 0;
  const size_t wsz = a.dtype == 1 ? 2 : 4;
  const bool vd = reinterpret_cast<uintptr_t>(a.q) % 16 == 0 && a.ld_q % 4 == 0 && a.gstride_q % 4 == 0 &&
                  reinterpret_cast<uintptr_t>(a.w) % (4 * wsz) == 0 && a.ld_w % 4 == 0 && a.gstride_w % 4 == 0;
  if (a.dtype == 1) {
    if (vd) return vh ? launch_output_error_typed<uint16_t, true, true>(a, stream)
                      : launch_output_error_typed<uint16_t, false, true>(a, stream);
    return vh ? launch_output_error_typed<uint16_t, true, false>(a, stream)
              : launch_output_error_typed<uint16_t, false, false>(a, stream);
  }
  if (vd) return vh ? launch_output_error_typed<float, true, true>(a, stream)
                    : launch_output_error_typed<float, false, true>(a, stream);
  return vh ? launch_output_error_typed<float, true, false>(a, stream)
            : launch_output_error_typed<float, false, false>(a, stream);
}

hipError_t launch_histogram(const HistogramArgs& a, hipStream_t stream) {
  if (a.n_groups == 0) return hipSuccess;
  const int64_t nc = a.n_groups * (a.n_bins + 1);
  zero_counts_kernel<<<dim3((unsigned)((nc + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream>>>(a.counts, nc);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.c_out == 0 || a.c_in == 0) return err;
  const int64_t total = a.c_out * a.c_in;
  int64_t blocks = (total + kThreads * 16 - 1) / (kThreads * 16);
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks, (unsigned)a.n_groups);
  if (a.dtype == 1)
    histogram_kernel<uint16_t><<<grid, dim3(kThreads), 0, stream>>>(
        static_cast<const uint16_t*>(a.w), a.c_out, a.c_in, a.ld_w, a.gstride_w, a.idx, a.amax, a.n_bins,
        a.bins_per_unit, a.counts);
  else
    histogram_kernel<float><<<grid, dim3(kThreads), 0, stream>>>(
        static_cast<const float*>(a.w), a.c_out, a.c_in, a.ld_w, a.gstride_w, a.idx, a.amax, a.n_bins,
        a.bins_per_unit, a.counts);
  return hipGetLastError();
}

}  // namespace lh
