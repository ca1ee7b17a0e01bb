// lh_quant.hip - NVFP4 fake-quant / packing with chosen block scales, and
// the per-group global amax.
//
// "Local-Hessian weight-scale guide" (xxmr.cn/news/266017):
//   "What is Local-Hessian": NVFP4 = E2M1 elements, one FP8 E4M3 scale per 16
//     weights, an FP32 per-tensor scale on top; the block scale maps the block
//     into [-6, 6]; max scaling takes the block's largest |w|.
//   "Algorithm principle": Q(W, s) = Cast(W / s) * s; the kernel receives the
//     global FP32 amax; candidate scales are bit-consistent with fake-quant.
// Both kernels are HBM-bound streaming passes.
#include <math.h>

#include "lh_device.h"
#include "lh_internal.h"

namespace lh {
namespace {

template <typename T, bool kVec>
__device__ __forceinline__ void load16(const T* p, float (&w)[16]) {
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

// One thread per 16-weight block.  Outputs are dense and each optional; the
// cast is nvfp4_cast_block, which the fused sweep uses too.  s == 0 (amax 0)
// gives x = 0 for every weight.  The workgroup's fp32 Q (256 blocks, 64
// contiguous bytes each) leaves through LDS, so that every store instruction
// writes 1 KiB of consecutive bytes: written from each thread, a wave's store
// put 16 of every 64 bytes over 4 KiB.  The nibbles and codes are
// consecutive per wave as they are.  In LDS the four 16-byte quarters of
// block i sit in the order rotated by i/2, so neither the writes (64-byte
// stride) nor the reads (16-byte stride) meet a bank twice in 8 lanes.
template <typename T, bool kVec>
__global__ __launch_bounds__(kThreads) void fake_quant_kernel(const T* __restrict__ wt, int64_t c_out,
                                                              int64_t ld_w, int64_t gstride_w, int64_t nb,
                                                              int64_t total, const uint8_t* __restrict__ idx,
                                                              const float* __restrict__ amax,
                                                              float* __restrict__ wq,
                                                              uint8_t* __restrict__ packed,
                                                              uint8_t* __restrict__ codes,
                                                              float* __restrict__ gscale, int64_t n_groups) {
  __shared__ float4 stage[kThreads * 4];
  const int tid = threadIdx.x;
  const int64_t f0 = (int64_t)blockIdx.x * kThreads;
  const int64_t f = f0 + tid;
  if (gscale && f < n_groups) gscale[f] = amax[f] / kAmaxDivisor;  // S_g, written once per group
  if (f < total) {
    const int64_t b = f % nb;
    const int64_t rg = f / nb;  // grp * c_out + row
    const int64_t grp = rg / c_out, row = rg - grp * c_out;
    const int k = idx[f];
    const float Sg = amax[grp] / kAmaxDivisor;
    const float s = e4m3_candidate(k) * Sg;
    float w[16];
    load16<T, kVec>(wt + grp * gstride_w + row * ld_w + 16 * b, w);
    uint32_t pk[2];
    nvfp4_cast_block(w, s, pk);
    nvfp4_emit_at(pk, s, k, f, nullptr, packed, codes);  // block f = rg * nb + b: nibbles and code
    if (wq) {
      float q[16];
      nvfp4_decode_block(pk, s, q);
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        stage[4 * tid + ((qd + (tid >> 1)) & 3)] = make_float4(q[4 * qd], q[4 * qd + 1], q[4 * qd + 2], q[4 * qd + 3]);
    }
  }
  if (wq == nullptr) return;  // the same for every thread
  __syncthreads();
  const int64_t live = total - f0 < kThreads ? total - f0 : kThreads;  // this workgroup's blocks
  float4* dst = reinterpret_cast<float4*>(wq + 16 * f0);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = tid + kThreads * r;  // 16-byte piece i of the workgroup's Q
    const int blk = i >> 2;
    if (blk < live) dst[i] = stage[4 * blk + (((i & 3) + (blk >> 1)) & 3)];
  }
}

__global__ void global_scale_kernel(const float* __restrict__ amax, float* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) out[i] = amax[i] / kAmaxDivisor;
}

template <typename T, bool kVec>
hipError_t launch_fq_typed(const FakeQuantArgs& a, hipStream_t stream) {
  const int64_t nb = a.c_in / 16;
  const int64_t total = a.n_groups * a.c_out * nb;
  if (total > 0 && (a.wq || a.packed || a.codes)) {
    // threads f < n_groups also write S_g, so the grid covers both
    const int64_t n = total > a.n_groups ? total : a.n_groups;
    const int64_t grid = (n + kThreads - 1) / kThreads;
    fake_quant_kernel<T, kVec><<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(
        static_cast<const T*>(a.w), a.c_out, a.ld_w, a.gstride_w, nb, total, a.idx, a.amax, a.wq, a.packed,
        a.codes, a.gscale, a.n_groups);
    return hipGetLastError();
  }
  if (a.gscale && a.n_groups > 0) {
    global_scale_kernel<<<dim3((unsigned)((a.n_groups + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream>>>(
        a.amax, a.gscale, a.n_groups);
    return hipGetLastError();
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Global amax: |w| as fp32 bits is monotone in |w|, so the reduction is an
// unsigned max; each workgroup folds its rows, then one atomicMax per
// workgroup into the zero-initialised output (order-independent, exact).
// ---------------------------------------------------------------------------
__global__ void absmax_init_kernel(float* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) out[i] = 0.0f;
}

// Contiguous groups (ld == cols): the group is one flat array of n16 16-byte
// vectors; grid-stride loop with four loads in flight per thread.
// Otherwise rows are walked one by one (kFlat == false), vectorised when the
// row length and strides allow (kVec).
template <typename T, bool kVec, bool kFlat>
__global__ __launch_bounds__(kThreads) void absmax_kernel(const T* __restrict__ w, int64_t rows, int64_t cols,
                                                          int64_t ld, int64_t gstride, int64_t per_group,
                                                          float* __restrict__ out) {
  const int64_t grp = (int64_t)blockIdx.x / per_group;
  const int64_t chunk = (int64_t)blockIdx.x - grp * per_group;
  const T* base = w + grp * gstride;
  constexpr bool kBf16 = sizeof(T) == 2;
  uint32_t t;
  if (kFlat) {
    t = absmax_flat_share<kBf16>(reinterpret_cast<const uint4*>(base), rows * cols * (int64_t)sizeof(T) / 16, chunk,
                                 per_group);
  } else {
    __shared__ uint32_t part[kThreads / 64];
    uint32_t m = 0;
    constexpr int kV = 16 / sizeof(T);
    for (int64_t r = chunk; r < rows; r += per_group) {
      const T* rp = base + r * ld;
      if (kVec) {
        for (int64_t c = (int64_t)threadIdx.x * kV; c < cols; c += (int64_t)kThreads * kV)
          m = absbits_max(m, *reinterpret_cast<const uint4*>(rp + c), kBf16);
      } else {
        for (int64_t c = threadIdx.x; c < cols; c += kThreads) {
          uint32_t bits;
          if constexpr (kBf16) bits = (uint32_t)rp[c] << 16;
          else bits = __float_as_uint(rp[c]);
          m = max(m, bits & 0x7FFFFFFFu);
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    t = part[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) t = max(t, part[i]);
  }
  if (threadIdx.x == 0) {
    // Atomics on one address serialise in L2; the stored value only grows, so
    // a workgroup whose maximum does not exceed what it reads (possibly a
    // stale, smaller value) has nothing to add.
    unsigned int* o = reinterpret_cast<unsigned int*>(out + grp);
    if (t > __atomic_load_n(o, __ATOMIC_RELAXED)) atomicMax(o, t);
  }
}

template <typename T, bool kVec, bool kFlat>
hipError_t launch_absmax_typed(const AbsmaxArgs& a, hipStream_t stream) {
  int64_t per_group;
  if (kFlat) {
    const int64_t n16 = a.rows * a.cols * (int64_t)sizeof(T) / 16;
    per_group = (1024 + a.n_groups - 1) / a.n_groups;              // ~4 workgroups per CU in total
    const int64_t need = (n16 + 4 * kThreads - 1) / (4 * kThreads);  // >= 4 vectors per thread
    if (per_group > need) per_group = need;
  } else {
    per_group = (2048 + a.n_groups - 1) / a.n_groups;
    if (per_group > a.rows) per_group = a.rows;
  }
  if (per_group < 1) per_group = 1;
  absmax_kernel<T, kVec, kFlat><<<dim3((unsigned)(per_group * a.n_groups)), dim3(kThreads), 0, stream>>>(
      static_cast<const T*>(a.w), a.rows, a.cols, a.ld, a.gstride, per_group, a.out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fake_quant(const FakeQuantArgs& a, hipStream_t stream) {
  const int64_t esz = a.dtype == 1 ? 2 : 4;
  const int64_t epv = 16 / esz;
  const bool aligned = (reinterpret_cast<uintptr_t>(a.w) % 16 == 0) && (a.ld_w % epv == 0) &&
                       (a.gstride_w % epv == 0);
  if (a.dtype == 1)
    return aligned ? launch_fq_typed<uint16_t, true>(a, stream) : launch_fq_typed<uint16_t, false>(a, stream);
  return aligned ? launch_fq_typed<float, true>(a, stream) : launch_fq_typed<float, false>(a, stream);
}

hipError_t launch_absmax(const AbsmaxArgs& a, hipStream_t stream) {
  if (a.n_groups == 0) return hipSuccess;
  absmax_init_kernel<<<dim3((unsigned)((a.n_groups + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream>>>(
      a.out, a.n_groups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.rows == 0 || a.cols == 0) return e;
  const int64_t esz = a.dtype == 1 ? 2 : 4;
  const int64_t epv = 16 / esz;
  const bool aligned = (reinterpret_cast<uintptr_t>(a.w) % 16 == 0) && (a.ld % epv == 0) &&
                       (a.gstride % epv == 0) && (a.cols % epv == 0);
  const bool flat = aligned && (a.ld == a.cols || a.rows == 1);
  if (a.dtype == 1) {
    if (flat) return launch_absmax_typed<uint16_t, true, true>(a, stream);
    return aligned ? launch_absmax_typed<uint16_t, true, false>(a, stream)
                   : launch_absmax_typed<uint16_t, false, false>(a, stream);
  }
  if (flat) return launch_absmax_typed<float, true, true>(a, stream);
  return aligned ? launch_absmax_typed<float, true, false>(a, stream) : launch_absmax_typed<float, false, false>(a, stream);
}

}  // namespace lh
