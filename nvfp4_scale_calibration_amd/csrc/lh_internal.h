// lh_internal.h - launchers shared between the C ABI front end (lh_api.hip)
// and the kernel translation units.  Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lh {

struct HessianArgs {
  const void* x;
  int dtype;      // 0 fp32, 1 bf16
  int layout;     // 0 channel-major, 1 token-major
  int64_t c_in, n_tok, ld, gstride;
  int64_t n_groups;
  float alpha, beta;
  float* h;
  int64_t h_gstride;
  void* ws;       // nullable
  size_t ws_bytes;
};

// Token-split plan: `nsplit` slices of `chunk` tokens each (chunk % 256 == 0).
struct HessianPlan {
  int64_t nsplit;
  int64_t chunk;
  int nw;  // channel-major: waves per workgroup (4, 8 or 16)
};
HessianPlan hessian_plan(int64_t c_in, int64_t n_tok, int64_t n_groups, int layout, bool have_ws);
size_t hessian_ws_bytes(int64_t c_in, int64_t n_tok, int64_t n_groups);
hipError_t launch_hessian(const HessianArgs& a, hipStream_t stream);

// The fused calibration prologue (channel-major X, flat W): partial Hessian
// sums for every token slice and partial |w| maxima, completed by
// launch_finalize_certify.
struct ProloguePlan {
  HessianPlan hess;       // always through the workspace (nsplit >= 1)
  int64_t abs_per_group;  // partial maxima per group
};
struct PrologueArgs {
  const void* x;
  int x_dtype;
  int64_t c_in, n_tok, ld_x, gstride_x, n_groups;
  const void* w;          // [n_groups][c_out][c_in], contiguous
  int w_dtype;
  int64_t c_out, gstride_w;
  float* h_part;          // [nsplit][n_groups][c_in/16][256]
  uint32_t* abs_part;     // [n_groups][abs_per_group]
};
ProloguePlan prologue_plan(int64_t c_in, int64_t n_tok, int64_t n_groups, int64_t w_elems);
size_t prologue_ws_bytes(int64_t c_in, int64_t n_tok, int64_t n_groups, int64_t w_elems);
hipError_t launch_prologue(const PrologueArgs& a, const ProloguePlan& q, hipStream_t stream);

struct HessianRaggedArgs {
  const void* x;          // token-major [n_rows][ld]
  int dtype;              // 0 fp32, 1 bf16
  int64_t c_in, ld, n_rows;
  const int64_t* offsets; // device [n_groups + 1]
  int64_t n_groups;
  float* h;
  int64_t h_gstride;
  int64_t* counts;        // nullable device [n_groups]: running mean
  int64_t max_group_rows; // host bound on any group's rows (0: unknown)
  void* ws;               // nullable
  size_t ws_bytes;
};
struct RaggedPlan {
  int64_t nsplit;
  int64_t slice_rows;     // 0: even split per group
};
RaggedPlan hessian_ragged_plan(int64_t c_in, int64_t n_rows, int64_t n_groups, int64_t max_group_rows,
                               bool have_ws);
size_t hessian_ragged_ws_bytes(int64_t c_in, int64_t n_rows, int64_t n_groups, int64_t max_group_rows);
hipError_t launch_hessian_ragged(const HessianRaggedArgs& a, hipStream_t stream);

struct SweepArgs {
  const void* w;
  int dtype;
  int64_t c_out, c_in, ld_w, n_groups, gstride_w;
  const float* h;  // nullptr: plain weight error (H = I)
  int64_t gstride_h;
  const float* amax;
  uint8_t* idx;
  float* err;
  float* best_amax;
  void* ws;       // nullable: per-block skip certificates
  size_t ws_bytes;
  int rule;       // 0: 126-value sweep, 1: max, 2: Four-Over-Six, 3: amax search
  // fused fake-quant outputs (rule 0 only; all nullptr: none), dense layouts
  float* wq = nullptr;
  uint8_t* packed = nullptr;
  uint8_t* codes = nullptr;
  float* gscale = nullptr;
  bool cert_ready = false;  // ws already holds the per-block certificates
};

struct FinalizeCertifyArgs {
  const float* h_part;    // the prologue's partial sums
  int64_t nsplit, n_groups, c_in;
  float alpha;
  float* h;
  int64_t h_gstride;
  float* cert;            // [n_groups][c_in/16]
  const uint32_t* abs_part;
  int64_t abs_per_group;
  float* amax;            // [n_groups]
};
// Whether launch_finalize_certify also writes the certificates for this many
// blocks (else the sweep computes them in its own pre-pass).
bool finalize_certifies(int64_t blocks);
// The sweep's certificate pre-pass alone: cert[g][b] for every block.
hipError_t launch_certificate(const float* h, int64_t gstride_h, int64_t c_in, int64_t n_groups, float* cert,
                              hipStream_t stream);
hipError_t launch_finalize_certify(const FinalizeCertifyArgs& a, hipStream_t stream);
size_t sweep_ws_bytes(int64_t c_in, int64_t n_groups);
hipError_t launch_sweep(const SweepArgs& a, hipStream_t stream);

struct FakeQuantArgs {
  const void* w;
  int dtype;
  int64_t c_out, c_in, ld_w, n_groups, gstride_w;
  const uint8_t* idx;
  const float* amax;
  float* wq;
  uint8_t* packed;
  uint8_t* codes;
  float* gscale;
};
hipError_t launch_fake_quant(const FakeQuantArgs& a, hipStream_t stream);

struct AbsmaxArgs {
  const void* w;
  int dtype;
  int64_t rows, cols, ld, n_groups, gstride;
  float* out;
};
hipError_t launch_absmax(const AbsmaxArgs& a, hipStream_t stream);

struct FullHessianArgs {
  const void* x;        // channel-major [n_groups][c_in][ld_x]
  int dtype;
  int64_t c_in, n_tok, ld_x, gstride_x, n_groups;
  float alpha;
  float* h;             // [n_groups][c_in][ld_h]
  int64_t ld_h, gstride_h;
};
hipError_t launch_full_hessian(const FullHessianArgs& a, hipStream_t stream);

struct OutputErrorArgs {
  const void* w;
  int dtype;
  const float* q;
  int64_t c_out, c_in, ld_w, ld_q, gstride_w, gstride_q, n_groups;
  const float* h;
  int64_t ld_h, gstride_h;
  float* err;           // [n_groups][c_out]
  void* ws;             // output_error_ws_bytes
};
size_t output_error_ws_bytes(int64_t c_out, int64_t c_in, int64_t n_groups);
hipError_t launch_output_error(const OutputErrorArgs& a, hipStream_t stream);

struct HistogramArgs {
  const void* w;
  int dtype;
  int64_t c_out, c_in, ld_w, gstride_w, n_groups;
  const uint8_t* idx;
  const float* amax;
  int n_bins;
  float bins_per_unit;
  unsigned long long* counts;  // [n_groups][n_bins + 1]
};
int histogram_max_bins();
hipError_t launch_histogram(const HistogramArgs& a, hipStream_t stream);

struct GptqPrepareArgs {
  const float* h;       // full Hessian [n][ld_h]
  int64_t n, ld_h;
  float damp;
  float* u;             // [n][ld_u]
  int64_t ld_u;
  void* ws;             // gptq_prepare_ws_bytes(n)
};
size_t gptq_prepare_ws_bytes(int64_t n);
hipError_t launch_gptq_prepare(const GptqPrepareArgs& a, hipStream_t stream);

struct GptqQuantizeArgs {
  const void* w;
  int dtype;
  int64_t c_out, c_in, ld_w;
  const uint8_t* idx;   // [c_out][c_in/16]
  const float* amax;    // device scalar
  const float* u;
  int64_t ld_u;
  float* q;             // [c_out][ld_q]
  int64_t ld_q;
  void* ws;             // gptq_quantize_ws_bytes(c_out, c_in)
};
size_t gptq_quantize_ws_bytes(int64_t c_out, int64_t c_in);
hipError_t launch_gptq_quantize(const GptqQuantizeArgs& a, hipStream_t stream);

}  // namespace lh
