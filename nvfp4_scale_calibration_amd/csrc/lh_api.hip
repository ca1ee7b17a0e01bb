// lh_api.hip - C ABI front end of liblh: argument validation (pure host code,
// no HIP call before it passes), launch, and error reporting.
// The contract of every entry point is documented in include/lh.h.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "lh.h"
#include "lh_internal.h"
#include <math.h>

namespace {

thread_local char g_msg[512] = "";

lh_status fail(lh_status st, const char* fmt, const char* what) {
  snprintf(g_msg, sizeof g_msg, fmt, what);
  return st;
}

lh_status hip_fail(hipError_t e, const char* where) {
  snprintf(g_msg, sizeof g_msg, "%s: %s", where, hipGetErrorString(e));
  return LH_ERR_HIP;
}

bool valid_dtype(int d) { return d == LH_DTYPE_F32 || d == LH_DTYPE_BF16; }
size_t elem_size(int d) { return d == LH_DTYPE_BF16 ? 2 : 4; }
bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

// The normalisation factor of a Hessian: the caller's alpha, or for NaN the
// normalised Hessian's fl32(1/N) (0 for N = 0), computed here once for every
// entry point so that callers do none of the method's arithmetic.
float hessian_alpha(float alpha, int64_t n_tokens) {
  if (!isnan(alpha)) return alpha;
  return n_tokens > 0 ? (float)(1.0 / (double)n_tokens) : 0.0f;
}

}  // namespace

extern "C" {

int lh_abi_version(void) { return 1; }

const char* lh_status_string(int status) {
  switch (status) {
    case LH_OK: return "LH_OK";
    case LH_ERR_NULL: return "LH_ERR_NULL: a required pointer is NULL";
    case LH_ERR_SHAPE: return "LH_ERR_SHAPE: invalid size, leading dimension or stride";
    case LH_ERR_DTYPE: return "LH_ERR_DTYPE: unknown dtype";
    case LH_ERR_LAYOUT: return "LH_ERR_LAYOUT: unknown layout";
    case LH_ERR_WORKSPACE: return "LH_ERR_WORKSPACE: workspace too small";
    case LH_ERR_ARG: return "LH_ERR_ARG: invalid argument";
    case LH_ERR_HIP: return "LH_ERR_HIP: HIP launch failed";
    default: return "unknown lh_status";
  }
}

const char* lh_last_error_message(void) { return g_msg; }

float lh_hessian_alpha(float alpha, int64_t n_tokens) { return hessian_alpha(alpha, n_tokens); }

lh_status lh_absmax(const void* w, int w_dtype, int64_t rows, int64_t cols, int64_t ld_w,
                    int64_t n_groups, int64_t group_stride_w, float* amax, void* stream) {
  g_msg[0] = '\0';
  if (!valid_dtype(w_dtype)) return fail(LH_ERR_DTYPE, "%s: w_dtype must be 0 (f32) or 1 (bf16)", "lh_absmax");
  if (rows < 0 || cols < 0 || n_groups < 0 || group_stride_w < 0)
    return fail(LH_ERR_SHAPE, "%s: negative size or stride", "lh_absmax");
  if (ld_w < cols) return fail(LH_ERR_SHAPE, "%s: ld_w < cols", "lh_absmax");
  if (n_groups > 0 && amax == nullptr) return fail(LH_ERR_NULL, "%s: amax is NULL", "lh_absmax");
  if (n_groups > 0 && rows > 0 && cols > 0 && w == nullptr) return fail(LH_ERR_NULL, "%s: w is NULL", "lh_absmax");
  if (!aligned(w, elem_size(w_dtype)) || !aligned(amax, 4))
    return fail(LH_ERR_ARG, "%s: pointer not aligned to its element size", "lh_absmax");
  if (n_groups == 0) return LH_OK;
  lh::AbsmaxArgs a{w, w_dtype, rows, cols, ld_w, n_groups, group_stride_w, amax};
  hipError_t e = lh::launch_absmax(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LH_OK : hip_fail(e, "lh_absmax");
}

size_t lh_hessian_workspace_bytes(int64_t c_in, int64_t n_tokens, int64_t n_groups) {
  if (c_in <= 0 || n_tokens <= 0 || n_groups <= 0 || c_in % 16 != 0) return 0;
  return lh::hessian_ws_bytes(c_in, n_tokens, n_groups);
}

lh_status lh_accumulate_hessian(const void* x, int x_dtype, int layout, int64_t c_in,
                                int64_t n_tokens, int64_t ld_x, int64_t n_groups,
                                int64_t group_stride_x, float alpha, float beta, float* h,
                                int64_t group_stride_h, void* workspace, size_t workspace_bytes,
                                void* stream) {
  const char* fn = "lh_accumulate_hessian";
  g_msg[0] = '\0';
  if (!valid_dtype(x_dtype)) return fail(LH_ERR_DTYPE, "%s: x_dtype must be 0 (f32) or 1 (bf16)", fn);
  if (layout != LH_LAYOUT_CHANNEL_MAJOR && layout != LH_LAYOUT_TOKEN_MAJOR)
    return fail(LH_ERR_LAYOUT, "%s: layout must be 0 (channel-major) or 1 (token-major)", fn);
  if (c_in < 0 || n_tokens < 0 || n_groups < 0 || group_stride_x < 0 || group_stride_h < 0)
    return fail(LH_ERR_SHAPE, "%s: negative size or stride", fn);
  if (c_in % 16 != 0) return fail(LH_ERR_SHAPE, "%s: c_in must be a multiple of 16", fn);
  const int64_t min_ld = layout == LH_LAYOUT_CHANNEL_MAJOR ? n_tokens : c_in;
  if (ld_x < min_ld || ld_x < 1) return fail(LH_ERR_SHAPE, "%s: ld_x smaller than the contiguous extent", fn);
  const int64_t nb = c_in / 16;
  if (n_groups > 1 && group_stride_h < nb * 256)
    return fail(LH_ERR_SHAPE, "%s: group_stride_h < (c_in/16)*256 would overlap outputs", fn);
  const bool work = n_groups > 0 && nb > 0;
  if (work && h == nullptr) return fail(LH_ERR_NULL, "%s: h is NULL", fn);
  if (work && n_tokens > 0 && x == nullptr) return fail(LH_ERR_NULL, "%s: x is NULL", fn);
  if (workspace == nullptr && workspace_bytes > 0) return fail(LH_ERR_NULL, "%s: workspace is NULL but workspace_bytes > 0", fn);
  if (!aligned(x, elem_size(x_dtype)) || !aligned(h, 4) || !aligned(workspace, 4))
    return fail(LH_ERR_ARG, "%s: pointer not aligned to its element size", fn);
  if (workspace != nullptr && workspace_bytes > 0 && work && n_tokens > 0) {
    const size_t need = lh::hessian_ws_bytes(c_in, n_tokens, n_groups);
    if (workspace_bytes < need) return fail(LH_ERR_WORKSPACE, "%s: workspace smaller than lh_hessian_workspace_bytes()", fn);
  }
  if (!work) return LH_OK;
  lh::HessianArgs a{x, x_dtype, layout, c_in, n_tokens, ld_x, group_stride_x, n_groups,
                    hessian_alpha(alpha, n_tokens), beta, h, group_stride_h, workspace, workspace_bytes};
  hipError_t e = lh::launch_hessian(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LH_OK : hip_fail(e, fn);
}

size_t lh_hessian_ragged_workspace_bytes(int64_t c_in, int64_t n_rows, int64_t n_groups, int64_t max_group_rows) {
  if (c_in <= 0 || n_rows <= 0 || n_groups <= 0 || c_in % 16 != 0 || max_group_rows < 0) return 0;
  return lh::hessian_ragged_ws_bytes(c_in, n_rows, n_groups, max_group_rows);
}

lh_status lh_accumulate_hessian_ragged(const void* x, int x_dtype, int64_t c_in, int64_t ld_x, int64_t n_rows,
                                       const int64_t* token_offsets, int64_t n_groups, int64_t max_group_rows,
                                       float* h, int64_t group_stride_h, int64_t* token_counts, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  const char* fn = "lh_accumulate_hessian_ragged";
  g_msg[0] = '\0';
  if (!valid_dtype(x_dtype)) return fail(LH_ERR_DTYPE, "%s: x_dtype must be 0 (f32) or 1 (bf16)", fn);
  if (c_in < 0 || n_rows < 0 || n_groups < 0 || group_stride_h < 0 || max_group_rows < 0)
    return fail(LH_ERR_SHAPE, "%s: negative size or stride", fn);
  if (c_in % 16 != 0) return fail(LH_ERR_SHAPE, "%s: c_in must be a multiple of 16", fn);
  if (ld_x < c_in || ld_x < 1) return fail(LH_ERR_SHAPE, "%s: ld_x < c_in", fn);
  const int64_t nb = c_in / 16;
  if (n_groups > 1 && group_stride_h < nb * 256)
    return fail(LH_ERR_SHAPE, "%s: group_stride_h < (c_in/16)*256 would overlap outputs", fn);
  const bool work = n_groups > 0 && nb > 0;
  if (work && (h == nullptr || token_offsets == nullptr))
    return fail(LH_ERR_NULL, "%s: h and token_offsets are required", fn);
  if (work && n_rows > 0 && x == nullptr) return fail(LH_ERR_NULL, "%s: x is NULL", fn);
  if (workspace == nullptr && workspace_bytes > 0) return fail(LH_ERR_NULL, "%s: workspace is NULL but workspace_bytes > 0", fn);
  if (!aligned(x, elem_size(x_dtype)) || !aligned(h, 4) || !aligned(workspace, 4) || !aligned(token_offsets, 8) ||
      !aligned(token_counts, 8))
    return fail(LH_ERR_ARG, "%s: pointer not aligned to its element size", fn);
  if (workspace != nullptr && workspace_bytes > 0 && work) {
    const size_t need = lh::hessian_ragged_ws_bytes(c_in, n_rows, n_groups, max_group_rows);
    if (workspace_bytes < need)
      return fail(LH_ERR_WORKSPACE, "%s: workspace smaller than lh_hessian_ragged_workspace_bytes()", fn);
  }
  if (!work) return LH_OK;
  lh::HessianRaggedArgs a{x, x_dtype, c_in, ld_x, n_rows, token_offsets, n_groups, h, group_stride_h,
                          token_counts, max_group_rows, workspace, workspace_bytes};
  hipError_t e = lh::launch_hessian_ragged(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LH_OK : hip_fail(e, fn);
}

size_t lh_sweep_workspace_bytes(int64_t c_in, int64_t n_groups) {
  if (c_in <= 0 || n_groups <= 0 || c_in % 16 != 0) return 0;
  return lh::sweep_ws_bytes(c_in, n_groups);
}

}  // extern "C"

namespace {

// Fake-quant outputs of the fused sweep (all NULL for the plain calls).
struct QuantPtrs {
  float* w_q;
  uint8_t* packed;
  uint8_t* codes;
  float* gscale;
};

// Shared by lh_scale_sweep (rule 0, Hessian required), lh_select_scales and
// lh_scale_sweep_fake_quant (rule 0, Hessian required, fake-quant outputs).
lh_status select_common(const char* fn, int rule, bool h_required, const void* w, int w_dtype, int64_t c_out,
                        int64_t c_in, int64_t ld_w, int64_t n_groups, int64_t group_stride_w, const float* h,
                        int64_t group_stride_h, const float* amax, uint8_t* best_idx, float* best_err,
                        float* best_amax, void* workspace, size_t workspace_bytes, void* stream,
                        QuantPtrs qp = QuantPtrs{nullptr, nullptr, nullptr, nullptr}, bool cert_ready = false,
                        bool launch = true) {
  g_msg[0] = '\0';
  if (rule < 0 || rule > 3) return fail(LH_ERR_ARG, "%s: rule must be 0..3", fn);
  if (!valid_dtype(w_dtype)) return fail(LH_ERR_DTYPE, "%s: w_dtype must be 0 (f32) or 1 (bf16)", fn);
  if (c_out < 0 || c_in < 0 || n_groups < 0 || group_stride_w < 0 || group_stride_h < 0)
    return fail(LH_ERR_SHAPE, "%s: negative size or stride", fn);
  if (c_in % 16 != 0) return fail(LH_ERR_SHAPE, "%s: c_in must be a multiple of 16", fn);
  if (ld_w < c_in) return fail(LH_ERR_SHAPE, "%s: ld_w < c_in", fn);
  const bool work = n_groups > 0 && c_out > 0 && c_in > 0;
  if (work && (w == nullptr || (h_required && h == nullptr) || amax == nullptr || best_idx == nullptr))
    return fail(LH_ERR_NULL, h_required ? "%s: w, h, amax and best_idx are required"
                                        : "%s: w, amax and best_idx are required", fn);
  if (!aligned(w, elem_size(w_dtype)) || !aligned(amax, 4) || !aligned(best_err, 4) || !aligned(best_amax, 4))
    return fail(LH_ERR_ARG, "%s: pointer not aligned to its element size", fn);
  if (h != nullptr && (!aligned(h, 16) || group_stride_h % 4 != 0))
    return fail(LH_ERR_ARG, "%s: h must be 16-byte aligned and group_stride_h a multiple of 4", fn);
  if (workspace == nullptr && workspace_bytes > 0) return fail(LH_ERR_NULL, "%s: workspace is NULL but workspace_bytes > 0", fn);
  if (!aligned(workspace, 4)) return fail(LH_ERR_ARG, "%s: workspace not 4-byte aligned", fn);
  if (workspace != nullptr && workspace_bytes > 0 && work && workspace_bytes < lh::sweep_ws_bytes(c_in, n_groups))
    return fail(LH_ERR_WORKSPACE, "%s: workspace smaller than lh_sweep_workspace_bytes()", fn);
  if (!aligned(qp.w_q, 16) || !aligned(qp.packed, 8) || !aligned(qp.gscale, 4))
    return fail(LH_ERR_ARG, "%s: misaligned pointer (w_q needs 16 bytes, packed_e2m1 8, global_scale 4)", fn);
  if (qp.gscale != nullptr && n_groups > 0 && amax == nullptr) return fail(LH_ERR_NULL, "%s: amax is NULL", fn);
  if (!launch) return LH_OK;   // arguments checked only
  if (!work) {
    if (qp.gscale == nullptr || n_groups == 0) return LH_OK;
    // no block, but S_g is still asked for
    lh::FakeQuantArgs f{w, w_dtype, c_out, c_in, ld_w, n_groups, group_stride_w, nullptr, amax,
                        nullptr, nullptr, nullptr, qp.gscale};
    hipError_t e = lh::launch_fake_quant(f, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LH_OK : hip_fail(e, fn);
  }
  lh::SweepArgs a{w, w_dtype, c_out, c_in, ld_w, n_groups, group_stride_w, h, group_stride_h, amax,
                  best_idx, best_err, best_amax, workspace, workspace_bytes, rule,
                  qp.w_q, qp.packed, qp.codes, qp.gscale, cert_ready};
  hipError_t e = lh::launch_sweep(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LH_OK : hip_fail(e, fn);
}

// Workspace of lh_calibrate_nvfp4: the per-block certificates, then the
// Hessian partial sums (of the fused prologue or of lh_accumulate_hessian),
// then the prologue's partial maxima.
size_t calibrate_cert_bytes(int64_t c_in, int64_t n_groups) {
  return ((size_t)n_groups * (size_t)(c_in / 16) * sizeof(float) + 255) & ~(size_t)255;
}

size_t calibrate_ws_bytes(int64_t c_out, int64_t c_in, int64_t n_tokens, int64_t n_groups) {
  const size_t fused = lh::prologue_ws_bytes(c_in, n_tokens, n_groups, c_out * c_in);
  const size_t plain = lh::hessian_ws_bytes(c_in, n_tokens, n_groups);
  return calibrate_cert_bytes(c_in, n_groups) + (fused > plain ? fused : plain);
}

// lh_calibrate_sweep; with launch == false only its arguments are checked
// (lh_calibrate_nvfp4 checks both halves before it enqueues anything).
lh_status calibrate_sweep(const char* fn, bool launch, const void* w, int w_dtype, int64_t c_out, int64_t c_in,
                          int64_t ld_w, int64_t n_groups, int64_t group_stride_w, const float* h,
                          int64_t group_stride_h, const float* amax, uint8_t* best_idx, float* best_err,
                          float* best_amax, QuantPtrs qp, void* workspace, size_t workspace_bytes, void* stream) {
  g_msg[0] = '\0';
  if (workspace == nullptr && n_groups > 0 && c_out > 0 && c_in > 0)
    return fail(LH_ERR_NULL, "%s: workspace (from lh_calibrate_prologue) is required", fn);
  if (!aligned(workspace, 256)) return fail(LH_ERR_ARG, "%s: workspace not 256-byte aligned", fn);
  if (workspace != nullptr && c_in >= 0 && n_groups >= 0 && workspace_bytes < calibrate_cert_bytes(c_in, n_groups))
    return fail(LH_ERR_WORKSPACE, "%s: workspace smaller than lh_calibrate_workspace_bytes()", fn);
  const size_t cert_bytes = c_in >= 0 && n_groups >= 0 ? calibrate_cert_bytes(c_in, n_groups) : 0;
  return select_common(fn, 0, true, w, w_dtype, c_out, c_in, ld_w, n_groups, group_stride_w, h, group_stride_h,
                       amax, best_idx, best_err, best_amax, workspace, cert_bytes, stream, qp, true, launch);
}

}  // namespace

extern "C" {

lh_status lh_scale_sweep(const void* w, int w_dtype, int64_t c_out, int64_t c_in, int64_t ld_w,
                         int64_t n_groups, int64_t group_stride_w, const float* h,
                         int64_t group_stride_h, const float* amax, uint8_t* best_idx,
                         float* best_err, float* best_amax, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return select_common("lh_scale_sweep", 0, true, w, w_dtype, c_out, c_in, ld_w, n_groups, group_stride_w, h,
                       group_stride_h, amax, best_idx, best_err, best_amax, workspace, workspace_bytes, stream);
}

lh_status lh_scale_sweep_fake_quant(const void* w, int w_dtype, int64_t c_out, int64_t c_in, int64_t ld_w,
                                    int64_t n_groups, int64_t group_stride_w, const float* h,
                                    int64_t group_stride_h, const float* amax, uint8_t* best_idx,
                                    float* best_err, float* best_amax, float* w_q, uint8_t* packed_e2m1,
                                    uint8_t* scale_e4m3, float* global_scale, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return select_common("lh_scale_sweep_fake_quant", 0, true, w, w_dtype, c_out, c_in, ld_w, n_groups,
                       group_stride_w, h, group_stride_h, amax, best_idx, best_err, best_amax, workspace,
                       workspace_bytes, stream, QuantPtrs{w_q, packed_e2m1, scale_e4m3, global_scale});
}

size_t lh_calibrate_workspace_bytes(int64_t c_out, int64_t c_in, int64_t n_tokens, int64_t n_groups) {
  if (c_out <= 0 || c_in <= 0 || n_groups <= 0 || n_tokens < 0 || c_in % 16 != 0) return 0;
  return calibrate_ws_bytes(c_out, c_in, n_tokens, n_groups);
}

lh_status lh_calibrate_prologue(const void* w, int w_dtype, int64_t c_out, int64_t c_in, int64_t ld_w,
                                int64_t n_groups, int64_t group_stride_w, const void* x, int x_dtype, int x_layout,
                                int64_t n_tokens, int64_t ld_x, int64_t group_stride_x, float* amax, float* h,
                                int64_t group_stride_h, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "lh_calibrate_prologue";
  g_msg[0] = '\0';
  if (!valid_dtype(w_dtype) || !valid_dtype(x_dtype))
    return fail(LH_ERR_DTYPE, "%s: w_dtype and x_dtype must be 0 (f32) or 1 (bf16)", fn);
  if (x_layout != LH_LAYOUT_CHANNEL_MAJOR && x_layout != LH_LAYOUT_TOKEN_MAJOR)
    return fail(LH_ERR_LAYOUT, "%s: x_layout must be 0 (channel-major) or 1 (token-major)", fn);
  if (c_out < 0 || c_in < 0 || n_groups < 0 || n_tokens < 0 || group_stride_w < 0 || group_stride_x < 0 ||
      group_stride_h < 0)
    return fail(LH_ERR_SHAPE, "%s: negative size or stride", fn);
  if (c_in % 16 != 0) return fail(LH_ERR_SHAPE, "%s: c_in must be a multiple of 16", fn);
  if (ld_w < c_in) return fail(LH_ERR_SHAPE, "%s: ld_w < c_in", fn);
  const int64_t min_ld = x_layout == LH_LAYOUT_CHANNEL_MAJOR ? n_tokens : c_in;
  if (ld_x < min_ld || ld_x < 1) return fail(LH_ERR_SHAPE, "%s: ld_x smaller than the contiguous extent", fn);
  const int64_t nb = c_in / 16;
  if (n_groups > 1 && group_stride_h < nb * 256)
    return fail(LH_ERR_SHAPE, "%s: group_stride_h < (c_in/16)*256 would overlap outputs", fn);
  const bool work = n_groups > 0 && c_out > 0 && c_in > 0;
  if (work && (w == nullptr || amax == nullptr || h == nullptr || workspace == nullptr ||
               (n_tokens > 0 && x == nullptr)))
    return fail(LH_ERR_NULL, "%s: w, x, amax, h and workspace are required", fn);
  if (!aligned(w, elem_size(w_dtype)) || !aligned(x, elem_size(x_dtype)) || !aligned(amax, 4) ||
      !aligned(workspace, 256))
    return fail(LH_ERR_ARG, "%s: misaligned pointer (workspace: 256 bytes)", fn);
  if (h != nullptr && (!aligned(h, 16) || group_stride_h % 4 != 0))
    return fail(LH_ERR_ARG, "%s: h must be 16-byte aligned and group_stride_h a multiple of 4", fn);
  if (!work) return LH_OK;
  if (workspace_bytes < calibrate_ws_bytes(c_out, c_in, n_tokens, n_groups))
    return fail(LH_ERR_WORKSPACE, "%s: workspace smaller than lh_calibrate_workspace_bytes()", fn);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* cert = reinterpret_cast<float*>(ws);
  char* rest = ws + calibrate_cert_bytes(c_in, n_groups);
  const size_t rest_bytes = workspace_bytes - calibrate_cert_bytes(c_in, n_groups);
  const float alpha = hessian_alpha(NAN, n_tokens);
  const int64_t epx = 16 / elem_size(x_dtype), epw = 16 / elem_size(w_dtype);
  const bool fused = x_layout == LH_LAYOUT_CHANNEL_MAJOR && n_tokens > 0 && aligned(x, 16) && ld_x % epx == 0 &&
                     group_stride_x % epx == 0 && aligned(w, 16) && ld_w == c_in && group_stride_w % epw == 0;
  hipError_t e;
  bool certified = false;
  if (fused) {
    const lh::ProloguePlan q = lh::prologue_plan(c_in, n_tokens, n_groups, c_out * c_in);
    float* part = reinterpret_cast<float*>(rest);
    uint32_t* abs_part = reinterpret_cast<uint32_t*>(part + q.hess.nsplit * n_groups * nb * 256);
    lh::PrologueArgs pa{x, x_dtype, c_in, n_tokens, ld_x, group_stride_x, n_groups, w, w_dtype, c_out,
                        group_stride_w, part, abs_part};
    e = lh::launch_prologue(pa, q, st);
    if (e != hipSuccess) return hip_fail(e, fn);
    lh::FinalizeCertifyArgs fa{part, q.hess.nsplit, n_groups, c_in, alpha, h, group_stride_h, cert, abs_part,
                               q.abs_per_group, amax};
    e = lh::launch_finalize_certify(fa, st);
    if (e != hipSuccess) return hip_fail(e, fn);
    certified = lh::finalize_certifies(n_groups * nb);
  } else {
    lh::AbsmaxArgs aa{w, w_dtype, c_out, c_in, ld_w, n_groups, group_stride_w, amax};
    e = lh::launch_absmax(aa, st);
    if (e != hipSuccess) return hip_fail(e, fn);
    lh::HessianArgs ha{x, x_dtype, x_layout, c_in, n_tokens, ld_x, group_stride_x, n_groups, alpha, 0.0f,
                       h, group_stride_h, rest, rest_bytes};
    e = lh::launch_hessian(ha, st);
    if (e != hipSuccess) return hip_fail(e, fn);
  }
  if (!certified) {
    e = lh::launch_certificate(h, group_stride_h, c_in, n_groups, cert, st);
    if (e != hipSuccess) return hip_fail(e, fn);
  }
  return LH_OK;
}

lh_status lh_calibrate_sweep(const void* w, int w_dtype, int64_t c_out, int64_t c_in, int64_t ld_w,
                             int64_t n_groups, int64_t group_stride_w, const float* h, int64_t group_stride_h,
                             const float* amax, uint8_t* best_idx, float* best_err, float* best_amax, float* w_q,
                             uint8_t* packed_e2m1, uint8_t* scale_e4m3, float* global_scale, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return calibrate_sweep("lh_calibrate_sweep", true, w, w_dtype, c_out, c_in, ld_w, n_groups, group_stride_w, h,
                         group_stride_h, amax, best_idx, best_err, best_amax,
                         QuantPtrs{w_q, packed_e2m1, scale_e4m3, global_scale}, workspace, workspace_bytes, stream);
}

lh_status lh_calibrate_nvfp4(const void* w, int w_dtype, int64_t c_out, int64_t c_in, int64_t ld_w, int64_t n_groups,
                             int64_t group_stride_w, const void* x, int x_dtype, int x_layout, int64_t n_tokens,
                             int64_t ld_x, int64_t group_stride_x, float* amax, float* h, int64_t group_stride_h,
                             uint8_t* best_idx, float* best_err, float* best_amax, float* w_q, uint8_t* packed_e2m1,
                             uint8_t* scale_e4m3, float* global_scale, void* workspace, size_t workspace_bytes,
                             void* stream) {
  const QuantPtrs qp{w_q, packed_e2m1, scale_e4m3, global_scale};
  lh_status st = calibrate_sweep("lh_calibrate_nvfp4", false, w, w_dtype, c_out, c_in, ld_w, n_groups,
                                 group_stride_w, h, group_stride_h, amax, best_idx, best_err, best_amax, qp, workspace,
                                 workspace_bytes, stream);
  if (st != LH_OK) return st;
  st = lh_calibrate_prologue(w, w_dtype, c_out, c_in, ld_w, n_groups, group_stride_w, x, x_dtype, x_layout,
                                       n_tokens, ld_x, group_stride_x, amax, h, group_stride_h, workspace,
                                       workspace_bytes, stream);
  if (st != LH_OK) return st;
  return calibrate_sweep("lh_calibrate_nvfp4", true, w, w_dtype, c_out, c_in, ld_w, n_groups, group_stride_w, h,
                         group_stride_h, amax, best_idx, best_err, best_amax, qp, workspace, workspace_bytes, stream);
}

lh_status lh_select_scales(int rule, const void* w, int w_dtype, int64_t c_out, int64_t c_in, int64_t ld_w,
                           int64_t n_groups, int64_t group_stride_w, const float* h, int64_t group_stride_h,
                           const float* amax, uint8_t* best_idx, float* best_err, float* best_amax,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return select_common("lh_select_scales", rule, false, w, w_dtype, c_out, c_in, ld_w, n_groups, group_stride_w,
                       h, group_stride_h, amax, best_idx, best_err, best_amax, workspace, workspace_bytes, stream);
}

lh_status lh_fake_quant_nvfp4(const void* w, int w_dtype, int64_t c_out, int64_t c_in, int64_t ld_w,
                              int64_t n_groups, int64_t group_stride_w, const uint8_t* best_idx,
                              const float* amax, float* w_q, uint8_t* packed_e2m1,
                              uint8_t* scale_e4m3, float* global_scale, void* stream) {
  const char* fn = "lh_fake_quant_nvfp4";
  g_msg[0] = '\0';
  if (!valid_dtype(w_dtype)) return fail(LH_ERR_DTYPE, "%s: w_dtype must be 0 (f32) or 1 (bf16)", fn);
  if (c_out < 0 || c_in < 0 || n_groups < 0 || group_stride_w < 0)
    return fail(LH_ERR_SHAPE, "%s: negative size or stride", fn);
  if (c_in % 16 != 0) return fail(LH_ERR_SHAPE, "%s: c_in must be a multiple of 16", fn);
  if (ld_w < c_in) return fail(LH_ERR_SHAPE, "%s: ld_w < c_in", fn);
  if (!w_q && !packed_e2m1 && !scale_e4m3 && !global_scale)
    return fail(LH_ERR_ARG, "%s: no output requested", fn);
  const bool blocks = n_groups > 0 && c_out > 0 && c_in > 0;
  if (n_groups > 0 && amax == nullptr) return fail(LH_ERR_NULL, "%s: amax is NULL", fn);
  if (blocks && (w_q || packed_e2m1 || scale_e4m3) && (w == nullptr || best_idx == nullptr))
    return fail(LH_ERR_NULL, "%s: w and best_idx are required for per-block outputs", fn);
  if (!aligned(w, elem_size(w_dtype)) || !aligned(amax, 4) || !aligned(global_scale, 4) ||
      !aligned(w_q, 16) || !aligned(packed_e2m1, 8))
    return fail(LH_ERR_ARG, "%s: misaligned pointer (w_q needs 16 bytes, packed_e2m1 8)", fn);
  if (n_groups == 0) return LH_OK;
  lh::FakeQuantArgs a{w, w_dtype, c_out, c_in, ld_w, n_groups, group_stride_w, best_idx, amax,
                      w_q, packed_e2m1, scale_e4m3, global_scale};
  hipError_t e = lh::launch_fake_quant(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LH_OK : hip_fail(e, fn);
}

size_t lh_output_error_workspace_bytes(int64_t c_out, int64_t c_in, int64_t n_groups) {
  if (c_out <= 0 || c_in <= 0 || n_groups <= 0 || c_in % 16 != 0) return 0;
  return lh::output_error_ws_bytes(c_out, c_in, n_groups);
}

lh_status lh_full_hessian(const void* x, int x_dtype, int64_t c_in, int64_t n_tokens, int64_t ld_x, int64_t n_groups,
                          int64_t group_stride_x, float alpha, float* h_full, int64_t ld_h, int64_t group_stride_h,
                          void* stream) {
  const char* fn = "lh_full_hessian";
  g_msg[0] = '\0';
  if (!valid_dtype(x_dtype)) return fail(LH_ERR_DTYPE, "%s: x_dtype must be 0 (f32) or 1 (bf16)", fn);
  if (c_in < 0 || n_tokens < 0 || n_groups < 0 || group_stride_x < 0 || group_stride_h < 0)
    return fail(LH_ERR_SHAPE, "%s: negative size or stride", fn);
  if (c_in % 16 != 0) return fail(LH_ERR_SHAPE, "%s: c_in must be a multiple of 16", fn);
  if (ld_x < n_tokens || ld_x < 1) return fail(LH_ERR_SHAPE, "%s: ld_x < n_tokens", fn);
  if (ld_h < c_in || ld_h < 1) return fail(LH_ERR_SHAPE, "%s: ld_h < c_in", fn);
  if (n_groups > 1 && group_stride_h < c_in * ld_h)
    return fail(LH_ERR_SHAPE, "%s: group_stride_h < c_in * ld_h would overlap outputs", fn);
  const bool work = n_groups > 0 && c_in > 0;
  if (work && h_full == nullptr) return fail(LH_ERR_NULL, "%s: h_full is NULL", fn);
  if (work && n_tokens > 0 && x == nullptr) return fail(LH_ERR_NULL, "%s: x is NULL", fn);
  if (!aligned(x, elem_size(x_dtype)) || !aligned(h_full, 4))
    return fail(LH_ERR_ARG, "%s: pointer not aligned to its element size", fn);
  if (!work) return LH_OK;
  lh::FullHessianArgs a{x, x_dtype, c_in, n_tokens, ld_x, group_stride_x, n_groups, hessian_alpha(alpha, n_tokens),
                        h_full, ld_h, group_stride_h};
  hipError_t e = lh::launch_full_hessian(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LH_OK : hip_fail(e, fn);
}

lh_status lh_output_error(const void* w, int w_dtype, const float* w_q, int64_t c_out, int64_t c_in, int64_t ld_w,
                          int64_t ld_q, int64_t n_groups, int64_t group_stride_w, int64_t group_stride_q,
                          const float* h_full, int64_t ld_h, int64_t group_stride_h, float* err, void* workspace,
                          size_t workspace_bytes, void* stream) {
  const char* fn = "lh_output_error";
  g_msg[0] = '\0';
  if (!valid_dtype(w_dtype)) return fail(LH_ERR_DTYPE, "%s: w_dtype must be 0 (f32) or 1 (bf16)", fn);
  if (c_out < 0 || c_in < 0 || n_groups < 0 || group_stride_w < 0 || group_stride_q < 0 || group_stride_h < 0)
    return fail(LH_ERR_SHAPE, "%s: negative size or stride", fn);
  if (c_in % 16 != 0) return fail(LH_ERR_SHAPE, "%s: c_in must be a multiple of 16", fn);
  if (ld_w < c_in || ld_q < c_in || ld_h < c_in) return fail(LH_ERR_SHAPE, "%s: a leading dimension < c_in", fn);
  const bool work = n_groups > 0 && c_out > 0 && c_in > 0;
  if (work && (w == nullptr || w_q == nullptr || h_full == nullptr || err == nullptr))
    return fail(LH_ERR_NULL, "%s: w, w_q, h_full and err are required", fn);
  if (work && workspace == nullptr) return fail(LH_ERR_NULL, "%s: workspace is required", fn);
  if (!aligned(w, elem_size(w_dtype)) || !aligned(w_q, 4) || !aligned(h_full, 4) || !aligned(err, 4) ||
      !aligned(workspace, 4))
    return fail(LH_ERR_ARG, "%s: pointer not aligned to its element size", fn);
  if (work && workspace_bytes < lh::output_error_ws_bytes(c_out, c_in, n_groups))
    return fail(LH_ERR_WORKSPACE, "%s: workspace smaller than lh_output_error_workspace_bytes()", fn);
  if (!work) return LH_OK;
  lh::OutputErrorArgs a{w, w_dtype, w_q, c_out, c_in, ld_w, ld_q, group_stride_w, group_stride_q, n_groups,
                        h_full, ld_h, group_stride_h, err, workspace};
  hipError_t e = lh::launch_output_error(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LH_OK : hip_fail(e, fn);
}

lh_status lh_scaled_histogram(const void* w, int w_dtype, int64_t c_out, int64_t c_in, int64_t ld_w,
                              int64_t n_groups, int64_t group_stride_w, const uint8_t* best_idx, const float* amax,
                              int n_bins, float bins_per_unit, uint64_t* counts, void* stream) {
  const char* fn = "lh_scaled_histogram";
  g_msg[0] = '\0';
  if (!valid_dtype(w_dtype)) return fail(LH_ERR_DTYPE, "%s: w_dtype must be 0 (f32) or 1 (bf16)", fn);
  if (c_out < 0 || c_in < 0 || n_groups < 0 || group_stride_w < 0)
    return fail(LH_ERR_SHAPE, "%s: negative size or stride", fn);
  if (c_in % 16 != 0) return fail(LH_ERR_SHAPE, "%s: c_in must be a multiple of 16", fn);
  if (ld_w < c_in) return fail(LH_ERR_SHAPE, "%s: ld_w < c_in", fn);
  if (n_bins < 1 || n_bins > lh::histogram_max_bins())
    return fail(LH_ERR_ARG, "%s: n_bins must be in [1, 4096]", fn);
  if (!(bins_per_unit > 0.0f) || !(bins_per_unit < INFINITY))
    return fail(LH_ERR_ARG, "%s: bins_per_unit must be positive and finite", fn);
  const bool blocks = n_groups > 0 && c_out > 0 && c_in > 0;
  if (n_groups > 0 && (counts == nullptr || amax == nullptr))
    return fail(LH_ERR_NULL, "%s: counts and amax are required", fn);
  if (blocks && (w == nullptr || best_idx == nullptr)) return fail(LH_ERR_NULL, "%s: w and best_idx are required", fn);
  if (!aligned(w, elem_size(w_dtype)) || !aligned(amax, 4) || !aligned(counts, 8))
    return fail(LH_ERR_ARG, "%s: pointer not aligned to its element size", fn);
  if (n_groups == 0) return LH_OK;
  lh::HistogramArgs a{w, w_dtype, c_out, c_in, ld_w, group_stride_w, n_groups, best_idx, amax, n_bins,
                      bins_per_unit, reinterpret_cast<unsigned long long*>(counts)};
  hipError_t e = lh::launch_histogram(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LH_OK : hip_fail(e, fn);
}

size_t lh_gptq_workspace_bytes(int64_t c_out, int64_t c_in) {
  if (c_out < 0 || c_in <= 0 || c_in % 16 != 0) return 0;
  const size_t a = lh::gptq_prepare_ws_bytes(c_in), b = lh::gptq_quantize_ws_bytes(c_out, c_in);
  return a > b ? a : b;
}

lh_status lh_gptq_prepare(const float* h_full, int64_t c_in, int64_t ld_h, float damp, float* u, int64_t ld_u,
                          void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "lh_gptq_prepare";
  g_msg[0] = '\0';
  if (c_in < 0) return fail(LH_ERR_SHAPE, "%s: negative size", fn);
  if (c_in % 16 != 0) return fail(LH_ERR_SHAPE, "%s: c_in must be a multiple of 16", fn);
  if (ld_h < c_in || ld_u < c_in) return fail(LH_ERR_SHAPE, "%s: a leading dimension < c_in", fn);
  if (!(damp >= 0.0f) || !(damp < INFINITY)) return fail(LH_ERR_ARG, "%s: damp must be finite and >= 0", fn);
  if (c_in == 0) return LH_OK;
  if (h_full == nullptr || u == nullptr || workspace == nullptr)
    return fail(LH_ERR_NULL, "%s: h_full, u and workspace are required", fn);
  if (!aligned(h_full, 4) || !aligned(u, 4) || !aligned(workspace, 16))
    return fail(LH_ERR_ARG, "%s: h_full and u need 4-byte, workspace 16-byte alignment", fn);
  if (workspace_bytes < lh::gptq_prepare_ws_bytes(c_in))
    return fail(LH_ERR_WORKSPACE, "%s: workspace smaller than lh_gptq_workspace_bytes()", fn);
  lh::GptqPrepareArgs a{h_full, c_in, ld_h, damp, u, ld_u, workspace};
  hipError_t e = lh::launch_gptq_prepare(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LH_OK : hip_fail(e, fn);
}

lh_status lh_gptq_quantize(const void* w, int w_dtype, int64_t c_out, int64_t c_in, int64_t ld_w,
                           const uint8_t* best_idx, const float* amax, const float* u, int64_t ld_u, float* w_q,
                           int64_t ld_q, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "lh_gptq_quantize";
  g_msg[0] = '\0';
  if (!valid_dtype(w_dtype)) return fail(LH_ERR_DTYPE, "%s: w_dtype must be 0 (f32) or 1 (bf16)", fn);
  if (c_out < 0 || c_in < 0) return fail(LH_ERR_SHAPE, "%s: negative size", fn);
  if (c_in % 16 != 0) return fail(LH_ERR_SHAPE, "%s: c_in must be a multiple of 16", fn);
  if (ld_w < c_in || ld_u < c_in || ld_q < c_in) return fail(LH_ERR_SHAPE, "%s: a leading dimension < c_in", fn);
  if (c_out == 0 || c_in == 0) return LH_OK;
  if (!w || !best_idx || !amax || !u || !w_q || !workspace)
    return fail(LH_ERR_NULL, "%s: w, best_idx, amax, u, w_q and workspace are required", fn);
  if (!aligned(w, elem_size(w_dtype)) || !aligned(amax, 4) || !aligned(u, 4) || !aligned(w_q, 4) ||
      !aligned(workspace, 16))
    return fail(LH_ERR_ARG, "%s: pointer not aligned to its element size (workspace: 16 bytes)", fn);
  if (workspace_bytes < lh::gptq_quantize_ws_bytes(c_out, c_in))
    return fail(LH_ERR_WORKSPACE, "%s: workspace smaller than lh_gptq_workspace_bytes()", fn);
  lh::GptqQuantizeArgs a{w, w_dtype, c_out, c_in, ld_w, best_idx, amax, u, ld_u, w_q, ld_q, workspace};
  hipError_t e = lh::launch_gptq_quantize(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LH_OK : hip_fail(e, fn);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The whole path for callers that cannot allocate (code under graph capture,
// tight serving loops, harnesses that forbid allocation).  The scratch that
// lh_calibrate_nvfp4 takes as its workspace (skip certificates, the
// Hessian's token-slice partial sums, the amax shares) lives in the
// file-scope device array `scratch` instead: each GPU the library runs on
// holds its own copy, kNoAllocScratchBytes, until the process ends.  In host
// code the array's name is only a stand-in, never a device address: the
// address on a device comes from hipGetSymbolAddress, looked up once per
// device (the first call with that device current) and kept.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
constexpr int kNoAllocMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kNoAllocMaxDevices];

// The address of this device's `scratch`, for the current device, which must
// also be the stream's.
lh_status noalloc_scratch(const char* fn, void* stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, fn);
  if (dev < 0 || dev >= kNoAllocMaxDevices) return fail(LH_ERR_ARG, "%s: device index out of range", fn);
  hipDevice_t sdev = -1;
  e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
  if (e != hipSuccess) return hip_fail(e, fn);
  if (sdev != dev) return fail(LH_ERR_ARG, "%s: the stream belongs to another device than the current one", fn);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, fn);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LH_OK;
}

}  // namespace

extern "C" lh_status lh_calibrate_nvfp4_noalloc(const void* w, int w_dtype, int64_t c_out, int64_t c_in,
                                                int64_t ld_w, int64_t n_groups, int64_t group_stride_w,
                                                const void* x, int x_dtype, int x_layout, int64_t n_tokens,
                                                int64_t ld_x, int64_t group_stride_x, float* amax, float* h,
                                                int64_t group_stride_h, uint8_t* best_idx, float* best_err,
                                                float* best_amax, float* w_q, uint8_t* packed_e2m1,
                                                uint8_t* scale_e4m3, float* global_scale, void* stream) {
  const char* fn = "lh_calibrate_nvfp4_noalloc";
  g_msg[0] = '\0';
  if (c_out > 0 && c_in > 0 && n_groups > 0 && n_tokens >= 0 && c_in % 16 == 0) {
    const size_t need = calibrate_ws_bytes(c_out, c_in, n_tokens, n_groups);
    if (need > kNoAllocScratchBytes) {
      snprintf(g_msg, sizeof g_msg,
               "%s: this layer needs %zu bytes of scratch, more than the %zu bytes the entry point holds on each "
               "device; call lh_calibrate_nvfp4 with a workspace instead",
               fn, need, kNoAllocScratchBytes);
      return LH_ERR_WORKSPACE;
    }
  }
  void* ws = nullptr;
  const lh_status st = noalloc_scratch(fn, stream, &ws);
  if (st != LH_OK) return st;
  return lh_calibrate_nvfp4(w, w_dtype, c_out, c_in, ld_w, n_groups, group_stride_w, x, x_dtype, x_layout, n_tokens,
                            ld_x, group_stride_x, amax, h, group_stride_h, best_idx, best_err, best_amax, w_q,
                            packed_e2m1, scale_e4m3, global_scale, ws, kNoAllocScratchBytes, stream);
}
