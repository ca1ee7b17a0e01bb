"""Local-Hessian NVFP4 weight-scale calibration on AMD Instinct MI355X.

Thin ctypes binding over the C ABI of ``liblh.so`` (declared in
``include/lh.h``).  The functions carry the C names and only marshal
arguments: tensor pointers, strides, dtypes and the current HIP stream.
Every step of the computation runs in the library's HIP kernels; there is no
CPU fallback.  If the library is missing the import raises.

Tensors must live on a ROCm device.  Shapes:
  weights      [c_out, c_in] or [n_groups, c_out, c_in], bf16 or fp32,
               last dim contiguous (any row / group stride)
  activations  channel-major [c_in, N] / [n_groups, c_in, N], or
               token-major   [N, c_in] / [n_groups, N, c_in]
  hessians     fp32 [n_groups, c_in/16, 16, 16]
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblh.so")

LH_DTYPE_F32, LH_DTYPE_BF16 = 0, 1
LH_LAYOUT_CHANNEL_MAJOR, LH_LAYOUT_TOKEN_MAJOR = 0, 1
LH_RULE_SWEEP, LH_RULE_MAX, LH_RULE_FOUR_OVER_SIX, LH_RULE_AMAX_SEARCH = 0, 1, 2, 3
N_CANDIDATES = 126
BLOCK = 16


class LHError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s (status %d)" % (message, status))
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("liblh.so not built: run __graft_entry__.build() or "
                          "python nvfp4_scale_calibration_amd/_build.py (%s)" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.lh_abi_version.restype = I
    lib.lh_status_string.argtypes = [I]
    lib.lh_status_string.restype = ctypes.c_char_p
    lib.lh_last_error_message.restype = ctypes.c_char_p
    lib.lh_absmax.argtypes = [P, I, I64, I64, I64, I64, I64, P, P]
    lib.lh_absmax.restype = I
    lib.lh_hessian_alpha.argtypes = [F, I64]
    lib.lh_hessian_alpha.restype = F
    lib.lh_hessian_workspace_bytes.argtypes = [I64, I64, I64]
    lib.lh_hessian_workspace_bytes.restype = SZ
    lib.lh_accumulate_hessian.argtypes = [P, I, I, I64, I64, I64, I64, I64, F, F, P, I64, P, SZ, P]
    lib.lh_accumulate_hessian.restype = I
    lib.lh_hessian_ragged_workspace_bytes.argtypes = [I64, I64, I64, I64]
    lib.lh_hessian_ragged_workspace_bytes.restype = SZ
    lib.lh_accumulate_hessian_ragged.argtypes = [P, I, I64, I64, I64, P, I64, I64, P, I64, P, P, SZ, P]
    lib.lh_accumulate_hessian_ragged.restype = I
    lib.lh_sweep_workspace_bytes.argtypes = [I64, I64]
    lib.lh_sweep_workspace_bytes.restype = SZ
    lib.lh_scale_sweep.argtypes = [P, I, I64, I64, I64, I64, I64, P, I64, P, P, P, P, P, SZ, P]
    lib.lh_scale_sweep.restype = I
    lib.lh_select_scales.argtypes = [I, P, I, I64, I64, I64, I64, I64, P, I64, P, P, P, P, P, SZ, P]
    lib.lh_select_scales.restype = I
    lib.lh_scale_sweep_fake_quant.argtypes = [P, I, I64, I64, I64, I64, I64, P, I64, P, P, P, P, P, P, P, P, P,
                                              SZ, P]
    lib.lh_scale_sweep_fake_quant.restype = I
    lib.lh_calibrate_workspace_bytes.argtypes = [I64, I64, I64, I64]
    lib.lh_calibrate_workspace_bytes.restype = SZ
    lib.lh_calibrate_nvfp4.argtypes = [P, I, I64, I64, I64, I64, I64, P, I, I, I64, I64, I64, P, P, I64, P, P, P, P, P,
                                       P, P, P, SZ, P]
    lib.lh_calibrate_nvfp4.restype = I
    lib.lh_calibrate_nvfp4_noalloc.argtypes = [P, I, I64, I64, I64, I64, I64, P, I, I, I64, I64, I64, P, P, I64, P, P,
                                               P, P, P, P, P, P]
    lib.lh_calibrate_nvfp4_noalloc.restype = I
    lib.lh_calibrate_prologue.argtypes = [P, I, I64, I64, I64, I64, I64, P, I, I, I64, I64, I64, P, P, I64, P, SZ, P]
    lib.lh_calibrate_prologue.restype = I
    lib.lh_calibrate_sweep.argtypes = [P, I, I64, I64, I64, I64, I64, P, I64, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.lh_calibrate_sweep.restype = I
    lib.lh_full_hessian.argtypes = [P, I, I64, I64, I64, I64, I64, F, P, I64, I64, P]
    lib.lh_full_hessian.restype = I
    lib.lh_output_error_workspace_bytes.argtypes = [I64, I64, I64]
    lib.lh_output_error_workspace_bytes.restype = SZ
    lib.lh_output_error.argtypes = [P, I, P, I64, I64, I64, I64, I64, I64, I64, P, I64, I64, P, P, SZ, P]
    lib.lh_output_error.restype = I
    lib.lh_scaled_histogram.argtypes = [P, I, I64, I64, I64, I64, I64, P, P, I, F, P, P]
    lib.lh_scaled_histogram.restype = I
    lib.lh_gptq_workspace_bytes.argtypes = [I64, I64]
    lib.lh_gptq_workspace_bytes.restype = SZ
    lib.lh_gptq_prepare.argtypes = [P, I64, I64, F, P, I64, P, SZ, P]
    lib.lh_gptq_prepare.restype = I
    lib.lh_gptq_quantize.argtypes = [P, I, I64, I64, I64, P, P, P, I64, P, I64, P, SZ, P]
    lib.lh_gptq_quantize.restype = I
    lib.lh_fake_quant_nvfp4.argtypes = [P, I, I64, I64, I64, I64, I64, P, P, P, P, P, P, P]
    lib.lh_fake_quant_nvfp4.restype = I
    return lib


lib = _load()
EXPORTS = ("lh_abi_version", "lh_status_string", "lh_last_error_message", "lh_absmax", "lh_hessian_alpha",
           "lh_hessian_workspace_bytes", "lh_accumulate_hessian", "lh_hessian_ragged_workspace_bytes",
           "lh_accumulate_hessian_ragged", "lh_sweep_workspace_bytes", "lh_scale_sweep",
           "lh_scale_sweep_fake_quant", "lh_calibrate_workspace_bytes", "lh_calibrate_nvfp4",
           "lh_calibrate_prologue", "lh_calibrate_sweep", "lh_calibrate_nvfp4_noalloc", "lh_select_scales", "lh_fake_quant_nvfp4", "lh_full_hessian", "lh_output_error_workspace_bytes",
           "lh_output_error", "lh_scaled_histogram", "lh_gptq_workspace_bytes", "lh_gptq_prepare",
           "lh_gptq_quantize")


def _check(status: int) -> None:
    if status != 0:
        msg = lib.lh_last_error_message().decode() or lib.lh_status_string(status).decode()
        raise LHError(status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LH_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return LH_DTYPE_BF16
    raise TypeError("expected float32 or bfloat16, got %s" % t.dtype)


def _as3(t: torch.Tensor) -> torch.Tensor:
    if t.dim() == 2:
        return t.unsqueeze(0)
    if t.dim() != 3:
        raise ValueError("expected a 2-D or 3-D tensor, got shape %s" % (tuple(t.shape),))
    return t


def _require_device(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("liblh works on device tensors only (got a %s tensor)" % t.device)


def _group_stride(t3: torch.Tensor) -> int:
    return t3.stride(0) if t3.shape[0] > 1 else 0


def _ld(t3: torch.Tensor) -> int:
    """Row stride; a dimension of size 1 has no meaningful stride (torch may
    report 1), so the contiguous extent is passed instead."""
    return t3.stride(1) if t3.shape[1] > 1 else t3.shape[2]


def lh_abi_version() -> int:
    return lib.lh_abi_version()


def lh_absmax(w: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Global amax per group: out[g] = max |w[g]| (fp32)."""
    _require_device(w)
    w3 = _as3(w)
    if w3.stride(-1) != 1:
        raise ValueError("last dim of w must be contiguous")
    g, rows, cols = w3.shape
    if out is None:
        out = torch.empty(g, dtype=torch.float32, device=w.device)
    _check(lib.lh_absmax(_ptr(w3), _dtype(w3), rows, cols, _ld(w3), g, _group_stride(w3),
                         _ptr(out), _stream(w)))
    return out


def lh_hessian_alpha(alpha: float, n_tokens: int) -> float:
    """The factor the Hessian calls apply for `alpha` (NaN: fl32(1/N))."""
    return float(lib.lh_hessian_alpha(float(alpha), int(n_tokens)))


def lh_hessian_workspace_bytes(c_in: int, n_tokens: int, n_groups: int = 1) -> int:
    return int(lib.lh_hessian_workspace_bytes(c_in, n_tokens, n_groups))


def lh_accumulate_hessian(x: torch.Tensor, layout: str = "channel", alpha: float | None = None,
                          beta: float = 0.0, h: torch.Tensor | None = None,
                          workspace: torch.Tensor | bool | None = True) -> torch.Tensor:
    """h = beta * h + alpha * X_b X_b^T for every 16-channel block.

    x: channel-major [.., c_in, N] (layout="channel") or token-major
    [.., N, c_in] (layout="token").  alpha defaults to 1/N (the normalised
    Hessian).  workspace=True allocates the split-token scratch buffer the
    library asks for, False/None runs without one, a uint8 device tensor is
    used as given."""
    _require_device(x, h)
    x3 = _as3(x)
    if x3.stride(-1) != 1:
        raise ValueError("last dim of x must be contiguous")
    lay = {"channel": LH_LAYOUT_CHANNEL_MAJOR, "token": LH_LAYOUT_TOKEN_MAJOR}[layout]
    g = x3.shape[0]
    c_in, n_tok = (x3.shape[1], x3.shape[2]) if lay == LH_LAYOUT_CHANNEL_MAJOR else (x3.shape[2], x3.shape[1])
    nb = c_in // BLOCK
    if alpha is None:
        alpha = float("nan")   # the library applies the normalised Hessian's 1/N
    if h is None:
        h = torch.empty((g, nb, BLOCK, BLOCK), dtype=torch.float32, device=x.device)
        if beta != 0.0:
            raise ValueError("beta != 0 needs an existing h")
    ws, ws_bytes = None, 0
    if workspace is True:
        ws_bytes = lh_hessian_workspace_bytes(c_in, n_tok, g)
        if ws_bytes:
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    elif isinstance(workspace, torch.Tensor):
        ws, ws_bytes = workspace, workspace.numel() * workspace.element_size()
    h_gstride = h.stride(0) if h.dim() == 4 and h.shape[0] > 1 else 0
    _check(lib.lh_accumulate_hessian(_ptr(x3), _dtype(x3), lay, c_in, n_tok, _ld(x3), g,
                                     _group_stride(x3), float(alpha), float(beta), _ptr(h), h_gstride,
                                     _ptr(ws), ws_bytes, _stream(x)))
    return h


def lh_hessian_ragged_workspace_bytes(c_in: int, n_rows: int, n_groups: int, max_group_rows: int = 0) -> int:
    return int(lib.lh_hessian_ragged_workspace_bytes(c_in, n_rows, n_groups, max_group_rows))


def lh_accumulate_hessian_ragged(x: torch.Tensor, offsets: torch.Tensor, h: torch.Tensor | None = None,
                                 counts: torch.Tensor | None = None,
                                 workspace: torch.Tensor | bool | None = True,
                                 max_group_rows: int = 0) -> torch.Tensor:
    """Per-group Hessians of token-major x [n_rows, c_in] whose rows
    offsets[g] .. offsets[g+1]-1 (device int64 [n_groups + 1]) belong to
    group g.  Without counts each group with tokens gets S_g / n_g; with a
    device int64 counts tensor the running mean (n_old H + S_g) / (n_old +
    n_g) is kept and counts is advanced.  Groups without tokens keep h (a
    new h starts at zero)."""
    _require_device(x, offsets, h, counts)
    if x.dim() != 2 or x.stride(-1) != 1:
        raise ValueError("x must be a 2-D token-major tensor with contiguous rows")
    if offsets.dtype != torch.int64 or counts is not None and counts.dtype != torch.int64:
        raise TypeError("offsets and counts must be int64")
    n_rows, c_in = x.shape
    g = offsets.numel() - 1
    nb = c_in // BLOCK
    if h is None:
        h = torch.zeros((g, nb, BLOCK, BLOCK), dtype=torch.float32, device=x.device)
    ws, ws_bytes = None, 0
    if workspace is True:
        ws_bytes = lh_hessian_ragged_workspace_bytes(c_in, n_rows, g, max_group_rows)
        if ws_bytes:
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    elif isinstance(workspace, torch.Tensor):
        ws, ws_bytes = workspace, workspace.numel() * workspace.element_size()
    h_gstride = h.stride(0) if h.dim() == 4 and h.shape[0] > 1 else 0
    ld = x.stride(0) if n_rows > 1 else c_in
    _check(lib.lh_accumulate_hessian_ragged(_ptr(x), _dtype(x), c_in, ld, n_rows, _ptr(offsets), g,
                                            int(max_group_rows), _ptr(h),
                                            h_gstride, _ptr(counts), _ptr(ws), ws_bytes, _stream(x)))
    return h


def lh_sweep_workspace_bytes(c_in: int, n_groups: int = 1) -> int:
    return int(lib.lh_sweep_workspace_bytes(c_in, n_groups))


def _select(rule, w, h, amax, best_idx, best_err, best_amax, workspace, quant=None):
    _require_device(w, h, amax)
    w3 = _as3(w)
    if w3.stride(-1) != 1:
        raise ValueError("last dim of w must be contiguous")
    g, c_out, c_in = w3.shape
    nb = c_in // BLOCK
    shape = (g, c_out, nb)
    dev = w.device
    if best_idx is None:
        best_idx = torch.empty(shape, dtype=torch.uint8, device=dev)
    if best_err is True:
        best_err = torch.empty(shape, dtype=torch.float32, device=dev)
    if best_amax is True:
        best_amax = torch.empty(shape, dtype=torch.float32, device=dev)
    best_err = best_err if isinstance(best_err, torch.Tensor) else None
    best_amax = best_amax if isinstance(best_amax, torch.Tensor) else None
    h_gstride = h.stride(0) if h is not None and h.dim() == 4 and h.shape[0] > 1 else 0
    ws, ws_bytes = None, 0
    if workspace is True:
        ws_bytes = lh_sweep_workspace_bytes(c_in, g) if h is not None and rule == LH_RULE_SWEEP else 0
        if ws_bytes:
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    elif isinstance(workspace, torch.Tensor):
        ws, ws_bytes = workspace, workspace.numel() * workspace.element_size()
    args = (_ptr(w3), _dtype(w3), c_out, c_in, _ld(w3), g, _group_stride(w3), _ptr(h), h_gstride, _ptr(amax),
            _ptr(best_idx), _ptr(best_err), _ptr(best_amax), _ptr(ws), ws_bytes, _stream(w))
    if quant is not None:
        _check(lib.lh_scale_sweep_fake_quant(*args[:13], *(_ptr(quant[k]) for k in _FQ_KEYS), *args[13:]))
    elif rule is None:
        _check(lib.lh_scale_sweep(*args))
    else:
        _check(lib.lh_select_scales(int(rule), *args))
    return best_idx, best_err, best_amax


def lh_scale_sweep(w: torch.Tensor, h: torch.Tensor, amax: torch.Tensor,
                   best_idx: torch.Tensor | None = None, best_err: torch.Tensor | bool | None = True,
                   best_amax: torch.Tensor | bool | None = True,
                   workspace: torch.Tensor | bool | None = True):
    """Per-block best candidate index (E4M3 code = idx + 1), its error
    dw^T H_b dw and the per-block amax 6 * s_idx.  Returns (idx, err, amax);
    err / amax are None when not requested (False/None).  workspace=True
    allocates the certificate scratch the library asks for (faster skipping),
    False/None runs without it, a device tensor is used as given."""
    if h is None:
        raise ValueError("lh_scale_sweep needs a Hessian (lh_select_scales takes h=None)")
    return _select(None, w, h, amax, best_idx, best_err, best_amax, workspace)


_FQ_KEYS = ("w_q", "packed", "scale_e4m3", "global_scale")


def _fq_outputs(w3, w_q, packed, scale_e4m3, global_scale) -> dict:
    g, c_out, c_in = w3.shape
    dev = w3.device

    def out(req, shape, dtype):
        if isinstance(req, torch.Tensor):
            return req
        return torch.empty(shape, dtype=dtype, device=dev) if req else None

    return dict(w_q=out(w_q, (g, c_out, c_in), torch.float32),
                packed=out(packed, (g, c_out, c_in // 2), torch.uint8),
                scale_e4m3=out(scale_e4m3, (g, c_out, c_in // BLOCK), torch.uint8),
                global_scale=out(global_scale, (g,), torch.float32))


def lh_scale_sweep_fake_quant(w: torch.Tensor, h: torch.Tensor, amax: torch.Tensor,
                              best_idx: torch.Tensor | None = None, best_err: torch.Tensor | bool | None = True,
                              best_amax: torch.Tensor | bool | None = True,
                              w_q: bool | torch.Tensor = True, packed: bool | torch.Tensor = False,
                              scale_e4m3: bool | torch.Tensor = False, global_scale: bool | torch.Tensor = False,
                              workspace: torch.Tensor | bool | None = True) -> dict:
    """lh_scale_sweep and lh_fake_quant_nvfp4 with its indices in one pass.
    Returns a dict with idx, err, amax (as lh_scale_sweep; None when not
    requested) and the requested fake-quant outputs (as lh_fake_quant_nvfp4)."""
    if h is None:
        raise ValueError("lh_scale_sweep_fake_quant needs a Hessian")
    _require_device(w)
    quant = _fq_outputs(_as3(w), w_q, packed, scale_e4m3, global_scale)
    idx, err, bam = _select(None, w, h, amax, best_idx, best_err, best_amax, workspace, quant=quant)
    res = dict(idx=idx, err=err, amax=bam)
    res.update({k: v for k, v in quant.items() if v is not None})
    return res


def lh_calibrate_workspace_bytes(c_out: int, c_in: int, n_tokens: int, n_groups: int = 1) -> int:
    return int(lib.lh_calibrate_workspace_bytes(c_out, c_in, n_tokens, n_groups))


def _calibrate_outputs(w3, x3, layout, out, best_err, best_amax, w_q, packed, scale_e4m3, global_scale):
    g, c_out, c_in = w3.shape
    if layout == "channel":
        lay, n_tok = LH_LAYOUT_CHANNEL_MAJOR, x3.shape[2]
    elif layout == "token":
        lay, n_tok = LH_LAYOUT_TOKEN_MAJOR, x3.shape[1]
    else:
        raise ValueError("layout must be 'channel' or 'token'")
    if n_tok > 0 and x3.stride(-1) != 1:
        raise ValueError("last dim of x must be contiguous")
    nb = c_in // BLOCK
    dev = w3.device
    out = dict(out or {})

    def get(name, req, shape, dtype):
        if name in out:
            return out[name]
        return torch.empty(shape, dtype=dtype, device=dev) if req else None

    res = dict(amax=get("amax", True, (g,), torch.float32),
               h=get("h", True, (g, nb, 16, 16), torch.float32),
               idx=get("idx", True, (g, c_out, nb), torch.uint8),
               err=get("err", best_err, (g, c_out, nb), torch.float32),
               amax_blk=get("amax_blk", best_amax, (g, c_out, nb), torch.float32),
               w_q=get("w_q", w_q, (g, c_out, c_in), torch.float32),
               packed=get("packed", packed, (g, c_out, c_in // 2), torch.uint8),
               scale_e4m3=get("scale_e4m3", scale_e4m3, (g, c_out, nb), torch.uint8),
               global_scale=get("global_scale", global_scale, (g,), torch.float32))
    if n_tok > 0:
        ld_x = _ld(x3)
    else:  # nothing is read; any row stride the boundary accepts
        ld_x = 1 if lay == LH_LAYOUT_CHANNEL_MAJOR else max(c_in, 1)
    return res, lay, n_tok, ld_x


def lh_calibrate_nvfp4(w: torch.Tensor, x: torch.Tensor, layout: str = "channel", out: dict | None = None,
                       best_err: bool = True, best_amax: bool = True, w_q: bool = True, packed: bool = False,
                       scale_e4m3: bool = False, global_scale: bool = False,
                       workspace: torch.Tensor | None = None, split: bool = False) -> dict:
    """The whole path: global amax, normalised local Hessians (x
    [.., c_in, N] channel-major or [.., N, c_in] token-major), the
    126-candidate sweep and the fake-quant of its result.  Returns a dict
    with amax, h, idx and the requested outputs (err, amax_blk, w_q, packed,
    scale_e4m3, global_scale); tensors given in `out` under those names are
    written in place.  split=True makes the same computation as the two calls
    lh_calibrate_prologue and lh_calibrate_sweep."""
    _require_device(w, x)
    w3, x3 = _as3(w), _as3(x)
    if w3.stride(-1) != 1:
        raise ValueError("last dim of w must be contiguous")
    g, c_out, c_in = w3.shape
    res, lay, n_tok, ld_x = _calibrate_outputs(w3, x3, layout, out, best_err, best_amax, w_q, packed, scale_e4m3,
                                               global_scale)
    if workspace is None:
        workspace = torch.empty(max(lh_calibrate_workspace_bytes(c_out, c_in, n_tok, g), 1), dtype=torch.uint8,
                                device=w.device)
    wsb = workspace.numel() * workspace.element_size()
    h = res["h"]
    h_gstride = h.stride(0) if h.dim() == 4 and h.shape[0] > 1 else 0
    wargs = (_ptr(w3), _dtype(w3), c_out, c_in, _ld(w3), g, _group_stride(w3))
    fq = (_ptr(res["w_q"]), _ptr(res["packed"]), _ptr(res["scale_e4m3"]), _ptr(res["global_scale"]))
    if split:
        _check(lib.lh_calibrate_prologue(*wargs, _ptr(x3), _dtype(x3), lay, n_tok, ld_x, _group_stride(x3),
                                         _ptr(res["amax"]), _ptr(h), h_gstride, _ptr(workspace), wsb, _stream(w)))
        _check(lib.lh_calibrate_sweep(*wargs, _ptr(h), h_gstride, _ptr(res["amax"]), _ptr(res["idx"]),
                                      _ptr(res["err"]), _ptr(res["amax_blk"]), *fq, _ptr(workspace), wsb,
                                      _stream(w)))
    else:
        _check(lib.lh_calibrate_nvfp4(*wargs, _ptr(x3), _dtype(x3), lay, n_tok, ld_x, _group_stride(x3),
                                      _ptr(res["amax"]), _ptr(h), h_gstride, _ptr(res["idx"]), _ptr(res["err"]),
                                      _ptr(res["amax_blk"]), *fq, _ptr(workspace), wsb, _stream(w)))
    return {k: v for k, v in res.items() if v is not None}


def lh_calibrate_nvfp4_noalloc(w: torch.Tensor, x: torch.Tensor, layout: str = "channel", out: dict | None = None,
                               best_err: bool = True, best_amax: bool = True, w_q: bool = True, packed: bool = False,
                               scale_e4m3: bool = False, global_scale: bool = False) -> dict:
    """lh_calibrate_nvfp4 through the entry point that takes no workspace
    (its scratch is a fixed device array in the library, 32 MiB per GPU).
    Outputs given in `out` are written in place; missing ones are created
    here (the C call itself allocates nothing)."""
    _require_device(w, x)
    w3, x3 = _as3(w), _as3(x)
    if w3.stride(-1) != 1:
        raise ValueError("last dim of w must be contiguous")
    g, c_out, c_in = w3.shape
    res, lay, n_tok, ld_x = _calibrate_outputs(w3, x3, layout, out, best_err, best_amax, w_q, packed, scale_e4m3,
                                               global_scale)
    h = res["h"]
    h_gstride = h.stride(0) if h.dim() == 4 and h.shape[0] > 1 else 0
    _check(lib.lh_calibrate_nvfp4_noalloc(_ptr(w3), _dtype(w3), c_out, c_in, _ld(w3), g, _group_stride(w3), _ptr(x3),
                                          _dtype(x3), lay, n_tok, ld_x, _group_stride(x3), _ptr(res["amax"]), _ptr(h),
                                          h_gstride, _ptr(res["idx"]), _ptr(res["err"]), _ptr(res["amax_blk"]),
                                          _ptr(res["w_q"]), _ptr(res["packed"]), _ptr(res["scale_e4m3"]),
                                          _ptr(res["global_scale"]), _stream(w)))
    return {k: v for k, v in res.items() if v is not None}


def lh_calibrate_prologue(w: torch.Tensor, x: torch.Tensor, amax: torch.Tensor, h: torch.Tensor,
                          workspace: torch.Tensor, layout: str = "channel") -> None:
    """amax, h and the sweep's certificates (left in workspace) for
    lh_calibrate_sweep; output tensors given."""
    _require_device(w, x, amax, h, workspace)
    w3, x3 = _as3(w), _as3(x)
    g, c_out, c_in = w3.shape
    _, lay, n_tok, ld_x = _calibrate_outputs(w3, x3, layout, dict(amax=amax, h=h, idx=None), False, False, False,
                                             False, False, False)
    h_gstride = h.stride(0) if h.dim() == 4 and h.shape[0] > 1 else 0
    _check(lib.lh_calibrate_prologue(_ptr(w3), _dtype(w3), c_out, c_in, _ld(w3), g, _group_stride(w3), _ptr(x3),
                                     _dtype(x3), lay, n_tok, ld_x, _group_stride(x3), _ptr(amax), _ptr(h), h_gstride,
                                     _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(w)))


def lh_calibrate_sweep(w: torch.Tensor, h: torch.Tensor, amax: torch.Tensor, workspace: torch.Tensor,
                       best_idx: torch.Tensor, best_err=None, best_amax=None, w_q=None, packed=None, scale_e4m3=None,
                       global_scale=None) -> None:
    """The sweep and fake-quant with the certificates lh_calibrate_prologue
    left in workspace; output tensors given (None to skip)."""
    _require_device(w, h, amax, workspace, best_idx)
    w3 = _as3(w)
    g, c_out, c_in = w3.shape
    h_gstride = h.stride(0) if h.dim() == 4 and h.shape[0] > 1 else 0
    _check(lib.lh_calibrate_sweep(_ptr(w3), _dtype(w3), c_out, c_in, _ld(w3), g, _group_stride(w3), _ptr(h),
                                  h_gstride, _ptr(amax), _ptr(best_idx), _ptr(best_err), _ptr(best_amax), _ptr(w_q),
                                  _ptr(packed), _ptr(scale_e4m3), _ptr(global_scale), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(w)))


def lh_select_scales(rule: int, w: torch.Tensor, h: torch.Tensor | None, amax: torch.Tensor,
                     best_idx: torch.Tensor | None = None, best_err: torch.Tensor | bool | None = True,
                     best_amax: torch.Tensor | bool | None = True,
                     workspace: torch.Tensor | bool | None = True):
    """Block scales by rule (LH_RULE_SWEEP / MAX / FOUR_OVER_SIX /
    AMAX_SEARCH) under dw^T H_b dw, or the plain weight error when h is
    None.  Same outputs as lh_scale_sweep."""
    return _select(rule, w, h, amax, best_idx, best_err, best_amax, workspace)


def lh_fake_quant_nvfp4(w: torch.Tensor, best_idx: torch.Tensor, amax: torch.Tensor,
                        w_q: bool | torch.Tensor = True, packed: bool | torch.Tensor = False,
                        scale_e4m3: bool | torch.Tensor = False,
                        global_scale: bool | torch.Tensor = False) -> dict:
    """NVFP4 fake-quant / packing with the chosen block scales.  Returns a
    dict with the requested outputs: w_q [g, c_out, c_in] fp32, packed
    [g, c_out, c_in/2] uint8, scale_e4m3 [g, c_out, c_in/16] uint8,
    global_scale [g] fp32."""
    _require_device(w, best_idx, amax)
    w3 = _as3(w)
    if w3.stride(-1) != 1:
        raise ValueError("last dim of w must be contiguous")
    g, c_out, c_in = w3.shape
    res = _fq_outputs(w3, w_q, packed, scale_e4m3, global_scale)
    _check(lib.lh_fake_quant_nvfp4(_ptr(w3), _dtype(w3), c_out, c_in, _ld(w3), g, _group_stride(w3),
                                   _ptr(best_idx), _ptr(amax), _ptr(res["w_q"]), _ptr(res["packed"]),
                                   _ptr(res["scale_e4m3"]), _ptr(res["global_scale"]), _stream(w)))
    return {k: v for k, v in res.items() if v is not None}


def lh_full_hessian(x: torch.Tensor, alpha: float | None = None, h: torch.Tensor | None = None) -> torch.Tensor:
    """Full C_in x C_in Hessian alpha X X^T of channel-major x [.., c_in, N]
    (alpha defaults to 1/N)."""
    _require_device(x, h)
    x3 = _as3(x)
    g, c_in, n = x3.shape
    if n > 0 and x3.stride(-1) != 1:
        raise ValueError("last dim of x must be contiguous")
    if alpha is None:
        alpha = float("nan")   # the library applies 1/N
    if h is None:
        h = torch.empty((g, c_in, c_in), dtype=torch.float32, device=x.device)
    h3 = _as3(h)
    ld = _ld(x3) if n > 0 else 1  # no token: nothing is read
    _check(lib.lh_full_hessian(_ptr(x3), _dtype(x3), c_in, n, ld, g, _group_stride(x3), float(alpha),
                               _ptr(h3), _ld(h3), _group_stride(h3), _stream(x)))
    return h


def lh_output_error_workspace_bytes(c_out: int, c_in: int, n_groups: int = 1) -> int:
    return int(lib.lh_output_error_workspace_bytes(c_out, c_in, n_groups))


def lh_output_error(w: torch.Tensor, w_q: torch.Tensor, h_full: torch.Tensor, err: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Per-row d H d^T with d = w_q - w ([n_groups, c_out])."""
    _require_device(w, w_q, h_full, err, workspace)
    w3, q3, h3 = _as3(w), _as3(w_q), _as3(h_full)
    if q3.dtype != torch.float32 or h3.dtype != torch.float32:
        raise TypeError("w_q and h_full must be float32")
    g, c_out, c_in = w3.shape
    if err is None:
        err = torch.empty((g, c_out), dtype=torch.float32, device=w.device)
    if workspace is None:
        workspace = torch.empty(max(lh_output_error_workspace_bytes(c_out, c_in, g), 4), dtype=torch.uint8,
                                device=w.device)
    _check(lib.lh_output_error(_ptr(w3), _dtype(w3), _ptr(q3), c_out, c_in, _ld(w3), _ld(q3), g,
                               _group_stride(w3), _group_stride(q3), _ptr(h3), _ld(h3), _group_stride(h3),
                               _ptr(err), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(w)))
    return err


def lh_scaled_histogram(w: torch.Tensor, best_idx: torch.Tensor, amax: torch.Tensor, n_bins: int = 160,
                        bins_per_unit: float = 20.0, counts: torch.Tensor | None = None) -> torch.Tensor:
    """Counts [n_groups, n_bins + 1] (int64 storage of uint64 counts) of
    W/s = fl32(|w| / s_k), bins of width 1/bins_per_unit, last = overflow."""
    _require_device(w, best_idx, amax, counts)
    w3 = _as3(w)
    g, c_out, c_in = w3.shape
    if counts is None:
        counts = torch.empty((g, n_bins + 1), dtype=torch.int64, device=w.device)
    _check(lib.lh_scaled_histogram(_ptr(w3), _dtype(w3), c_out, c_in, _ld(w3), g, _group_stride(w3),
                                   _ptr(best_idx), _ptr(amax), int(n_bins), float(bins_per_unit), _ptr(counts),
                                   _stream(w)))
    return counts


def lh_gptq_workspace_bytes(c_out: int, c_in: int) -> int:
    return int(lib.lh_gptq_workspace_bytes(c_out, c_in))


def _gptq_ws(c_out, c_in, device, workspace):
    if workspace is not None:
        return workspace
    return torch.empty(max(lh_gptq_workspace_bytes(c_out, c_in), 16), dtype=torch.uint8, device=device)


def lh_gptq_prepare(h_full: torch.Tensor, damp: float = 0.01, u: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Upper u with (H + damp mean(diag H) I)^-1 = u^T u, from one layer's
    full Hessian [c_in, c_in] (fp32)."""
    _require_device(h_full, u, workspace)
    h2 = h_full.reshape(h_full.shape[-2], h_full.shape[-1])
    c_in = h2.shape[0]
    if u is None:
        u = torch.empty((c_in, c_in), dtype=torch.float32, device=h_full.device)
    ws = _gptq_ws(0, c_in, h_full.device, workspace)
    _check(lib.lh_gptq_prepare(_ptr(h2), c_in, h2.stride(0), float(damp), _ptr(u), u.stride(0), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(h_full)))
    return u


def lh_gptq_quantize(w: torch.Tensor, best_idx: torch.Tensor, amax: torch.Tensor, u: torch.Tensor,
                     w_q: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """GPTQ rounding of one layer's w [c_out, c_in] with fixed block scales
    (best_idx [c_out, c_in/16], global amax device scalar); returns the
    dequantised fp32 weights."""
    _require_device(w, best_idx, amax, u, w_q, workspace)
    w2 = w.reshape(w.shape[-2], w.shape[-1])
    if w2.stride(-1) != 1:
        raise ValueError("last dim of w must be contiguous")
    c_out, c_in = w2.shape
    if w_q is None:
        w_q = torch.empty((c_out, c_in), dtype=torch.float32, device=w.device)
    ws = _gptq_ws(c_out, c_in, w.device, workspace)
    ld_w = w2.stride(0) if c_out > 1 else c_in
    _check(lib.lh_gptq_quantize(_ptr(w2), _dtype(w2), c_out, c_in, ld_w, _ptr(best_idx), _ptr(amax), _ptr(u),
                                u.stride(0), _ptr(w_q), w_q.stride(0) if c_out > 1 else c_in, _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(w)))
    return w_q
