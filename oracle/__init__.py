"""CPU oracle for Local-Hessian NVFP4 scale calibration (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU leg of
the benchmark may import this package.  The HIP library never links, loads or
calls it, and it shares no code with that library.

The arithmetic lives in ``lh_oracle.c`` (plain C, fp64 sums, the fp32 cast
operations spelled out); this module only marshals numpy arrays.  Every
function follows the "Local-Hessian weight-scale guide" (xxmr.cn/news/266017):
sections "What is Local-Hessian" (NVFP4 format, 126-candidate sweep) and
"Algorithm principle" (Q = Cast(W/s)*s, block error E_b = Delta_b H_b
Delta_b^T with H_b = X_b X_b^T, kernel interface).  The readings taken where
the page is silent are listed at the top of ``lh_oracle.c``.

bf16 arrays are passed as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lh_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblh_oracle.so")

F32, BF16 = 0, 1
RULE_SWEEP, RULE_MAX, RULE_FOUR_OVER_SIX, RULE_AMAX_SEARCH = 0, 1, 2, 3
CHANNEL_MAJOR, TOKEN_MAJOR = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
               "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    alt = os.environ.get("LH_ORACLE_LIB")  # a variant build, used only by the mutation tests
    if alt:
        lib = ctypes.CDLL(alt)
    else:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I32, D, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_float
    lib.oracle_e4m3_value.argtypes = [I32]
    lib.oracle_e4m3_value.restype = D
    lib.oracle_candidate_scales.argtypes = [F, P]
    lib.oracle_e2m1_code.argtypes = [F]
    lib.oracle_e2m1_code.restype = I32
    lib.oracle_quantize.argtypes = [F, F, P]
    lib.oracle_quantize.restype = F
    lib.oracle_block_errors.argtypes = [P, P, F, P]
    lib.oracle_absmax.argtypes = [P, I32, I64, I64, I64, I64, I64, P]
    lib.oracle_hessian.argtypes = [P, I32, I32, I64, I64, I64, I64, D, D, P, I64, P, P]
    lib.oracle_sweep.argtypes = [P, I32, I64, I64, I64, I64, P, I64, P, P, I64, P, P, P, P, P, P, P, P, P]
    lib.oracle_fake_quant.argtypes = [P, I32, I64, I64, I64, I64, P, P, P, I64, P, P, P]
    lib.oracle_e4m3_round_code.argtypes = [F]
    lib.oracle_e4m3_round_code.restype = I32
    lib.oracle_amax_multiplier.argtypes = [I32]
    lib.oracle_amax_multiplier.restype = F
    lib.oracle_rule_candidates.argtypes = [I32, P, F, P]
    lib.oracle_rule_candidates.restype = I32
    lib.oracle_select.argtypes = [I32, P, I32, I64, I64, I64, I64, P, I64, P, P, I64, P, P, P, P, P, P, P, P, P]
    lib.oracle_hessian_ragged.argtypes = [P, I32, I64, I64, P, I64, P, P, I64, P, P, P]
    lib.oracle_full_hessian.argtypes = [P, I32, I64, I64, I64, D, P]
    lib.oracle_output_error.argtypes = [P, I32, P, I64, I64, I64, P, P, I64, P]
    lib.oracle_scaled_histogram.argtypes = [P, I32, I64, I64, I64, P, F, I32, F, P]
    lib.oracle_gptq_u.argtypes = [P, I64, D, P]
    lib.oracle_gptq_u.restype = I32
    lib.oracle_gptq_sweep.argtypes = [P, I32, I64, I64, P, F, P, P, I32, P, I64, P]
    lib.oracle_num_threads.restype = I32
    lib.oracle_set_num_threads.argtypes = [I32]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("oracle inputs are float32 or uint16 (bf16 bits), got %s" % a.dtype)


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def e4m3_value(code: int) -> float:
    return _load().oracle_e4m3_value(int(code))


def candidate_scales(g: float) -> np.ndarray:
    out = np.empty(126, np.float32)
    _load().oracle_candidate_scales(float(np.float32(g)), _ptr(out))
    return out


def e2m1_code(x: float) -> int:
    return _load().oracle_e2m1_code(float(np.float32(x)))


def quantize(w: float, s: float) -> tuple[float, int]:
    code = ctypes.c_int(0)
    q = _load().oracle_quantize(float(np.float32(w)), float(np.float32(s)), ctypes.byref(code))
    return float(np.float32(q)), code.value


def block_errors(w16, H, g: float) -> np.ndarray:
    w16 = np.ascontiguousarray(w16, np.float32).reshape(16)
    H = np.ascontiguousarray(H, np.float32).reshape(256)
    out = np.empty(126, np.float64)
    _load().oracle_block_errors(_ptr(w16), _ptr(H), float(np.float32(g)), _ptr(out))
    return out


def absmax(w: np.ndarray, c_out: int, c_in: int, ld_w: int | None = None,
           n_groups: int = 1, group_stride_w: int | None = None) -> np.ndarray:
    w = np.ascontiguousarray(w)
    ld_w = c_in if ld_w is None else ld_w
    gs = c_out * ld_w if group_stride_w is None else group_stride_w
    out = np.empty(n_groups, np.float32)
    _load().oracle_absmax(_ptr(w), _dtype_code(w), c_out, c_in, ld_w, n_groups, gs, _ptr(out))
    return out


def hessian(x: np.ndarray, c_in: int, n_tok: int, layout: int = CHANNEL_MAJOR,
            ld_x: int | None = None, n_groups: int = 1, group_stride_x: int | None = None,
            alpha: float | None = None, beta: float = 0.0, h_old: np.ndarray | None = None,
            sel: np.ndarray | None = None):
    """Returns (h64, h32) of shape [n_sel, 16, 16] for the selected flat
    (group * c_in/16 + block) indices (all when ``sel`` is None).
    alpha defaults to 1/N (the normalised Hessian)."""
    x = np.ascontiguousarray(x)
    nb = c_in // 16
    if ld_x is None:
        ld_x = n_tok if layout == CHANNEL_MAJOR else c_in
    if group_stride_x is None:
        group_stride_x = c_in * ld_x if layout == CHANNEL_MAJOR else n_tok * ld_x
    if alpha is None:
        alpha = 1.0 / n_tok if n_tok > 0 else 0.0
    sel = np.arange(n_groups * nb, dtype=np.int64) if sel is None else np.ascontiguousarray(sel, np.int64)
    h64 = np.empty((len(sel), 16, 16), np.float64)
    if h_old is not None:
        h32 = np.ascontiguousarray(h_old, np.float32).reshape(len(sel), 16, 16).copy()
    else:
        h32 = np.zeros((len(sel), 16, 16), np.float32)
    _load().oracle_hessian(_ptr(x), _dtype_code(x), layout, c_in, n_tok, ld_x, group_stride_x,
                           float(alpha), float(beta), _ptr(sel), len(sel), _ptr(h64), _ptr(h32))
    return h64, h32


def _probe_outputs(n: int, probe, forms: bool) -> dict:
    out = {}
    if probe is not None:
        out["e_probe"] = np.empty(n, np.float64)
    if forms:
        out["s_best"] = np.empty(n, np.float64)
        if probe is not None:
            out["s_probe"] = np.empty(n, np.float64)
    return out


def sweep(w: np.ndarray, H: np.ndarray, amax: np.ndarray, c_out: int, c_in: int,
          ld_w: int | None = None, n_groups: int = 1, group_stride_w: int | None = None,
          group_stride_h: int | None = None, sel: np.ndarray | None = None, probe: np.ndarray | None = None,
          forms: bool = False) -> dict:
    """Exhaustive 126-candidate sweep for the selected flat block indices
    ((group * c_out + row) * c_in/16 + b).  H is the fp32 Hessian tensor the
    sweep consumes ([n_groups][c_in/16][16][16]).  Returns a dict of compact
    arrays: idx, e1 (best error), e2 (second best), err (fl32(e1)), amax.
    With ``probe`` (one candidate index per selected block, e.g. another
    implementation's pick) also e_probe = the error at that candidate; with
    ``forms`` also s_best (and s_probe) = sum_ij |H_ij| |dw_i| |dw_j| at the
    best (and the probed) candidate, which sizes fp32 rounding in checks."""
    w = np.ascontiguousarray(w)
    H = np.ascontiguousarray(H, np.float32)
    amax = np.ascontiguousarray(amax, np.float32).reshape(-1)
    nb = c_in // 16
    ld_w = c_in if ld_w is None else ld_w
    gsw = c_out * ld_w if group_stride_w is None else group_stride_w
    gsh = nb * 256 if group_stride_h is None else group_stride_h
    sel = np.arange(n_groups * c_out * nb, dtype=np.int64) if sel is None else np.ascontiguousarray(sel, np.int64)
    n = len(sel)
    out = dict(idx=np.empty(n, np.int32), e1=np.empty(n, np.float64), e2=np.empty(n, np.float64),
               err=np.empty(n, np.float32), amax=np.empty(n, np.float32))
    pr = None if probe is None else np.ascontiguousarray(probe, np.int32).reshape(n)
    out.update(_probe_outputs(n, pr, forms))
    _load().oracle_sweep(_ptr(w), _dtype_code(w), c_out, c_in, ld_w, gsw, _ptr(H), gsh, _ptr(amax),
                         _ptr(sel), n, _ptr(out["idx"]), _ptr(out["e1"]), _ptr(out["e2"]),
                         _ptr(out["err"]), _ptr(out["amax"]), _ptr(pr), _ptr(out.get("e_probe")),
                         _ptr(out.get("s_probe")), _ptr(out.get("s_best")))
    return out


def fake_quant(w: np.ndarray, idx: np.ndarray, amax: np.ndarray, c_out: int, c_in: int,
               ld_w: int | None = None, n_groups: int = 1, group_stride_w: int | None = None,
               sel: np.ndarray | None = None) -> dict:
    """NVFP4 fake-quant of the selected blocks with per-block candidate index
    ``idx`` (full [n_groups][c_out][c_in/16] uint8 array).  Returns compact
    q [n,16] fp32, packed [n,8] uint8 and code [n] uint8 (= idx + 1)."""
    w = np.ascontiguousarray(w)
    idx = np.ascontiguousarray(idx, np.uint8).reshape(-1)
    amax = np.ascontiguousarray(amax, np.float32).reshape(-1)
    nb = c_in // 16
    ld_w = c_in if ld_w is None else ld_w
    gsw = c_out * ld_w if group_stride_w is None else group_stride_w
    sel = np.arange(n_groups * c_out * nb, dtype=np.int64) if sel is None else np.ascontiguousarray(sel, np.int64)
    n = len(sel)
    out = dict(q=np.empty((n, 16), np.float32), packed=np.empty((n, 8), np.uint8),
               code=np.empty(n, np.uint8))
    _load().oracle_fake_quant(_ptr(w), _dtype_code(w), c_out, c_in, ld_w, gsw, _ptr(idx),
                              _ptr(amax), _ptr(sel), n, _ptr(out["q"]), _ptr(out["packed"]),
                              _ptr(out["code"]))
    return out


def e4m3_round_code(t: float) -> int:
    """E4M3 byte (1..126) stored for a wanted block-scale value t (nearest,
    ties to the even code, saturating at 448, never zero)."""
    return int(_load().oracle_e4m3_round_code(float(t)))


def amax_multiplier(i: int) -> float:
    """The i-th multiplier of the amax search (0.25 + 0.1 i)."""
    return float(_load().oracle_amax_multiplier(int(i)))


def rule_candidates(rule: int, w16, g: float) -> np.ndarray:
    """Distinct candidate indices (ascending) that a scale rule considers."""
    w16 = np.ascontiguousarray(w16, np.float32)
    out = np.empty(126, np.int32)
    n = _load().oracle_rule_candidates(int(rule), _ptr(w16), float(g), _ptr(out))
    return out[:n].copy()


def select(rule: int, w: np.ndarray, H, amax: np.ndarray, c_out: int, c_in: int,
           ld_w: int | None = None, n_groups: int = 1, group_stride_w: int | None = None,
           group_stride_h: int | None = None, sel: np.ndarray | None = None, probe: np.ndarray | None = None,
           forms: bool = False) -> dict:
    """Scale selection by rule (RULE_SWEEP: all 126 candidates, RULE_MAX,
    RULE_FOUR_OVER_SIX, RULE_AMAX_SEARCH) for the selected flat block
    indices.  H is the fp32 Hessian tensor, or None for the plain weight
    error (H = I).  Returns idx, e1, e2, err, amax like ``sweep``, and the
    same optional probe / form outputs (under the rule's objective)."""
    w = np.ascontiguousarray(w)
    Hc = None if H is None else np.ascontiguousarray(H, np.float32)
    amax = np.ascontiguousarray(amax, np.float32).reshape(-1)
    nb = c_in // 16
    ld_w = c_in if ld_w is None else ld_w
    gsw = c_out * ld_w if group_stride_w is None else group_stride_w
    gsh = nb * 256 if group_stride_h is None else group_stride_h
    sel = np.arange(n_groups * c_out * nb, dtype=np.int64) if sel is None else np.ascontiguousarray(sel, np.int64)
    n = len(sel)
    out = dict(idx=np.empty(n, np.int32), e1=np.empty(n, np.float64), e2=np.empty(n, np.float64),
               err=np.empty(n, np.float32), amax=np.empty(n, np.float32))
    pr = None if probe is None else np.ascontiguousarray(probe, np.int32).reshape(n)
    out.update(_probe_outputs(n, pr, forms))
    _load().oracle_select(int(rule), _ptr(w), _dtype_code(w), c_out, c_in, ld_w, gsw,
                          None if Hc is None else _ptr(Hc), gsh, _ptr(amax), _ptr(sel), n,
                          _ptr(out["idx"]), _ptr(out["e1"]), _ptr(out["e2"]), _ptr(out["err"]),
                          _ptr(out["amax"]), _ptr(pr), _ptr(out.get("e_probe")), _ptr(out.get("s_probe")),
                          _ptr(out.get("s_best")))
    return out


def hessian_ragged(x: np.ndarray, c_in: int, offsets, h_old: np.ndarray, counts=None, ld_x: int | None = None,
                   sel: np.ndarray | None = None):
    """Per-group Hessians of token-major x [rows][ld_x] whose rows
    offsets[g] .. offsets[g+1]-1 belong to group g.  h_old is the previous
    fp32 Hessian tensor [n_groups][c_in/16][16][16]; without counts each
    group with tokens gets S_g / n_g, with counts the running mean
    (n_old H + S_g) / (n_old + n_g); groups without tokens keep h_old.
    Returns (h64, h32) compact over the selected flat blocks, and the
    updated counts (or None)."""
    x = np.ascontiguousarray(x)
    offsets = np.ascontiguousarray(offsets, np.int64)
    n_groups = len(offsets) - 1
    nb = c_in // 16
    ld_x = c_in if ld_x is None else ld_x
    sel = np.arange(n_groups * nb, dtype=np.int64) if sel is None else np.ascontiguousarray(sel, np.int64)
    hold = np.ascontiguousarray(np.asarray(h_old, np.float32).reshape(n_groups * nb, 256)[sel])
    cnt = None if counts is None else np.ascontiguousarray(counts, np.int64)
    h64 = np.zeros((len(sel), 16, 16), np.float64)
    h32 = np.zeros((len(sel), 16, 16), np.float32)
    _load().oracle_hessian_ragged(_ptr(x), _dtype_code(x), c_in, ld_x, _ptr(offsets), n_groups,
                                  None if cnt is None else _ptr(cnt), _ptr(sel), len(sel), _ptr(hold),
                                  _ptr(h64), _ptr(h32))
    new_counts = None if cnt is None else cnt + np.diff(offsets)
    return h64, h32, new_counts


def full_hessian(x: np.ndarray, c_in: int, n_tok: int, ld_x: int | None = None, alpha: float | None = None):
    """Full C_in x C_in Hessian alpha X X^T (fp64) of one channel-major group
    (alpha defaults to 1/N)."""
    x = np.ascontiguousarray(x)
    ld_x = n_tok if ld_x is None else ld_x
    alpha = (1.0 / n_tok if n_tok else 0.0) if alpha is None else alpha
    h = np.zeros((c_in, c_in), np.float64)
    _load().oracle_full_hessian(_ptr(x), _dtype_code(x), c_in, n_tok, ld_x, float(alpha), _ptr(h))
    return h


def output_error(w: np.ndarray, q: np.ndarray, h: np.ndarray, c_in: int, rows: np.ndarray | None = None,
                 ld_w: int | None = None, ld_q: int | None = None) -> np.ndarray:
    """(q - w) H (q - w)^T per selected row of one group (fp64), with the
    fp32 full Hessian h [c_in][c_in]."""
    w = np.ascontiguousarray(w)
    q = np.ascontiguousarray(q, np.float32)
    h = np.ascontiguousarray(h, np.float32)
    n = w.shape[0] if w.ndim == 2 else w.size // (ld_w or c_in)
    rows = np.arange(n, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    ld_w = c_in if ld_w is None else ld_w
    ld_q = c_in if ld_q is None else ld_q
    e = np.zeros(len(rows), np.float64)
    _load().oracle_output_error(_ptr(w), _dtype_code(w), _ptr(q), c_in, ld_w, ld_q, _ptr(h), _ptr(rows),
                                len(rows), _ptr(e))
    return e


def scaled_histogram(w: np.ndarray, idx: np.ndarray, g: float, c_out: int, c_in: int, n_bins: int,
                     bins_per_unit: float, ld_w: int | None = None) -> np.ndarray:
    """Counts [n_bins + 1] of x = fl32(|w| / s_k) over one group (bin
    floor(fl32(x * bins_per_unit)), last bin = overflow)."""
    w = np.ascontiguousarray(w)
    idx = np.ascontiguousarray(idx, np.uint8)
    ld_w = c_in if ld_w is None else ld_w
    counts = np.zeros(n_bins + 1, np.uint64)
    _load().oracle_scaled_histogram(_ptr(w), _dtype_code(w), c_out, c_in, ld_w, _ptr(idx), float(g), int(n_bins),
                                    float(bins_per_unit), _ptr(counts))
    return counts


def gptq_u(h: np.ndarray, damp: float = 0.01) -> np.ndarray:
    """Upper U (fp64) with (H + damp mean(diag H) I)^-1 = U^T U, from the fp32
    full Hessian h [n][n]."""
    h = np.ascontiguousarray(h, np.float32)
    n = h.shape[0]
    U = np.zeros((n, n), np.float64)
    if _load().oracle_gptq_u(_ptr(h), n, float(damp), _ptr(U)) != 0:
        raise ValueError("damped Hessian is not positive definite")
    return U


def gptq_sweep(w: np.ndarray, idx: np.ndarray, g: float, c_in: int, U32: np.ndarray | None = None,
               U64: np.ndarray | None = None, rows: np.ndarray | None = None, ld_w: int | None = None) -> np.ndarray:
    """GPTQ rounding of the selected rows of one group with fixed block
    scales.  With U32 (fp32) the fp32 sweep (fused multiply-adds in column
    order), with U64 the fp64 sweep.  Returns q [n_rows][c_in] fp32."""
    w = np.ascontiguousarray(w)
    idx = np.ascontiguousarray(idx, np.uint8)
    ld_w = c_in if ld_w is None else ld_w
    n_all = w.size // ld_w
    rows = np.arange(n_all, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    prec = 32 if U32 is not None else 64
    u32 = None if U32 is None else np.ascontiguousarray(U32, np.float32)
    u64 = None if U64 is None else np.ascontiguousarray(U64, np.float64)
    q = np.zeros((len(rows), c_in), np.float32)
    _load().oracle_gptq_sweep(_ptr(w), _dtype_code(w), c_in, ld_w, _ptr(idx), float(g),
                              None if u32 is None else _ptr(u32), None if u64 is None else _ptr(u64), prec,
                              _ptr(rows), len(rows), _ptr(q))
    return q
