"""Parity rules between the HIP library and the CPU oracle (used by the GPU
tests, the smoke check and the benchmark's self-check).

Rules (the repository's design notes derive them):
  * Hessian: |H_gpu - H_oracle|_ij <= 1e-3 * sqrt(H_ii H_jj) (+1e-30): relative
    on the diagonal, Cauchy-Schwarz-scaled off it; the oracle sums in fp64.
  * Sweep (judged on the same fp32 H fed to both sides): the GPU evaluates
    E = dw^T H dw in fp32, so its forward error is bounded by
    gamma * S with S = sum_ij |H_ij| |dw_i| |dw_j| and gamma = 4e-6 (about
    twice the 35 unit roundoffs of the evaluation: dw = fl(Q - w), 16-term
    fused dot products, the 16-term outer sum).  Where the quadratic form
    cancels (e.g. a rank-1 H from one token) S >> E and no fp32 evaluation
    can reach a relative tolerance, so:
      - the chosen index is bit-exact unless the oracle's best and
        second-best errors differ by less than max(1e-5 * e2, 2 gamma S)
        (or e2 == 0);
      - the error is within max(1e-4 * e1, gamma * S);
    S is taken at the oracle's best candidate.  The per-block amax is
    bit-exact where the index agrees.
  * Fake-quant: Q, packed nibbles and E4M3 codes bit-exact for the same indices.
  * Global amax: bit-exact.
"""
from __future__ import annotations

import numpy as np

import oracle

H_RTOL = 1e-3
TIE_RTOL = 1e-5
ERR_RTOL = 1e-4
FP32_GAMMA = 4e-6


def check_hessian(h_gpu: np.ndarray, h_or64: np.ndarray, what: str = "") -> float:
    """h_gpu, h_or64: [n, 16, 16].  Returns the worst normalised deviation."""
    h_gpu = np.asarray(h_gpu, np.float64).reshape(-1, 16, 16)
    ref = np.asarray(h_or64, np.float64).reshape(-1, 16, 16)
    d = np.sqrt(np.abs(np.einsum("nii->ni", ref)))
    scale = d[:, :, None] * d[:, None, :]
    dev = np.abs(h_gpu - ref)
    bad = dev > H_RTOL * scale + 1e-30
    if bad.any():
        n, i, j = np.argwhere(bad)[0]
        raise AssertionError("%s Hessian mismatch at block %d (%d,%d): gpu %r oracle %r (allowed %r); %d bad" % (
            what, n, i, j, h_gpu[n, i, j], ref[n, i, j], H_RTOL * scale[n, i, j], bad.sum()))
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(scale > 0, dev / scale, 0.0)
    return float(rel.max()) if rel.size else 0.0


def abs_form(w_sel: np.ndarray, q_sel: np.ndarray, h_sel: np.ndarray) -> np.ndarray:
    """S = sum_ij |H_ij| |dw_i| |dw_j| for each selected block (fp64)."""
    dw = np.abs(q_sel.astype(np.float64) - w_sel.astype(np.float64))
    return np.einsum("ni,nij,nj->n", dw, np.abs(h_sel.astype(np.float64)), dw)


def check_sweep(gpu_idx, gpu_err, gpu_amax, orc: dict, S: np.ndarray, what: str = "") -> dict:
    """gpu_* are compact arrays for the same selected blocks as the oracle
    dict; S = sum |H||dw||dw| at the oracle's best candidate."""
    gi = np.asarray(gpu_idx).astype(np.int64)
    oi = orc["idx"].astype(np.int64)
    e1, e2 = orc["e1"], orc["e2"]
    bound = FP32_GAMMA * S
    near_tie = (e2 == 0) | ((e2 - e1) < np.maximum(TIE_RTOL * e2, 2 * bound))
    mism = (gi != oi) & ~near_tie
    if mism.any():
        n = int(np.flatnonzero(mism)[0])
        raise AssertionError("%s index mismatch at selected block %d: gpu %d oracle %d (e1 %r e2 %r); %d of %d" % (
            what, n, gi[n], oi[n], e1[n], e2[n], int(mism.sum()), len(gi)))
    stats = dict(n=len(gi), near_tie=int(near_tie.sum()), idx_diff_in_ties=int(((gi != oi) & near_tie).sum()))
    if gpu_err is not None:
        ge = np.asarray(gpu_err, np.float64)
        tol = np.maximum(ERR_RTOL * e1, bound)
        bad = np.abs(ge - e1) > tol
        if bad.any():
            n = int(np.flatnonzero(bad)[0])
            raise AssertionError("%s error mismatch at selected block %d: gpu %r oracle %r tol %r; %d bad" % (
                what, n, ge[n], e1[n], tol[n], int(bad.sum())))
        with np.errstate(invalid="ignore", divide="ignore"):
            stats["err_rel_max"] = float(np.nanmax(np.where(e1 > 0, np.abs(ge - e1) / e1, 0.0))) if len(ge) else 0.0
    if gpu_amax is not None:
        same = gi == oi
        ga = np.asarray(gpu_amax, np.float32)
        if not np.array_equal(ga[same], orc["amax"][same]):
            n = int(np.flatnonzero(same & (ga != orc["amax"]))[0])
            raise AssertionError("%s amax mismatch at %d: gpu %r oracle %r" % (what, n, ga[n], orc["amax"][n]))
    return stats


def block_rows(w_np: np.ndarray, sel: np.ndarray, c_out: int, c_in: int) -> np.ndarray:
    """[n, 16] fp32 weights of the selected flat blocks (w_np [G, c_out, c_in],
    fp32 or bf16 bits)."""
    nb = c_in // 16
    b = sel % nb
    rg = sel // nb
    flat = w_np.reshape(-1, c_in)
    cols = (16 * b)[:, None] + np.arange(16)[None, :]
    vals = flat[rg[:, None], cols]
    if vals.dtype == np.uint16:
        vals = (vals.astype(np.uint32) << 16).view(np.float32)
    return vals.astype(np.float32)


def sweep_against_oracle(w_np, h_np, amax_np, c_out, c_in, n_groups, sel, gpu_idx_full, gpu_err_full,
                         gpu_amax_full, what=""):
    """Run the oracle sweep on `sel` with the GPU's H and compare."""
    nb = c_in // 16
    res = oracle.sweep(w_np, h_np, amax_np, c_out, c_in, n_groups=n_groups, sel=sel)
    # S from the oracle's chosen candidate
    idx_full = np.zeros(n_groups * c_out * nb, np.uint8)
    idx_full[sel] = res["idx"].astype(np.uint8)
    fq = oracle.fake_quant(w_np, idx_full, amax_np, c_out, c_in, n_groups=n_groups, sel=sel)
    grp = sel // (c_out * nb)
    hb = h_np.reshape(n_groups, nb, 16, 16)[grp, sel % nb]
    S = abs_form(block_rows(w_np, sel, c_out, c_in), fq["q"], hb)
    ge = None if gpu_err_full is None else gpu_err_full.reshape(-1)[sel]
    ga = None if gpu_amax_full is None else gpu_amax_full.reshape(-1)[sel]
    return check_sweep(gpu_idx_full.reshape(-1)[sel], ge, ga, res, S, what)


def fake_quant_against_oracle(w_np, idx_full, amax_np, c_out, c_in, n_groups, sel, gpu: dict, what=""):
    nb = c_in // 16
    fq = oracle.fake_quant(w_np, idx_full.reshape(-1), amax_np, c_out, c_in, n_groups=n_groups, sel=sel)
    rg, b = sel // nb, sel % nb
    if "w_q" in gpu:
        q = gpu["w_q"].reshape(-1, c_in)
        cols = (16 * b)[:, None] + np.arange(16)[None, :]
        got = q[rg[:, None], cols]
        if not np.array_equal(got.view(np.uint32), fq["q"].view(np.uint32)):
            n = int(np.argwhere(got.view(np.uint32) != fq["q"].view(np.uint32))[0][0])
            raise AssertionError("%s fake-quant Q mismatch at block %d: gpu %r oracle %r" % (what, n, got[n], fq["q"][n]))
    if "packed" in gpu:
        p = gpu["packed"].reshape(-1, c_in // 2)
        cols = (8 * b)[:, None] + np.arange(8)[None, :]
        got = p[rg[:, None], cols]
        assert np.array_equal(got, fq["packed"]), "%s packed nibbles differ" % what
    if "scale_e4m3" in gpu:
        assert np.array_equal(gpu["scale_e4m3"].reshape(-1)[sel], fq["code"]), "%s E4M3 codes differ" % what


def select_against_oracle(rule, w_np, h_np, amax_np, c_out, c_in, n_groups, sel, gpu_idx_full, gpu_err_full,
                          gpu_amax_full, what=""):
    """Scale selection by rule (h_np None = plain weight error) against the
    oracle on `sel`, with the sweep's rules; S uses H = I without a Hessian."""
    nb = c_in // 16
    res = oracle.select(rule, w_np, h_np, amax_np, c_out, c_in, n_groups=n_groups, sel=sel)
    idx_full = np.zeros(n_groups * c_out * nb, np.uint8)
    idx_full[sel] = res["idx"].astype(np.uint8)
    fq = oracle.fake_quant(w_np, idx_full, amax_np, c_out, c_in, n_groups=n_groups, sel=sel)
    if h_np is None:
        hb = np.broadcast_to(np.eye(16, dtype=np.float32), (len(sel), 16, 16))
    else:
        grp = sel // (c_out * nb)
        hb = h_np.reshape(n_groups, nb, 16, 16)[grp, sel % nb]
    S = abs_form(block_rows(w_np, sel, c_out, c_in), fq["q"], hb)
    ge = None if gpu_err_full is None else gpu_err_full.reshape(-1)[sel]
    ga = None if gpu_amax_full is None else gpu_amax_full.reshape(-1)[sel]
    return check_sweep(gpu_idx_full.reshape(-1)[sel], ge, ga, res, S, what)
