"""Parity rules between the HIP library and the CPU oracle (used by the GPU
tests, the smoke check and the benchmark's self-check).

Rules (the repository's design notes derive them):
  * Hessian: |H_gpu - H_oracle|_ij <= 1e-3 * sqrt(H_ii H_jj) (+1e-30): relative
    on the diagonal, Cauchy-Schwarz-scaled off it; the oracle sums in fp64.
  * Sweep, compared on the same fp32 H fed to both sides.  For every block the
    oracle also evaluates its error E_or[k_gpu] at the candidate the GPU
    chose (exact, fp64), so a different pick is accepted only when it is
    itself a near-tie of the best, and the GPU's reported error is compared
    with the error of the candidate it actually reports:
      - index: k_gpu == k_or, or E_or[k_gpu] - e1 <= 1e-5 * E_or[k_gpu]
        (then the oracle's best and second-best differ by less than 1e-5
        relative, the stated near-tie exemption);
      - error: |err_gpu - E_or[k_gpu]| <= 1e-4 * |E_or[k_gpu]|;
      - amax: bit-exact fl32(6 s_k) of the GPU's own index.
    The GPU evaluates E = dw^T H dw in fp32; its forward error is at most
    gamma * S with S = sum_ij |H_ij| |dw_i| |dw_j| and gamma = 4e-6 (twice
    the 35 unit roundoffs of dw = fl(Q - w), the 16-term fused rows and the
    16-term outer sum).  Where the form cancels (S >> E, e.g. a rank-1 H
    from one token) no fp32 evaluation meets a relative tolerance, so a
    block also passes when the pick is within gamma (S_best + S_pick) of the
    best, or the error within gamma * S_pick.  Blocks that pass only through
    these gamma terms are counted (``gamma_only_idx``, ``gamma_only_err``);
    with ``strict=True`` there must be none.
  * Fake-quant: Q, packed nibbles and E4M3 codes bit-exact for the same indices.
  * Global amax: bit-exact.
"""
from __future__ import annotations

import numpy as np

import oracle

# One line per parity case (what was compared and how it came out); the test
# session prints them in its summary, so a quiet run's log carries them too.
SUMMARY: list = []


def note(line: str) -> None:
    SUMMARY.append(line)


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


def check_sweep(gpu_idx, gpu_err, gpu_amax, orc: dict, scales: np.ndarray, grp: np.ndarray, what: str = "",
                strict: bool = False) -> dict:
    """gpu_* are compact arrays for the same selected blocks as the oracle
    dict, which holds e_probe / s_probe / s_best for the GPU's indices
    (oracle.sweep or oracle.select with probe=gpu_idx, forms=True);
    scales[g] are the oracle's 126 candidate scales of group g and grp the
    group of each selected block."""
    gi = np.asarray(gpu_idx).astype(np.int64)
    oi = orc["idx"].astype(np.int64)
    e1, e2, ep = orc["e1"], orc["e2"], orc["e_probe"]
    sb, sp = orc["s_best"], orc["s_probe"]
    n = len(gi)
    diff = gi != oi
    gap = ep - e1                                   # >= 0 for any candidate of the set: e1 is its minimum
    finite2 = np.isfinite(e2)
    # the stated near-tie band: the oracle's best two within 1e-5 relative, and
    # the GPU's pick itself within that band of the best
    ns_ok = finite2 & (gap >= 0) & (gap <= TIE_RTOL * np.abs(e2)) & ((e2 - e1) <= TIE_RTOL * np.abs(e2))
    g_ok = finite2 & (gap >= 0) & (gap <= FP32_GAMMA * (sb + sp))   # fp32 evaluation of cancelling forms
    bad = diff & ~(ns_ok | g_ok)
    if bad.any():
        k = int(np.flatnonzero(bad)[0])
        raise AssertionError("%s index mismatch at selected block %d: gpu %d oracle %d (e1 %r, e2 %r, oracle error "
                             "at the gpu's pick %r); %d of %d" % (what, k, gi[k], oi[k], e1[k], e2[k], ep[k],
                                                                 int(bad.sum()), n))
    stats = dict(n=n, idx_diff=int(diff.sum()), idx_diff_near_tie=int((diff & ns_ok).sum()),
                 gamma_only_idx=int((diff & ~ns_ok).sum()),
                 near_tie_blocks=int((finite2 & ((e2 - e1) <= TIE_RTOL * np.abs(e2))).sum()))
    if gpu_err is not None:
        ge = np.asarray(gpu_err, np.float64)
        dev = np.abs(ge - ep)
        ns_e = dev <= ERR_RTOL * np.abs(ep)
        g_e = dev <= FP32_GAMMA * sp
        bad = ~(ns_e | g_e)
        if bad.any():
            k = int(np.flatnonzero(bad)[0])
            raise AssertionError("%s error mismatch at selected block %d: gpu %r oracle %r at the gpu's index %d "
                                 "(tol %r); %d bad" % (what, k, ge[k], ep[k], gi[k], ERR_RTOL * abs(ep[k]),
                                                       int(bad.sum())))
        stats["gamma_only_err"] = int((~ns_e).sum())
        with np.errstate(invalid="ignore", divide="ignore"):
            rel = np.where(ep != 0, dev / np.abs(ep), np.where(dev == 0, 0.0, np.inf))
        stats["err_rel_max"] = float(rel.max()) if n else 0.0
    if gpu_amax is not None:
        ga = np.asarray(gpu_amax, np.float32)
        want = np.float32(6.0) * scales[grp, gi]
        if not np.array_equal(ga.view(np.uint32), want.view(np.uint32)):
            k = int(np.flatnonzero(ga.view(np.uint32) != want.view(np.uint32))[0])
            raise AssertionError("%s amax mismatch at %d: gpu %r, fl32(6 s_k) of its index %r" % (what, k, ga[k],
                                                                                                 want[k]))
    if strict:
        assert stats["gamma_only_idx"] == 0 and stats.get("gamma_only_err", 0) == 0, \
            "%s: blocks pass only through the fp32 allowance: %s" % (what, stats)
    return stats


def _scales(amax_np) -> np.ndarray:
    return np.stack([oracle.candidate_scales(float(g)) for g in np.asarray(amax_np, np.float32).reshape(-1)])


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
                         gpu_amax_full, what="", strict=False):
    """Run the oracle sweep on `sel` with the GPU's H and compare."""
    nb = c_in // 16
    gi = gpu_idx_full.reshape(-1)[sel]
    res = oracle.sweep(w_np, h_np, amax_np, c_out, c_in, n_groups=n_groups, sel=sel, probe=gi, forms=True)
    ge = None if gpu_err_full is None else gpu_err_full.reshape(-1)[sel]
    ga = None if gpu_amax_full is None else gpu_amax_full.reshape(-1)[sel]
    return check_sweep(gi, ge, ga, res, _scales(amax_np), sel // (c_out * nb), what, strict)


def fake_quant_against_oracle(w_np, idx_full, amax_np, c_out, c_in, n_groups, sel, gpu: dict, what=""):
    nb = c_in // 16
    fq = oracle.fake_quant(w_np, idx_full.reshape(-1), amax_np, c_out, c_in, n_groups=n_groups, sel=sel)
    if len(sel) == n_groups * c_out * nb and np.array_equal(sel, np.arange(len(sel))):
        # every block in order: compare the whole tensors
        if "w_q" in gpu:
            got = gpu["w_q"].reshape(-1, 16).view(np.uint32)
            badq = np.flatnonzero((got != fq["q"].view(np.uint32)).any(1))
            if len(badq):
                n = int(badq[0])
                raise AssertionError("%s fake-quant Q mismatch at block %d: gpu %r oracle %r; %d blocks" % (
                    what, n, gpu["w_q"].reshape(-1, 16)[n], fq["q"][n], len(badq)))
        if "packed" in gpu:
            assert np.array_equal(gpu["packed"].reshape(-1, 8), fq["packed"]), "%s packed nibbles differ" % what
        if "scale_e4m3" in gpu:
            assert np.array_equal(gpu["scale_e4m3"].reshape(-1), fq["code"]), "%s E4M3 codes differ" % what
        return
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
                          gpu_amax_full, what="", strict=False):
    """Scale selection by rule (h_np None = plain weight error) against the
    oracle on `sel`, with the sweep's rules (forms under the rule's
    objective: H = I without a Hessian)."""
    nb = c_in // 16
    gi = gpu_idx_full.reshape(-1)[sel]
    res = oracle.select(rule, w_np, h_np, amax_np, c_out, c_in, n_groups=n_groups, sel=sel, probe=gi, forms=True)
    grp = sel // (c_out * nb)
    # a pick that differs must still be one of the rule's own candidates
    diff = np.flatnonzero(gi.astype(np.int64) != res["idx"])
    if len(diff):
        rows = block_rows(w_np, sel[diff], c_out, c_in)
        amax_f = np.asarray(amax_np, np.float32).reshape(-1)
        for j, k in enumerate(diff):
            cands = oracle.rule_candidates(rule, rows[j], float(amax_f[grp[k]]))
            assert int(gi[k]) in cands, "%s: gpu pick %d at block %d is not a candidate of the rule" % (what, gi[k], k)
    ge = None if gpu_err_full is None else gpu_err_full.reshape(-1)[sel]
    ga = None if gpu_amax_full is None else gpu_amax_full.reshape(-1)[sel]
    return check_sweep(gi, ge, ga, res, _scales(amax_np), grp, what, strict)
