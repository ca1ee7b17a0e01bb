"""CPU checks of the parity checker itself (tests/parity.py) and of the
oracle's probe outputs it relies on: a checker that waves wrong results
through would make every GPU parity claim void.  The "GPU" results here are
the oracle's own, with mistakes planted in them."""
import numpy as np
import pytest

import oracle
import parity


def _layer(seed, c_out=24, c_in=64, n_tok=200):
    rng = np.random.default_rng(seed)
    w = (rng.standard_t(4, size=(1, c_out, c_in)) * 0.02).astype(np.float32)
    x = rng.standard_normal((c_in, n_tok)).astype(np.float32)
    _, h = oracle.hessian(x, c_in, n_tok)
    amax = oracle.absmax(w, c_out, c_in)
    return w, h.reshape(1, c_in // 16, 16, 16), amax


def test_probe_outputs_are_the_block_errors():
    """e_probe is the oracle's own 126-vector at the probed index; the
    absolute form equals E for H = I and for a diagonal H, bounds |E|, and
    scales with H."""
    w, h, amax = _layer(1)
    c_out, c_in = w.shape[1:]
    nb = c_in // 16
    sel = np.arange(c_out * nb)
    rng = np.random.default_rng(2)
    probe = rng.integers(0, 126, len(sel)).astype(np.int32)
    res = oracle.sweep(w, h, amax, c_out, c_in, sel=sel, probe=probe, forms=True)
    for n in range(0, len(sel), 7):
        r, b = divmod(n, nb)
        E = oracle.block_errors(w[0, r, 16 * b:16 * b + 16], h[0, b], amax[0])
        assert res["e_probe"][n] == E[probe[n]]
        assert res["e1"][n] == E.min() and res["idx"][n] == int(np.argmin(E))
    assert np.all(res["s_best"] >= np.abs(res["e1"]) * (1 - 1e-12))
    assert np.all(res["s_probe"] >= np.abs(res["e_probe"]) * (1 - 1e-12))
    res_self = oracle.sweep(w, h, amax, c_out, c_in, sel=sel, probe=res["idx"], forms=True)
    assert np.array_equal(res_self["e_probe"], res_self["e1"])
    assert np.array_equal(res_self["s_probe"], res_self["s_best"])
    eye = np.broadcast_to(np.eye(16, dtype=np.float32), h.shape).copy()
    ri = oracle.sweep(w, eye, amax, c_out, c_in, sel=sel, probe=probe, forms=True)
    np.testing.assert_allclose(ri["s_probe"], ri["e_probe"], rtol=1e-15)
    dg = eye * np.float32(3.0)
    rd = oracle.sweep(w, dg, amax, c_out, c_in, sel=sel, probe=probe, forms=True)
    np.testing.assert_allclose(rd["s_probe"], rd["e_probe"], rtol=1e-15)
    r4 = oracle.sweep(w, h * np.float32(4.0), amax, c_out, c_in, sel=sel, probe=probe, forms=True)
    assert np.array_equal(r4["s_probe"], 4.0 * res["s_probe"])
    # without a Hessian (the plain weight error) the form is the error itself
    rm = oracle.select(oracle.RULE_SWEEP, w, None, amax, c_out, c_in, sel=sel, probe=probe, forms=True)
    np.testing.assert_allclose(rm["s_probe"], rm["e_probe"], rtol=1e-15)


def _as_gpu(res, amax):
    scales = oracle.candidate_scales(float(amax[0]))
    return res["idx"].copy(), res["err"].astype(np.float32), (np.float32(6.0) * scales[res["idx"]]).astype(np.float32)


def test_checker_accepts_the_oracle_and_rejects_planted_mistakes():
    w, h, amax = _layer(3)
    c_out, c_in = w.shape[1:]
    nb = c_in // 16
    sel = np.arange(c_out * nb)
    res = oracle.sweep(w, h, amax, c_out, c_in, sel=sel)
    gi, ge, ga = _as_gpu(res, amax)
    full = lambda a: a.reshape(1, c_out, nb)
    st = parity.sweep_against_oracle(w, h, amax, c_out, c_in, 1, sel, full(gi), full(ge), full(ga), "self",
                                     strict=True)
    assert st["idx_diff"] == 0 and st["gamma_only_idx"] == 0 and st["gamma_only_err"] == 0
    # a second-best pick on a block whose best two are far apart: rejected
    k = int(np.argmax((res["e2"] - res["e1"]) / res["e2"]))
    E = oracle.block_errors(w[0, k // nb, 16 * (k % nb):16 * (k % nb) + 16], h[0, k % nb], amax[0])
    order = np.argsort(E, kind="stable")
    bad = gi.copy()
    bad[k] = order[1]
    with pytest.raises(AssertionError, match="index mismatch"):
        parity.sweep_against_oracle(w, h, amax, c_out, c_in, 1, sel, full(bad), full(ge), full(ga), "planted")
    # an error 2e-4 off (relative): rejected
    bad_e = ge.copy()
    bad_e[k] = np.float32(ge[k] * (1 + 2e-4))
    with pytest.raises(AssertionError, match="error mismatch"):
        parity.sweep_against_oracle(w, h, amax, c_out, c_in, 1, sel, full(gi), full(bad_e), full(ga), "planted")
    # an amax one ulp off: rejected
    bad_a = ga.copy()
    bad_a[k] = np.nextafter(ga[k], np.float32(1.0))
    with pytest.raises(AssertionError, match="amax mismatch"):
        parity.sweep_against_oracle(w, h, amax, c_out, c_in, 1, sel, full(gi), full(ge), full(bad_a), "planted")


def test_checker_near_tie_needs_the_pick_itself_in_the_band():
    """A block whose best two candidates tie exactly (two identical weight
    halves under a block-symmetric H give no tie, so the tie is built from
    the error vector directly): the second-best pick passes, a third-best
    pick outside the band fails even though the best two are a near-tie."""
    e1 = np.array([1.0])
    orc = dict(idx=np.array([5]), e1=e1, e2=np.array([1.0 + 5e-6]), s_best=np.array([1.0]),
               e_probe=np.array([1.0 + 5e-6]), s_probe=np.array([1.0]))
    scales = oracle.candidate_scales(1.0)[None, :]
    grp = np.zeros(1, np.int64)
    st = parity.check_sweep(np.array([6]), None, None, orc, scales, grp, "tie")
    assert st["idx_diff_near_tie"] == 1 and st["gamma_only_idx"] == 0
    # the GPU's pick is a third candidate, 1e-3 above the best: rejected
    orc3 = dict(orc, e_probe=np.array([1.001]), s_probe=np.array([1.001]))
    with pytest.raises(AssertionError, match="index mismatch"):
        parity.check_sweep(np.array([9]), None, None, orc3, scales, grp, "third")
    # its error must match the error of the candidate it picked, not e1
    with pytest.raises(AssertionError, match="error mismatch"):
        parity.check_sweep(np.array([6]), np.array([1.0 + 5e-6 + 2e-4]), None, orc, scales, grp, "err")
    # a pick that passes only through the fp32 allowance is counted, and
    # refused in strict mode
    orcg = dict(idx=np.array([5]), e1=np.array([1e-3]), e2=np.array([1.2e-3]), s_best=np.array([100.0]),
                e_probe=np.array([1.2e-3]), s_probe=np.array([100.0]))
    st = parity.check_sweep(np.array([6]), None, None, orcg, scales, grp, "gamma")
    assert st["gamma_only_idx"] == 1
    with pytest.raises(AssertionError, match="fp32 allowance"):
        parity.check_sweep(np.array([6]), None, None, orcg, scales, grp, "gamma", strict=True)


def test_checker_rule_pick_must_be_a_candidate_of_the_rule():
    w, h, amax = _layer(4)
    c_out, c_in = w.shape[1:]
    nb = c_in // 16
    sel = np.arange(c_out * nb)
    res = oracle.select(oracle.RULE_MAX, w, h, amax, c_out, c_in, sel=sel)
    gi, ge, ga = _as_gpu(res, amax)
    full = lambda a: a.reshape(1, c_out, nb)
    parity.select_against_oracle(oracle.RULE_MAX, w, h, amax, c_out, c_in, 1, sel, full(gi), full(ge), full(ga),
                                 "max", strict=True)
    bad = gi.copy()
    bad[0] = (gi[0] + 1) % 126
    with pytest.raises(AssertionError):
        parity.select_against_oracle(oracle.RULE_MAX, w, h, amax, c_out, c_in, 1, sel, full(bad), None, None, "max")
