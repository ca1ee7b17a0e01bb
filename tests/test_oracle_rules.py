"""Pins for the oracle's scale-rule variants (max scaling, Four-Over-Six, the
amax multiplier search and the plain-MSE 126-value sweep).

Sources: "Local-Hessian weight-scale guide" (xxmr.cn/news/266017), section
"What is Local-Hessian" (max scaling takes the block scale from the block's
largest |w|; Four-Over-Six chooses between two candidate scales by the
in-block error; the MSE method sweeps all 126 positive FP8 values) and
section "Entry API and calibration flow" (amax search from multiplier 0.25
to 4.0 in steps of 0.1).

Each test checks the oracle against something other than itself: torch's
float8_e4m3fn encoder (round to nearest even), planted blocks whose answer
is known in closed form, brute-force errors from tests/_brute.py (torch
decoder + midpoint cast table, errors from the activations), and the
superset invariant (the 126-value sweep is never worse than a rule that
searches a subset of its candidates).
"""
import numpy as np
import pytest
import torch

import _brute as brute

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

RULES = ("SWEEP", "MAX", "FOUR_OVER_SIX", "AMAX_SEARCH")


def torch_e4m3_code(t):
    """E4M3FN byte of fp32 values by torch's encoder (valid for t <= 464)."""
    v = torch.from_numpy(np.ascontiguousarray(t, np.float32)).to(torch.float8_e4m3fn)
    return v.view(torch.uint8).numpy().astype(np.int64)


def stored_code(t):
    """The byte a wanted block-scale value t stores: torch's encoder, with
    values beyond 448 saturating and zero raised to the smallest value."""
    t = np.asarray(t, np.float32)
    c = torch_e4m3_code(np.minimum(t, np.float32(448.0)))
    return np.maximum(c, 1)


# ------------------------------------------------------------ E4M3 rounding

def test_e4m3_round_matches_torch_encoder(orc):
    rng = np.random.default_rng(7)
    t = np.exp2(rng.uniform(-12, 9.2, 20000)).astype(np.float32)
    t = t[t <= 464]
    got = np.array([orc.e4m3_round_code(v) for v in t])
    np.testing.assert_array_equal(got, stored_code(t))


def test_e4m3_round_midpoints_and_neighbours(orc):
    vals = np.concatenate([[0.0], brute.e4m3_candidates().astype(np.float64)])
    for i in range(len(vals) - 1):
        lo, hi = vals[i], vals[i + 1]
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2  # midpoints are exact in fp32
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(np.inf))
        code_lo, code_hi = max(i, 1), i + 1
        assert orc.e4m3_round_code(below) == code_lo
        assert orc.e4m3_round_code(above) == code_hi
        even = i if i % 2 == 0 else i + 1
        assert orc.e4m3_round_code(mid) == max(even, 1)
        assert orc.e4m3_round_code(mid) == stored_code([mid])[0]


def test_e4m3_round_saturates_and_never_zero(orc):
    for t in (448.0, 460.0, 464.0, 470.0, 1e6, 3e38, np.inf):
        assert orc.e4m3_round_code(t) == 126
    for t in (0.0, 1e-30, 2.0 ** -10, -1.0):
        assert orc.e4m3_round_code(t) == 1


# ------------------------------------------------------- multiplier grid

def test_amax_multiplier_grid(orc):
    m = np.array([orc.amax_multiplier(i) for i in range(38)], np.float32)
    ref = np.arange(0.25, 4.0, 0.1).astype(np.float32)  # stop value exclusive
    assert len(ref) == 38
    np.testing.assert_array_equal(m, ref)
    assert m[0] == np.float32(0.25) and m[-1] == np.float32(3.95)


# --------------------------------------------------- candidate sets by rule

def planted_block(rng, k, Sg, top=6.0):
    """16 weights whose largest magnitude is exactly top * s_k (s_k = fl32(c_k S_g))."""
    c = brute.e4m3_candidates()[k]
    sk = np.float32(c * np.float32(Sg))
    w = (rng.uniform(-1, 1, 16) * float(sk) * top * 0.9).astype(np.float32)
    w[rng.integers(16)] = np.float32(top * sk) * (1 if rng.random() < 0.5 else -1)
    return w


def test_max_rule_planted(orc):
    """A block whose largest |w| is 6 s_k (k not in the subnormal range,
    where fl32 rounding of amax/6 and of the division cannot leave the
    nearest E4M3 value) selects exactly k."""
    rng = np.random.default_rng(11)
    for g in (1.0, 0.37, 13.5, 2.0 ** -20, 2.0 ** 30):
        Sg = np.float32(g) / np.float32(2688.0)
        for k in range(8, 126):
            w = planted_block(rng, k, Sg)
            assert list(orc.rule_candidates(orc.RULE_MAX, w, g)) == [k]
            # largest |w| = 4 s_k: Four-Over-Six's second candidate is k
            w4 = planted_block(rng, k, Sg, top=4.0)
            assert k in list(orc.rule_candidates(orc.RULE_FOUR_OVER_SIX, w4, g))


def test_rule_candidates_match_torch_encoder(orc):
    rng = np.random.default_rng(12)
    for trial in range(400):
        g = float(np.float32(np.exp2(rng.uniform(-30, 30))))
        Sg = np.float32(g) / np.float32(2688.0)
        w = (rng.standard_normal(16) * g * np.exp2(rng.uniform(-14, 0))).astype(np.float32)
        ab = np.abs(w).max()
        k6 = stored_code([(ab / np.float32(6)) / Sg])[0] - 1
        k4 = stored_code([(ab / np.float32(4)) / Sg])[0] - 1
        assert list(orc.rule_candidates(orc.RULE_MAX, w, g)) == [k6]
        assert list(orc.rule_candidates(orc.RULE_FOUR_OVER_SIX, w, g)) == sorted({k6, k4})
        mult = np.arange(0.25, 4.0, 0.1).astype(np.float32)
        ks = stored_code(((mult * ab) / np.float32(6)) / Sg) - 1
        assert list(orc.rule_candidates(orc.RULE_AMAX_SEARCH, w, g)) == sorted(set(ks.tolist()))
        assert list(orc.rule_candidates(orc.RULE_SWEEP, w, g)) == list(range(126))


def test_rule_degenerate_blocks(orc):
    z = np.zeros(16, np.float32)
    w = np.linspace(-1, 1, 16).astype(np.float32)
    for rule in range(4):
        cands = orc.rule_candidates(rule, w, 0.0)
        assert cands[0] == 0
        if rule != orc.RULE_SWEEP:
            assert list(cands) == [0]            # g = 0: every Q is 0
            assert list(orc.rule_candidates(rule, z, 1.0)) == [0]  # zero block: smallest scale
    res = orc.select(orc.RULE_MAX, w.reshape(1, 16), None, np.zeros(1, np.float32), 1, 16)
    assert res["idx"][0] == 0 and res["e1"][0] == float(np.sum(w.astype(np.float64) ** 2))


# ------------------------------------------------ selection by brute force

def brute_select(rule, orc, w16, g, xb=None):
    cands = orc.rule_candidates(rule, w16, g)
    if xb is None:
        E = brute.block_errors_mse(w16, g)
    else:
        E = brute.block_errors_from_x(w16, xb, g)
    sub = E[cands]
    return int(cands[int(np.flatnonzero(sub == sub.min())[0])]), E


@pytest.mark.parametrize("rule", [0, 1, 2, 3])
@pytest.mark.parametrize("weighted", [False, True])
def test_select_matches_brute_force(orc, rule, weighted):
    rng = np.random.default_rng(100 + 10 * rule + weighted)
    c_out, c_in, n_tok = 6, 64, 40
    w = (0.02 * rng.standard_t(4, (c_out, c_in))).astype(np.float32)
    x = (rng.standard_normal((c_in, n_tok)) * np.exp(rng.standard_normal((c_in, 1)))).astype(np.float32)
    g = float(np.abs(w).max())
    amax = np.array([g], np.float32)
    if weighted:
        _, H = orc.hessian(x, c_in, n_tok)
        H = H.reshape(1, c_in // 16, 16, 16)
    else:
        H = None
    res = orc.select(rule, w, H, amax, c_out, c_in)
    nb = c_in // 16
    s = brute.scales(g)
    for f in range(c_out * nb):
        row, b = divmod(f, nb)
        w16 = w[row, 16 * b:16 * b + 16]
        xb = x[16 * b:16 * b + 16] if weighted else None
        k, E = brute_select(rule, orc, w16, g, xb)
        # the oracle reads the fp32-rounded H, the brute force the exact X:
        # errors agree to the rounding of H (relative 2^-24 per entry)
        rtol = 1e-6 if weighted else 1e-12
        if res["e2"][f] - res["e1"][f] > 10 * rtol * res["e2"][f]:
            assert res["idx"][f] == k
        assert np.isclose(res["e1"][f], E[res["idx"][f]], rtol=rtol, atol=0)
        assert res["amax"][f] == np.float32(6) * s[res["idx"][f]]


def test_sweep_rule_with_hessian_equals_the_sweep(orc):
    rng = np.random.default_rng(5)
    c_out, c_in, n_tok = 8, 48, 33
    w = (0.05 * rng.standard_normal((c_out, c_in))).astype(np.float32)
    x = rng.standard_normal((c_in, n_tok)).astype(np.float32)
    _, H = orc.hessian(x, c_in, n_tok)
    amax = np.array([np.abs(w).max()], np.float32)
    a = orc.select(orc.RULE_SWEEP, w, H, amax, c_out, c_in)
    b = orc.sweep(w, H, amax, c_out, c_in)
    for key in ("idx", "e1", "e2", "err", "amax"):
        np.testing.assert_array_equal(a[key], b[key])
    eye = np.broadcast_to(np.eye(16, dtype=np.float32), (c_in // 16, 16, 16)).copy()
    m = orc.select(orc.RULE_SWEEP, w, None, amax, c_out, c_in)
    i = orc.sweep(w, eye, amax, c_out, c_in)
    for key in ("idx", "e1", "e2", "err", "amax"):
        np.testing.assert_array_equal(m[key], i[key])


def test_exhaustive_sweep_is_never_worse_than_a_rule(orc):
    rng = np.random.default_rng(6)
    c_out, c_in, n_tok = 16, 64, 128
    w = (0.02 * rng.standard_t(3, (c_out, c_in))).astype(np.float32)
    x = rng.standard_normal((c_in, n_tok)).astype(np.float32)
    _, H = orc.hessian(x, c_in, n_tok)
    amax = np.array([np.abs(w).max()], np.float32)
    for Hx in (H, None):
        full = orc.select(orc.RULE_SWEEP, w, Hx, amax, c_out, c_in)
        for rule in (1, 2, 3):
            r = orc.select(rule, w, Hx, amax, c_out, c_in)
            assert np.all(full["e1"] <= r["e1"])
        # Four-Over-Six contains the max-scaling candidate.  (The amax search
        # need not: 0.25 + 0.1 i never equals 1.)
        mx = orc.select(orc.RULE_MAX, w, Hx, amax, c_out, c_in)
        fo = orc.select(orc.RULE_FOUR_OVER_SIX, w, Hx, amax, c_out, c_in)
        assert np.all(fo["e1"] <= mx["e1"])


def test_select_is_invariant_to_power_of_two_rescaling(orc):
    """W and g scaled together by 2^m leave every rule's choice unchanged and
    scale its errors by 4^m (all the rule's fp32 steps commute with it)."""
    rng = np.random.default_rng(8)
    c_out, c_in = 8, 32
    w = (0.03 * rng.standard_normal((c_out, c_in))).astype(np.float32)
    amax = np.array([np.abs(w).max()], np.float32)
    for rule in range(4):
        a = orc.select(rule, w, None, amax, c_out, c_in)
        for m in (-9, 5):
            b = orc.select(rule, np.ldexp(w, m), None, np.ldexp(amax, m), c_out, c_in)
            np.testing.assert_array_equal(a["idx"], b["idx"])
            np.testing.assert_array_equal(np.ldexp(a["e1"], 2 * m), b["e1"])
