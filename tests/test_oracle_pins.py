"""Pins for the CPU oracle: each test checks it against something other than
itself - a library decoder, a golden fixture with its citation, a closed form
computed from the activations, a special case that reduces to a textbook
routine, an exact invariance, or a planted solution.

Sources: "Local-Hessian weight-scale guide" (xxmr.cn/news/266017), sections
"What is Local-Hessian" (NVFP4 format, 126 FP8 candidates, E2M1 range [-6,6])
and "Algorithm principle" (Q = Cast(W/s)*s, E_b = Delta_b X_b X_b^T
Delta_b^T, kernel interface); "ModelOpt overview" (linlog.top/article/1517),
"Local-Hessian" (126 candidates, block-diagonal approximation).
"""
import numpy as np
import pytest
import torch

import _brute as brute

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def f32(x):
    return np.float32(x)


def bf16_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_vals(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()


# ---------------------------------------------------------------- format facts

def test_golden_format_facts(orc):
    fmt = brute.load_format()
    vals = np.array([orc.e4m3_value(c) for c in range(1, 127)])
    assert int(fmt["n_candidates"]) == len(vals) == len(brute.e4m3_candidates())
    assert np.all(vals > 0) and np.all(np.isfinite(vals))
    assert vals.max() == fmt["e4m3_max"]
    assert brute.GRID.max() == fmt["e2m1_max"]
    assert int(fmt["block_size"]) == 16


def test_e4m3_table_matches_library_decoder(orc):
    ours = np.array([orc.e4m3_value(c) for c in range(1, 127)])
    lib = brute.e4m3_candidates().astype(np.float64)
    np.testing.assert_array_equal(ours, lib)
    assert np.all(np.diff(ours) > 0)
    assert ours[0] == 2.0 ** -9 and ours[7] == 2.0 ** -6 and ours[125] == 448.0
    # code 0x7F is the only non-finite positive code: the set has exactly 126
    assert np.isnan(torch.tensor([0x7F], dtype=torch.uint8).view(torch.float8_e4m3fn).float().item())


def test_largest_candidate_reproduces_max_scaling(orc):
    rng = np.random.default_rng(1)
    for g in np.exp(rng.uniform(-30, 30, 3000)).astype(np.float32):
        s = orc.candidate_scales(g)
        assert np.all(np.diff(s) > 0)
        # 6 * s_125 within one ulp of g: the top candidate is per-tensor max scaling
        assert abs(6.0 * float(s[125]) - float(g)) <= np.spacing(g)
        np.testing.assert_array_equal(s, brute.scales(g))


# ---------------------------------------------------------------- E2M1 cast

def _expected_code_at(mid_index, where):
    lower, upper = mid_index, mid_index + 1
    if where < 0:
        return lower
    if where > 0:
        return upper
    return upper if upper % 2 == 0 else lower


def test_e2m1_thresholds_nextafter(orc):
    for i, m in enumerate(brute.MIDPOINTS):
        m32 = f32(m)
        assert float(m32) == m  # thresholds are exact in fp32
        for where, x in ((-1, np.nextafter(m32, f32(-np.inf))), (0, m32), (1, np.nextafter(m32, f32(np.inf)))):
            assert orc.e2m1_code(x) == _expected_code_at(i, where), (m, where)
            assert brute.cast_codes(np.array([x], np.float32))[0] == _expected_code_at(i, where)


def test_e2m1_grid_points_and_saturation(orc):
    for c, v in enumerate(brute.GRID):
        assert orc.e2m1_code(v) == c
        assert orc.e2m1_value(c) == v if hasattr(orc, "e2m1_value") else True
    for x in (6.0, 6.5, 7.0, 1e30, np.inf):
        assert orc.e2m1_code(x) == 7
    assert orc.e2m1_code(0.0) == 0
    assert orc.e2m1_code(1e-40) == 0


def test_cast_through_division_near_every_threshold(orc):
    """w placed so that fl32(|w|/s) falls just below / at / above each
    rounding threshold, for many scales; the expected code is the golden
    threshold table applied to the IEEE fp32 quotient."""
    rng = np.random.default_rng(2)
    s_all = np.exp(rng.uniform(-20, 5, 150)).astype(np.float32)
    for s in s_all:
        for m in brute.MIDPOINTS:
            w0 = f32(f32(m) * s)
            cands = [w0]
            for _ in range(4):
                cands.append(np.nextafter(cands[-1], f32(np.inf)))
            lo = w0
            for _ in range(4):
                lo = np.nextafter(lo, f32(-np.inf))
                cands.append(lo)
            for w in cands:
                x = np.abs(np.float32(w)) / s
                want = brute.cast_codes(np.array([x], np.float32))[0]
                q, code = orc.quantize(w, s)
                assert code == want, (w, s, x)
                assert q == brute.quantize(np.array([w]), s)[0]


def test_cast_symmetric_and_grid_reproduced(orc):
    rng = np.random.default_rng(3)
    for s in np.exp(rng.uniform(-15, 3, 200)).astype(np.float32):
        for v in brute.GRID:
            w = f32(f32(v) * s)
            q, _ = orc.quantize(w, s)
            assert q == w  # values already on the grid x s come back unchanged
            qn, _ = orc.quantize(-w, s)
            assert qn == (-w if w != 0 else 0.0)
        for w in rng.normal(0, 10 * s, 20).astype(np.float32):
            q1, c1 = orc.quantize(w, s)
            q2, c2 = orc.quantize(-w, s)
            assert c1 == c2 and q2 == (-q1 if q1 != 0 else 0.0)
    q, c = orc.quantize(f32(0.3), f32(0.0))
    assert q == 0.0 and c == 0
    q, _ = orc.quantize(f32(-1e-3), f32(1.0))
    assert q == 0.0 and not np.signbit(q)  # -0 written as +0


# ---------------------------------------------------------------- Hessian

@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hessian_equals_gram_matrix(orc, layout, dtype):
    rng = np.random.default_rng(4)
    G, c_in, n = 2, 48, 37
    x = rng.standard_normal((G, c_in, n)).astype(np.float32)
    if dtype == "bf16":
        bits = bf16_bits(x)
        x = bf16_vals(bits)
    xs = x if layout == 0 else np.ascontiguousarray(x.transpose(0, 2, 1))
    arr = xs if dtype == "f32" else bf16_bits(xs)
    h64, h32 = orc.hessian(arr, c_in, n, layout=layout, n_groups=G)
    h64 = h64.reshape(G, c_in // 16, 16, 16)
    for g in range(G):
        for b in range(c_in // 16):
            xb = x[g, 16 * b:16 * b + 16].astype(np.float64)
            ref = (xb @ xb.T) / n
            np.testing.assert_allclose(h64[g, b], ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(h32, h64.reshape(h32.shape).astype(np.float32))


def test_hessian_invariants(orc):
    rng = np.random.default_rng(5)
    c_in, n = 32, 50
    x = rng.standard_normal((c_in, n)).astype(np.float32)
    h64, _ = orc.hessian(x, c_in, n)
    for hb, xb in zip(h64, (x[:16], x[16:])):
        np.testing.assert_array_equal(hb, hb.T)
        ev = np.linalg.eigvalsh(hb)
        assert ev.min() >= -1e-12 * np.trace(hb)
        np.testing.assert_allclose(np.trace(hb), (xb.astype(np.float64) ** 2).sum() / n, rtol=1e-12)
    # X -> -X leaves H unchanged; X -> 2^m X multiplies it by 4^m exactly
    hn, _ = orc.hessian(-x, c_in, n)
    np.testing.assert_array_equal(hn, h64)
    h8, _ = orc.hessian(x * np.float32(8.0), c_in, n)
    np.testing.assert_array_equal(h8, h64 * 64.0)


def test_hessian_single_token_and_orthogonal_rows(orc):
    rng = np.random.default_rng(6)
    x1 = rng.standard_normal((16, 1)).astype(np.float32)
    h, _ = orc.hessian(x1, 16, 1)
    np.testing.assert_array_equal(h[0], np.outer(x1[:, 0].astype(np.float64), x1[:, 0]))
    # rows of a 16x16 Hadamard matrix are orthogonal: H = (16/16) I exactly
    had = np.array([[1.0]])
    while had.shape[0] < 16:
        had = np.block([[had, had], [had, -had]])
    h, _ = orc.hessian(had.astype(np.float32), 16, 16)
    np.testing.assert_array_equal(h[0], np.eye(16))


def test_hessian_chunks_equal_one_shot(orc):
    rng = np.random.default_rng(7)
    c_in, n1, n2 = 32, 40, 23
    x = rng.standard_normal((c_in, n1 + n2)).astype(np.float32)
    _, one = orc.hessian(x, c_in, n1 + n2, alpha=1.0)
    _, a = orc.hessian(np.ascontiguousarray(x[:, :n1]), c_in, n1, alpha=1.0)
    _, ab = orc.hessian(np.ascontiguousarray(x[:, n1:]), c_in, n2, alpha=1.0, beta=1.0, h_old=a)
    np.testing.assert_allclose(ab, one, rtol=2e-7, atol=1e-6)
    # zero tokens: h = beta * h_old
    _, z = orc.hessian(np.zeros((c_in, 1), np.float32), c_in, 0, alpha=1.0, beta=0.5, h_old=one)
    np.testing.assert_array_equal(z, (one.astype(np.float64) * 0.5).astype(np.float32))


# ---------------------------------------------------------------- sweep errors

def _int_activations(rng, c_in, n):
    # small integers and a power-of-two token count: X X^T / N is exact in fp32
    return rng.integers(-3, 4, size=(c_in, n)).astype(np.float32)


def test_block_errors_equal_output_error_closed_form(orc):
    rng = np.random.default_rng(8)
    c_in, n = 32, 64
    x = _int_activations(rng, c_in, n)
    _, h32 = orc.hessian(x, c_in, n)
    for t in range(12):
        w = rng.standard_normal(c_in).astype(np.float32) * f32(0.05)
        g = f32(np.abs(w).max() * rng.uniform(1.0, 3.0))
        for b in range(2):
            e_or = orc.block_errors(w[16 * b:16 * b + 16], h32[b], g)
            e_bf = brute.block_errors_from_x(w[16 * b:16 * b + 16], x[16 * b:16 * b + 16], g)
            np.testing.assert_allclose(e_or, e_bf, rtol=1e-12, atol=1e-18)
            assert brute.argmin_lowest(e_or) == brute.argmin_lowest(e_bf)


def test_sweep_matches_brute_force_random_activations(orc):
    rng = np.random.default_rng(9)
    c_out, c_in, n = 6, 48, 80
    x = rng.standard_normal((c_in, n)).astype(np.float32)
    w = (rng.standard_t(3, size=(c_out, c_in)) * 0.02).astype(np.float32)
    g = orc.absmax(w, c_out, c_in)
    _, h32 = orc.hessian(x, c_in, n)
    res = orc.sweep(w, h32, g, c_out, c_in)
    nb = c_in // 16
    for f in range(c_out * nb):
        r, b = divmod(f, nb)
        e_bf = brute.block_errors_from_x(w[r, 16 * b:16 * b + 16], x[16 * b:16 * b + 16], g[0])
        srt = np.sort(e_bf)
        if srt[1] - srt[0] >= 1e-5 * srt[1]:  # H's fp32 rounding only matters inside near-ties
            assert res["idx"][f] == brute.argmin_lowest(e_bf)
        np.testing.assert_allclose(res["e1"][f], e_bf.min(), rtol=1e-6)
        assert res["e2"][f] >= res["e1"][f]
        assert res["err"][f] == np.float32(res["e1"][f])
        s = orc.candidate_scales(g[0])
        assert res["amax"][f] == np.float32(np.float32(6.0) * s[res["idx"][f]])


def test_identity_hessian_is_mse_sweep(orc):
    rng = np.random.default_rng(10)
    eye = np.eye(16, dtype=np.float32)
    for _ in range(20):
        w = rng.standard_normal(16).astype(np.float32) * f32(0.03)
        g = f32(np.abs(w).max() * rng.uniform(1, 4))
        np.testing.assert_allclose(orc.block_errors(w, eye, g), brute.block_errors_mse(w, g), rtol=1e-13, atol=1e-20)


def test_single_token_error_is_squared_projection(orc):
    rng = np.random.default_rng(11)
    for _ in range(20):
        xv = rng.integers(-4, 5, 16).astype(np.float32)
        H = np.outer(xv, xv).astype(np.float32)  # exact
        w = rng.standard_normal(16).astype(np.float32) * f32(0.03)
        g = f32(np.abs(w).max())
        e = orc.block_errors(w, H, g)
        s = brute.scales(g)
        for k in range(0, 126, 7):
            dw = brute.quantize(w, s[k]).astype(np.float64) - w
            assert e[k] == pytest.approx(float(xv.astype(np.float64) @ dw) ** 2, rel=1e-9, abs=1e-20)


def test_error_invariances(orc):
    rng = np.random.default_rng(12)
    x = rng.standard_normal((16, 40)).astype(np.float32)
    _, h = orc.hessian(x, 16, 40)
    h = h[0]
    w = rng.standard_normal(16).astype(np.float32) * f32(0.02)
    g = f32(np.abs(w).max() * 1.3)
    e = orc.block_errors(w, h, g)
    p = rng.permutation(16)
    np.testing.assert_allclose(orc.block_errors(w[p], h[np.ix_(p, p)], g), e, rtol=1e-12)
    np.testing.assert_array_equal(orc.block_errors(-w, h, g), e)
    # H * 2^m: errors scale by 2^m exactly, argmin identical
    np.testing.assert_array_equal(orc.block_errors(w, h * f32(4.0), g), e * 4.0)
    # W and g scaled together by 2^m: errors scale by 4^m exactly
    np.testing.assert_array_equal(orc.block_errors(w * f32(8.0), h, g * f32(8.0)), e * 64.0)
    # any positive rescaling of H leaves the argmin (outside near-ties) unchanged
    e3 = orc.block_errors(w, h * f32(3.7), g)
    if np.sort(e)[1] - e.min() > 1e-5 * np.sort(e)[1]:
        assert brute.argmin_lowest(e3) == brute.argmin_lowest(e)


def test_chosen_error_never_exceeds_max_scaling(orc):
    rng = np.random.default_rng(13)
    c_out, c_in, n = 16, 64, 48
    x = rng.standard_normal((c_in, n)).astype(np.float32)
    w = (rng.standard_t(4, size=(c_out, c_in)) * 0.02).astype(np.float32)
    g = orc.absmax(w, c_out, c_in)
    _, h = orc.hessian(x, c_in, n)
    res = orc.sweep(w, h, g, c_out, c_in)
    cands = brute.e4m3_candidates()
    sg = f32(g[0]) / f32(2688.0)
    nb = c_in // 16
    for f in range(c_out * nb):
        r, b = divmod(f, nb)
        wb = w[r, 16 * b:16 * b + 16]
        e = orc.block_errors(wb, h[b], g[0])
        assert res["e1"][f] <= e[125]
        # the scale max calibration would pick: E4M3 RNE of amax_b / 6 / S_g
        want = f32(f32(np.abs(wb).max()) / f32(6.0)) / sg
        c8 = torch.tensor([min(float(want), 448.0)]).to(torch.float8_e4m3fn).float().item()
        c8 = max(c8, float(cands[0]))
        kmax = int(np.flatnonzero(cands == np.float32(c8))[0])
        assert res["e1"][f] <= e[kmax]


def test_zero_block_and_zero_amax(orc):
    h = np.eye(16, dtype=np.float32)
    e = orc.block_errors(np.zeros(16, np.float32), h, f32(0.5))
    assert np.all(e == 0.0)
    w = np.zeros((1, 16), np.float32)
    res = orc.sweep(w, h.reshape(1, 16, 16), np.array([0.5], np.float32), 1, 16)
    assert res["idx"][0] == 0 and res["e1"][0] == 0.0
    fq = orc.fake_quant(w, res["idx"].astype(np.uint8), np.array([0.5], np.float32), 1, 16)
    assert np.all(fq["q"] == 0) and not np.any(np.signbit(fq["q"]))
    # g = 0: every scale is 0, every Q is 0, all errors equal, index 0
    w = np.full((1, 16), 0.25, np.float32)
    res = orc.sweep(w, h.reshape(1, 16, 16), np.array([0.0], np.float32), 1, 16)
    assert res["idx"][0] == 0 and res["e1"][0] == pytest.approx(16 * 0.0625)


def test_planted_solution_is_unique_zero_error_minimiser(orc):
    rng = np.random.default_rng(14)
    x = rng.standard_normal((16, 64)).astype(np.float32)
    _, h = orc.hessian(x, 16, 64)
    for t in range(40):
        g = f32(np.exp(rng.uniform(-6, 2)))
        s = orc.candidate_scales(g)
        kp = int(rng.integers(0, 126))
        codes = rng.integers(0, 8, 16)
        codes[rng.integers(0, 16)] = 1  # a +-0.5
        j = rng.integers(0, 16)
        while codes[j] == 1 and np.count_nonzero(codes == 1) == 1:
            j = rng.integers(0, 16)
        codes[j] = 7  # a +-6
        sign = np.where(rng.random(16) < 0.5, -1.0, 1.0)
        w = (sign * brute.GRID[codes]).astype(np.float32) * s[kp]
        w = w.astype(np.float32)
        res = orc.sweep(w.reshape(1, 16), h, np.array([g], np.float32), 1, 16)
        assert res["idx"][0] == kp and res["e1"][0] == 0.0 and res["e2"][0] > 0.0


# ---------------------------------------------------------------- fake-quant

def test_fake_quant_consistent_with_sweep(orc):
    rng = np.random.default_rng(15)
    c_out, c_in, n = 8, 64, 32
    x = rng.standard_normal((c_in, n)).astype(np.float32)
    w = (rng.standard_normal((c_out, c_in)) * 0.02).astype(np.float32)
    g = orc.absmax(w, c_out, c_in)
    _, h = orc.hessian(x, c_in, n)
    res = orc.sweep(w, h, g, c_out, c_in)
    idx = res["idx"].astype(np.uint8)
    fq = orc.fake_quant(w, idx, g, c_out, c_in)
    s = orc.candidate_scales(g[0])
    nb = c_in // 16
    for f in range(c_out * nb):
        r, b = divmod(f, nb)
        q = fq["q"][f].astype(np.float64)
        sk = float(s[idx[f]])
        ratio = np.abs(q) / sk
        nearest = brute.GRID[np.abs(ratio[:, None] - brute.GRID[None, :]).argmin(1)]
        np.testing.assert_allclose(ratio, nearest, rtol=1e-6, atol=0)
        dw = q - w[r, 16 * b:16 * b + 16].astype(np.float64)
        np.testing.assert_allclose(dw @ h[b].astype(np.float64) @ dw, res["e1"][f], rtol=1e-12, atol=1e-20)
        assert fq["code"][f] == idx[f] + 1
        nib = np.stack([fq["packed"][f] & 15, fq["packed"][f] >> 4], 1).reshape(16)
        val = brute.GRID[nib & 7] * np.where(nib & 8, -1.0, 1.0)
        qq = (np.abs(val).astype(np.float32) * np.float32(sk)).astype(np.float32) * np.sign(val)
        np.testing.assert_array_equal(qq + 0.0, fq["q"][f])
    # idempotent: quantising Q with the same indices returns Q
    qfull = fq["q"].reshape(c_out, nb, 16).reshape(c_out, c_in)
    fq2 = orc.fake_quant(qfull, idx, g, c_out, c_in)
    np.testing.assert_array_equal(fq2["q"], fq["q"])


def test_absmax_bf16_and_groups(orc):
    rng = np.random.default_rng(16)
    w = rng.standard_normal((3, 5, 32)).astype(np.float32)
    bits = bf16_bits(w)
    vals = bf16_vals(bits)
    got = orc.absmax(bits, 5, 32, n_groups=3)
    np.testing.assert_array_equal(got, np.abs(vals).reshape(3, -1).max(1))
