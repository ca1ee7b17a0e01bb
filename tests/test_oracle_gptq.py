"""Pins for the oracle's GPTQ rounding with fixed Local-Hessian scales.

Sources: "Local-Hessian weight-scale guide" (xxmr.cn/news/266017), section
"Combining with GPTQ" (scales from Local-Hessian, GPTQ replaces the
round-to-nearest step); the GPTQ method itself is the published one
(Frantar et al., ICLR 2023): columns in order, each rounding error fed to
the remaining columns through the inverse Hessian.

Checked against: numpy's matrix inverse (U^T U = H'^-1), optimal-brain-
surgeon updates recomputed with an explicit inverse of the remaining
Hessian at every step, the diagonal-Hessian case (no feedback: plain
round-to-nearest, bit for bit), and the method's purpose (lower output
error than round-to-nearest with the same scales).
"""
import numpy as np

import _brute as brute


def layer(rng, c_out, c_in, n, corr=0.6):
    w = (0.02 * rng.standard_t(4, (c_out, c_in))).astype(np.float32)
    z = rng.standard_normal((c_in, n))
    mix = np.eye(c_in) + corr * rng.standard_normal((c_in, c_in)) / np.sqrt(c_in)  # correlated channels
    x = (mix @ z).astype(np.float32)
    return w, x


def test_u_is_the_upper_cholesky_factor_of_the_damped_inverse(orc):
    rng = np.random.default_rng(1)
    _, x = layer(rng, 4, 48, 100)
    h = orc.full_hessian(x, 48, 100).astype(np.float32)
    U = orc.gptq_u(h, 0.01)
    hd = h.astype(np.float64) + 0.01 * np.mean(np.diag(h).astype(np.float64)) * np.eye(48)
    inv = np.linalg.inv(hd)
    np.testing.assert_allclose(U.T @ U, inv, rtol=0, atol=1e-10 * np.abs(inv).max())
    assert np.all(np.tril(U, -1) == 0) and np.all(np.diag(U) > 0)
    eye = orc.gptq_u(np.zeros((16, 16), np.float32))          # no signal at all: H' = I
    np.testing.assert_array_equal(eye, np.eye(16))


def test_sweep_equals_obs_updates_with_explicit_inverses(orc):
    rng = np.random.default_rng(2)
    c_out, c_in, n = 5, 32, 80
    w, x = layer(rng, c_out, c_in, n)
    h = orc.full_hessian(x, c_in, n).astype(np.float32)
    g = float(np.abs(w).max())
    idx = rng.integers(60, 110, (c_out, c_in // 16)).astype(np.uint8)
    q = orc.gptq_sweep(w, idx, g, c_in, U64=orc.gptq_u(h))
    hd = h.astype(np.float64) + 0.01 * np.mean(np.diag(h).astype(np.float64)) * np.eye(c_in)
    s = brute.scales(g)
    for r in range(c_out):
        wr = w[r].astype(np.float64)
        for i in range(c_in):
            qi = brute.quantize(np.array([wr[i]], np.float32), s[idx[r, i // 16]])[0]
            assert qi == q[r, i], "row %d column %d" % (r, i)
            hinv = np.linalg.inv(hd[i:, i:])                     # remaining columns i..n-1
            wr[i + 1:] -= (wr[i] - qi) / hinv[0, 0] * hinv[0, 1:]


def test_diagonal_hessian_is_round_to_nearest(orc):
    rng = np.random.default_rng(3)
    c_out, c_in = 6, 32
    w = (0.02 * rng.standard_normal((c_out, c_in))).astype(np.float32)
    h = np.diag(rng.uniform(0.5, 2.0, c_in)).astype(np.float32)
    g = float(np.abs(w).max())
    idx = rng.integers(50, 120, (c_out, c_in // 16)).astype(np.uint8)
    rtn = orc.fake_quant(w, idx, np.array([g], np.float32), c_out, c_in)["q"].reshape(c_out, c_in)
    U = orc.gptq_u(h)
    assert np.all(U == np.diag(np.diag(U)))
    np.testing.assert_array_equal(orc.gptq_sweep(w, idx, g, c_in, U64=U), rtn)
    np.testing.assert_array_equal(orc.gptq_sweep(w, idx, g, c_in, U32=U.astype(np.float32)), rtn)


def test_gptq_lowers_the_output_error_and_fp32_agrees(orc):
    rng = np.random.default_rng(4)
    c_out, c_in, n = 24, 64, 256
    w, x = layer(rng, c_out, c_in, n)
    h = orc.full_hessian(x, c_in, n).astype(np.float32)
    g = np.abs(w).max()
    _, hb = orc.hessian(x, c_in, n)
    idx = orc.sweep(w, hb, np.array([g], np.float32), c_out, c_in)["idx"].astype(np.uint8).reshape(c_out, -1)
    rtn = orc.fake_quant(w, idx, np.array([g], np.float32), c_out, c_in)["q"].reshape(c_out, c_in)
    U = orc.gptq_u(h)
    q64 = orc.gptq_sweep(w, idx, g, c_in, U64=U)
    q32 = orc.gptq_sweep(w, idx, g, c_in, U32=U.astype(np.float32))
    e_rtn = orc.output_error(w, rtn, h, c_in).sum()
    e_gptq = orc.output_error(w, q64, h, c_in).sum()
    assert e_gptq < 0.9 * e_rtn                # measured: 18% lower on this layer
    assert np.mean(q32 == q64) > 0.97          # fp32 decisions differ only near rounding thresholds
    s = brute.scales(g)                         # every code sits on its block's fixed grid
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    ratio = np.abs(q32).astype(np.float64) / s[np.repeat(idx, 16, axis=1)]   # Q = fl32(r s): within an ulp
    assert np.all(np.min(np.abs(ratio[..., None] - grid), axis=-1) <= 2.0 ** -22 * 6)
