"""Pins for the oracle's approximation diagnostics.

Source: "Local-Hessian weight-scale guide" (xxmr.cn/news/266017), section
"Algorithm principle" (output error ||Delta X||_F^2 = tr(Delta X X^T
Delta^T); the method keeps only the diagonal 16x16 blocks of X X^T) and
"How scaling reshapes the weight distribution" (histogram of W/s, the values
fed to the E2M1 rounding).

Checked against numpy's X X^T / N, the output error computed straight from
the activations ||(q - w) X||^2 / N (never forming H), the H = I special
case, the block-diagonal restriction that reproduces the sweep's own block
errors, and a brute-force histogram with torch's E4M3 decoder.
"""
import numpy as np

import _brute as brute


def test_full_hessian_is_the_gram_matrix(orc):
    rng = np.random.default_rng(1)
    c_in, n = 48, 37
    x = (rng.standard_normal((c_in, n)) * np.exp(rng.standard_normal((c_in, 1)))).astype(np.float32)
    h = orc.full_hessian(x, c_in, n)
    ref = x.astype(np.float64) @ x.astype(np.float64).T / n
    np.testing.assert_allclose(h, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    assert np.array_equal(h, h.T)
    h64_blocks, _ = orc.hessian(x, c_in, n)
    for b in range(c_in // 16):
        np.testing.assert_allclose(h[16 * b:16 * b + 16, 16 * b:16 * b + 16], h64_blocks[b], rtol=1e-12)


def test_output_error_is_the_output_error(orc):
    rng = np.random.default_rng(2)
    c_out, c_in, n = 9, 64, 50
    w = (0.02 * rng.standard_t(3, (c_out, c_in))).astype(np.float32)
    x = rng.standard_normal((c_in, n)).astype(np.float32)
    g = float(np.abs(w).max())
    idx = rng.integers(30, 126, (c_out, c_in // 16)).astype(np.uint8)
    q = orc.fake_quant(w, idx, np.array([g], np.float32), c_out, c_in)["q"].reshape(c_out, c_in)
    h32 = orc.full_hessian(x, c_in, n).astype(np.float32)
    e = orc.output_error(w, q, h32, c_in)
    d = q.astype(np.float64) - w.astype(np.float64)
    direct = np.sum((d @ x.astype(np.float64)) ** 2, axis=1) / n   # ||Delta X||^2 / N per row
    np.testing.assert_allclose(e, direct, rtol=2e-6)                # H rounded to fp32
    eye = np.eye(c_in, dtype=np.float32)
    np.testing.assert_allclose(orc.output_error(w, q, eye, c_in), np.sum(d * d, axis=1), rtol=1e-14)
    # keeping only the diagonal 16x16 blocks gives the sum of the sweep's block errors
    bd = np.zeros_like(h32)
    for b in range(c_in // 16):
        bd[16 * b:16 * b + 16, 16 * b:16 * b + 16] = h32[16 * b:16 * b + 16, 16 * b:16 * b + 16]
    e_bd = orc.output_error(w, q, bd, c_in)
    blocks = bd.reshape(c_in // 16, 16, c_in // 16, 16)[np.arange(c_in // 16), :, np.arange(c_in // 16), :]
    per_block = np.array([[orc.block_errors(w[r, 16 * b:16 * b + 16], blocks[b], g)[idx[r, b]]
                           for b in range(c_in // 16)] for r in range(c_out)])
    np.testing.assert_allclose(e_bd, per_block.sum(1), rtol=1e-12)


def test_scaled_histogram_brute_force(orc):
    rng = np.random.default_rng(3)
    c_out, c_in = 7, 48
    w = (0.03 * rng.standard_normal((c_out, c_in))).astype(np.float32)
    w[0, :16] = 0.0
    g = float(np.abs(w).max())
    idx = rng.integers(0, 126, (c_out, c_in // 16)).astype(np.uint8)
    n_bins, per_unit = 160, np.float32(20.0)
    counts = orc.scaled_histogram(w, idx, g, c_out, c_in, n_bins, per_unit)
    s = brute.scales(g)
    want = np.zeros(n_bins + 1, np.uint64)
    for r in range(c_out):
        for c in range(c_in):
            x = np.float32(abs(w[r, c])) / s[idx[r, c // 16]]
            y = np.float32(x * per_unit)
            want[n_bins if y >= n_bins else int(np.floor(y))] += 1
    np.testing.assert_array_equal(counts, want)
    assert counts.sum() == c_out * c_in
    zero = orc.scaled_histogram(w, idx, 0.0, c_out, c_in, n_bins, per_unit)   # s = 0: every x is 0
    assert zero[0] == c_out * c_in
