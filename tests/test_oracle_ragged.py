"""Pins for the oracle's ragged / streaming Hessian accumulation.

Source: "Local-Hessian weight-scale guide" (xxmr.cn/news/266017), section
"Entry API and calibration flow": phase 2 accumulates X^T X per module from
hooked inputs batch by batch (MoE experts see only their routed tokens, so
counts differ and can be zero); phase 3 uses the Hessian normalised by the
token count.

Checked against numpy's Gram matrix of each group's own token rows (fp64),
the running-mean identity (three batches equal one shot over their
concatenation), and the untouched-H rule for groups without tokens.
"""
import numpy as np
import torch


def ragged_case(rng, n_groups, c_in, counts, dtype="f32", ld_extra=0):
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    rows = int(offsets[-1])
    x = rng.standard_normal((rows, c_in + ld_extra)).astype(np.float32)
    x *= np.exp(rng.standard_normal(c_in + ld_extra)).astype(np.float32)
    if dtype == "bf16":
        bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
        return bits, vals, offsets
    return x, x, offsets


def gram_blocks(xv, c_in):
    """Block-diagonal 16x16 blocks of X^T X (fp64) for token-major rows xv."""
    nb = c_in // 16
    x64 = xv[:, :c_in].astype(np.float64)
    return np.stack([x64[:, 16 * b:16 * b + 16].T @ x64[:, 16 * b:16 * b + 16] for b in range(nb)])


def test_ragged_equals_per_group_gram(orc):
    rng = np.random.default_rng(1)
    c_in = 48
    counts = np.array([5, 0, 17, 1, 0, 40, 3])
    for dtype, extra in (("f32", 0), ("bf16", 8)):
        x, xv, off = ragged_case(rng, len(counts), c_in, counts, dtype, extra)
        G, nb = len(counts), c_in // 16
        h_old = rng.standard_normal((G, nb, 16, 16)).astype(np.float32)
        h64, h32, cnt = orc.hessian_ragged(x, c_in, off, h_old, ld_x=c_in + extra)
        assert cnt is None
        h64 = h64.reshape(G, nb, 16, 16)
        h32 = h32.reshape(G, nb, 16, 16)
        for g in range(G):
            if counts[g] == 0:
                np.testing.assert_array_equal(h32[g], h_old[g])  # no tokens: the caller's H stays
                continue
            ref = gram_blocks(xv[off[g]:off[g + 1]], c_in) / counts[g]
            np.testing.assert_allclose(h64[g], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
            np.testing.assert_array_equal(h32[g], h64[g].astype(np.float32))


def test_running_mean_over_batches_equals_one_shot(orc):
    rng = np.random.default_rng(2)
    c_in, G = 32, 5
    nb = c_in // 16
    batches = [rng.integers(0, 30, G) for _ in range(3)]
    batches[0][2] = 0          # an expert that sees no token in the first batch
    for bt in batches:
        bt[4] = 0              # an expert that never sees a token
    h = np.full((G, nb, 16, 16), 7.0, np.float32)  # caller's fallback for empty experts
    counts = np.zeros(G, np.int64)
    seen = [[] for _ in range(G)]
    for bt in batches:
        x, xv, off = ragged_case(rng, G, c_in, bt)
        _, h32, counts = orc.hessian_ragged(x, c_in, off, h, counts=counts)
        h = h32.reshape(G, nb, 16, 16)
        for g in range(G):
            seen[g].append(xv[off[g]:off[g + 1]])
    np.testing.assert_array_equal(counts, np.sum(batches, axis=0))
    for g in range(G):
        allx = np.concatenate(seen[g])
        if len(allx) == 0:
            np.testing.assert_array_equal(h[g], np.float32(7.0))
            continue
        ref = gram_blocks(allx, c_in) / len(allx)
        d = np.sqrt(np.abs(np.einsum("bii->bi", ref)))
        # fp32 storage between batches: a few units of roundoff per batch
        assert np.all(np.abs(h[g] - ref) <= 1e-6 * d[:, :, None] * d[:, None, :] + 1e-30)


def test_ragged_sampled_blocks_match_full(orc):
    rng = np.random.default_rng(3)
    c_in = 64
    counts = np.array([9, 0, 33])
    x, _, off = ragged_case(rng, 3, c_in, counts)
    h_old = np.zeros((3, 4, 16, 16), np.float32)
    _, full, _ = orc.hessian_ragged(x, c_in, off, h_old)
    sel = np.array([1, 5, 10, 11])
    _, part, _ = orc.hessian_ragged(x, c_in, off, h_old, sel=sel)
    np.testing.assert_array_equal(part, full[sel])
