"""GPU parity of the approximation diagnostics (lh_full_hessian,
lh_output_error, lh_scaled_histogram) against the CPU oracle, on ragged
shapes, several groups, both dtypes, and the dense-4096 layer (sampled rows).

Tolerances (derived from the fp32 arithmetic):
  * full Hessian: each entry is an fp32 sum of N exact bf16/fp32 products,
    |dH_ij| <= N u sum_t |x_it x_jt| <= N u sqrt(H_ii H_jj) * N/N, so the
    Hessian rule |dH| <= 1e-3 sqrt(H_ii H_jj) holds for N up to ~16k;
  * output error: T = d H (fp32, K = c_in terms) then a 64-term row dot
    and an ordered sum over c_in/64 tiles: |de| <= (c_in + 64 + c_in/64) u S
    with S = sum |d_n| |H_nk| |d_k|;
  * histogram: integer counts, bit-exact.
"""
import numpy as np
import pytest
import torch

import lh_workloads as wl
import oracle
import parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
U = 2.0 ** -24


@pytest.fixture(scope="module")
def lh():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import nvfp4_scale_calibration_amd as m
    return m


def check_full_hessian(h_gpu, x_np_g, c_in, n, rows=None):
    if rows is None:
        ref = oracle.full_hessian(x_np_g, c_in, n)
        got = h_gpu
    else:
        xv = x_np_g if x_np_g.dtype == np.float32 else (x_np_g.astype(np.uint32) << 16).view(np.float32)
        x64 = xv.astype(np.float64)
        ref = x64[rows] @ x64.T / n
        got = h_gpu[rows]
        dref = np.einsum("ij,ij->i", x64, x64) / n
        scale = np.sqrt(np.abs(dref[rows]))[:, None] * np.sqrt(np.abs(dref))[None, :]
        bad = np.abs(got - ref) > 1e-3 * scale + 1e-30
        assert not bad.any(), "full Hessian mismatch in sampled rows: %d entries" % bad.sum()
        return
    d = np.sqrt(np.abs(np.diag(ref)))
    bad = np.abs(got - ref) > 1e-3 * d[:, None] * d[None, :] + 1e-30
    assert not bad.any(), "full Hessian mismatch: %d entries, first %s" % (bad.sum(), np.argwhere(bad)[0])


def check_output_error(err_gpu, w_np_g, q_np_g, h32, c_in, rows):
    e = oracle.output_error(w_np_g, q_np_g, h32, c_in, rows=rows)
    wv = w_np_g if w_np_g.dtype == np.float32 else (w_np_g.astype(np.uint32) << 16).view(np.float32)
    d = np.abs(q_np_g[rows].astype(np.float64) - wv[rows].astype(np.float64))
    S = np.einsum("ri,ij,rj->r", d, np.abs(h32.astype(np.float64)), d)
    tol = (c_in + 64 + c_in // 64 + 8) * U * S + 1e-30
    bad = np.abs(err_gpu[rows] - e) > tol
    assert not bad.any(), "output error mismatch at rows %s: gpu %s oracle %s tol %s" % (
        rows[bad][:4], err_gpu[rows][bad][:4], e[bad][:4], tol[bad][:4])
    return e


def run_layer(lh, work):
    wd, xd = work.w.to(DEV), work.x.to(DEV)
    amax = lh.lh_absmax(wd)
    h = lh.lh_accumulate_hessian(xd)
    idx, err, _ = lh.lh_scale_sweep(wd, h, amax)
    q = lh.lh_fake_quant_nvfp4(wd, idx, amax, w_q=True)["w_q"]
    hf = lh.lh_full_hessian(xd)
    e_full = lh.lh_output_error(wd, q, hf)
    counts = lh.lh_scaled_histogram(wd, idx, amax)
    torch.cuda.synchronize()
    return dict(amax=amax.cpu().numpy(), h=h.cpu().numpy(), idx=idx.cpu().numpy(), err=err.cpu().numpy(),
                q=q.cpu().numpy(), hf=hf.cpu().numpy(), e_full=e_full.cpu().numpy(), counts=counts.cpu().numpy())


@pytest.mark.parametrize("G,c_out,c_in,n,dtype", [(2, 37, 48, 77, "f32"), (1, 129, 272, 300, "bf16"),
                                                   (3, 70, 1040, 130, "bf16")])
def test_diagnostics_ragged(lh, G, c_out, c_in, n, dtype):
    work = wl.make_custom(c_out, c_in, n, n_groups=G, dtype=dtype, seed=c_in + n, w_dist="t3", x_dist="lognormal")
    print("case diag G=%d %dx%d N=%d %s" % (G, c_out, c_in, n, dtype), flush=True)
    got = run_layer(lh, work)
    w_np, x_np = wl.np_bits(work.w), wl.np_bits(work.x)
    for g in range(G):
        check_full_hessian(got["hf"][g], x_np[g], c_in, n)
        # its diagonal blocks are the local Hessians
        for b in range(c_in // 16):
            blk = got["hf"][g][16 * b:16 * b + 16, 16 * b:16 * b + 16]
            d = np.sqrt(np.abs(np.diag(blk)))
            assert np.all(np.abs(blk - got["h"][g, b]) <= 2e-3 * d[:, None] * d[None, :] + 1e-30)
        check_output_error(got["e_full"][g], w_np[g], got["q"][g], got["hf"][g], c_in, np.arange(c_out))
        counts = oracle.scaled_histogram(w_np[g], got["idx"][g], float(got["amax"][g]), c_out, c_in, 160, 20.0)
        np.testing.assert_array_equal(got["counts"][g].astype(np.uint64), counts)


@pytest.mark.parametrize("G,c_in,n", [(8, 1040, 304), (4, 784, 77), (1, 4096, 96), (2, 2048, 40), (1, 4096, 256)])
def test_full_hessian_large_tiles(lh, G, c_in, n):
    """Shapes whose full Hessian runs on the large-tile kernel (at least 128
    tiles of 256 x 256 in the square): a ragged last tile row and column, a
    partial last 64-token
    step with 16-byte aligned rows (304 = 4 x 64 + 48, 96 = 64 + 32),
    fewer tokens than one step (40), whole steps only (256), unaligned rows
    (N = 77), and a whole 4096-channel layer; every entry against the
    oracle."""
    work = wl.make_custom(16, c_in, n, n_groups=G, dtype="bf16", seed=c_in + 7 * n, w_dist="t3", x_dist="lognormal")
    print("case full Hessian G=%d c_in=%d N=%d" % (G, c_in, n), flush=True)
    hf = lh.lh_full_hessian(work.x.to(DEV)).cpu().numpy()
    x_np = wl.np_bits(work.x)
    for g in range(G):
        check_full_hessian(hf[g], x_np[g], c_in, n)


@pytest.mark.parametrize("G,c_in,n,pad", [(1, 5120, 96, 0), (3, 2608, 200, 0), (3, 2608, 200, 1), (3, 2608, 40, 0),
                                          (1, 4096, 200, 0), (2, 2048, 72, 1)])
def test_full_hessian_syrk(lh, G, c_in, n, pad):
    """The large-tile kernel computes the lower triangle of output tiles and
    mirrors it: 256 x 256 tiles (5120; 2608 = 10 x 256 + 48, a ragged last
    tile row, several groups) or 192 x 192 tiles where that takes cheaper
    rounds (4096 = 21 x 192 + 64; 2048 in two groups); partial last K steps
    (or only one, N = 40), and H rows that are not 16-byte aligned (pad = 1:
    row stride c_in + 1, scalar mirrored stores).  Every entry against the
    oracle; entries outside the diagonal tiles (of either size) are exact
    mirrors."""
    work = wl.make_custom(16, c_in, n, n_groups=G, dtype="bf16", seed=c_in + 3 * n, w_dist="t3", x_dist="lognormal")
    print("case full Hessian syrk G=%d c_in=%d N=%d pad=%d" % (G, c_in, n, pad), flush=True)
    hbuf = torch.full((G, c_in, c_in + pad), float("nan"), dtype=torch.float32, device=DEV)
    hv = hbuf[:, :, :c_in]
    lh.lh_full_hessian(work.x.to(DEV), h=hv)
    hf = hv.cpu().numpy()
    x_np = wl.np_bits(work.x)
    t256, t192 = np.arange(c_in) // 256, np.arange(c_in) // 192
    off = (t256[:, None] != t256[None, :]) & (t192[:, None] != t192[None, :])
    for g in range(G):
        assert np.isfinite(hf[g]).all()
        np.testing.assert_array_equal(hf[g][off], hf[g].T[off])
        check_full_hessian(hf[g], x_np[g], c_in, n)
    if pad:
        assert torch.isnan(hbuf[:, :, c_in:]).all()  # the padding column is never written


def test_diagnostics_zero_weights_and_no_tokens(lh):
    work = wl.make_custom(16, 32, 0, dtype="f32", seed=1, w_dist="zeros")
    wd = work.w.to(DEV)
    amax = lh.lh_absmax(wd)
    idx, _, _ = lh.lh_scale_sweep(wd, torch.eye(16, device=DEV).expand(1, 2, 16, 16).contiguous(), amax)
    hf = lh.lh_full_hessian(work.x.to(DEV))
    q = lh.lh_fake_quant_nvfp4(wd, idx, amax, w_q=True)["w_q"]
    e = lh.lh_output_error(wd, q, hf)
    counts = lh.lh_scaled_histogram(wd, idx, amax)
    torch.cuda.synchronize()
    assert torch.count_nonzero(hf) == 0 and torch.count_nonzero(e) == 0
    assert counts[0, 0].item() == 16 * 32 and counts.sum().item() == 16 * 32


def test_diagnostics_dense_4096_sampled(lh):
    work = wl.make(2)
    c_in, n = work.c_in, work.n_tok
    print("case diag dense-4096", flush=True)
    got = run_layer(lh, work)
    w_np, x_np = wl.np_bits(work.w)[0], wl.np_bits(work.x)[0]
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(c_in, 12, replace=False))
    check_full_hessian(got["hf"][0], x_np, c_in, n, rows=rows)
    orows = np.sort(rng.choice(work.c_out, 8, replace=False))
    e = check_output_error(got["e_full"][0], w_np, got["q"][0], got["hf"][0], c_in, orows)
    # the block-diagonal part the sweep minimised is a share of the full error
    e_bd = got["err"][0].astype(np.float64).sum(axis=1)
    print("  rows %s: full %s block-diagonal %s" % (orows[:4], e[:4], e_bd[orows][:4]), flush=True)
    counts = oracle.scaled_histogram(w_np, got["idx"][0], float(got["amax"][0]), work.c_out, c_in, 160, 20.0)
    np.testing.assert_array_equal(got["counts"][0].astype(np.uint64), counts)


@pytest.mark.parametrize("n_bins,bins_per_unit", [(3000, 400.0), (1023, 150.0)])
def test_histogram_many_bins(lh, n_bins, bins_per_unit):
    """Bin counts too large for a copy of the bins per wave (one shared copy
    per workgroup) and at the four-copy limit, against the oracle; two
    groups, a ragged row count."""
    work = wl.make_custom(70, 96, 8, n_groups=2, dtype="bf16", seed=17, w_dist="t3")
    wd = work.w.to(DEV)
    amax = lh.lh_absmax(wd)
    h = torch.eye(16, device=DEV).expand(2, 6, 16, 16).contiguous()
    idx, _, _ = lh.lh_scale_sweep(wd, h, amax)
    counts = lh.lh_scaled_histogram(wd, idx, amax, n_bins=n_bins, bins_per_unit=bins_per_unit)
    torch.cuda.synchronize()
    w_np = wl.np_bits(work.w)
    idx_np, amax_np, got = idx.cpu().numpy(), amax.cpu().numpy(), counts.cpu().numpy()
    for g in range(2):
        ref = oracle.scaled_histogram(w_np[g], idx_np[g], float(amax_np[g]), 70, 96, n_bins, bins_per_unit)
        np.testing.assert_array_equal(got[g].astype(np.uint64), ref)
        assert int(got[g].sum()) == 70 * 96
