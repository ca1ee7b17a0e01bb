"""GPU parity of lh_scale_sweep_fake_quant, the sweep and the fake-quant of
its result in one pass.

Checked two ways on the same seeded inputs:
* against the oracle: the sweep's parity rules on every block (small cases)
  or on a sample (full size), and the fake-quant outputs bit-exact given the
  GPU's indices;
* against the two separate calls (lh_scale_sweep, then lh_fake_quant_nvfp4
  with its indices): every output bit for bit, since the fused kernel must
  write exactly what the pair writes.
Cases: the small named layer, ragged shapes (fp32 and bf16, several groups,
block counts off the wave width), an unaligned leading dimension and base
pointer, degenerate amax (zero, far below and far above the weights: rows
whose working exponent is not S_g's), no certificate workspace, weights on
the rounding thresholds of the chosen scale, the dense 4096 x 4096 layer at
full size in the benchmark's launch configuration, and empty problems.
"""
import numpy as np
import pytest
import torch

import lh_workloads as wl
import oracle
import parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FQ = ("w_q", "packed", "scale_e4m3", "global_scale")


@pytest.fixture(scope="module")
def lh():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import nvfp4_scale_calibration_amd as m
    return m


def fused_and_separate(lh, wd, h, amax, workspace=True):
    fused = lh.lh_scale_sweep_fake_quant(wd, h, amax, w_q=True, packed=True, scale_e4m3=True, global_scale=True,
                                         workspace=workspace)
    idx, err, bam = lh.lh_scale_sweep(wd, h, amax, workspace=workspace)
    sep = lh.lh_fake_quant_nvfp4(wd, idx, amax, w_q=True, packed=True, scale_e4m3=True, global_scale=True)
    sep.update(idx=idx, err=err, amax=bam)
    torch.cuda.synchronize()
    return fused, sep


def assert_same(fused, sep, what):
    for k in ("idx", "err", "amax") + FQ:
        a, b = fused[k], sep[k]
        assert a.shape == b.shape, (what, k)
        if a.dtype == torch.float32:
            a, b = a.view(torch.int32), b.view(torch.int32)   # bit patterns (NaN-safe)
        bad = (a != b).nonzero()
        assert bad.numel() == 0, "%s: %s differs from the separate calls at %s" % (what, k, bad[0].tolist())


def against_oracle(w_np, fused, c_out, c_in, G, sel, what):
    h_np = fused["h"].cpu().numpy()
    amax_np = fused["amax_in"].cpu().numpy()
    idx_np = fused["idx"].cpu().numpy()
    stats = parity.sweep_against_oracle(w_np, h_np, amax_np, c_out, c_in, G, sel, idx_np,
                                        fused["err"].cpu().numpy(), fused["amax"].cpu().numpy(), what)
    parity.fake_quant_against_oracle(w_np, idx_np, amax_np, c_out, c_in, G, sel,
                                     {k: fused[k].cpu().numpy() for k in FQ}, what)
    np.testing.assert_array_equal(fused["global_scale"].cpu().numpy(), amax_np / np.float32(2688.0))
    return stats


def run_case(lh, w, x, what, sel=None, workspace=True, amax_scale=None):
    """w [G, c_out, c_in], x channel-major [G, c_in, N] (host tensors)."""
    G, c_out, c_in = w.shape
    print("case fused %s G=%d c_out=%d c_in=%d %s" % (what, G, c_out, c_in, w.dtype), flush=True)
    wd, xd = w.to(DEV), x.to(DEV)
    amax = lh.lh_absmax(wd)
    if amax_scale is not None:
        amax = amax * amax_scale
    h = lh.lh_accumulate_hessian(xd)
    fused, sep = fused_and_separate(lh, wd, h, amax, workspace)
    assert_same(fused, sep, what)
    fused.update(h=h, amax_in=amax)
    w_np = wl.np_bits(w)
    if sel is None:
        sel = np.arange(G * c_out * (c_in // 16))
    stats = against_oracle(w_np, fused, c_out, c_in, G, sel, what)
    print("  ok: %s" % stats, flush=True)
    return stats


def test_fused_small_layer(lh):
    work = wl.make(1)
    stats = run_case(lh, work.w, work.x, work.name)
    assert stats["n"] == 4096


@pytest.mark.parametrize("G,c_out,c_in,n,dtype", [
    (3, 37, 48, 77, "bf16"),
    (2, 5, 16, 1, "f32"),
    (1, 129, 1040, 300, "bf16"),
    (4, 64, 64, 1000, "f32"),
    (2, 70, 112, 513, "bf16"),
])
def test_fused_ragged_shapes(lh, G, c_out, c_in, n, dtype):
    work = wl.make_custom(c_out, c_in, n, n_groups=G, dtype=dtype, seed=c_out + n, w_dist="t3",
                          x_dist="lognormal")
    run_case(lh, work.w, work.x, "ragged")


def test_fused_without_workspace_and_degenerate_amax(lh):
    work = wl.make_custom(40, 96, 200, dtype="bf16", seed=31, w_dist="t3")
    run_case(lh, work.w, work.x, "no workspace", workspace=False)
    for scale in (0.0, 2.0 ** -100, 2.0 ** 90, 0.25):   # zero, far below / above, below max|w| (saturation)
        run_case(lh, work.w, work.x, "amax x %g" % scale, amax_scale=scale)


def test_fused_unaligned_leading_dimension(lh):
    rng = np.random.default_rng(24)
    c_out, c_in, n = 33, 64, 203
    wbig = torch.from_numpy((rng.standard_normal((c_out, c_in + 3)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    x = torch.from_numpy(rng.standard_normal((1, c_in, n)).astype(np.float32)).to(torch.bfloat16)
    wd = wbig.to(DEV)[:, 1:1 + c_in]   # ld = c_in + 3, base offset by one element: scalar loads
    amax = lh.lh_absmax(wd)
    h = lh.lh_accumulate_hessian(x.to(DEV))
    fused, sep = fused_and_separate(lh, wd, h, amax)
    assert_same(fused, sep, "unaligned")
    fused.update(h=h, amax_in=amax)
    w_np = wl.np_bits(wd.cpu().contiguous()).reshape(1, c_out, c_in)
    against_oracle(w_np, fused, c_out, c_in, 1, np.arange(c_out * c_in // 16), "unaligned")


def test_fused_weights_on_rounding_thresholds_of_the_chosen_scale(lh):
    """Blocks planted on candidate k's grid except two weights within 3 ulps
    of a rounding threshold of k (x = 0.25, 0.75, ..., 5), so that k is
    usually the chosen scale and the fused cast of the chosen candidate
    decides those thresholds; every output must equal the separate calls
    and the oracle's fake-quant."""
    rng = np.random.default_rng(41)
    g = np.float32(1.7)
    s = oracle.candidate_scales(g)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    grid = np.array([1.5, 2.0, 3.0, 4.0, 6.0], np.float32)
    blocks, planted = [], []
    for _ in range(1024):
        k = int(rng.integers(20, 126))
        vals = (grid[rng.integers(0, 5, 16)] * s[k]).astype(np.float32)
        for i in rng.choice(16, 2, replace=False):
            base = np.array([mids[rng.integers(0, 7)] * s[k]], np.float32)
            vals[i] = (base.view(np.int32) + np.int32(rng.integers(-3, 4))).view(np.float32)[0]
        vals *= np.where(rng.random(16) < 0.5, -1, 1).astype(np.float32)
        blocks.append(vals)
        planted.append(k)
    c_out, c_in = 128, 128
    w = np.stack(blocks).reshape(c_out, c_in)
    wd = torch.from_numpy(w).to(DEV)
    hd = torch.eye(16, device=DEV).expand(1, c_in // 16, 16, 16).contiguous()
    am = torch.tensor([g], device=DEV)
    fused, sep = fused_and_separate(lh, wd, hd, am)
    assert_same(fused, sep, "thresholds")
    idx = fused["idx"].cpu().numpy().reshape(-1)
    hit = float(np.mean(idx == np.array(planted)))
    print("  chosen scale = planted scale in %.0f%% of blocks" % (100 * hit), flush=True)
    assert hit > 0.5
    fused.update(h=hd, amax_in=am)
    against_oracle(w.reshape(1, c_out, c_in), fused, c_out, c_in, 1, np.arange(idx.size), "thresholds")


def test_fused_dense_4096_full_size(lh):
    """The benchmark's layer and launch configuration: every output equal to
    the separate calls, a sample of blocks against the oracle."""
    work = wl.make(2)
    total = work.n_blocks
    sel = np.sort(np.random.default_rng(2).choice(total, 2000, replace=False))
    run_case(lh, work.w, work.x, work.name, sel=sel)


def test_fused_empty_problems(lh):
    amax = torch.tensor([3.0, 0.5], device=DEV)
    w = torch.zeros((2, 0, 64), dtype=torch.bfloat16, device=DEV)
    h = torch.zeros((2, 4, 16, 16), device=DEV)
    out = lh.lh_scale_sweep_fake_quant(w, h, amax, global_scale=True)
    torch.cuda.synchronize()
    assert out["idx"].numel() == 0 and out["w_q"].numel() == 0
    # no block, but S_g is still written
    np.testing.assert_array_equal(out["global_scale"].cpu().numpy(),
                                  np.array([3.0, 0.5], np.float32) / np.float32(2688.0))
