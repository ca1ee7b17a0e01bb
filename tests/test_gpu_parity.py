"""GPU parity: the HIP library (called through its C ABI via the thin
binding) against the CPU oracle on identical seeded inputs.

Covers: the small named workload end to end; ragged shapes (block counts
that are not multiples of the wave width, token counts that end mid-tile,
several groups, unaligned leading dimensions, both activation layouts, fp32
and bf16); split-token vs one-pass Hessians and their determinism; alpha /
beta chunking and empty token sets; degenerate amax (zero, tiny, huge,
smaller than the weights); all-zero blocks; planted exact solutions;
weights placed on both sides of every rounding threshold.
"""
import numpy as np
import pytest
import torch

import lh_workloads as wl
import oracle
import parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def lh():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import nvfp4_scale_calibration_amd as m
    return m


def _np(t):
    t = t.detach().cpu().contiguous()
    return wl.np_bits(t) if t.dtype in (torch.bfloat16, torch.float32) else t.numpy()


def run_path(lh, w, x, layout="channel", workspace=True):
    """absmax -> Hessian -> sweep -> fake-quant on the GPU."""
    wd, xd = w.to(DEV), x.to(DEV)
    if layout == "token":
        xd = xd.transpose(1, 2).contiguous()
    amax = lh.lh_absmax(wd)
    h = lh.lh_accumulate_hessian(xd, layout=layout, workspace=workspace)
    idx, err, bam = lh.lh_scale_sweep(wd, h, amax)
    fq = lh.lh_fake_quant_nvfp4(wd, idx, amax, w_q=True, packed=True, scale_e4m3=True, global_scale=True)
    torch.cuda.synchronize()
    return dict(amax=amax.cpu().numpy(), h=h.cpu().numpy(), idx=idx.cpu().numpy(), err=err.cpu().numpy(),
                bam=bam.cpu().numpy(), fq={k: v.cpu().numpy() for k, v in fq.items()})


def check_all(lh, work: wl.Workload, layout="channel", n_hess_sel=None, n_sweep_sel=None, seed=0, strict=False):
    G, c_out, c_in, n = work.n_groups, work.c_out, work.c_in, work.n_tok
    nb = c_in // 16
    print("case %s G=%d c_out=%d c_in=%d N=%d %s %s" % (work.name, G, c_out, c_in, n, work.dtype, layout), flush=True)
    got = run_path(lh, work.w, work.x, layout)
    w_np, x_np = wl.np_bits(work.w), wl.np_bits(work.x)
    # global amax: exact
    np.testing.assert_array_equal(got["amax"], oracle.absmax(w_np, c_out, c_in, n_groups=G))
    rng = np.random.default_rng(seed)
    # Hessian
    hsel = np.arange(G * nb) if n_hess_sel is None else np.sort(rng.choice(G * nb, min(n_hess_sel, G * nb), replace=False))
    h64, _ = oracle.hessian(x_np, c_in, n, n_groups=G, sel=hsel)
    parity.check_hessian(got["h"].reshape(G * nb, 16, 16)[hsel], h64, work.name)
    # sweep on the GPU's H
    total = G * c_out * nb
    ssel = np.arange(total) if n_sweep_sel is None else np.sort(rng.choice(total, min(n_sweep_sel, total), replace=False))
    stats = parity.sweep_against_oracle(w_np, got["h"], got["amax"], c_out, c_in, G, ssel, got["idx"], got["err"],
                                        got["bam"], work.name, strict=strict)
    # fake-quant with the GPU's indices: bit-exact
    parity.fake_quant_against_oracle(w_np, got["idx"], got["amax"], c_out, c_in, G, ssel, got["fq"], work.name)
    np.testing.assert_array_equal(got["fq"]["global_scale"], got["amax"] / np.float32(2688.0))
    print("  ok: %s" % stats, flush=True)
    return got, stats


def test_linear_256_end_to_end(lh):
    work = wl.make(1)
    got, stats = check_all(lh, work, strict=True)
    assert stats["n"] == 4096
    parity.note("%s (separate calls, every block): %s" % (work.name, stats))
    # end to end, each side with its own H: report the index agreement
    _, h32 = oracle.hessian(wl.np_bits(work.x), 256, 128)
    res = oracle.sweep(wl.np_bits(work.w), h32, got["amax"], 256, 256)
    agree = float((res["idx"] == got["idx"].reshape(-1)).mean())
    print("  end-to-end index agreement with the oracle's own H: %.5f" % agree)
    assert agree > 0.99


@pytest.mark.parametrize("G,c_out,c_in,n,dtype,layout", [
    (3, 37, 48, 77, "bf16", "channel"),
    (2, 5, 16, 1, "f32", "token"),
    (1, 129, 1040, 300, "bf16", "token"),
    (4, 64, 64, 1000, "f32", "channel"),
    (1, 3, 2064, 2500, "bf16", "channel"),
    (2, 70, 112, 513, "bf16", "token"),
    (1, 5, 48, 3 * 1024 + 37, "f32", "channel"),
])
def test_ragged_shapes(lh, G, c_out, c_in, n, dtype, layout):
    work = wl.make_custom(c_out, c_in, n, n_groups=G, dtype=dtype, seed=c_out + n, w_dist="t3",
                          x_dist="lognormal")
    check_all(lh, work, layout=layout)


@pytest.mark.parametrize("c_in,n", [(256, 8192 + 77), (9600, 2048 + 77), (48, 3 * 1024 + 50)])
def test_hessian_split_vs_one_pass_and_determinism(lh, c_in, n):
    """16 blocks over 8269 tokens: the channel-major plan keeps one slice
    (16-wave workgroups, all resident at once), the token-major one splits;
    600 blocks over 2125 tokens: the channel-major plan splits the tokens in
    two slices of 16-wave workgroups, the second one ragged; 3 blocks over
    3122 tokens: three full steps (an odd count, so the walk ends on one
    slab) from starts 0, 17 and 34 of 48 slabs (the walk wraps), then a
    ragged rest of 50 tokens."""
    work = wl.make_custom(8, c_in, n, dtype="bf16", seed=5, x_dist="lognormal")
    xd = work.x.to(DEV)
    assert lh.lh_hessian_workspace_bytes(c_in, n, 1) > 0
    h_split = lh.lh_accumulate_hessian(xd, workspace=True)
    h_split2 = lh.lh_accumulate_hessian(xd, workspace=True)
    h_one = lh.lh_accumulate_hessian(xd, workspace=False)
    torch.cuda.synchronize()
    assert torch.equal(h_split, h_split2)  # fixed reduction order
    h64, _ = oracle.hessian(wl.np_bits(work.x), c_in, n)
    parity.check_hessian(h_split.cpu().numpy(), h64, "split")
    parity.check_hessian(h_one.cpu().numpy(), h64, "one-pass")
    # token-major gives the same matrix within tolerance
    h_tm = lh.lh_accumulate_hessian(xd.transpose(1, 2).contiguous(), layout="token")
    parity.check_hessian(h_tm.cpu().numpy(), h64, "token-major")


def test_hessian_alpha_beta_chunks_and_empty(lh):
    work = wl.make_custom(4, 64, 600, dtype="bf16", seed=9)
    x = work.x.to(DEV)
    h = lh.lh_accumulate_hessian(x[:, :, :250].contiguous(), alpha=1.0, beta=0.0)
    h = lh.lh_accumulate_hessian(x[:, :, 250:].contiguous(), alpha=1.0, beta=1.0, h=h)
    h64, _ = oracle.hessian(wl.np_bits(work.x), 64, 600, alpha=1.0)
    parity.check_hessian(h.cpu().numpy(), h64, "chunks")
    # strided view (ld > N) without a copy
    hv = lh.lh_accumulate_hessian(x[:, :, 100:400], alpha=1.0)
    hv64, _ = oracle.hessian(np.ascontiguousarray(wl.np_bits(work.x)[:, :, 100:400]), 64, 300, alpha=1.0)
    parity.check_hessian(hv.cpu().numpy(), hv64, "strided")
    # zero tokens: h = beta * h
    h0 = h.clone()
    lh.lh_accumulate_hessian(x[:, :, :0], alpha=1.0, beta=0.5, h=h0)
    torch.cuda.synchronize()
    assert torch.equal(h0, h * 0.5)


def test_hessian_alpha_nan_is_the_normalised_factor(lh):
    """alpha = NaN (the binding's default) makes the library apply
    fl32(1/N) itself: bit-identical to passing that factor explicitly, for
    the local and the full Hessian, and equal to the oracle's 1/N Hessian."""
    work = wl.make_custom(4, 64, 777, dtype="bf16", seed=19)
    x = work.x.to(DEV)
    a = float(np.float32(1.0 / 777))
    h_nan = lh.lh_accumulate_hessian(x, alpha=float("nan"))
    h_exp = lh.lh_accumulate_hessian(x, alpha=a)
    h_def = lh.lh_accumulate_hessian(x)
    f_nan = lh.lh_full_hessian(x, alpha=float("nan"))
    f_exp = lh.lh_full_hessian(x, alpha=a)
    torch.cuda.synchronize()
    assert torch.equal(h_nan.view(torch.int32), h_exp.view(torch.int32))
    assert torch.equal(h_def.view(torch.int32), h_exp.view(torch.int32))
    assert torch.equal(f_nan.view(torch.int32), f_exp.view(torch.int32))
    h64, _ = oracle.hessian(wl.np_bits(work.x), 64, 777)
    parity.check_hessian(h_nan.cpu().numpy(), h64, "alpha NaN")


def _sweep_case(lh, w_np32, h_np, amax_val, what, check_err=True):
    """w_np32: [c_out, c_in] fp32; H [nb,16,16]; explicit amax."""
    c_out, c_in = w_np32.shape
    w = torch.from_numpy(w_np32).to(DEV)
    hd = torch.from_numpy(np.ascontiguousarray(h_np, np.float32)).reshape(1, c_in // 16, 16, 16).to(DEV)
    am = torch.tensor([amax_val], dtype=torch.float32, device=DEV)
    idx, err, bam = lh.lh_scale_sweep(w, hd, am)
    fq = lh.lh_fake_quant_nvfp4(w, idx, am, w_q=True, packed=True, scale_e4m3=True)
    torch.cuda.synchronize()
    am_np = np.array([amax_val], np.float32)
    sel = np.arange(c_out * (c_in // 16))
    stats = parity.sweep_against_oracle(w_np32.reshape(1, c_out, c_in), hd.cpu().numpy(), am_np, c_out, c_in, 1, sel,
                                        idx.cpu().numpy(), err.cpu().numpy() if check_err else None,
                                        bam.cpu().numpy(), what)
    parity.fake_quant_against_oracle(w_np32.reshape(1, c_out, c_in), idx.cpu().numpy(), am_np, c_out, c_in, 1, sel,
                                     {k: v.cpu().numpy() for k, v in fq.items()}, what)
    return idx.cpu().numpy().reshape(-1), err.cpu().numpy().reshape(-1), stats


def _spd(rng, nb, n=64, scale=1.0):
    x = rng.standard_normal((nb * 16, n)).astype(np.float32) * np.float32(scale)
    _, h32 = oracle.hessian(x, nb * 16, n)
    return h32


def test_degenerate_amax_and_zero_blocks(lh):
    rng = np.random.default_rng(21)
    h = _spd(rng, 4)
    w = (rng.standard_normal((8, 64)) * 0.02).astype(np.float32)
    w[0, :16] = 0.0           # all-zero block
    w[1, 16:32] = -0.0
    g = float(np.abs(w).max())
    idx, err, _ = _sweep_case(lh, w, h, g, "zero-blocks")
    assert idx[0] == 0 and err[0] == 0.0 and idx[4 + 1] == 0
    _sweep_case(lh, w, h, 0.0, "amax=0")                     # every scale 0: Q = 0, index 0
    _sweep_case(lh, w, h, g * 0.3, "amax<max|w|")           # saturation region
    for scale in (2.0 ** -70, 2.0 ** -100, 1e-33, 2.0 ** 90, 1e30):
        ws = (w.astype(np.float64) * scale).astype(np.float32)
        gs = float(np.abs(ws).max())
        hs = h * np.float32(1.0 / scale) if scale > 1 else h  # keep E inside fp32 range
        _sweep_case(lh, ws, hs, gs, "scaled %g" % scale, check_err=(2.0 ** -40 <= scale <= 2.0 ** 100))  # tiny weights: E underflows fp32


def test_level1_scan_stop_on_saturating_blocks(lh):
    """Blocks built around the stop of the top-down level-1 scan: leading
    elements that saturate together or far apart, one dominant weight,
    equal magnitudes, weights on exact multiples of 6 x a candidate scale,
    log-uniform magnitudes over twenty octaves, and channel scales that make
    the bound elements (largest H_ee w^2) differ from the largest |w|; two
    global amax values (the weights' own, and a third of it so that whole
    blocks sit in the saturation region)."""
    rng = np.random.default_rng(26)
    c_out, nb = 192, 8
    w = (rng.standard_normal((c_out, nb, 16)) * 0.01).astype(np.float32)
    sign = np.where(rng.random((c_out, 16)) < 0.5, -1.0, 1.0).astype(np.float32)
    big = np.exp(rng.uniform(-3, 0, c_out)).astype(np.float32)
    w[:, 0, :2] = big[:, None] * sign[:, :2]                                  # two equal leaders
    w[:, 1, 0] = big * sign[:, 0]
    w[:, 1, 1] = big / np.float32(37.0) * sign[:, 1]                          # leaders far apart
    w[:, 2, 5] = big * np.float32(4.0) * sign[:, 5]                           # one dominant weight
    w[:, 3, :] = big[:, None] * sign                                          # sixteen equal magnitudes
    w[:, 5, :] = (np.exp2(rng.uniform(-20, 0, (c_out, 16))) * sign).astype(np.float32)
    w[:, 6, :] = w[:, 6, :] * np.float32(1e-3)                                # far below the amax
    w[:, 7, :] = (rng.standard_t(2, (c_out, 16)) * 0.02).astype(np.float32)
    g = float(np.abs(w).max())
    s = oracle.candidate_scales(np.float32(g))                                # 6 * s[125] is g (to an ulp)
    k = rng.integers(0, 126, c_out)
    w[:, 4, :4] = (np.float32(6.0) * s[k])[:, None] * sign[:, :4]             # exactly 6 x a candidate
    w = w.reshape(c_out, nb * 16)
    x = rng.standard_normal((nb * 16, 96)).astype(np.float32)
    x *= np.exp(rng.standard_normal((nb * 16, 1))).astype(np.float32)         # channel scales
    _, h = oracle.hessian(x, nb * 16, 96)
    _sweep_case(lh, w, h, g, "scan-stop")
    _sweep_case(lh, w, h, g / 3.0, "scan-stop amax/3")
    _sweep_case(lh, w, _spd(rng, nb), g, "scan-stop white H")


def test_planted_solutions(lh):
    rng = np.random.default_rng(22)
    c_out, c_in = 64, 128
    h = _spd(rng, c_in // 16)
    g = np.float32(0.37)
    s = oracle.candidate_scales(g)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    w = np.empty((c_out, c_in), np.float32)
    want = rng.integers(0, 126, (c_out, c_in // 16))
    for r in range(c_out):
        for b in range(c_in // 16):
            codes = rng.integers(0, 8, 16)
            codes[0], codes[1] = 1, 7
            rng.shuffle(codes)
            sign = np.where(rng.random(16) < 0.5, -1, 1).astype(np.float32)
            w[r, 16 * b:16 * b + 16] = (sign * grid[codes]) * s[want[r, b]]
    g_act = float(np.abs(w).max())
    assert g_act <= g * (1 + 1e-6)  # 6 * s_125 is within one ulp of g
    idx, err, _ = _sweep_case(lh, w, h, float(g), "planted")
    np.testing.assert_array_equal(idx, want.reshape(-1))
    assert np.all(err == 0.0)


def test_weights_on_every_rounding_threshold(lh):
    """Weights within a few ulps of x = 0.25, 0.75, ..., 5 times a candidate
    scale, so that fl32(|w| / s) falls below, on and above each threshold."""
    rng = np.random.default_rng(23)
    g = np.float32(1.7)
    s = oracle.candidate_scales(g)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    rows = []
    for t in range(512):
        k = int(rng.integers(0, 126))
        m = mids[rng.integers(0, 7, 16)]
        base = (m * s[k]).astype(np.float32)
        off = rng.integers(-3, 4, 16).astype(np.int32)
        v = base.view(np.int32) + off
        vals = v.view(np.float32) * np.where(rng.random(16) < 0.5, -1, 1).astype(np.float32)
        rows.append(vals)
    w = np.stack(rows).reshape(64, 128).astype(np.float32)
    w[0, 0] = g  # keep the global amax
    h = _spd(rng, 8)
    _sweep_case(lh, w, h, float(g), "thresholds")
    # fake-quant with random indices: every cast bit-exact
    c_out, c_in = w.shape
    idx = torch.from_numpy(rng.integers(0, 126, (1, c_out, c_in // 16)).astype(np.uint8)).to(DEV)
    wd = torch.from_numpy(w).to(DEV)
    am = torch.tensor([g], device=DEV)
    fq = lh.lh_fake_quant_nvfp4(wd, idx, am, w_q=True, packed=True, scale_e4m3=True)
    torch.cuda.synchronize()
    parity.fake_quant_against_oracle(w.reshape(1, c_out, c_in), idx.cpu().numpy(), np.array([g], np.float32),
                                     c_out, c_in, 1, np.arange(c_out * c_in // 16),
                                     {k: v.cpu().numpy() for k, v in fq.items()}, "thresholds-fq")


def test_unaligned_leading_dimensions(lh):
    rng = np.random.default_rng(24)
    c_out, c_in, n = 33, 64, 203
    wbig = torch.from_numpy((rng.standard_normal((c_out, c_in + 3)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    xbig = torch.from_numpy(rng.standard_normal((c_in, n + 5)).astype(np.float32)).to(torch.bfloat16)
    wd = wbig.to(DEV)[:, 1:1 + c_in]   # ld = c_in + 3, base offset by one element
    xd = xbig.to(DEV)[:, 2:2 + n]
    amax = lh.lh_absmax(wd)
    h = lh.lh_accumulate_hessian(xd)
    idx, err, bam = lh.lh_scale_sweep(wd, h, amax)
    fq = lh.lh_fake_quant_nvfp4(wd, idx, amax, w_q=True, packed=True)
    torch.cuda.synchronize()
    w_np = wl.np_bits(wd.cpu().contiguous()).reshape(1, c_out, c_in)
    x_np = wl.np_bits(xd.cpu().contiguous())
    np.testing.assert_array_equal(amax.cpu().numpy(), oracle.absmax(w_np, c_out, c_in))
    h64, _ = oracle.hessian(x_np, c_in, n)
    parity.check_hessian(h.cpu().numpy(), h64, "unaligned")
    sel = np.arange(c_out * c_in // 16)
    parity.sweep_against_oracle(w_np, h.cpu().numpy(), amax.cpu().numpy(), c_out, c_in, 1, sel,
                                idx.cpu().numpy(), err.cpu().numpy(), bam.cpu().numpy(), "unaligned")
    parity.fake_quant_against_oracle(w_np, idx.cpu().numpy(), amax.cpu().numpy(), c_out, c_in, 1, sel,
                                     {k: v.cpu().numpy() for k, v in fq.items()}, "unaligned")


def test_empty_problems(lh):
    w = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    amax = lh.lh_absmax(w)
    torch.cuda.synchronize()
    assert amax.item() == 0.0
    h = torch.zeros((1, 4, 16, 16), device=DEV)
    idx, err, bam = lh.lh_scale_sweep(w, h, amax)
    assert idx.numel() == 0


@pytest.mark.timeout(900)
@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_full_size_benchmarked_pair_every_block(lh, n):
    """The named workloads at full size through the two calls the benchmark
    times (lh_calibrate_prologue, then lh_calibrate_sweep, with the
    benchmark's buffers), every output of every block against the oracle:
    global amax bit-exact, every Hessian block, every block's index, error
    and amax under the near-tie rules with no block passing only through the
    fp32 allowance, and Q, nibbles and E4M3 codes bit-exact.  The separate
    calls (lh_absmax, lh_accumulate_hessian, lh_fake_quant_nvfp4) and the
    sweep without certificates (lh_scale_sweep without a workspace, which
    evaluates without the prologue's skip bounds) must give the same bits."""
    work = wl.make(n)
    G, c_out, c_in, N = work.n_groups, work.c_out, work.c_in, work.n_tok
    nb = c_in // 16
    print("case full-size %s G=%d c_out=%d c_in=%d N=%d" % (work.name, G, c_out, c_in, N), flush=True)
    w, x = work.w.to(DEV), work.x.to(DEV)
    amax = torch.empty(G, dtype=torch.float32, device=DEV)
    h = torch.empty((G, nb, 16, 16), dtype=torch.float32, device=DEV)
    cws = torch.empty(lh.lh_calibrate_workspace_bytes(c_out, c_in, N, G), dtype=torch.uint8, device=DEV)
    idx = torch.empty((G, c_out, nb), dtype=torch.uint8, device=DEV)
    err = torch.empty((G, c_out, nb), dtype=torch.float32, device=DEV)
    bam = torch.empty((G, c_out, nb), dtype=torch.float32, device=DEV)
    wq = torch.empty((G, c_out, c_in), dtype=torch.float32, device=DEV)
    packed = torch.empty((G, c_out, c_in // 2), dtype=torch.uint8, device=DEV)
    codes = torch.empty((G, c_out, nb), dtype=torch.uint8, device=DEV)
    gscale = torch.empty(G, dtype=torch.float32, device=DEV)
    lh.lh_calibrate_prologue(w, x, amax, h, cws)
    lh.lh_calibrate_sweep(w, h, amax, cws, idx, err, bam, wq, packed, codes, gscale)
    # the separate calls and the certificate-free sweep: the same bits
    amax2 = lh.lh_absmax(w)
    h2 = lh.lh_accumulate_hessian(x)
    i2, e2, b2 = lh.lh_scale_sweep(w, h, amax, workspace=False)
    fq2 = lh.lh_fake_quant_nvfp4(w, idx, amax, w_q=True, packed=True, scale_e4m3=True, global_scale=True)
    torch.cuda.synchronize()
    for name, a, b in (("amax", amax, amax2), ("h", h, h2), ("idx", idx, i2), ("err", err, e2), ("amax_blk", bam, b2),
                       ("w_q", wq, fq2["w_q"]), ("packed", packed, fq2["packed"]),
                       ("scale_e4m3", codes, fq2["scale_e4m3"]), ("global_scale", gscale, fq2["global_scale"])):
        if a.dtype == torch.float32:
            a, b = a.view(torch.int32), b.view(torch.int32)
        assert torch.equal(a, b), "%s: %s differs between the benchmarked pair and the separate calls" % (work.name,
                                                                                                          name)
    del amax2, h2, i2, e2, b2, fq2, x
    got = dict(amax=amax.cpu().numpy(), h=h.cpu().numpy(), idx=idx.cpu().numpy(), err=err.cpu().numpy(),
               bam=bam.cpu().numpy(), fq=dict(w_q=wq.cpu().numpy(), packed=packed.cpu().numpy(),
                                              scale_e4m3=codes.cpu().numpy()))
    gs = gscale.cpu().numpy()
    w_np, x_np = wl.np_bits(work.w), wl.np_bits(work.x)
    np.testing.assert_array_equal(got["amax"], oracle.absmax(w_np, c_out, c_in, n_groups=G))
    np.testing.assert_array_equal(gs, got["amax"] / np.float32(2688.0))
    h64, _ = oracle.hessian(x_np, c_in, N, n_groups=G)
    hdev = parity.check_hessian(got["h"], h64, work.name)
    del h64, x_np
    sel = np.arange(G * c_out * nb, dtype=np.int64)
    stats = parity.sweep_against_oracle(w_np, got["h"], got["amax"], c_out, c_in, G, sel, got["idx"], got["err"],
                                        got["bam"], work.name, strict=True)
    parity.fake_quant_against_oracle(w_np, got["idx"], got["amax"], c_out, c_in, G, sel, got["fq"], work.name)
    print("  ok %s: every block; Hessian worst normalised deviation %.3g; %s" % (work.name, hdev, stats), flush=True)
    parity.note("%s (benchmarked pair, every block): Hessian worst |dH|/sqrt(Hii Hjj) %.3g; %s" % (work.name, hdev,
                                                                                                 stats))


def test_sweep_waves_walking_several_chunks_with_a_partial_last_chunk(lh):
    """Enough input blocks that each wave of the sweep walks several chunks
    of 64 rows of its block (3 x 1024 blocks: waves take every 11th of the
    16 chunks), and 1000 rows, so the last chunk holds 40 rows and 24 idle
    lanes.  The whole path (certificates from the prologue) is sampled
    against the oracle, every output of the fused sweep on the sample, and
    the certificate-free sweep of the same H must give the same bits."""
    work = wl.make_custom(1000, 16384, 64, n_groups=3, dtype="bf16", seed=77, w_dist="t3", x_dist="lognormal")
    G, c_out, c_in = work.n_groups, work.c_out, work.c_in
    nb = c_in // 16
    print("case multi-chunk G=%d c_out=%d c_in=%d" % (G, c_out, c_in), flush=True)
    wd, xd = work.w.to(DEV), work.x.to(DEV)
    res = lh.lh_calibrate_nvfp4(wd, xd, packed=True, scale_e4m3=True, global_scale=True, split=True)
    # the same H through the certificate-free path (in-kernel Gershgorin): same results
    idx2, err2, bam2 = lh.lh_scale_sweep(wd, res["h"], res["amax"])
    torch.cuda.synchronize()
    for a, b in ((res["idx"], idx2), (res["err"], err2), (res["amax_blk"], bam2)):
        assert torch.equal(a, b)
    w_np = wl.np_bits(work.w)
    amax_np, h_np = res["amax"].cpu().numpy(), res["h"].cpu().numpy()
    sel = np.sort(np.random.default_rng(77).choice(G * c_out * nb, 4000, replace=False))
    idx_np = res["idx"].cpu().numpy()
    stats = parity.sweep_against_oracle(w_np, h_np, amax_np, c_out, c_in, G, sel, idx_np, res["err"].cpu().numpy(),
                                        res["amax_blk"].cpu().numpy(), "multi-chunk")
    parity.fake_quant_against_oracle(w_np, idx_np, amax_np, c_out, c_in, G, sel,
                                     {k: res[k].cpu().numpy() for k in ("w_q", "packed", "scale_e4m3")}, "multi-chunk")
    print("  ok: %s" % stats, flush=True)


def test_skipping_never_changes_results(lh):
    """The sweep with the certificate pre-pass, with the on-the-fly
    certificate, and on Hessians that admit no certificate (rank-deficient,
    indefinite) returns bit-identical indices, errors and amax, and matches
    the oracle."""
    rng = np.random.default_rng(25)
    c_out, c_in = 96, 256
    nb = c_in // 16
    w = torch.from_numpy((rng.standard_t(4, size=(c_out, c_in)) * 0.02).astype(np.float32)).to(DEV)
    amax = lh.lh_absmax(w)
    cases = []
    for n_tok in (512, 3):  # well-conditioned; rank 3 < 16 (singular)
        x = torch.from_numpy(rng.standard_normal((c_in, n_tok)).astype(np.float32)).to(DEV)
        cases.append(("N=%d" % n_tok, lh.lh_accumulate_hessian(x)))
    h_ind = cases[0][1].clone()
    h_ind[:, :, 3, 3] = -h_ind[:, :, 3, 3]  # indefinite: no certificate
    cases.append(("indefinite", h_ind))
    for name, h in cases:
        outs = [lh.lh_scale_sweep(w, h, amax, workspace=ws) for ws in (True, False)]
        torch.cuda.synchronize()
        for a, b in zip(outs[0], outs[1]):
            assert torch.equal(a, b), name
        sel = np.arange(c_out * nb)
        w_np = w.cpu().numpy().reshape(1, c_out, c_in)
        parity.sweep_against_oracle(w_np, h.cpu().numpy(), amax.cpu().numpy(), c_out, c_in, 1, sel,
                                    outs[0][0].cpu().numpy(), outs[0][1].cpu().numpy(), outs[0][2].cpu().numpy(),
                                    name)


@pytest.mark.parametrize("copies", [1, 7])   # 320 blocks (one workgroup per block), 2240 (one lane per tau)
def test_certificate_is_a_valid_eigenvalue_bound(lh, copies):
    """The per-block skip certificate left in the sweep's workspace is a
    lower bound on the smallest eigenvalue of C = D^-1/2 S D^-1/2
    (S = (H + H^T)/2, D = diag S), checked in fp64 with numpy: 0 where no
    bound is certified (singular, indefinite, zero diagonal), else at least
    0.02 and within 1/16 + 2e-3 below the best grid value q/16 that the
    exact eigenvalue allows (or at the Gershgorin bound)."""
    rng = np.random.default_rng(26)
    hs = []
    for n_tok in (2000, 100, 40, 17, 3):
        x = rng.standard_normal((64 * 16, n_tok)) * np.exp(rng.standard_normal((64 * 16, 1)))
        hs.append(oracle.hessian(x.astype(np.float32), 64 * 16, n_tok)[1].reshape(64, 16, 16))
    h = np.concatenate(hs)
    h[3, 5, 5] = -h[3, 5, 5]            # indefinite
    h[7, 2, :] = h[7, :, 2] = 0.0       # zero row: diagonal not positive
    h[9] *= np.float32(2.0 ** 60)       # scale leaves C unchanged
    h[11, 0, 1] += np.float32(0.3) * np.sqrt(h[11, 0, 0] * h[11, 1, 1])   # non-symmetric
    h = np.ascontiguousarray(np.tile(h, (copies, 1, 1)))
    nb = h.shape[0]
    c_in = nb * 16
    w = torch.from_numpy((rng.standard_normal((4, c_in)) * 0.02).astype(np.float32)).to(DEV)
    hd = torch.from_numpy(h).reshape(1, nb, 16, 16).to(DEV)
    amax = lh.lh_absmax(w)
    ws = torch.full((lh.lh_sweep_workspace_bytes(c_in, 1) // 4,), -1.0, dtype=torch.float32, device=DEV)
    lh.lh_scale_sweep(w, hd, amax, workspace=ws.view(torch.uint8))
    torch.cuda.synchronize()
    cert = ws.cpu().numpy()
    n_pos = 0
    for b in range(nb):
        s = (h[b].astype(np.float64) + h[b].T.astype(np.float64)) / 2
        d = np.diag(s)
        if not np.all(d > 0):
            assert cert[b] == 0.0, b
            continue
        c = s / np.sqrt(np.outer(d, d))
        lam = np.linalg.eigvalsh(c).min()
        assert cert[b] == 0.0 or 0.02 <= cert[b] <= lam, (b, cert[b], lam)
        rho = (np.abs(c).sum(1) - 1).max()
        best = max(np.floor(16 * lam - 1e-3) / 16, 1 - rho - 1e-3)   # what the grid and Gershgorin allow
        if best >= 0.1 and 35 * 2.0 ** -24 * (1 + rho) / best <= 2.0 ** -12:
            assert cert[b] >= best - 1 / 16 - 2e-3, (b, cert[b], lam)
        n_pos += cert[b] > 0
    print("  %d of %d blocks certified" % (n_pos, nb), flush=True)
    assert n_pos > nb // 4
