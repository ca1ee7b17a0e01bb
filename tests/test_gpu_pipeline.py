"""GPU parity of lh_calibrate_nvfp4, the whole path in one call (global
amax, normalised local Hessians, the 126-candidate sweep and the fake-quant
of its result), and of its two halves lh_calibrate_prologue and
lh_calibrate_sweep called in turn.

Every output must equal, bit for bit, what the separate calls write
(lh_absmax, lh_accumulate_hessian with alpha = 1/N, lh_scale_sweep_fake_quant),
which the other GPU tests hold to the oracle; the small layer is also
checked against the oracle directly.  Cases cover both code paths: the fused
prologue (channel-major X, contiguous W: one launch for amax and the
Hessian's slices, one for the Hessian's finalisation with the certificates)
with one and with several token slices, and the separate kernels
(token-major X, a W row stride larger than c_in), mixed dtypes, several
groups, more blocks than the finalisation certifies (the certificates then
come from their own pass), no tokens, and the dense 4096 x 4096 layer at
full size.
"""
import numpy as np
import pytest
import torch

import lh_workloads as wl
import oracle
import parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
KEYS = ("amax", "h", "idx", "err", "amax_blk", "w_q", "packed", "scale_e4m3", "global_scale")


@pytest.fixture(scope="module")
def lh():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import nvfp4_scale_calibration_amd as m
    return m


def separate(lh, wd, xd, layout):
    amax = lh.lh_absmax(wd)
    h = lh.lh_accumulate_hessian(xd, layout=layout)
    r = lh.lh_scale_sweep_fake_quant(wd, h, amax, w_q=True, packed=True, scale_e4m3=True, global_scale=True)
    return dict(amax=amax, h=h, idx=r["idx"], err=r["err"], amax_blk=r["amax"], w_q=r["w_q"], packed=r["packed"],
                scale_e4m3=r["scale_e4m3"], global_scale=r["global_scale"])


def compare(lh, wd, xd, layout, what):
    print("case pipeline %s w %s x %s %s" % (what, tuple(wd.shape), tuple(xd.shape), layout), flush=True)
    got = lh.lh_calibrate_nvfp4(wd, xd, layout=layout, packed=True, scale_e4m3=True, global_scale=True)
    halves = lh.lh_calibrate_nvfp4(wd, xd, layout=layout, packed=True, scale_e4m3=True, global_scale=True,
                                   split=True)
    ref = separate(lh, wd, xd, layout)
    torch.cuda.synchronize()
    for name, res in (("one call", got), ("two halves", halves)):
        assert_same(res, ref, "%s, %s" % (what, name))
    return got


def assert_same(got, ref, what):
    for k in KEYS:
        a, b = got[k], ref[k]
        assert a.shape == b.shape, (what, k)
        if a.dtype == torch.float32:
            a, b = a.view(torch.int32), b.view(torch.int32)
        bad = (a != b).nonzero()
        assert bad.numel() == 0, "%s: %s differs from the separate calls at %s" % (what, k, bad[0].tolist())


def test_pipeline_small_layer_against_oracle(lh):
    work = wl.make(1)
    got = compare(lh, work.w.to(DEV), work.x.to(DEV), "channel", work.name)
    G, c_out, c_in, n = work.n_groups, work.c_out, work.c_in, work.n_tok
    w_np, x_np = wl.np_bits(work.w), wl.np_bits(work.x)
    np.testing.assert_array_equal(got["amax"].cpu().numpy(), oracle.absmax(w_np, c_out, c_in, n_groups=G))
    h64, _ = oracle.hessian(x_np, c_in, n, n_groups=G)
    parity.check_hessian(got["h"].cpu().numpy().reshape(-1, 16, 16), h64, "pipeline")
    sel = np.arange(G * c_out * (c_in // 16))
    h_np, amax_np = got["h"].cpu().numpy(), got["amax"].cpu().numpy()
    parity.sweep_against_oracle(w_np, h_np, amax_np, c_out, c_in, G, sel, got["idx"].cpu().numpy(),
                                got["err"].cpu().numpy(), got["amax_blk"].cpu().numpy(), "pipeline")
    parity.fake_quant_against_oracle(w_np, got["idx"].cpu().numpy(), amax_np, c_out, c_in, G, sel,
                                     {k: got[k].cpu().numpy() for k in ("w_q", "packed", "scale_e4m3")}, "pipeline")


@pytest.mark.parametrize("G,c_out,c_in,n,wdt,xdt,layout", [
    (3, 37, 48, 77, "bf16", "bf16", "channel"),      # fused, one token slice
    (2, 70, 112, 4100, "bf16", "bf16", "channel"),   # fused, several slices
    (1, 33, 272, 2500, "f32", "bf16", "channel"),    # fused, mixed dtypes
    (4, 16, 64, 300, "f32", "f32", "channel"),
    (1, 129, 1040, 300, "bf16", "f32", "token"),     # separate kernels
    (2, 5, 16, 1, "f32", "f32", "token"),
    (9, 8, 4096, 40, "bf16", "bf16", "channel"),     # 2304 blocks: certificates in their own pass
])
def test_pipeline_matches_separate_calls(lh, G, c_out, c_in, n, wdt, xdt, layout):
    work = wl.make_custom(c_out, c_in, n, n_groups=G, dtype=wdt, seed=c_out + n, w_dist="t3", x_dist="lognormal")
    x = work.x if xdt == wdt else work.x.to(torch.bfloat16 if xdt == "bf16" else torch.float32)
    xd = x.to(DEV)
    if layout == "token":
        xd = xd.transpose(1, 2).contiguous()
    compare(lh, work.w.to(DEV), xd, layout, "%s/%s" % (wdt, xdt))


def test_pipeline_strided_w_and_no_tokens(lh):
    rng = np.random.default_rng(7)
    c_out, c_in, n = 40, 96, 500
    wbig = torch.from_numpy((rng.standard_normal((c_out, c_in + 32)) * 0.02).astype(np.float32)).to(DEV)
    wd = wbig[:, :c_in]                      # row stride c_in + 32: the separate kernels
    x = torch.from_numpy(rng.standard_normal((1, c_in, n)).astype(np.float32)).to(DEV)
    compare(lh, wd, x, "channel", "strided w")
    got = lh.lh_calibrate_nvfp4(wd.contiguous(), x[:, :, :0], layout="channel")
    torch.cuda.synchronize()
    assert torch.count_nonzero(got["h"]) == 0            # no token: H = 0
    assert torch.all(got["err"] == 0)                     # every block error is then zero
    assert torch.all(got["idx"] == 0)                     # and the lowest index wins


def test_pipeline_dense_4096_full_size(lh):
    work = wl.make(2)
    compare(lh, work.w.to(DEV), work.x.to(DEV), "channel", work.name)


def test_pipeline_halves_reuse_one_workspace(lh):
    """Two layers of different shapes through lh_calibrate_prologue and
    lh_calibrate_sweep with one workspace sized for the larger, in stream
    order, the smaller second: each equal to the separate calls."""
    big = wl.make_custom(64, 512, 700, n_groups=2, dtype="bf16", seed=5, w_dist="t3", x_dist="lognormal")
    small = wl.make_custom(24, 128, 90, n_groups=1, dtype="bf16", seed=6, w_dist="t3", x_dist="lognormal")
    ws = torch.empty(lh.lh_calibrate_workspace_bytes(64, 512, 700, 2), dtype=torch.uint8, device=DEV)
    for work in (big, small):
        print("case halves G=%d c_out=%d c_in=%d" % (work.n_groups, work.c_out, work.c_in), flush=True)
        wd, xd = work.w.to(DEV), work.x.to(DEV)
        G, c_out, c_in = work.n_groups, work.c_out, work.c_in
        nb = c_in // 16
        amax = torch.empty(G, device=DEV)
        h = torch.empty(G, nb, 16, 16, device=DEV)
        idx = torch.empty(G, c_out, nb, dtype=torch.uint8, device=DEV)
        err = torch.empty(G, c_out, nb, device=DEV)
        bam = torch.empty(G, c_out, nb, device=DEV)
        w_q = torch.empty(G, c_out, c_in, device=DEV)
        packed = torch.empty(G, c_out, c_in // 2, dtype=torch.uint8, device=DEV)
        codes = torch.empty(G, c_out, nb, dtype=torch.uint8, device=DEV)
        gsc = torch.empty(G, device=DEV)
        lh.lh_calibrate_prologue(wd, xd, amax, h, ws)
        lh.lh_calibrate_sweep(wd, h, amax, ws, idx, err, bam, w_q, packed, codes, gsc)
        ref = separate(lh, wd, xd, "channel")
        torch.cuda.synchronize()
        got = dict(amax=amax, h=h, idx=idx, err=err, amax_blk=bam, w_q=w_q, packed=packed, scale_e4m3=codes,
                   global_scale=gsc)
        assert_same(got, ref, "halves c_in=%d" % c_in)
