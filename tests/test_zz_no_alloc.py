"""lh_calibrate_nvfp4_noalloc, the whole path without a workspace argument
(its scratch is a device array inside the library), called through the C ABI:
every output must equal lh_calibrate_nvfp4 with a caller-provided workspace,
bit for bit, on two calls in a row (the second with a smaller layer, so the
array holds the first call's data when the second starts), and a layer whose
scratch would exceed the array is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import lh_workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
KEYS = ("amax", "h", "idx", "err", "amax_blk", "w_q", "packed", "scale_e4m3", "global_scale")


@pytest.fixture(scope="module")
def lh():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import nvfp4_scale_calibration_amd as m
    return m


def _same(a, b, what):
    for k in KEYS:
        x, y = a[k], b[k]
        assert x.shape == y.shape, (what, k)
        if x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), "%s: %s differs from lh_calibrate_nvfp4 with a workspace" % (what, k)


def test_noalloc_matches_workspace_call_twice_then_smaller(lh):
    cases = [wl.make_custom(300, 4096, 1500, n_groups=2, dtype="bf16", seed=41, w_dist="t3", x_dist="lognormal"),
             wl.make_custom(70, 272, 333, n_groups=1, dtype="bf16", seed=42, w_dist="t3", x_dist="lognormal")]
    for work in cases:
        print("case noalloc G=%d c_out=%d c_in=%d N=%d" % (work.n_groups, work.c_out, work.c_in, work.n_tok),
              flush=True)
        w, x = work.w.to(DEV), work.x.to(DEV)
        got = lh.lh_calibrate_nvfp4_noalloc(w, x, packed=True, scale_e4m3=True, global_scale=True)
        ref = lh.lh_calibrate_nvfp4(w, x, packed=True, scale_e4m3=True, global_scale=True)
        torch.cuda.synchronize()
        _same(got, ref, work.name)


def test_noalloc_full_size_mlp_down(lh):
    """The benchmark's largest layer (17 MiB of scratch) fits the array."""
    work = wl.make(5)
    w, x = work.w.to(DEV), work.x.to(DEV)
    got = lh.lh_calibrate_nvfp4_noalloc(w, x, packed=True, scale_e4m3=True, global_scale=True)
    ref = lh.lh_calibrate_nvfp4(w, x, packed=True, scale_e4m3=True, global_scale=True)
    torch.cuda.synchronize()
    _same(got, ref, work.name)
