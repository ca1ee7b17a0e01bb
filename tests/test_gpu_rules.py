"""GPU parity of the scale-rule variants (lh_select_scales) against the CPU
oracle: the 126-value sweep under the plain weight error (H = I), max
scaling, Four-Over-Six and the amax multiplier search, each with the local
Hessian and with the plain weight error, on ragged shapes, degenerate amax
values and a full-size layer (sampled)."""
import numpy as np
import pytest
import torch

import lh_workloads as wl
import oracle
import parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
RULE_NAMES = {0: "sweep", 1: "max", 2: "four-over-six", 3: "amax-search"}


@pytest.fixture(scope="module")
def lh():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import nvfp4_scale_calibration_amd as m
    return m


def run_rule(lh, rule, wd, h, amax):
    idx, err, bam = lh.lh_select_scales(rule, wd, h, amax)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), err.cpu().numpy(), bam.cpu().numpy()


def check_rule(lh, work, rule, weighted, sel=None, amax_override=None):
    G, c_out, c_in = work.n_groups, work.c_out, work.c_in
    print("case rule=%s weighted=%s %s G=%d %dx%d N=%d %s" % (RULE_NAMES[rule], weighted, work.name, G, c_out, c_in,
                                                              work.n_tok, work.dtype), flush=True)
    wd = work.w.to(DEV)
    amax = lh.lh_absmax(wd) if amax_override is None else torch.tensor(amax_override, dtype=torch.float32, device=DEV)
    h = lh.lh_accumulate_hessian(work.x.to(DEV)) if weighted else None
    idx, err, bam = run_rule(lh, rule, wd, h, amax)
    w_np = wl.np_bits(work.w)
    total = G * c_out * (c_in // 16)
    sel = np.arange(total) if sel is None else sel
    h_np = None if h is None else h.cpu().numpy()
    stats = parity.select_against_oracle(rule, w_np, h_np, amax.cpu().numpy(), c_out, c_in, G, sel, idx, err, bam,
                                         "%s/%s" % (work.name, RULE_NAMES[rule]))
    print("  ok: %s" % stats, flush=True)
    return idx, err, bam


@pytest.mark.parametrize("rule", [0, 1, 2, 3])
@pytest.mark.parametrize("weighted", [True, False])
@pytest.mark.parametrize("G,c_out,c_in,n,dtype", [(3, 37, 48, 77, "bf16"), (1, 129, 1040, 300, "f32")])
def test_rules_ragged(lh, rule, weighted, G, c_out, c_in, n, dtype):
    if rule == 0 and weighted:
        pytest.skip("the Local-Hessian sweep itself is covered by test_gpu_parity")
    work = wl.make_custom(c_out, c_in, n, n_groups=G, dtype=dtype, seed=31 * rule + c_out, w_dist="t3",
                          x_dist="lognormal")
    check_rule(lh, work, rule, weighted)


def test_select_sweep_with_hessian_is_lh_scale_sweep(lh):
    work = wl.make_custom(64, 256, 512, dtype="bf16", seed=4, w_dist="t3")
    wd = work.w.to(DEV)
    amax = lh.lh_absmax(wd)
    h = lh.lh_accumulate_hessian(work.x.to(DEV))
    a = lh.lh_scale_sweep(wd, h, amax)
    b = lh.lh_select_scales(lh.LH_RULE_SWEEP, wd, h, amax)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("rule", [0, 1, 2, 3])
def test_rules_degenerate_amax(lh, rule):
    """amax = 0 (every rule picks 0), amax below the weights (saturating
    scales beyond 448), tiny and huge amax (subnormal candidate scales and
    the definition-based fallback), all-zero blocks."""
    work = wl.make_custom(24, 64, 40, n_groups=5, dtype="f32", seed=9, w_dist="t3")
    w = work.w.clone()
    w[1, 3:7] = 0.0                                  # zero blocks
    work.w = w
    g = np.abs(wl.np_bits(w).reshape(5, -1)).max(1).astype(np.float32)
    amax = np.array([0.0, g[1], g[2] * 0.01, g[3] * 2.0 ** -100, g[4] * 2.0 ** 90], np.float32)
    for weighted in (False, True):
        idx, err, _ = check_rule(lh, work, rule, weighted, amax_override=amax)
        assert np.all(idx.reshape(5, -1)[0] == 0)


@pytest.mark.parametrize("rule", [0, 1, 2, 3])
def test_rules_full_size_sampled(lh, rule):
    work = wl.make(2)
    rng = np.random.default_rng(rule)
    total = work.n_blocks
    sel = np.sort(rng.choice(total, 2000, replace=False))
    for weighted in ((True, False) if rule else (False,)):
        check_rule(lh, work, rule, weighted, sel=sel)
