"""GPU parity of GPTQ rounding with fixed Local-Hessian scales
(lh_gptq_prepare, lh_gptq_quantize) against the CPU oracle.

* U (upper factor of the damped inverse Hessian): upper with a positive
  diagonal and exact zeros below; close to the oracle's fp64 factor of the
  same fp32 H, within the first-order fp32 bound of a Cholesky-based
  inverse, 8 n u cond(H') relative to the row's largest entry.
* Quantised weights: the rounding decisions are taken in fp32 on both sides
  (the kernel's precision), every update one fused multiply-add in column
  order, so with the GPU's own U fed to the oracle the results are bit-exact.
* A diagonal Hessian reproduces round-to-nearest (the fake-quant kernel)
  bit for bit, and GPTQ lowers the layer output error.
"""
import numpy as np
import pytest
import torch

import lh_workloads as wl
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
U32 = 2.0 ** -24


@pytest.fixture(scope="module")
def lh():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import nvfp4_scale_calibration_amd as m
    return m


def correlated(c_out, c_in, n, seed, dtype):
    rng = np.random.default_rng(seed)
    w = (0.02 * rng.standard_t(4, (c_out, c_in))).astype(np.float32)
    mix = np.eye(c_in) + 0.6 * rng.standard_normal((c_in, c_in)) / np.sqrt(c_in)
    x = (mix @ rng.standard_normal((c_in, n))).astype(np.float32)
    wt = torch.from_numpy(w)
    xt = torch.from_numpy(x)
    if dtype == "bf16":
        wt, xt = wt.to(torch.bfloat16), xt.to(torch.bfloat16)
    return wt, xt


def run(lh, w, x):
    wd, xd = w.to(DEV), x.to(DEV)
    amax = lh.lh_absmax(wd)
    h = lh.lh_accumulate_hessian(xd)
    idx, _, _ = lh.lh_scale_sweep(wd, h, amax)
    hf = lh.lh_full_hessian(xd)
    u = lh.lh_gptq_prepare(hf)
    q = lh.lh_gptq_quantize(wd, idx, amax, u)
    rtn = lh.lh_fake_quant_nvfp4(wd, idx, amax, w_q=True)["w_q"]
    e_g = lh.lh_output_error(wd, q, hf)
    e_r = lh.lh_output_error(wd, rtn, hf)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in dict(amax=amax, idx=idx, hf=hf, u=u, q=q, rtn=rtn, e_g=e_g,
                                                 e_r=e_r).items()}


def check_u(u_gpu, hf):
    n = hf.shape[0]
    assert np.all(np.tril(u_gpu, -1) == 0) and np.all(np.diag(u_gpu) > 0)
    ref = oracle.gptq_u(hf)
    hd = hf.astype(np.float64) + 0.01 * np.mean(np.diag(hf).astype(np.float64)) * np.eye(n)
    cond = np.linalg.cond(hd)
    tol = 8 * n * U32 * cond
    rel = np.abs(u_gpu - ref) / np.abs(ref).max(axis=1, keepdims=True)
    print("  U: cond %.3g, worst row-relative deviation %.3g (bound %.3g)" % (cond, rel.max(), tol), flush=True)
    assert rel.max() <= tol


@pytest.mark.parametrize("c_out,c_in,n,dtype", [(37, 64, 200, "f32"), (129, 272, 600, "bf16"),
                                                 (70, 1040, 2000, "bf16")])
def test_gptq_ragged(lh, c_out, c_in, n, dtype):
    print("case gptq %dx%d N=%d %s" % (c_out, c_in, n, dtype), flush=True)
    w, x = correlated(c_out, c_in, n, c_in, dtype)
    got = run(lh, w, x)
    check_u(got["u"], got["hf"][0])
    w_np = wl.np_bits(w)
    q_or = oracle.gptq_sweep(w_np, got["idx"][0], float(got["amax"][0]), c_in, U32=got["u"])
    mism = got["q"].view(np.uint32) != q_or.view(np.uint32)
    assert not mism.any(), "GPTQ mismatch at %s: gpu %r oracle %r" % (
        np.argwhere(mism)[0], got["q"][mism][0], q_or[mism][0])
    assert got["e_g"].sum() < got["e_r"].sum()
    print("  output error: GPTQ %.6g vs round-to-nearest %.6g" % (got["e_g"].sum(), got["e_r"].sum()), flush=True)


def test_gptq_diagonal_hessian_is_round_to_nearest(lh):
    rng = np.random.default_rng(5)
    c_out, c_in = 40, 128
    w = torch.from_numpy((0.02 * rng.standard_normal((c_out, c_in))).astype(np.float32)).to(DEV)
    amax = lh.lh_absmax(w)
    idx = torch.from_numpy(rng.integers(40, 120, (1, c_out, c_in // 16)).astype(np.uint8)).to(DEV)
    hf = torch.diag(torch.from_numpy(rng.uniform(0.5, 2.0, c_in).astype(np.float32))).to(DEV)
    u = lh.lh_gptq_prepare(hf)
    q = lh.lh_gptq_quantize(w, idx, amax, u)
    rtn = lh.lh_fake_quant_nvfp4(w, idx, amax, w_q=True)["w_q"]
    torch.cuda.synchronize()
    assert torch.count_nonzero(torch.triu(u, 1)) == 0
    assert torch.equal(q, rtn.reshape(c_out, c_in))


def test_gptq_dense_4096_sampled_rows(lh):
    work = wl.make(2)
    print("case gptq dense-4096", flush=True)
    got = run(lh, work.w[0], work.x[0])
    c_in = work.c_in
    rows = np.sort(np.random.default_rng(1).choice(work.c_out, 6, replace=False))
    q_or = oracle.gptq_sweep(wl.np_bits(work.w)[0], got["idx"][0], float(got["amax"][0]), c_in, U32=got["u"],
                             rows=rows)
    assert np.array_equal(got["q"][rows].view(np.uint32), q_or.view(np.uint32))
    hf = got["hf"][0]
    assert np.all(np.tril(got["u"], -1) == 0) and np.all(np.diag(got["u"]) > 0)
    # residual of the factor on a few rows: (U^T U H')[r] = e_r
    hd = hf.astype(np.float64) + 0.01 * np.mean(np.diag(hf).astype(np.float64)) * np.eye(c_in)
    u64 = got["u"].astype(np.float64)
    for r in rows[:3]:
        res = (u64[:, r] @ u64) @ hd
        res[r] -= 1.0
        assert np.abs(res).max() < 1e-2
    print("  output error: GPTQ %.6g vs round-to-nearest %.6g" % (got["e_g"].sum(), got["e_r"].sum()), flush=True)
    assert got["e_g"].sum() < got["e_r"].sum()
