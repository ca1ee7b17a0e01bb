"""The whole path (the separate calls, the fused sweep + fake-quant call and
the two halves lh_calibrate_prologue and lh_calibrate_sweep) captured in one
HIP graph: every replay, with eager work and synchronisations between replays,
reproduces the eager results bit for bit (the library records only kernel
launches: no memset, copy, sync or allocation)."""
import pytest
import torch

import lh_workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def lh():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import nvfp4_scale_calibration_amd as m
    return m


def test_path_in_hip_graph_replays_match_eager(lh):
    work = wl.make_custom(96, 512, 4096 + 100, n_groups=2, dtype="bf16", seed=12, w_dist="t3", x_dist="lognormal")
    G, c_out, c_in, n = work.n_groups, work.c_out, work.c_in, work.n_tok
    nb = c_in // 16
    w, x = work.w.to(DEV), work.x.to(DEV)
    xt = x.transpose(1, 2).contiguous().view(-1, c_in)       # token-major, for the ragged call
    off = torch.tensor([0, 1000, 1000, 2 * n], dtype=torch.int64, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    u8 = dict(dtype=torch.uint8, device=DEV)
    out = dict(amax=torch.empty(G, **f32), h=torch.empty((G, nb, 16, 16), **f32),
               hr=torch.zeros((3, nb, 16, 16), **f32),
               idx=torch.empty((G, c_out, nb), **u8), err=torch.empty((G, c_out, nb), **f32),
               bam=torch.empty((G, c_out, nb), **f32), idx4=torch.empty((G, c_out, nb), **u8),
               wq=torch.empty((G, c_out, c_in), **f32), packed=torch.empty((G, c_out, c_in // 2), **u8),
               codes=torch.empty((G, c_out, nb), **u8), gs=torch.empty(G, **f32),
               f_idx=torch.empty((G, c_out, nb), **u8), f_wq=torch.empty((G, c_out, c_in), **f32),
               f_packed=torch.empty((G, c_out, c_in // 2), **u8), f_codes=torch.empty((G, c_out, nb), **u8),
               c_amax=torch.empty(G, **f32), c_h=torch.empty((G, nb, 16, 16), **f32),
               c_idx=torch.empty((G, c_out, nb), **u8), c_wq=torch.empty((G, c_out, c_in), **f32),
               c_packed=torch.empty((G, c_out, c_in // 2), **u8), c_codes=torch.empty((G, c_out, nb), **u8))
    hws = torch.empty(max(lh.lh_hessian_workspace_bytes(c_in, n, G), 4), **u8)
    rws = torch.empty(max(lh.lh_hessian_ragged_workspace_bytes(c_in, 2 * n, 3), 4), **u8)
    sws = torch.empty(max(lh.lh_sweep_workspace_bytes(c_in, G), 4), **u8)
    cws = torch.empty(lh.lh_calibrate_workspace_bytes(c_out, c_in, n, G), **u8)
    assert hws.numel() > 4  # the split-token path with its finalize kernel is part of the graph

    def step():
        lh.lh_absmax(w, out=out["amax"])
        lh.lh_accumulate_hessian(x, h=out["h"], workspace=hws)
        lh.lh_accumulate_hessian_ragged(xt, off, h=out["hr"], workspace=rws)
        lh.lh_scale_sweep(w, out["h"], out["amax"], best_idx=out["idx"], best_err=out["err"],
                          best_amax=out["bam"], workspace=sws)
        lh.lh_select_scales(lh.LH_RULE_FOUR_OVER_SIX, w, out["h"], out["amax"], best_idx=out["idx4"],
                            best_err=False, best_amax=False)
        lh.lh_fake_quant_nvfp4(w, out["idx"], out["amax"], w_q=out["wq"], packed=out["packed"],
                               scale_e4m3=out["codes"], global_scale=out["gs"])
        lh.lh_scale_sweep_fake_quant(w, out["h"], out["amax"], best_idx=out["f_idx"], best_err=False,
                                     best_amax=False, w_q=out["f_wq"], packed=out["f_packed"],
                                     scale_e4m3=out["f_codes"], workspace=sws)
        lh.lh_calibrate_prologue(w, x, out["c_amax"], out["c_h"], cws)
        lh.lh_calibrate_sweep(w, out["c_h"], out["c_amax"], cws, out["c_idx"], w_q=out["c_wq"],
                              packed=out["c_packed"], scale_e4m3=out["c_codes"])

    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in out.items()}
    for k in ("idx", "wq", "packed", "codes"):     # the fused call writes what the two separate calls write
        assert torch.equal(eager["f_" + k], eager[k]), k
    for k in ("amax", "h", "idx", "wq", "packed", "codes"):   # and so do the two halves of the whole path
        assert torch.equal(eager["c_" + k], eager[k]), k
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for v in out.values():      # eager work between replays
            v.fill_(7)
        out["hr"].zero_()           # in/out: the empty group keeps the caller's H, as in the eager run
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            assert torch.equal(v, eager[k]), "replay %d: %s differs from the eager result" % (rep, k)
        print("replay %d matches" % rep, flush=True)
