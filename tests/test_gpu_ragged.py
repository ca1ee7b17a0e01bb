"""GPU parity of the ragged / streaming Hessian (lh_accumulate_hessian_ragged)
against the CPU oracle: skewed per-group token counts with empty groups,
both dtypes, padded rows, with and without the split workspace (and bit-
identical reruns), the running mean over batches with token counts, offsets
outside the buffer (clamped), and the MoE capture at full size (sampled)."""
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


def run(lh, cap, h0, counts=None, workspace=True, ld_pad=0, max_group_rows=0):
    xd = cap.x.to(DEV)
    if ld_pad:  # rows padded in memory: a view with row stride c_in + ld_pad
        xd = torch.cat([xd, torch.zeros((xd.shape[0], ld_pad), dtype=xd.dtype, device=DEV)], 1)[:, :cap.c_in]
    off = torch.from_numpy(cap.offsets).to(DEV)
    h = torch.from_numpy(h0.copy()).to(DEV)
    cnt = None if counts is None else torch.from_numpy(counts.copy()).to(DEV)
    lh.lh_accumulate_hessian_ragged(xd, off, h=h, counts=cnt, workspace=workspace, max_group_rows=max_group_rows)
    torch.cuda.synchronize()
    return h.cpu().numpy(), (None if cnt is None else cnt.cpu().numpy())


def check(cap, h_gpu, h0, counts=None, sel=None, what=""):
    G, nb = cap.n_groups, cap.c_in // 16
    sel = np.arange(G * nb) if sel is None else sel
    h64, _, new_counts = oracle.hessian_ragged(wl.np_bits(cap.x), cap.c_in, cap.offsets, h0, counts=counts, sel=sel)
    parity.check_hessian(h_gpu.reshape(G * nb, 16, 16)[sel], h64, what)
    empty = np.flatnonzero(np.diff(cap.offsets) == 0)
    if counts is None:
        for g in empty:  # groups without rows keep the caller's H bit for bit
            np.testing.assert_array_equal(h_gpu[g], h0[g])
    return new_counts


@pytest.mark.parametrize("dtype,c_in,ld_pad", [("bf16", 48, 0), ("f32", 64, 4), ("bf16", 272, 8)])
def test_ragged_small(lh, dtype, c_in, ld_pad):
    cap = wl.make_ragged(9, c_in, 700, dtype=dtype, seed=c_in, concentration=0.4, n_empty=2)
    print("case ragged G=9 c_in=%d rows=700 %s pad=%d counts=%s" % (c_in, dtype, ld_pad, np.diff(cap.offsets)),
          flush=True)
    rng = np.random.default_rng(1)
    h0 = rng.standard_normal((9, c_in // 16, 16, 16)).astype(np.float32)
    h, _ = run(lh, cap, h0, ld_pad=ld_pad)
    check(cap, h, h0, what="ragged-small")


def test_ragged_split_matches_one_pass_and_is_deterministic(lh):
    cap = wl.make_ragged(3, 256, 3 * 9000 + 13, dtype="bf16", seed=7, concentration=2.0)
    assert lh.lh_hessian_ragged_workspace_bytes(256, cap.x.shape[0], 3) > 0
    print("case ragged split G=3 rows=%d counts=%s" % (cap.x.shape[0], np.diff(cap.offsets)), flush=True)
    h0 = np.zeros((3, 16, 16, 16), np.float32)
    a, _ = run(lh, cap, h0, workspace=True)
    b, _ = run(lh, cap, h0, workspace=True)
    c, _ = run(lh, cap, h0, workspace=False)
    assert np.array_equal(a, b)  # fixed reduction order
    check(cap, a, h0, what="split")
    check(cap, c, h0, what="one-pass")


def test_ragged_running_mean_over_batches(lh):
    G, c_in = 6, 96
    h = np.full((G, c_in // 16, 16, 16), 3.0, np.float32)   # the caller's fallback
    counts = np.zeros(G, np.int64)
    for i in range(3):
        cap = wl.make_ragged(G, c_in, 300 + 50 * i, dtype="bf16", seed=40 + i, concentration=0.5, n_empty=1 + i % 2)
        print("case running mean batch %d counts=%s" % (i, np.diff(cap.offsets)), flush=True)
        h_new, c_new = run(lh, cap, h, counts=counts)
        want_counts = check(cap, h_new, h, counts=counts, what="batch %d" % i)
        np.testing.assert_array_equal(c_new, want_counts)
        h, counts = h_new, c_new


def test_ragged_offsets_are_clamped(lh):
    """Each group's range is [clamp(off[g]), max(that, clamp(off[g+1]))) with
    clamp to [0, n_rows]: negative and too-large offsets stay inside the
    buffer and a decreasing pair gives an empty group."""
    cap = wl.make_ragged(6, 32, 200, dtype="f32", seed=3)
    n = cap.x.shape[0]
    bad = np.array([-7, 40, 30, 150, 10 ** 9, 10 ** 12, 5], np.int64)
    h0 = np.ones((6, 2, 16, 16), np.float32)
    cap_bad = wl.RaggedCapture(cap.name, cap.description, cap.c_in, cap.dtype, cap.x, bad)
    h, _ = run(lh, cap_bad, h0)
    x_np = wl.np_bits(cap.x)
    for g in range(6):
        r0 = min(max(int(bad[g]), 0), n)
        r1 = max(r0, min(max(int(bad[g + 1]), 0), n))
        h64, _, _ = oracle.hessian_ragged(x_np, 32, np.array([r0, r1]), h0[g:g + 1])
        parity.check_hessian(h[g], h64, "clamped group %d [%d, %d)" % (g, r0, r1))
        if r1 == r0:
            np.testing.assert_array_equal(h[g], h0[g])


def test_ragged_moe_capture_full_size_sampled(lh):
    cap = wl.make_ragged_moe()
    G, nb = cap.n_groups, cap.c_in // 16
    print("case ragged MoE capture rows=%d" % cap.x.shape[0], flush=True)
    h0 = np.zeros((G, nb, 16, 16), np.float32)
    h, _ = run(lh, cap, h0, max_group_rows=int(np.diff(cap.offsets).max()))  # as the benchmark runs it
    rng = np.random.default_rng(0)
    heavy = int(np.argmax(np.diff(cap.offsets)))
    sel = np.unique(np.concatenate([rng.choice(G * nb, 40, replace=False), heavy * nb + np.arange(4)]))
    check(cap, h, h0, sel=sel, what="moe-capture")


@pytest.mark.parametrize("hint", ["exact", "too small", "none"])
def test_ragged_largest_group_hint(lh, hint):
    """With a bound on the largest group the rows are cut into 1024-row
    slices (unused slices skipped by the finalize kernel); a bound that is
    too small only changes the split.  Results match the oracle either way
    and reruns are bit-identical."""
    cap = wl.make_ragged(12, 128, 20000, dtype="bf16", seed=77, concentration=0.2, n_empty=3)
    largest = int(np.diff(cap.offsets).max())
    mx = {"exact": largest, "too small": max(1, largest // 5), "none": 0}[hint]
    print("case ragged hint=%s largest=%d max_group_rows=%d" % (hint, largest, mx), flush=True)
    h0 = np.full((12, 8, 16, 16), 2.0, np.float32)
    counts = np.arange(12, dtype=np.int64) * 7      # running mean on top of earlier batches
    a, ca = run(lh, cap, h0, counts=counts, max_group_rows=mx)
    b, cb = run(lh, cap, h0, counts=counts, max_group_rows=mx)
    assert np.array_equal(a, b) and np.array_equal(ca, cb)
    want = check(cap, a, h0, counts=counts, what="hint %s" % hint)
    np.testing.assert_array_equal(ca, want)
