#!/usr/bin/env python3
"""Benchmark of the Local-Hessian NVFP4 calibration hot path on one MI355X.

One step = the whole path over one layer's synthetic inputs, inputs resident
in HBM: global amax and local Hessians (lh_calibrate_prologue), then the
126-candidate scale sweep and the NVFP4 fake-quant of its result
(dequantised fp32 weights + packed E2M1 nibbles + E4M3 scale codes + S_g,
lh_calibrate_sweep).  The default layer is the largest named workload, the
MLP down projection W[5120 x 17408] with X[17408 x 16384 tokens] (5,570,560
blocks; the only one whose activations exceed the 256 MB last-level cache).
W warm-up steps, then K timed steps between device synchronisations; the
sweep's launch is also timed with HIP events recorded on the stream it is
launched on (the current torch stream, which the binding passes to the
library).

Prints ONE JSON line.  value = NVFP4 blocks scale-swept per second over the
whole step.  The line also carries the Hessian pass in GB/s measured after
a last-level-cache flush (per named workload), the roofline of the dominant
kernel (the sweep: VALU issue, from the rocprofv3 counters of one dispatch
committed under profiles/ for these kernel sources) and the CPU oracle's
rate on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 blocks/s scale-swept (126 cand) + Hessian-accum GB/s, % roofline"
HBM_PEAK_GBPS = 8000.0
FP32_NONPACKED_TFLOPS = 78.6          # 256 CU x 4 SIMD x 16 lanes x 2 flop x 2.4 GHz (packed FP32 is off)
N_SIMD = 256 * 4                      # MI355X: 256 CUs x 4 SIMDs
N_XCD = 8                             # GRBM_GUI_ACTIVE reads summed over the 8 XCDs
CLOCK_GHZ = 2.4                       # published peak engine clock
VALU_QUAD_PEAK_G = N_SIMD * CLOCK_GHZ / 4   # G quad-cycles/s: one wave64 VALU issue per SIMD per 4 clocks
SWEEP_FLOP_PER_BLOCK = 126 * (16 * 16 + 16) * 2   # 68,544: dense dw^T H dw of every candidate
PROFILES = os.path.join(ROOT, "profiles")
COUNTERS = os.path.join(PROFILES, "counters.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", type=int, default=5, help="named workload 1..5 (default: mlp-down-5120x17408)")
    p.add_argument("--extras-workload", type=int, default=2,
                   help="named workload of the adjacent parts (rules, ragged, diagnostics, GPTQ)")
    p.add_argument("--cold", default="2,3,4,5", help="named workloads whose Hessian is timed cache-cold")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the cold-cache Hessian timings and the adjacent parts")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run a plain 256 MiB device copy 5 times (HBM counter calibration)")
    p.add_argument("--summarize-profiles", metavar="DIR",
                   help="only turn the rocprofv3 runs under DIR into profiles/counters.json and the summaries")
    p.add_argument("--profile-workloads", default="5,1,2,3,4", help="workloads to summarise from DIR")
    return p.parse_args()


def copy_probe() -> None:
    """A plain copy kernel of known size: reads and writes 256 MiB per launch.
    Its FETCH_SIZE / WRITE_SIZE counter readings scale the counters taken on
    the library's kernels to bytes."""
    import torch
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_per_launch": n}), flush=True)


# the sources the step's kernels (prologue and sweep) are built from
KERNEL_SOURCES = ("lh_device.h", "lh_sweep.hip", "lh_hessian.hip")


def kernel_source_hash() -> str:
    """Hash of the step kernels' sources: counter readings taken on other
    sources no longer describe the kernels and are not reported."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "nvfp4_scale_calibration_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def profile_entry(kernel: str, workload: str, src_hash: str):
    """The committed rocprofv3 counter summary of one kernel on one workload
    (profiles/counters.json), or None when absent or taken on other kernel
    sources."""
    if not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as f:
        data = json.load(f)
    ent = data.get("kernels", {}).get("%s/%s" % (kernel, workload))
    if not ent or ent.get("source_hash") != src_hash:
        return None
    return ent


def sweep_roofline(ent, live_ms: float, blocks: int) -> dict:
    """Roofline of the sweep kernel, bound by VALU issue.

    From one dispatch's counters (deterministic instruction counts; the
    issue counters of the same dispatch): busy = SQ_ACTIVE_INST_VALU -
    SQ_ACTIVE_INST_VALU2, the SIMD quad-cycles in which the VALU issued at
    least one wave64 instruction (gfx950 can issue two VALU instructions in
    one quad-cycle; ACTIVE_INST_VALU counts both, VALU2 counts such
    quad-cycles once).  achieved = busy quad-cycles per launch / the live
    HIP-event launch time; peak = 1024 SIMDs x 2.4 GHz / 4; frac = their
    ratio.  frac_dispatch uses the dispatch's own cycle count
    (GRBM_GUI_ACTIVE / 8 XCDs) instead of the published clock."""
    if ent is None or "valu" not in ent:
        return {"bound": "alu", "achieved": None, "peak": VALU_QUAD_PEAK_G, "unit": "Gquad/s", "frac": None,
                "traffic": None, "note": "no counter summary for these kernel sources"}
    v = ent["valu"]
    busy = v["SQ_ACTIVE_INST_VALU"] - v["SQ_ACTIVE_INST_VALU2"]
    cycles = v["GRBM_GUI_ACTIVE"] / N_XCD
    achieved = busy / (live_ms / 1e3) / 1e9
    out = {"bound": "alu", "achieved": achieved, "peak": VALU_QUAD_PEAK_G, "unit": "Gquad/s",
           "frac": achieved / VALU_QUAD_PEAK_G,
           "traffic": ent.get("bytes_per_launch"),
           "frac_dispatch": busy / (N_SIMD * cycles / 4),
           "dispatch_clock_ghz": cycles / v["dispatch_ns"],
           "valu_instr_per_block": v["SQ_INSTS_VALU"] * 64 / blocks,
           "instr_per_busy_quad": v["SQ_INSTS_VALU"] / busy,
           "lanes_active": v["SQ_THREAD_CYCLES_VALU"] / (64.0 * v["SQ_ACTIVE_INST_VALU"]),
           "source": "rocprofv3 --pmc, one dispatch (profiles/counters.json, hash %s)" % ent["source_hash"]}
    ops = ent.get("ops")
    if ops:
        flop = 64.0 * (2 * ops["SQ_INSTS_VALU_FMA_F32"] + ops["SQ_INSTS_VALU_MUL_F32"] + ops["SQ_INSTS_VALU_ADD_F32"])
        out["fp32_executed_tflops"] = flop / (live_ms / 1e3) / 1e12
        out["fp32_executed_frac_78_6"] = out["fp32_executed_tflops"] / FP32_NONPACKED_TFLOPS
    return out


def copy_gbps(device) -> float:
    """Bandwidth of a plain 256 MiB device copy (read + write), for the
    'fraction of a measured copy' figures."""
    import torch
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device=device).fill_(1)
    b = torch.empty_like(a)
    t = graph_time(lambda: b.copy_(a), reps=5)
    return 2 * n / (t / 1e3) / 1e9


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def timed(fn, stream, reps: int, before=None):
    """Per-rep durations (ms) of fn() with HIP events on `stream`; before()
    runs outside the bracket."""
    import torch
    out = []
    for _ in range(reps):
        if before is not None:
            before()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        out.append(e0.elapsed_time(e1))
    return out


def graph_time(fn, reps: int = 20) -> float:
    """GPU time (ms) of one fn() launch: `reps` launches captured back to
    back in one HIP graph and replayed between two events, so host-side
    launch overhead does not leave the GPU idle between short kernels.
    fn must not allocate (buffers are passed in)."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def pct(v, q):
    import numpy as np
    return float(np.percentile(np.asarray(v), q))


def read_flush(device):
    """A 1 GiB buffer whose read (a sum) evicts the 256 MB last-level cache
    and the L2s before a cold rep; reading leaves no dirty lines whose
    write-back could overlap the timed launch."""
    import torch
    buf = torch.ones(1 << 28, dtype=torch.float32, device=device)
    out = torch.empty((), dtype=torch.float32, device=device)
    return lambda: torch.sum(buf, dim=0, out=out)   # fp32 in, fp32 out: a pure read of 1 GiB


def cold_prologue_and_hessian(lh, work, stream, reps: int = 9, w=None, x=None) -> dict:
    """The Hessian pass (lh_accumulate_hessian with its split-token
    workspace) and the step's prologue (lh_calibrate_prologue: amax, H and
    the skip certificates) timed with HIP events right after a read flush of
    the last-level cache; median and p10/p90 over `reps`.  GB/s counts the
    algorithmic bytes: X read once (Hessian), W + X (prologue)."""
    import torch
    dev = torch.device("cuda:0")
    G, c_out, c_in, n = work.n_groups, work.c_out, work.c_in, work.n_tok
    nb = c_in // 16
    w = work.w.to(dev) if w is None else w
    x = work.x.to(dev) if x is None else x
    h = torch.empty((G, nb, 16, 16), dtype=torch.float32, device=dev)
    amax = torch.empty(G, dtype=torch.float32, device=dev)
    ws_bytes = lh.lh_hessian_workspace_bytes(c_in, n, G)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    cws = torch.empty(lh.lh_calibrate_workspace_bytes(c_out, c_in, n, G), dtype=torch.uint8, device=dev)
    flush = read_flush(dev)
    hess = timed(lambda: lh.lh_accumulate_hessian(x, h=h, workspace=ws if ws_bytes else None), stream, reps,
                 before=flush)
    pro = timed(lambda: lh.lh_calibrate_prologue(w, x, amax, h, cws), stream, reps, before=flush)
    xb = work.x_bytes
    wb = work.w.numel() * work.w.element_size()
    med_h, med_p = pct(hess, 50), pct(pro, 50)
    return {"workload": work.name, "x_bytes": xb, "w_bytes": wb,
            "hessian_ms": med_h, "hessian_p10_ms": pct(hess, 10), "hessian_p90_ms": pct(hess, 90),
            "hessian_gbps": xb / (med_h / 1e3) / 1e9, "hessian_frac_hbm": xb / (med_h / 1e3) / 1e9 / HBM_PEAK_GBPS,
            "prologue_ms": med_p, "prologue_p10_ms": pct(pro, 10), "prologue_p90_ms": pct(pro, 90),
            "prologue_gbps": (xb + wb) / (med_p / 1e3) / 1e9,
            "prologue_frac_hbm": (xb + wb) / (med_p / 1e3) / 1e9 / HBM_PEAK_GBPS}


def extras(lh, work, stream) -> dict:
    """Outside the timed steps, on workload `work` (a layer resident in
    HBM): every scale rule of lh_select_scales with the local Hessian and
    with the plain weight error (N2); the ragged MoE capture with a running
    mean (N1); the approximation diagnostics and GPTQ (N3, N4)."""
    import torch
    dev = torch.device("cuda:0")
    G, c_out, c_in, n = work.n_groups, work.c_out, work.c_in, work.n_tok
    nb = c_in // 16
    w, x = work.w.to(dev), work.x.to(dev)
    amax = lh.lh_absmax(w)
    h = lh.lh_accumulate_hessian(x)
    idx = torch.empty((G, c_out, nb), dtype=torch.uint8, device=dev)
    err = torch.empty((G, c_out, nb), dtype=torch.float32, device=dev)
    bam = torch.empty((G, c_out, nb), dtype=torch.float32, device=dev)
    blocks = work.n_blocks
    rules = {}
    names = {0: "sweep126", 1: "max", 2: "four_over_six", 3: "amax_search"}
    for rule in (0, 1, 2, 3):
        for weighted in (True, False):
            hh = h if weighted else None
            fn = (lambda r=rule, hh=hh: lh.lh_select_scales(r, w, hh, amax, best_idx=idx, best_err=err,
                                                              best_amax=bam))
            fn()
            t = timed(fn, stream, 5)
            ms = sorted(t)[len(t) // 2]
            rules["%s/%s" % (names[rule], "hessian" if weighted else "mse")] = {
                "ms": ms, "blocks_per_s": blocks / (ms / 1e3)}
    # ragged / streaming Hessian on the MoE layer's capture (skewed routing)
    import lh_workloads as wl
    cap = wl.make_ragged_moe()
    xr = cap.x.to(dev)
    off = torch.from_numpy(cap.offsets).to(dev)
    hr = torch.zeros((cap.n_groups, cap.c_in // 16, 16, 16), dtype=torch.float32, device=dev)
    cnt = torch.zeros(cap.n_groups, dtype=torch.int64, device=dev)
    largest = int((cap.offsets[1:] - cap.offsets[:-1]).max())   # known where the tokens were routed
    rb = lh.lh_hessian_ragged_workspace_bytes(cap.c_in, xr.shape[0], cap.n_groups, largest)
    rws = torch.empty(max(rb, 1), dtype=torch.uint8, device=dev)
    fn = (lambda: lh.lh_accumulate_hessian_ragged(xr, off, h=hr, counts=cnt, workspace=rws if rb else None,
                                                  max_group_rows=largest))
    fn()
    warm = timed(fn, stream, 15)
    launch_ms = graph_time(fn)
    rcold = timed(fn, stream, 15, before=read_flush(dev))
    counts = cap.offsets[1:] - cap.offsets[:-1]
    diag = diagnostics(lh, work, w, x, h, amax, idx, err, bam)
    return {"workload": work.name,
            "hessian_ragged": {"workload": cap.description, "x_bytes": cap.x_bytes,
                               "max_group_rows": int(counts.max()), "empty_groups": int((counts == 0).sum()),
                               "running_mean": True,
                               "launch_ms": launch_ms, "launch_gbps": cap.x_bytes / (launch_ms / 1e3) / 1e9,
                               "warm_median_ms": pct(warm, 50), "warm_gbps": cap.x_bytes / (pct(warm, 50) / 1e3) / 1e9,
                               "cold_median_ms": pct(rcold, 50), "cold_p10_ms": pct(rcold, 10),
                               "cold_p90_ms": pct(rcold, 90),
                               "cold_gbps": cap.x_bytes / (pct(rcold, 50) / 1e3) / 1e9,
                               "flush": "1 GiB device read before every cold rep"},
            "scale_rules": rules,
            "diagnostics": diag}


def full_hessian_wide(lh, work, x) -> dict:
    """The full C_in x C_in Hessian of a wide layer's X (N3): at C_in = 17408
    the kernel computes the lower triangle of 256 x 256 tiles (2346 of 4624)
    and mirrors it.  Two rates: the full product's 2 C_in^2 N flop per
    second (what a square GEMM would have to reach for the same result) and
    the symmetric product's C_in (C_in + 1) N flop per second (work that no
    C_in x C_in result can avoid); the MFMA peak applies to the second."""
    import torch
    c_in, n = work.c_in, work.n_tok
    hf = torch.empty((1, c_in, c_in), dtype=torch.float32, device=x.device)
    t = graph_time(lambda: lh.lh_full_hessian(x, h=hf), reps=3)
    del hf
    sym = float(c_in) * (c_in + 1) * n / (t / 1e3) / 1e12
    return {"workload": work.description, "c_in": c_in, "n_tokens": n, "ms": t,
            "full_product_tflops": 2.0 * c_in * c_in * n / (t / 1e3) / 1e12,
            "symmetric_tflops": sym, "symmetric_frac_bf16_peak": sym / 2500.0}


def diagnostics(lh, work, w, x, h, amax, idx, err, bam) -> dict:
    """How much of the layer's output error the block-diagonal objective
    sees, per scale rule: the full error sum_r (q-w) H_full (q-w)^T (H_full =
    X X^T / N on matrix cores) against the sweep's block errors, and where
    the W/s values fall relative to the E2M1 grid.  Timed: the full Hessian
    (bf16 MFMA, 2 C_in^2 N flop) and the output error (fp32 MFMA, 2 C_out
    C_in^2 flop)."""
    import torch
    G, c_out, c_in, n = work.n_groups, work.c_out, work.c_in, work.n_tok
    if G != 1:
        return {"skipped": "grouped layers: per-expert full Hessians not measured here"}
    hf = torch.empty((1, c_in, c_in), dtype=torch.float32, device=w.device)
    t_hf = graph_time(lambda: lh.lh_full_hessian(x, h=hf), reps=3)
    wq = torch.empty((1, c_out, c_in), dtype=torch.float32, device=w.device)
    e = torch.empty((1, c_out), dtype=torch.float32, device=w.device)
    ows = torch.empty(max(lh.lh_output_error_workspace_bytes(c_out, c_in, 1), 4), dtype=torch.uint8, device=w.device)
    counts = torch.empty((1, 161), dtype=torch.int64, device=w.device)
    grid = torch.tensor([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=torch.float64)
    centers = (torch.arange(160, dtype=torch.float64) + 0.5) / 20.0
    near_grid = (centers[:, None] - grid[None, :]).abs().min(1).values < 0.05
    sym = float(c_in) * (c_in + 1) * n / (t_hf / 1e3) / 1e12
    out = {"full_hessian_ms": t_hf, "full_hessian_tflops": 2.0 * c_in * c_in * n / (t_hf / 1e3) / 1e12,
           "full_hessian_symmetric_tflops": sym, "full_hessian_symmetric_frac_bf16_peak": sym / 2500.0,
           "full_hessian_note": "full_hessian_tflops counts the full product (2 C_in^2 N flop); wide bf16 layers "
                                "compute one triangle of tiles and mirror it, so the symmetric product's "
                                "C_in (C_in + 1) N flop is the work no C_in x C_in result can avoid"}
    rules = {"local_hessian": (0, h), "mse": (0, None), "max": (1, h), "four_over_six": (2, None)}
    for name, (rule, hh) in rules.items():
        ri, re_, _ = lh.lh_select_scales(rule, w, hh, amax, best_idx=torch.empty_like(idx), best_err=True,
                                         best_amax=False)
        lh.lh_fake_quant_nvfp4(w, ri, amax, w_q=wq)
        fn = (lambda: lh.lh_output_error(w, wq, hf, err=e, workspace=ows))
        t_e = graph_time(fn, reps=3) if name == "local_hessian" else None
        fn()
        lh.lh_scaled_histogram(w, ri, amax, counts=counts)
        torch.cuda.synchronize()
        c = counts[0].double().cpu()
        tot = float(c.sum())
        ent = {"output_error": float(e.double().sum()),
               "w_over_s_near_grid": float(c[:160][near_grid].sum()) / tot,
               "w_over_s_at_least_5_5": float(c[110:].sum()) / tot}
        if rule == 0 and hh is not None:
            ent["block_diagonal_error"] = float(re_.double().sum())
        if t_e is not None:
            out["output_error_ms"] = t_e
            out["output_error_tflops"] = 2.0 * c_out * c_in * c_in / (t_e / 1e3) / 1e12
        out[name] = ent
    # GPTQ rounding with fixed scales (Local-Hessian and max), on the same layer
    gws = torch.empty(max(lh.lh_gptq_workspace_bytes(c_out, c_in), 16), dtype=torch.uint8, device=w.device)
    u = torch.empty((c_in, c_in), dtype=torch.float32, device=w.device)
    gq = torch.empty((c_out, c_in), dtype=torch.float32, device=w.device)
    t_prep = graph_time(lambda: lh.lh_gptq_prepare(hf, u=u, workspace=gws), reps=1)
    for name, (rule, hh) in (("local_hessian_gptq", (0, h)), ("max_gptq", (1, h))):
        ri, _, _ = lh.lh_select_scales(rule, w, hh, amax, best_idx=torch.empty_like(idx), best_err=False,
                                       best_amax=False)
        fn = (lambda ri=ri: lh.lh_gptq_quantize(w, ri, amax, u, w_q=gq, workspace=gws))
        t_q = graph_time(fn, reps=1)
        fn()
        lh.lh_output_error(w, gq.view(1, c_out, c_in), hf, err=e, workspace=ows)
        torch.cuda.synchronize()
        out[name] = {"output_error": float(e.double().sum()), "quantize_ms": t_q}
    out["gptq_prepare_ms"] = t_prep
    return out


def cpu_baseline(work, budget_s: float) -> dict:
    """The oracle as it stands, on host cores, on a bounded sample: Hessians
    of a few input blocks and the sweep + fake-quant of the first rows; the
    per-unit costs are scaled to the whole step of the workload."""
    import numpy as np
    import lh_workloads as wl
    import oracle

    G, c_out, c_in, n = work.n_groups, work.c_out, work.c_in, work.n_tok
    nb = c_in // 16
    w_np, x_np = wl.np_bits(work.w), wl.np_bits(work.x)
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    amax = oracle.absmax(w_np, c_out, c_in, n_groups=G)
    t_amax = time.perf_counter() - t0
    # Hessian: grow the sample until it costs ~15% of the budget
    hs = max(1, threads)
    while True:
        sel = np.arange(min(hs, G * nb), dtype=np.int64)
        t0 = time.perf_counter()
        _, h32s = oracle.hessian(x_np, c_in, n, n_groups=G, sel=sel)
        th = time.perf_counter() - t0
        if th > 0.15 * budget_s or len(sel) >= G * nb:
            break
        hs *= 4
    t_hess_total = th / len(sel) * (G * nb)
    h_full = np.zeros((G * nb, 16, 16), np.float32)
    h_full[: len(sel)] = h32s
    h_full[len(sel):] = np.eye(16, dtype=np.float32)  # blocks outside the sample: any valid H
    # sweep + fake-quant on the first rows of group 0 (blocks b < len(sel) use the oracle's H)
    nsw = max(threads * 8, 64)
    while True:
        ssel = np.arange(min(nsw, G * c_out * nb), dtype=np.int64)
        t0 = time.perf_counter()
        res = oracle.sweep(w_np, h_full, amax, c_out, c_in, n_groups=G, sel=ssel)
        idx_full = np.zeros(G * c_out * nb, np.uint8)
        idx_full[ssel] = res["idx"].astype(np.uint8)
        oracle.fake_quant(w_np, idx_full, amax, c_out, c_in, n_groups=G, sel=ssel)
        ts = time.perf_counter() - t0
        if ts > 0.6 * budget_s or len(ssel) >= G * c_out * nb:
            break
        nsw *= 4
    blocks = G * c_out * nb
    step_s = t_amax + t_hess_total + ts / len(ssel) * blocks
    return {
        "value": blocks / step_s, "unit": "blocks/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
        "sample": "Hessians of %d of %d input blocks (all %d tokens) + sweep and fake-quant of the first %d of "
                  "%d blocks, per-unit times scaled to the whole step; global amax over the full tensor"
                  % (len(sel), G * nb, n, len(ssel), blocks),
        "hessian_gbps": work.x_bytes / t_hess_total / 1e9,
        "sweep_blocks_per_s": len(ssel) / ts,
        "est_step_s": step_s,
    }


# ---------------------------------------------------------------------------
# Profile summaries: rocprofv3 CSVs -> profiles/counters.json and
# profiles/pipeline_<workload>.md (python3 bench.py --summarize-profiles DIR).
# DIR holds the runs named in the summaries' command lists: trace_w<n>,
# valu_w<n>, ops_w<n>, fetch_w<n>, write_w<n> (each with the run's log
# <run>.log beside it), copy_fetch, copy_write and, for the adjacent parts,
# trace_extras_w2.
# ---------------------------------------------------------------------------
PROF_VALU = ("SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_VALU2 SQ_THREAD_CYCLES_VALU SQ_WAVES SQ_BUSY_CYCLES "
             "GRBM_GUI_ACTIVE")
PROF_OPS = ("SQ_INSTS_VALU_FMA_F32 SQ_INSTS_VALU_ADD_F32 SQ_INSTS_VALU_MUL_F32 SQ_INSTS_VALU_TRANS_F32 "
            "SQ_INSTS_VALU_CVT SQ_INSTS_SALU SQ_INSTS_LDS GRBM_GUI_ACTIVE")


def _short_kernel_name(name: str) -> str:
    """A demangled kernel name without 'void ', the library's namespace and
    the parameter list."""
    s = name[5:] if name.startswith("void ") else name
    s = s.replace("lh::(anonymous namespace)::", "")
    if s.endswith(")"):
        depth = 0
        for i in range(len(s) - 1, -1, -1):
            if s[i] == ")":
                depth += 1
            elif s[i] == "(":
                depth -= 1
                if depth == 0:
                    return s[:i]
    return s


def _one_file(d: str, pattern: str) -> str:
    import glob
    fs = glob.glob(os.path.join(d, pattern), recursive=True)
    if len(fs) != 1:
        raise SystemExit("expected one %s under %s, found %d" % (pattern, d, len(fs)))
    return fs[0]


def _counter_dispatches(d: str, run: str) -> dict:
    """Dispatch id -> {name, grid, ns, counters} of one --pmc run."""
    import csv
    out = {}
    with open(_one_file(d, run + "/**/pmc_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            e = out.setdefault(int(r["Dispatch_Id"]), {
                "name": _short_kernel_name(r["Kernel_Name"]), "grid": int(r["Grid_Size"]),
                "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), "c": {}})
            e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _trace_rows(d: str, run: str) -> list:
    import csv
    rows = []
    with open(_one_file(d, run + "/**/trace_kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            rows.append({"name": _short_kernel_name(r["Kernel_Name"]),
                         "grid": int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]),
                         "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
    return rows


def _trace_stats(d: str, run: str) -> list:
    import csv
    out = []
    with open(_one_file(d, run + "/**/trace_kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            out.append((_short_kernel_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                        float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return out


def _copy_scales(d: str) -> dict:
    """FETCH_SIZE / WRITE_SIZE of a plain 256 MiB device copy -> bytes per counter KiB."""
    import statistics

    def kib(run, cname):
        v = [e["c"][cname] for e in _counter_dispatches(d, run).values() if e["name"] == "__amd_rocclr_copyBuffer"]
        return statistics.median(v)
    n = 256 << 20
    fk, wk = kib("copy_fetch", "FETCH_SIZE"), kib("copy_write", "WRITE_SIZE")
    return {"calibration": "plain 256 MiB device copy (python3 bench.py --copy-probe): FETCH_SIZE %d KiB, "
                           "WRITE_SIZE %d KiB per launch" % (round(fk), round(wk)),
            "fetch_scale": n / (fk * 1024), "write_scale": n / (wk * 1024)}


def summarize_workload(d: str, w: int, data: dict, src_hash: str) -> None:
    """counters.json entries (sweep, prologue, Hessian) and the pipeline
    summary of named workload w.  The sweep's counters are those of the
    median-duration dispatch of the workload's grid, leaving out the
    kernel's first dispatch (its GRBM_GUI_ACTIVE spans more than the
    dispatch); traffic is the mean over the workload's dispatches, scaled by
    the copy calibration."""
    import statistics
    from collections import Counter
    valu, ops = _counter_dispatches(d, "valu_w%d" % w), _counter_dispatches(d, "ops_w%d" % w)
    fetch, write = _counter_dispatches(d, "fetch_w%d" % w), _counter_dispatches(d, "write_w%d" % w)
    names = Counter(e["name"] for e in valu.values())
    sweep = [n for n in names if n.startswith("sweep_rows") and n.endswith("true, true, true>")]
    if len(sweep) != 1:
        raise SystemExit("workload %d: expected one fused sweep kernel, found %r" % (w, sweep))
    sweep = sweep[0]
    grids = {}
    for e in valu.values():
        grids.setdefault(e["name"], Counter())[e["grid"]] += 1

    def sel(dd, name):
        g = grids[name].most_common(1)[0][0]
        return [e for e in dd.values() if e["name"] == name and e["grid"] == g]

    def median_dispatch(dd, name):
        first = min(k for k, v in dd.items() if v["name"] == name)
        es = sorted([e for e in sel(dd, name) if e is not dd[first]], key=lambda e: e["ns"])
        e = es[len(es) // 2]
        if "GRBM_GUI_ACTIVE" in e["c"] and e["ns"] > 100000 and e["c"]["GRBM_GUI_ACTIVE"] / N_XCD / e["ns"] >= 2.45:
            raise SystemExit("workload %d: implausible dispatch clock in %s" % (w, name))
        return e, [k for k, v in dd.items() if v is e][0], len(es)

    ev, vid, nv = median_dispatch(valu, sweep)
    eo, oid, _ = median_dispatch(ops, sweep)
    tr = _trace_rows(d, "trace_w%d" % w)
    g_sweep = grids[sweep].most_common(1)[0][0]
    tsw = [r["ns"] for r in tr if r["name"] == sweep and r["grid"] == g_sweep]
    cp = data["copy"]

    def traffic(kernels):
        rd = sum(statistics.mean([e["c"]["FETCH_SIZE"] for e in sel(fetch, k)]) for k in kernels)
        wr = sum(statistics.mean([e["c"]["WRITE_SIZE"] for e in sel(write, k)]) for k in kernels)
        return rd * 1024 * cp["fetch_scale"], wr * 1024 * cp["write_scale"]

    def trace_avg(kernels):
        tot = 0.0
        for k in kernels:
            g = grids[k].most_common(1)[0][0]
            tot += statistics.mean([r["ns"] for r in tr if r["name"] == k and r["grid"] == g])
        return tot

    with open(os.path.join(d, "valu_w%d.log" % w)) as f:
        cfg = json.loads([l for l in f if l.startswith("{")][0])["config"]
    wl, blocks = cfg["name"], cfg["blocks"]
    # the calls' kernels: the prologue's certificates come from the lane
    # pre-pass above 2048 input blocks
    pro_k = [n for n in names if n.startswith("prologue_cm_kernel")] + ["finalize_certify_kernel"]
    if cfg["n_groups"] * cfg["c_in"] // 16 > 2048:
        pro_k.append("sweep_certificate_lane_kernel")
    hes_k = [n for n in names if n.startswith("hessian_cm_kernel")]
    if "hessian_finalize_kernel" in names:
        hes_k.append("hessian_finalize_kernel")
    kern = data["kernels"]
    rd, wr = traffic([sweep])
    vc = dict(ev["c"]); vc.update(dispatch_id=vid, dispatch_ns=ev["ns"], n_dispatches=nv)
    oc = dict(eo["c"]); oc.update(dispatch_id=oid, dispatch_ns=eo["ns"])
    kern["sweep/%s" % wl] = {"avg_ns": statistics.mean(tsw), "bytes_per_launch": rd + wr, "kernel": sweep,
                             "ops": oc, "read_bytes": rd, "source_hash": src_hash, "trace_dispatches": len(tsw),
                             "valu": vc, "write_bytes": wr}
    prd, pwr = traffic(pro_k)
    kern["prologue/%s" % wl] = {"avg_ns": trace_avg(pro_k), "bytes_per_launch": prd + pwr, "kernels": pro_k,
                                "read_bytes": prd, "source_hash": src_hash, "write_bytes": pwr}
    hrd, hwr = traffic(hes_k)
    hns = sum(statistics.mean([e["ns"] for e in sel(fetch, k)]) for k in hes_k)
    kern["hessian/%s" % wl] = {"avg_ns_counter_run": hns, "bytes_per_launch": hrd + hwr, "kernels": hes_k,
                               "read_bytes": hrd, "source_hash": src_hash, "write_bytes": hwr}

    tr_cmd = ("python3 bench.py" if w == 5 else
              "python3 bench.py --workload %d --steps 20 --warmup 3 --no-cpu-baseline --no-extras" % w)
    short_cmd = "python3 bench.py --workload %d --steps 2 --warmup 1 --no-cpu-baseline --no-extras" % w
    L = ["# Kernel profile: the benchmark step on workload %s (MI355X)\n" % wl,
         "Commands (on the GPU box, from the repository root; each profiler run is started from `/tmp` with "
         "`TMPDIR=/tmp`, for the profiler's files, and `-d` pointing back under `gpurun_out/prof/`):\n",
         "```",
         "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof/trace_w%d -o trace -- %s" % (w, tr_cmd),
         "rocprofv3 --kernel-trace --pmc %s --output-format csv -d gpurun_out/prof/valu_w%d -o pmc -- %s"
         % (PROF_VALU, w, short_cmd),
         "rocprofv3 --kernel-trace --pmc %s --output-format csv -d gpurun_out/prof/ops_w%d -o pmc -- %s"
         % (PROF_OPS, w, short_cmd),
         "rocprofv3 --kernel-trace --pmc FETCH_SIZE --output-format csv -d gpurun_out/prof/fetch_w%d -o pmc -- %s"
         % (w, short_cmd),
         "rocprofv3 --kernel-trace --pmc WRITE_SIZE --output-format csv -d gpurun_out/prof/write_w%d -o pmc -- %s"
         % (w, short_cmd),
         "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/prof/copy_fetch -o pmc -- python3 bench.py "
         "--copy-probe",
         "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/prof/copy_write -o pmc -- python3 bench.py "
         "--copy-probe",
         "python3 bench.py --summarize-profiles gpurun_out/prof   # this summary and profiles/counters.json",
         "```\n",
         "kernel source hash: `%s`\n" % src_hash,
         "| kernel | calls | avg us | min us | max us | % time |",
         "|---|---|---|---|---|---|"]
    for n, c, a, mn, mx, pc in _trace_stats(d, "trace_w%d" % w):
        L.append("| %s | %d | %.1f | %.1f | %.1f | %.1f |" % (n, c, a, mn, mx, pc))
    L.append("")
    L.append("Benchmarked sweep launch (`%s`): %d dispatches of this workload in the trace run "
             "(matched by grid size), average %.1f us.\n" % (sweep, len(tsw), statistics.mean(tsw) / 1e3))
    c = ev["c"]
    L.append("VALU counters of one dispatch (id %d, %.1f us under the counter pass; median of %d):\n"
             % (vid, ev["ns"] / 1e3, nv))
    L += ["| counter | value |", "|---|---|"]
    L += ["| %s | %d |" % (k, c[k]) for k in PROF_VALU.split()]
    L.append("")
    L.append("Instruction mix of one dispatch (id %d):\n" % oid)
    L += ["| counter | value |", "|---|---|"]
    L += ["| %s | %d |" % (k, eo["c"][k]) for k in PROF_OPS.split()[:-1]]
    L.append("")
    cyc = c["GRBM_GUI_ACTIVE"] / N_XCD
    busy = c["SQ_ACTIVE_INST_VALU"] - c["SQ_ACTIVE_INST_VALU2"]
    avg_s = statistics.mean(tsw) / 1e9
    flop = 64.0 * (2 * eo["c"]["SQ_INSTS_VALU_FMA_F32"] + eo["c"]["SQ_INSTS_VALU_MUL_F32"]
                   + eo["c"]["SQ_INSTS_VALU_ADD_F32"])
    L += ["Derived (one dispatch):\n",
          "* dispatch cycles = GRBM_GUI_ACTIVE / 8 XCDs = %d (clock %.2f GHz over the dispatch)" % (cyc, cyc / ev["ns"]),
          "* VALU-busy SIMD quad-cycles = SQ_ACTIVE_INST_VALU - SQ_ACTIVE_INST_VALU2 = %d; **VALU busy = %.3f** of "
          "1024 SIMDs x %d quad-cycles" % (busy, busy / (N_SIMD * cyc / 4), cyc / 4),
          "* at the published 2.4 GHz over the trace average: %.3f of 614.4 G quad-cycles/s"
          % (busy / avg_s / (VALU_QUAD_PEAK_G * 1e9)),
          "* wave64 VALU instructions per busy quad-cycle = %.3f (gfx950 dual issue: %.1f%% of busy quad-cycles issue two)"
          % (c["SQ_INSTS_VALU"] / busy, 100 * c["SQ_ACTIVE_INST_VALU2"] / busy),
          "* lanes active per VALU instruction = %.4f" % (c["SQ_THREAD_CYCLES_VALU"] / (64.0 * c["SQ_ACTIVE_INST_VALU"])),
          "* VALU instructions per block = %.1f (per lane-row block; 126 x 207 = 26,082 for an exhaustive evaluation)"
          % (c["SQ_INSTS_VALU"] * 64 / blocks),
          "* executed fp32 arithmetic = %.1f GFLOP per launch, %.1f TFLOP/s over the trace average = %.3f of the "
          "78.6 TFLOP/s non-packed fp32 peak" % (flop / 1e9, flop / avg_s / 1e12, flop / avg_s / 1e12 / FP32_NONPACKED_TFLOPS),
          "* dense-equivalent rate (68,544 flop per block, not executed work) = %.0f TFLOP/s\n"
          % (SWEEP_FLOP_PER_BLOCK * blocks / avg_s / 1e12),
          "HBM traffic (counter KiB x 1024 x the copy factor: FETCH_SIZE x %.3f, WRITE_SIZE x %.3f; %s):\n"
          % (cp["fetch_scale"], cp["write_scale"], cp["calibration"]),
          "| call | kernels | avg us | read MB | written MB |",
          "|---|---|---|---|---|"]
    e1, e2, e3 = kern["sweep/%s" % wl], kern["prologue/%s" % wl], kern["hessian/%s" % wl]
    L.append("| lh_calibrate_sweep | %s | %.1f | %.1f | %.1f |"
             % (sweep, e1["avg_ns"] / 1e3, e1["read_bytes"] / 1e6, e1["write_bytes"] / 1e6))
    L.append("| lh_calibrate_prologue | %s | %.1f | %.1f | %.1f |"
             % (" + ".join(pro_k), e2["avg_ns"] / 1e3, e2["read_bytes"] / 1e6, e2["write_bytes"] / 1e6))
    L.append("| lh_accumulate_hessian | %s | %.1f (counter run) | %.1f | %.1f |"
             % (" + ".join(hes_k), e3["avg_ns_counter_run"] / 1e3, e3["read_bytes"] / 1e6, e3["write_bytes"] / 1e6))
    with open(os.path.join(PROFILES, "pipeline_%s.md" % wl), "w") as f:
        f.write("\n".join(L) + "\n")


def summarize_extras(d: str, src_hash: str) -> None:
    """profiles/extras_dense-4096.md from the trace of the adjacent parts."""
    L = ["# Kernel profile: adjacent parts on workload dense-4096 (MI355X)\n",
         "Ragged Hessian of the MoE capture (N1), the scale rules (N2), the full Hessian,\n"
         "output error and W/s histogram (N3), GPTQ factorisation and sweep (N4), plus\n"
         "the hot path itself, as bench.py runs them (its extras).\n",
         "```",
         "# on the GPU box, from the repository root; the profiler run is started from /tmp with TMPDIR=/tmp",
         "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof/trace_extras_w2 -o trace -- python3 "
         "bench.py --workload 2 --steps 3 --warmup 1 --no-cpu-baseline --cold \"\"",
         "python3 bench.py --summarize-profiles gpurun_out/prof   # this summary",
         "```\n",
         "kernel source hash: `%s` (lh_dense.hip is not part of it)\n" % src_hash,
         "| kernel | calls | avg us | min us | max us | % time |",
         "|---|---|---|---|---|---|"]
    for n, c, a, mn, mx, pc in _trace_stats(d, "trace_extras_w2"):
        L.append("| %s | %d | %.1f | %.1f | %.1f | %.1f |" % (n, c, a, mn, mx, pc))
    with open(os.path.join(PROFILES, "extras_dense-4096.md"), "w") as f:
        f.write("\n".join(L) + "\n")


def summarize_profiles(d: str, workloads: list) -> None:
    data = {"kernels": {}}
    if os.path.exists(COUNTERS):
        with open(COUNTERS) as f:
            data = json.load(f)
    h = kernel_source_hash()
    if os.path.isdir(os.path.join(d, "copy_fetch")):
        data["copy"] = _copy_scales(d)
    if "copy" not in data:
        raise SystemExit("no copy calibration: profile bench.py --copy-probe first")
    for w in workloads:
        summarize_workload(d, w, data, h)
    if os.path.isdir(os.path.join(d, "trace_extras_w2")):
        summarize_extras(d, h)
    data["kernels"] = dict(sorted(data["kernels"].items()))
    with open(COUNTERS, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")


def main():
    args = parse()
    if args.copy_probe:
        copy_probe()
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, [int(v) for v in args.profile_workloads.split(",") if v])
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (asked for %d)." % max(args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    import torch
    import lh_workloads as wl
    import nvfp4_scale_calibration_amd as lh

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    work = wl.make(args.workload)
    G, c_out, c_in, n = work.n_groups, work.c_out, work.c_in, work.n_tok
    nb = c_in // 16
    blocks = work.n_blocks
    w = work.w.to(dev)
    x = work.x.to(dev)
    amax = torch.empty(G, dtype=torch.float32, device=dev)
    h = torch.empty((G, nb, 16, 16), dtype=torch.float32, device=dev)
    ws_bytes = lh.lh_hessian_workspace_bytes(c_in, n, G)
    cws = torch.empty(lh.lh_calibrate_workspace_bytes(c_out, c_in, n, G), dtype=torch.uint8, device=dev)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    sws = torch.empty(max(lh.lh_sweep_workspace_bytes(c_in, G), 4), dtype=torch.uint8, device=dev)
    idx = torch.empty((G, c_out, nb), dtype=torch.uint8, device=dev)
    err = torch.empty((G, c_out, nb), dtype=torch.float32, device=dev)
    bam = torch.empty((G, c_out, nb), dtype=torch.float32, device=dev)
    wq = torch.empty((G, c_out, c_in), dtype=torch.float32, device=dev)
    packed = torch.empty((G, c_out, c_in // 2), dtype=torch.uint8, device=dev)
    codes = torch.empty((G, c_out, nb), dtype=torch.uint8, device=dev)
    gscale = torch.empty(G, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    # HIP events bracket the dominant launch (the sweep with its fake-quant,
    # one kernel) in every timed step; the other calls' GPU times come from
    # graph replays (launch_ms), so the timed steps carry no further records.
    def step(ev=None):
        lh.lh_calibrate_prologue(w, x, amax, h, cws)
        if ev is not None:
            ev[0].record(stream)
        lh.lh_calibrate_sweep(w, h, amax, cws, idx, err, bam, wq, packed, codes, gscale)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_kernel_ms = {"calibrate_sweep": sum(e[0].elapsed_time(e[1]) for e in events) / args.steps}
    # per-call GPU time, free of host launch overhead: the step's two calls,
    # and for comparison the separate calls that compute the same
    launch_ms = {
        "calibrate_prologue": graph_time(lambda: lh.lh_calibrate_prologue(w, x, amax, h, cws)),
        "calibrate_sweep": graph_time(lambda: lh.lh_calibrate_sweep(w, h, amax, cws, idx, err, bam, wq, packed,
                                                                    codes, gscale), reps=5),
        "absmax": graph_time(lambda: lh.lh_absmax(w, out=amax)),
        "hessian": graph_time(lambda: lh.lh_accumulate_hessian(x, h=h, workspace=ws if ws_bytes else None)),
        "sweep_fake_quant": graph_time(lambda: lh.lh_scale_sweep_fake_quant(
            w, h, amax, best_idx=idx, best_err=err, best_amax=bam, w_q=wq, packed=packed, scale_e4m3=codes,
            global_scale=gscale, workspace=sws), reps=5),
        "sweep": graph_time(lambda: lh.lh_scale_sweep(w, h, amax, best_idx=idx, best_err=err, best_amax=bam,
                                                      workspace=sws), reps=5),
        "fake_quant": graph_time(lambda: lh.lh_fake_quant_nvfp4(w, idx, amax, w_q=wq, packed=packed,
                                                                scale_e4m3=codes, global_scale=gscale)),
    }
    ms_per_step = wall * 1e3 / args.steps
    sweep_ms = per_kernel_ms["calibrate_sweep"]
    w_bytes = work.w.numel() * work.w.element_size()
    src_hash = kernel_source_hash()
    name = wl.SHORT_NAMES[args.workload]
    sweep_ent = profile_entry("sweep", name, src_hash)
    pro_ent = profile_entry("prologue", name, src_hash)
    copy_bw = copy_gbps(dev)
    # the headline Hessian figure: this layer, after a read flush of the last-level cache
    cold = cold_prologue_and_hessian(lh, work, stream, w=w, x=x)
    # fake-quant: W + indices read, Q + nibbles + codes written (algorithmic bytes)
    fq_bytes = w_bytes + blocks + blocks * 16 * 4 + blocks * 8 + blocks
    dense_tflops = SWEEP_FLOP_PER_BLOCK * blocks / (sweep_ms / 1e3) / 1e12
    out = {
        "metric": METRIC,
        "value": blocks / (ms_per_step / 1e3),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": work.description, "name": name, "n_groups": G,
                   "c_out": c_out, "c_in": c_in, "n_tokens": n, "blocks": blocks, "storage": work.dtype},
        "roofline": sweep_roofline(sweep_ent, sweep_ms, blocks),
        "kernels_ms": per_kernel_ms,
        "launch_ms": launch_ms,
        "sweep": {"blocks_per_s": blocks / (sweep_ms / 1e3),
                  "dense_equivalent_tflops": dense_tflops,
                  "dense_equivalent_note": "68,544 flop per block (every candidate's dense dw^T H dw); the kernel "
                                           "skips candidates it proves cannot win, so this is not executed work"},
        "fake_quant": {"gbps": fq_bytes / (launch_ms["fake_quant"] / 1e3) / 1e9, "bytes": fq_bytes},
        "copy_gbps": copy_bw,
        "hessian": {"gbps": cold["hessian_gbps"], "frac_hbm": cold["hessian_frac_hbm"],
                    "frac_copy": cold["hessian_gbps"] / copy_bw, "median_ms": cold["hessian_ms"],
                    "p10_ms": cold["hessian_p10_ms"], "p90_ms": cold["hessian_p90_ms"], "x_bytes": work.x_bytes,
                    "cold": "1 GiB device read before every rep (last-level cache flushed, nothing dirty)",
                    "warm_graph_gbps": work.x_bytes / (launch_ms["hessian"] / 1e3) / 1e9,
                    "traffic": None if profile_entry("hessian", name, src_hash) is None
                    else profile_entry("hessian", name, src_hash).get("bytes_per_launch")},
        "prologue": {"gbps": cold["prologue_gbps"], "frac_hbm": cold["prologue_frac_hbm"],
                     "median_ms": cold["prologue_ms"], "bytes": work.x_bytes + w_bytes, "cold": True,
                     "traffic": None if pro_ent is None else pro_ent.get("bytes_per_launch")},
        "source_hash": src_hash,
    }
    if not args.no_extras:
        per = {}
        for k in [int(v) for v in args.cold.split(",") if v.strip()]:
            if k == args.workload:
                per[wl.SHORT_NAMES[k]] = cold
            else:
                other = wl.make(k)
                per[wl.SHORT_NAMES[k]] = cold_prologue_and_hessian(lh, other, stream)
                del other
                torch.cuda.empty_cache()
        out["hessian_cold"] = per
        if G == 1:
            out["full_hessian_wide"] = full_hessian_wide(lh, work, x)
            torch.cuda.empty_cache()
        ework = work if args.extras_workload == args.workload else wl.make(args.extras_workload)
        out["extras"] = extras(lh, ework, stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(work, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
