"""Seeded synthetic inputs for Local-Hessian NVFP4 scale calibration.

Shared by the tests, the benchmark and the smoke check, on both the HIP side
and the oracle side.  This module only draws random numbers and rounds them
to the storage dtype; it holds none of the method's arithmetic (no amax, no
Hessian, no scale, no cast).

The five named workloads stand in for the calibration data the pages use (a
real model's layers fed 512 samples x 2048 tokens of text, "Enabling
Local-Hessian" section of the Local-Hessian weight-scale guide,
xxmr.cn/news/266017).  They take the shapes of such layers with synthetic
values: weights ~ N(0, sigma^2) or scaled Student-t, a few outlier weights,
activations ~ N(0, 1) with outlier / near-zero / log-normal channel scales.

Generator: numpy PCG64 via SeedSequence(1000 + workload number).spawn(4),
one stream each for weight values, weight outlier picks, activation values
and activation channel picks (the MoE workload first spawns one sequence per
expert).  Values are drawn in fp32, outliers applied, then rounded to bf16
with round-to-nearest-even (torch's conversion).  Outlier sets are drawn
uniformly without replacement, counts = round(fraction * size).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

F32, BF16 = "f32", "bf16"


@dataclass
class Workload:
    name: str
    description: str
    c_out: int
    c_in: int
    n_tok: int
    n_groups: int
    dtype: str           # storage dtype of W and X: "f32" or "bf16"
    w: torch.Tensor      # [n_groups, c_out, c_in], CPU
    x: torch.Tensor      # [n_groups, c_in, n_tok], CPU (channel-major)

    @property
    def n_blocks(self) -> int:
        return self.n_groups * self.c_out * (self.c_in // 16)

    @property
    def x_bytes(self) -> int:
        return self.x.numel() * self.x.element_size()


def np_bits(t: torch.Tensor) -> np.ndarray:
    """numpy view for the oracle: float32 stays float32, bf16 -> uint16 bits."""
    t = t.contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    raise TypeError(t.dtype)


def _store(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t if dtype == F32 else t.to(torch.bfloat16)


def _pick(rng: np.random.Generator, size: int, frac: float) -> np.ndarray:
    return rng.choice(size, size=int(round(frac * size)), replace=False)


def _normal(rng, shape, sigma=1.0):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)


WORKLOADS = {
    1: "linear-256: W[256x256] fp32 ~N(0,0.02^2), X[256x128] fp32 ~N(0,1)",
    2: "dense-4096: W[4096x4096] bf16 ~N(0,0.02^2) with 0.1% of entries x20, "
       "X[4096x4096 tokens] bf16 ~N(0,1) with 1% of channels x30",
    3: "mlp-up-12288x4096: W[12288x4096] bf16 0.02*t(4), X[4096x8192 tokens] bf16 "
       "with per-channel log-normal scales (sigma=1)",
    4: "moe-64x1024x2048: 64 experts, each W[1024x2048] bf16 ~N(0,0.02^2) and "
       "X[2048x512 routed tokens] bf16 ~N(0,1), own Hessians and amax",
    5: "mlp-down-5120x17408: W[5120x17408] bf16 0.015*t(3), X[17408x16384 tokens] bf16 "
       "with 0.5% outlier channels x50 and 10% near-zero channels x1e-3",
}
SHORT_NAMES = {1: "linear-256", 2: "dense-4096", 3: "mlp-up-12288x4096",
               4: "moe-64x1024x2048", 5: "mlp-down-5120x17408"}


def make(n: int) -> Workload:
    """Build named workload n (1..5) on the CPU."""
    if n == 4:
        return _make_moe()
    ss = np.random.SeedSequence(1000 + n)
    r_wv, r_wp, r_xv, r_xp = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(4)]
    if n == 1:
        c_out, c_in, n_tok, dt = 256, 256, 128, F32
        w = _normal(r_wv, (c_out, c_in), 0.02)
        x = _normal(r_xv, (c_in, n_tok))
    elif n == 2:
        c_out, c_in, n_tok, dt = 4096, 4096, 4096, BF16
        w = _normal(r_wv, (c_out, c_in), 0.02)
        wf = w.reshape(-1)
        wf[_pick(r_wp, wf.size, 0.001)] *= np.float32(20.0)
        x = _normal(r_xv, (c_in, n_tok))
        x[_pick(r_xp, c_in, 0.01)] *= np.float32(30.0)
    elif n == 3:
        c_out, c_in, n_tok, dt = 12288, 4096, 8192, BF16
        w = (r_wv.standard_t(4, size=(c_out, c_in)) * 0.02).astype(np.float32)
        z = r_xp.standard_normal(c_in).astype(np.float32)
        x = _normal(r_xv, (c_in, n_tok))
        x *= np.exp(z)[:, None]
    elif n == 5:
        c_out, c_in, n_tok, dt = 5120, 17408, 16384, BF16
        w = (r_wv.standard_t(3, size=(c_out, c_in)) * 0.015).astype(np.float32)
        x = _normal(r_xv, (c_in, n_tok))
        picks = r_xp.permutation(c_in)
        n_hi, n_lo = int(round(0.005 * c_in)), int(round(0.10 * c_in))
        x[picks[:n_hi]] *= np.float32(50.0)
        x[picks[n_hi:n_hi + n_lo]] *= np.float32(1e-3)
    else:
        raise ValueError("workloads are numbered 1..5")
    return Workload(SHORT_NAMES[n], WORKLOADS[n], c_out, c_in, n_tok, 1, dt,
                    _store(w, dt).reshape(1, c_out, c_in), _store(x, dt).reshape(1, c_in, n_tok))


def _make_moe() -> Workload:
    G, c_out, c_in, n_tok = 64, 1024, 2048, 512
    experts = np.random.SeedSequence(1004).spawn(G)
    w = np.empty((G, c_out, c_in), np.float32)
    x = np.empty((G, c_in, n_tok), np.float32)
    for e, ss in enumerate(experts):
        r_wv, _r_wp, r_xv, _r_xp = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(4)]
        w[e] = _normal(r_wv, (c_out, c_in), 0.02)
        x[e] = _normal(r_xv, (c_in, n_tok))
    return Workload(SHORT_NAMES[4], WORKLOADS[4], c_out, c_in, n_tok, G, BF16,
                    _store(w, BF16), _store(x, BF16))


def make_custom(c_out: int, c_in: int, n_tok: int, n_groups: int = 1, dtype: str = BF16,
                seed: int = 0, w_sigma: float = 0.02, w_dist: str = "normal",
                x_dist: str = "normal") -> Workload:
    """Small seeded cases for parity tests (ragged shapes, several groups).
    w_dist: "normal" | "t3" | "zeros"; x_dist: "normal" | "lognormal" | "zeros"."""
    ss = np.random.SeedSequence([seed, c_out, c_in, n_tok, n_groups])
    r_w, r_x, r_z = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(3)]
    shape_w = (n_groups, c_out, c_in)
    if w_dist == "normal":
        w = _normal(r_w, shape_w, w_sigma)
    elif w_dist == "t3":
        w = (r_w.standard_t(3, size=shape_w) * w_sigma).astype(np.float32)
    elif w_dist == "zeros":
        w = np.zeros(shape_w, np.float32)
    else:
        raise ValueError(w_dist)
    shape_x = (n_groups, c_in, n_tok)
    if x_dist == "normal":
        x = _normal(r_x, shape_x)
    elif x_dist == "lognormal":
        x = _normal(r_x, shape_x) * np.exp(r_z.standard_normal((n_groups, c_in, 1)).astype(np.float32))
    elif x_dist == "zeros":
        x = np.zeros(shape_x, np.float32)
    else:
        raise ValueError(x_dist)
    return Workload("custom-%dx%dx%dx%d" % (n_groups, c_out, c_in, n_tok), "custom", c_out, c_in,
                    n_tok, n_groups, dtype, _store(w, dtype), _store(x, dtype))


@dataclass
class RaggedCapture:
    """Token-major activations of several groups (MoE experts) in one buffer:
    rows offsets[g] .. offsets[g+1]-1 belong to group g."""
    name: str
    description: str
    c_in: int
    dtype: str
    x: torch.Tensor          # [n_rows, c_in], CPU, token-major
    offsets: np.ndarray      # int64 [n_groups + 1]

    @property
    def n_groups(self) -> int:
        return len(self.offsets) - 1

    @property
    def x_bytes(self) -> int:
        return self.x.numel() * self.x.element_size()


def make_ragged(n_groups: int, c_in: int, n_rows: int, dtype: str = BF16, seed: int = 0,
                concentration: float = 0.3, n_empty: int = 0) -> RaggedCapture:
    """Skewed routing: group shares ~ Dirichlet(concentration) (small values
    give a few heavy experts and many light ones), `n_empty` groups forced to
    zero rows, counts rounded so they sum to n_rows; rows ~ N(0, 1) with a
    log-normal scale per channel.  Streams: SeedSequence(seed).spawn(3) for
    the shares, the empty picks and the values."""
    s_share, s_empty, s_val = [np.random.default_rng(q) for q in np.random.SeedSequence(seed).spawn(3)]
    share = s_share.dirichlet(np.full(n_groups, concentration))
    if n_empty:
        share[s_empty.choice(n_groups, n_empty, replace=False)] = 0.0
        share /= share.sum()
    counts = np.floor(share * n_rows).astype(np.int64)
    rest = n_rows - int(counts.sum())
    order = np.argsort(-(share * n_rows - counts))  # largest remainders first
    counts[order[:rest]] += 1
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    x = _normal(s_val, (n_rows, c_in)) * np.exp(s_val.standard_normal(c_in)).astype(np.float32)
    desc = ("ragged capture: %d groups, X[%d tokens x %d] %s token-major, Dirichlet(%g) routing shares, "
            "%d empty groups, channel scales exp(N(0,1))" % (n_groups, n_rows, c_in, dtype, concentration, n_empty))
    return RaggedCapture("ragged-%dx%d" % (n_groups, c_in), desc, c_in, dtype, _store(x, dtype), offsets)


def make_ragged_moe() -> RaggedCapture:
    """The MoE layer's activations as hooks would capture them: 64 experts,
    C_in 2048, the 32768 routed tokens (64 x 512 on average) split by skewed
    routing, 4 experts without tokens."""
    return make_ragged(64, 2048, 64 * 512, BF16, seed=2004, concentration=0.3, n_empty=4)
