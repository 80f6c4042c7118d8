"""Seeded synthetic attention inputs shaped like the video-DiT layers on the PARK pages.

This module only draws random numbers. It holds none of the retrieval or attention arithmetic,
so both the oracle side and the HIP side of the tests may use it.

Workload recipe (one latent token per (t, y, x) grid cell, row-major order):
  * one set of ``centres`` Gaussian directions per head, each scaled to norm ``norm``;
  * the grid is cut into ``patch`` = (pt, ph, pw) spatio-temporal patches (edge patches may be
    partial); every patch draws one centre uniformly;
  * each token takes its patch's centre, except a ``reassign`` fraction that draws a centre
    uniformly from all of them (one Bernoulli draw per token);
  * q = centre + N(0, I), k = centre + N(0, I) (independent noise), v = N(0, I);
  * bf16 workloads round fp32 values to bfloat16 (round to nearest even);
  * heads draw from independent generator streams.
The PARK pages measure on real HunyuanVideo / Wan activations, which are not available here; the
shapes below stand in for them (PARK page, Tables 1-3 and 7-8 name the models).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    grid: tuple  # (T, H, W) latent grid
    d: int
    dtype: str  # "f32" or "bf16"
    centres: int
    norm: float
    patch: tuple
    reassign: float
    cq: int
    ck: int
    iters: int
    p: float
    steps: int = 1
    anchors: tuple = (0,)
    warm_iters: int = 2
    drift: tuple = (0.95, 0.31)

    @property
    def n(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


WORKLOADS = {
    # 1 head, d=64, fp32, 4x16x32 grid, 16 centres of norm 6, 2x4x8 patches, Cq=16, Ck=32.
    "tiny": Workload("tiny", 1, (4, 16, 32), 64, "f32", 16, 6.0, (2, 4, 8), 0.2, 16, 32, 10, 0.9),
    # Wan-shaped layer: 40 heads, d=128, bf16, 21x45x80 = 75,600 tokens, Cq=100, Ck=500.
    "wan": Workload("wan", 40, (21, 45, 80), 128, "bf16", 64, 8.0, (3, 5, 5), 0.2, 100, 500, 10, 0.9),
    # HunyuanVideo-shaped layer: 24 heads, 33x45x80 = 118,800 tokens, Cq=128, Ck=512.
    "hunyuan": Workload("hunyuan", 24, (33, 45, 80), 128, "bf16", 64, 8.0, (3, 5, 5), 0.2, 128, 512, 10, 0.9),
    # One GPU's share of the Wan-shaped layer when its 40 heads are split over eight GPUs (heads are
    # independent, so a head shard runs the same path): heads 0-4 of the Wan layer.
    "wan_shard8": Workload("wan_shard8", 5, (21, 45, 80), 128, "bf16", 64, 8.0, (3, 5, 5), 0.2, 100, 500, 10, 0.9),
    # Long clip: 40 heads, 61x45x80 = 219,600 tokens, Cq=200, Ck=1000, 10 drifting steps,
    # full K-means at steps 0 and 5, two warm-started iterations otherwise.
    "long": Workload("long", 40, (61, 45, 80), 128, "bf16", 64, 8.0, (3, 5, 5), 0.2, 200, 1000, 10, 0.9,
                     steps=10, anchors=(0, 5), warm_iters=2),
}

# Sparsity sweep on the Wan-shaped layer.
SWEEP_P = (0.5, 0.7, 0.9, 0.95, 1.0)
SWEEP_CK = (250, 500, 1000)


def _head_generator(seed: int, head: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + head * 7919 + 17) & ((1 << 63) - 1))
    return g


def token_centres(w: Workload, seed: int, head: int, device="cpu") -> torch.Tensor:
    """Latent centre index of every token of one head (int64 [N])."""
    g = _head_generator(seed, head, device)
    T, H, W = w.grid
    pt, ph, pw = w.patch
    nt, nh, nw = -(-T // pt), -(-H // ph), -(-W // pw)
    patch_centre = torch.randint(0, w.centres, (nt * nh * nw,), generator=g, device=device)
    t = torch.arange(T, device=device).view(T, 1, 1) // pt
    y = torch.arange(H, device=device).view(1, H, 1) // ph
    x = torch.arange(W, device=device).view(1, 1, W) // pw
    pid = ((t * nh + y) * nw + x).reshape(-1)
    cen = patch_centre[pid]
    moved = torch.rand(w.n, generator=g, device=device) < w.reassign
    other = torch.randint(0, w.centres, (w.n,), generator=g, device=device)
    return torch.where(moved, other, cen)


def _head_fp32(w: Workload, seed: int, head: int, device):
    cen = token_centres(w, seed, head, device)
    g2 = _head_generator(seed + 0x5151, head, device)
    dirs = torch.randn(w.centres, w.d, generator=g2, device=device)
    dirs = dirs / dirs.norm(dim=1, keepdim=True) * w.norm
    q = dirs[cen] + torch.randn(w.n, w.d, generator=g2, device=device)
    k = dirs[cen] + torch.randn(w.n, w.d, generator=g2, device=device)
    v = torch.randn(w.n, w.d, generator=g2, device=device)
    return q, k, v


def make_qkv(w: Workload, seed: int = 0, device="cpu", heads=None, keep_fp32: bool = False):
    """Q, K, V as contiguous [heads, N, d] tensors of the workload's dtype.

    ``heads`` limits generation to the first ``heads`` heads (sampled tests). With ``keep_fp32`` the
    fp32 masters of Q and K are returned as well (used by the drifting multi-step workload).
    """
    nh = w.heads if heads is None else heads
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    Q = torch.empty(nh, w.n, w.d, dtype=dt, device=device)
    K = torch.empty_like(Q)
    V = torch.empty_like(Q)
    if keep_fp32:
        Qm = torch.empty(nh, w.n, w.d, dtype=torch.float32, device=device)
        Km = torch.empty_like(Qm)
    for h in range(nh):
        q, k, v = _head_fp32(w, seed, h, device)
        Q[h].copy_(q)
        K[h].copy_(k)
        V[h].copy_(v)
        if keep_fp32:
            Qm[h].copy_(q)
            Km[h].copy_(k)
    if keep_fp32:
        return Q, K, V, Qm, Km
    return Q, K, V


def drift_step(w: Workload, master: torch.Tensor, seed: int, step: int, which: int) -> torch.Tensor:
    """One denoising-step drift x_t = a * x_{t-1} + b * N(0, 1) on an fp32 master, in place.

    Returns the master rounded to the workload dtype.
    """
    a, b = w.drift
    g = torch.Generator(device=master.device)
    g.manual_seed((seed * 2_000_029 + step * 131 + which * 7 + 3) & ((1 << 63) - 1))
    noise = torch.randn(master.shape, generator=g, device=master.device, dtype=torch.float32)
    master.mul_(a).add_(noise, alpha=b)
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    return master.to(dt).contiguous()


def custom(name="custom", heads=1, grid=(4, 16, 32), d=64, dtype="f32", centres=16, norm=6.0,
           patch=(2, 4, 8), reassign=0.2, cq=16, ck=32, iters=10, p=0.9) -> Workload:
    """A workload of the same recipe with other sizes (parity cases with ragged tails)."""
    return Workload(name, heads, tuple(grid), d, dtype, centres, norm, tuple(patch), reassign, cq, ck,
                    iters, p)
