"""Shared helpers of the GPU parity tests (test code only)."""
import numpy as np
import torch

import oracle as O
import synth

TAU = 1e-5  # near-tie threshold: decisions closer than this to their boundary are counted, not failed
ATTN_MAX_ABS = 2e-2
ATTN_MEAN_ABS = 2e-3
# log-sum-exp: the attention weights are rounded to bf16 before they meet V on the MFMA, and the
# normaliser is the sum of those same rounded weights. bf16 keeps 8 significant bits (7 stored and
# the implicit one), so round-to-nearest has a relative error of at most the unit roundoff 2^-8
# (reached just above a power of two: 1 + 2^-8 rounds to 1); a sum of positive values each off by
# at most a relative 2^-8 is off by at most a relative 2^-8, so |d lse| <= log(1 + 2^-8) = 3.90e-3.
# The fp32 terms on top (scores accumulated from 128 bf16 products, running sums over N / 32 tiles)
# stay below 1e-4 at these sizes. Measured: at most 3.5e-3 on small hand-built selections where a
# query sees a few keys (no averaging of the rounding), at most 4.4e-4 on the full-size layers.
LSE_ABS = 4e-3
MAP_ABS = 1e-5


def to64(t):
    """Exact float64 copy of a device tensor (bf16 and fp32 values are exact in fp64)."""
    return t.detach().to(torch.float64).cpu().numpy()


def np_i(t):
    return t.detach().cpu().numpy().astype(np.int64)


SMALL = {
    # several 128-row attention tiles, 1024-token sort chunks and a 4096-token metric block, all with
    # ragged tails
    "small": synth.custom("small", heads=2, grid=(6, 15, 37), d=128, dtype="bf16", centres=24, norm=8.0,
                          patch=(3, 5, 5), cq=24, ck=96, iters=4, p=0.9),
    "small64": synth.custom("small64", heads=2, grid=(5, 12, 31), d=64, dtype="bf16", centres=16, norm=6.0,
                            patch=(2, 4, 8), cq=16, ck=40, iters=4, p=0.9),
    "tiny": synth.WORKLOADS["tiny"],
    # more heads than the cooperative seeding can hold on the CUs (the single-work-group seeding
    # runs for every head and side)
    "many_heads": synth.custom("many_heads", heads=1000, grid=(4, 32, 32), d=64, dtype="bf16", centres=16,
                               norm=6.0, patch=(2, 4, 8), cq=32, ck=64, iters=2, p=0.9),
    # both sides at the ABI's cluster limit (2048), two tokens per cluster on average
    "maxc": synth.custom("maxc", heads=1, grid=(4, 32, 32), d=128, dtype="bf16", centres=24, norm=8.0,
                         patch=(2, 4, 8), cq=2048, ck=2048, iters=1, p=0.9),
    # fp32 data at d = 128 (fp32 assignment and map kernels, 128-query fp32 attention work items)
    "small32": synth.custom("small32", heads=2, grid=(5, 13, 29), d=128, dtype="f32", centres=16, norm=8.0,
                            patch=(2, 4, 8), cq=20, ck=60, iters=4, p=0.9),
}


def inputs(w, seed=0, heads=None):
    Q, K, V = synth.make_qkv(w, seed=seed, heads=heads)
    return Q.cuda(), K.cuda(), V.cuda()


def attn_view(w, x):
    """Values the attention kernels read: bf16 (fp32 data is rounded on load)."""
    x = to64(x)
    return x if w.dtype == "bf16" else O.round_bf16(x)


def cols_list(counts_h, cols_h):
    return [cols_h[i, :counts_h[i]] for i in range(counts_h.shape[0])]


def check_topp_rows(A, sizes, p, counts_g, cols_g, keys_g):
    """Compare GPU top-p rows with the oracle fed the GPU map. Returns (near_ties, bad_rows)."""
    mask_o, counts_o, cols_o, keys_o, margin = O.select_topp(A, sizes, p, return_margin=True)
    near, bad = 0, []
    for i in range(A.shape[0]):
        cg = cols_g[i, :counts_g[i]]
        if np.array_equal(cg, cols_o[i]) and keys_g[i] == keys_o[i]:
            continue
        # a differing row is a near-tie when the cumulative sum at the cut is within TAU of p, or
        # when the blocks that differ have importances within TAU of each other
        diff = np.setxor1d(cg, cols_o[i])
        vals = A[i, diff]
        kept = A[i, cols_o[i]]
        tie_val = kept.size and np.all(np.abs(vals - kept.min()) <= TAU)
        if margin[i] <= TAU or tie_val:
            near += 1
        else:
            bad.append(i)
    return near, bad
