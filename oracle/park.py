"""fp64 reference of every step of PARK retrieval and the block-sparse attention it drives.

TEST INFRASTRUCTURE ONLY (see the package docstring). Per attention head; heads are independent.

Notation (per head): X is an [N, d] array of queries or keys, s the softmax scale (1/sqrt(d) by
default), C a number of clusters. All arithmetic is numpy float64 unless a function says it models
how a stored value is rounded (``round_bf16``, ``round_f32``): those roundings are part of what the
method consumes, not of how it is computed.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "EUCLID", "QRKC", "SIDE_Q", "SIDE_K",
    "splitmix64_next", "splitmix64_first", "kpp_uniform",
    "round_f32", "round_bf16",
    "qrkc_metric", "metric_distance", "candidate_rows", "kmeanspp", "consumed_centroids",
    "assign", "assign_near_tie", "cluster_order", "update", "lloyd", "subset_rows", "lloyd_subset", "cluster",
    "pama", "select_topp", "topk_count", "select_topk", "merge_cost", "merge_clusters", "merged_order", "key_runs", "sparse_attention", "dense_attention",
    "SIDE_SIP", "sip_uniform", "sip_probabilities", "select_sip", "weighted_sparse_attention",
    "recall", "density", "estimator_maps", "estimator_block_maps", "tv_to_full", "raw_key_mse", "qk_score_sq_error",
    "centered_log_mass_error", "retrieve", "forward",
]

EUCLID = 0
QRKC = 1
SIDE_Q = 0
SIDE_K = 1
SIDE_SIP = 2  # random stream of the block sampling (select_sip)

_M64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15


# --------------------------------------------------------------------------------------------
# Random draws. SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
# generators", OOPSLA 2014): the state advances by the golden-ratio increment and each output is
# the state passed through a 64-bit finaliser (two xor-shift-multiply rounds and a xor-shift).
# --------------------------------------------------------------------------------------------

def _mix64(z: int) -> int:
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def splitmix64_next(state: int):
    """One SplitMix64 step: returns (new_state, output)."""
    state = (state + _GAMMA) & _M64
    return state, _mix64(state)


def splitmix64_first(seed: int) -> int:
    """First output of a SplitMix64 generator seeded with ``seed``."""
    return splitmix64_next(seed & _M64)[1]


def kpp_uniform(seed: int, head: int, side: int, m: int) -> float:
    """The m-th uniform draw in [0, 1) of the k-means++ seeding of (head, side).

    Reading (the pages give no initialisation): a counter-based stream, u_m = 53 high bits of the
    first SplitMix64 output seeded with seed ^ (head << 32) ^ (side << 24) ^ m, times 2^-53.
    """
    key = (seed ^ (head << 32) ^ (side << 24) ^ m) & _M64
    return (splitmix64_first(key) >> 11) * (2.0 ** -53)


# --------------------------------------------------------------------------------------------
# Roundings of stored values
# --------------------------------------------------------------------------------------------

def round_f32(x):
    """Round to the nearest float32 (ties to even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(x):
    """Round float32 values to bfloat16 (nearest, ties to even), returned as float64.

    Works on the float32 bit pattern: add 0x7FFF plus the lowest kept bit, then clear the 16 low
    bits. Inputs are first rounded to float32.
    """
    b = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------------------------
# QRKC key metric
# --------------------------------------------------------------------------------------------

def qrkc_metric(Q):
    """Query-derived key metric M = (1/N) * sum_t q_t q_t^T (uncentered second moment).

    PARK page, Figure 2 caption and abstract: keys are transformed with a metric derived from the
    current queries so that keys that receive similar QK scores are grouped together. Reading: the
    key distance is D_M(k, c) = (k - c)^T M (k - c) = mean over the current queries q of
    (q.k - q.c)^2, the mean squared QK-score difference; full rank, uniform query weights.
    """
    Q = np.asarray(Q, dtype=np.float64)
    return Q.T @ Q / Q.shape[0]


def metric_distance(P, c, M=None):
    """Squared distance of each row of P to c: Euclidean when M is None, else (p-c)^T M (p-c)."""
    diff = np.asarray(P, dtype=np.float64) - np.asarray(c, dtype=np.float64)[None, :]
    if M is None:
        return np.einsum("ij,ij->i", diff, diff)
    return ((diff @ np.asarray(M, dtype=np.float64)) * diff).sum(axis=1)


# --------------------------------------------------------------------------------------------
# Initialisation: k-means++ (Arthur & Vassilvitskii 2007), single trial
# --------------------------------------------------------------------------------------------

def candidate_rows(n: int, c: int):
    """Rows that k-means++ samples from: floor(i * n / S) for i < S, S = min(n, max(4096, 8c)).

    Reading: the pages give no initialisation; seeding from a strided subsample keeps the
    sequential seeding cheap at video token counts, and uses every row when n <= 4096.
    """
    S = min(n, max(4096, 8 * c))
    return (np.arange(S, dtype=np.int64) * n) // S


def kmeanspp(X, C, M=None, seed=0, head=0, side=SIDE_Q, draws=None, return_trace=False):
    """k-means++ seeding of C centres from the candidate rows of X.

    First centre: candidate floor(u_0 * S). Centre m >= 1: the smallest candidate t whose running
    sum of D^2 exceeds u_m * sum(D^2), where D^2 is each candidate's distance to its nearest chosen
    centre (Euclidean, or the QRKC metric when M is given). When every D^2 is zero the lowest
    unchosen candidate is taken. ``draws(m)`` overrides the uniform stream (used by fixtures).
    Returns the chosen centres (float64 copies of rows of X) and, with ``return_trace``, the chosen
    candidate indices and each step's relative margin to the nearest sampling boundary.
    """
    X = np.asarray(X, dtype=np.float64)
    n = X.shape[0]
    if not 1 <= C <= n:
        raise ValueError("need 1 <= C <= N")
    rows = candidate_rows(n, C)
    P = X[rows]
    S = P.shape[0]
    u = draws if draws is not None else (lambda m: kpp_uniform(seed, head, side, m))
    chosen = [min(int(u(0) * S), S - 1)]
    margins = [1.0]
    D2 = metric_distance(P, P[chosen[0]], M)
    D2[chosen[0]] = 0.0
    taken = np.zeros(S, dtype=bool)
    taken[chosen[0]] = True
    for m in range(1, C):
        prefix = np.cumsum(D2)
        total = prefix[-1]
        if not total > 0.0:
            t = int(np.flatnonzero(~taken)[0])
            margins.append(0.0)
        else:
            v = u(m) * total
            t = int(np.searchsorted(prefix, v, side="right"))
            if t >= S:  # v rounded up to the total: take the last candidate with mass
                t = int(np.flatnonzero(D2 > 0)[-1])
            lo = prefix[t - 1] if t > 0 else 0.0
            margins.append(min(prefix[t] - v, v - lo) / total)
        chosen.append(t)
        taken[t] = True
        D2 = np.minimum(D2, metric_distance(P, P[t], M))
        D2[t] = 0.0
    cent = P[np.asarray(chosen)].copy()
    if return_trace:
        return cent, rows[np.asarray(chosen)], np.asarray(margins)
    return cent


# --------------------------------------------------------------------------------------------
# Lloyd iterations
# --------------------------------------------------------------------------------------------

def consumed_centroids(cent, metric=EUCLID, M=None, bf16=True):
    """The (g, b) pairs an assignment compares a point against: label = argmin_j b_j - 2 x.g_j.

    The fp32 centroid c_j is what is stored. Euclidean: g_j = c_j (rounded to bf16 for bf16 data),
    b_j = ||g_j||^2 rounded to fp32, so b_j - 2 x.g_j = ||x - g_j||^2 - ||x||^2. QRKC: y_j = M c_j,
    g_j = y_j rounded to fp32 (then to bf16 for bf16 data), b_j = c_j^T M c_j rounded to fp32, so
    b_j - 2 x.g_j = D_M(x, c_j) - x^T M x. The dropped term does not depend on j.
    """
    c = round_f32(cent)
    if metric == EUCLID:
        g = round_bf16(c) if bf16 else c
        b = round_f32(np.einsum("ij,ij->i", g, g))
    else:
        y = c @ np.asarray(M, dtype=np.float64).T
        g = round_f32(y)
        if bf16:
            g = round_bf16(g)
        b = round_f32(np.einsum("ij,ij->i", c, y))
    return g, b


def assign(X, g, b):
    """Nearest centre of every row: argmin_j (b_j - 2 x.g_j), ties to the lowest j.

    PARK page, Figure 2 caption: queries are clustered with Euclidean K-means, keys with the
    query-derived metric; this is the assignment half of a Lloyd iteration for either.
    """
    f = np.asarray(b, dtype=np.float64)[None, :] - 2.0 * (np.asarray(X, dtype=np.float64)
                                                          @ np.asarray(g, dtype=np.float64).T)
    return np.argmin(f, axis=1).astype(np.int32)


def assign_near_tie(X, g, b, labels_other, tau=1e-5):
    """Rows where ``labels_other`` differs from the fp64 argmin, split into near-ties and errors.

    A differing row is a near-tie when f(j_other) - f(j_best) <= tau * (1 + |f(j_best)| +
    2 ||x|| ||g_best||): the gap is within what fp32 accumulation of the dot products can flip.
    Returns (n_near_ties, bad_rows).
    """
    X = np.asarray(X, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    labels_other = np.asarray(labels_other)
    jb = assign(X, g, b)
    diff = np.flatnonzero(jb != labels_other)
    if diff.size == 0:
        return 0, diff
    x = X[diff]
    fb = b[jb[diff]] - 2.0 * np.einsum("ij,ij->i", x, g[jb[diff]])
    fo = b[labels_other[diff]] - 2.0 * np.einsum("ij,ij->i", x, g[labels_other[diff]])
    bound = tau * (1.0 + np.abs(fb) + 2.0 * np.linalg.norm(x, axis=1) * np.linalg.norm(g[jb[diff]], axis=1))
    ok = (fo - fb) <= bound
    return int(ok.sum()), diff[~ok]


def cluster_order(labels, C):
    """Cluster-contiguous token order (the "Clustered" ordering of PARK Tables 1 and 10).

    A stable counting sort: offsets[j] = number of rows with label < j, and rows of one cluster
    keep their original order. Returns (perm, offsets): perm[p] is the original row at sorted
    position p; cluster j occupies positions offsets[j] .. offsets[j+1]-1.
    """
    labels = np.asarray(labels, dtype=np.int64)
    counts = np.zeros(C, dtype=np.int64)
    for lab in labels:
        counts[lab] += 1
    offsets = np.zeros(C + 1, dtype=np.int64)
    for j in range(C):
        offsets[j + 1] = offsets[j] + counts[j]
    cursor = offsets[:-1].copy()
    perm = np.empty(labels.shape[0], dtype=np.int64)
    for t, lab in enumerate(labels):
        perm[cursor[lab]] = t
        cursor[lab] += 1
    return perm.astype(np.int32), offsets.astype(np.int32)


def update(X, labels, C, previous):
    """Centroid update: c_j = mean of the rows labelled j, stored in fp32; empty clusters keep
    their previous centroid. (A Lloyd iteration's second half; under the QRKC metric the mean is
    still the minimiser because M is positive semi-definite.)"""
    X = np.asarray(X, dtype=np.float64)
    labels = np.asarray(labels)
    out = round_f32(previous).copy()
    for j in range(C):
        rows = X[labels == j]
        if rows.shape[0]:
            out[j] = rows.sum(axis=0) / rows.shape[0]
    return round_f32(out)


def lloyd(X, init, iters, metric=EUCLID, M=None, bf16=True, trace=None):
    """``iters`` Lloyd iterations (assign against the consumed centroids, then update).

    Returns (labels of the last assignment, centroids after the last update). ``trace`` (a list)
    receives (labels, centroids) after every iteration.
    """
    c = round_f32(init)
    labels = None
    for _ in range(iters):
        g, b = consumed_centroids(c, metric, M, bf16)
        labels = assign(X, g, b)
        c = update(X, labels, c.shape[0], c)
        if trace is not None:
            trace.append((labels, c))
    return labels, c


def subset_rows(n: int, stride: int, phase: int):
    """Tokens a subset update re-assigns: phase, phase + stride, phase + 2 stride, ... below n.

    HyperVAttention page, abstract: between anchor steps only a subset of the tokens is updated.
    Reading (the page does not say which subset): a strided one, so that successive steps with
    phase = step mod stride cover every token once per stride steps, with the subset spread
    evenly over the spatio-temporal grid.
    """
    return np.arange(phase, n, stride, dtype=np.int64)


def lloyd_subset(X, init, labels, iters, stride, phase, metric=EUCLID, M=None, bf16=True):
    """Subset update of a clustering (hybrid clustering between anchor steps, HyperVAttention page,
    abstract): ``iters`` iterations, each re-assigning only the rows of ``subset_rows`` against the
    consumed form of the current centroids (the other rows keep their labels, e.g. from the previous
    denoising step), then setting every centroid to the mean of its members under the combined
    labels, over the current values of all rows (empty clusters keep their centroid).
    Returns (labels, centroids). stride = 1 is a full warm-started Lloyd iteration.
    """
    X = np.asarray(X, dtype=np.float64)
    lab = np.asarray(labels, dtype=np.int64).copy()
    rows = subset_rows(X.shape[0], stride, phase)
    c = round_f32(init)
    for _ in range(iters):
        g, b = consumed_centroids(c, metric, M, bf16)
        lab[rows] = assign(X[rows], g, b)
        c = update(X, lab, c.shape[0], c)
    return lab.astype(np.int32), c


def cluster(X, C, iters, metric=EUCLID, M=None, seed=0, head=0, side=SIDE_Q, bf16=True, init=None):
    """Seed (k-means++, or ``init`` for a warm start) and run ``iters`` Lloyd iterations.

    Returns dict(labels, centroids, perm, offsets). With iters == 0 only the centroids are set.
    """
    c0 = kmeanspp(X, C, M if metric == QRKC else None, seed, head, side) if init is None else init
    labels, c = lloyd(X, c0, iters, metric, M, bf16)
    out = {"centroids": round_f32(c) if iters == 0 else c, "labels": labels}
    if labels is not None:
        out["perm"], out["offsets"] = cluster_order(labels, C)
    return out


# --------------------------------------------------------------------------------------------
# PAMA block-importance map
# --------------------------------------------------------------------------------------------

def pama(Q, q_perm, q_offsets, k_cent, k_sizes, scale, rows=None):
    """Block-importance map A [Cq, Ck].

    PARK page, Figure 2 caption and abstract: every original query keeps its own softmax over the
    key centroids, and these distributions are averaged within each query block. Readings: the
    logit of key cluster j is s * q.c_j + ln n_j (a cluster of n_j keys that all score q.c_j
    carries n_j * exp(s q.c_j) of the softmax mass); empty key clusters get weight 0; the average
    is the unweighted mean over the block's queries; an empty query block gives a zero row.
    ``k_cent`` are the key centroids as consumed. ``rows`` limits the result to some query blocks.
    """
    Q = np.asarray(Q, dtype=np.float64)
    k_cent = np.asarray(k_cent, dtype=np.float64)
    k_sizes = np.asarray(k_sizes, dtype=np.int64)
    cq = len(q_offsets) - 1
    ck = k_cent.shape[0]
    logn = np.full(ck, -np.inf)
    logn[k_sizes > 0] = np.log(k_sizes[k_sizes > 0].astype(np.float64))
    A = np.zeros((cq, ck))
    for i in (range(cq) if rows is None else rows):
        t = np.asarray(q_perm[q_offsets[i]:q_offsets[i + 1]])
        if t.size == 0:
            continue
        lg = scale * (Q[t] @ k_cent.T) + logn[None, :]
        lg -= lg.max(axis=1, keepdims=True)
        w = np.exp(lg)
        w /= w.sum(axis=1, keepdims=True)
        A[i] = w.mean(axis=0)
    return A


# --------------------------------------------------------------------------------------------
# Top-p selection
# --------------------------------------------------------------------------------------------

def select_topp(A, k_sizes, p, return_margin=False):
    """Row-wise top-p cut of the block map (PARK page, Table 1 caption: top-p retrieval, p = 0.9).

    For each row: order key clusters by importance (descending, ties to the lower index) and keep
    the shortest prefix whose cumulative importance reaches p. Readings: p >= 1 keeps every
    non-empty key cluster; when rounding keeps the row total below p, every block with positive
    importance is kept; empty key clusters are never kept; an all-zero row keeps nothing.
    Returns (mask bool [Cq, Ck], counts [Cq], cols list of ascending int arrays, keys [Cq]) where
    keys[i] is the number of keys row i attends to. With ``return_margin`` also the per-row
    distance of the deciding cumulative sum to p (np.inf when no cut was made).
    """
    A = np.asarray(A, dtype=np.float64)
    k_sizes = np.asarray(k_sizes, dtype=np.int64)
    cq, ck = A.shape
    mask = np.zeros((cq, ck), dtype=bool)
    margin = np.full(cq, np.inf)
    for i in range(cq):
        row = A[i]
        if not (row > 0).any():
            continue
        if p >= 1.0:
            mask[i] = k_sizes > 0
            continue
        order = np.lexsort((np.arange(ck), -row))
        cum = np.cumsum(row[order])
        hit = np.flatnonzero(cum >= p)
        if hit.size:
            k = int(hit[0])
            mask[i, order[:k + 1]] = True
            margin[i] = min(cum[k] - p, p - cum[k - 1] if k > 0 else np.inf)
        else:
            mask[i] = row > 0
        mask[i] &= k_sizes > 0
    counts = mask.sum(axis=1).astype(np.int32)
    cols = [np.flatnonzero(mask[i]).astype(np.int32) for i in range(cq)]
    keys = (mask * k_sizes[None, :]).sum(axis=1).astype(np.int64)
    if return_margin:
        return mask, counts, cols, keys, margin
    return mask, counts, cols, keys


def topk_count(k_sizes, rho):
    """Blocks a top-k row keeps at retrieval ratio rho (PARK-p2 Table 10: top-k retrieval at a fixed
    ratio rho = 0.1). Reading: rho is the share of the head's non-empty key blocks, rounded up,
    k = ceil(rho * C_ne - 1e-9) clamped to [1, C_ne] (the 1e-9 keeps an exact product such as
    0.3 * 10 from rounding up to the next integer)."""
    c_ne = int((np.asarray(k_sizes) > 0).sum())
    if c_ne == 0:
        return 0
    return int(min(max(math.ceil(rho * c_ne - 1e-9), 1), c_ne))


def select_topk(A, k_sizes, rho):
    """Row-wise top-k cut of the block map: every row with positive importance keeps the k
    non-empty key blocks of highest importance (ties to the lower index), k = topk_count(rho);
    rows without positive importance (empty query blocks) keep nothing. Returns the same
    (mask, counts, cols, keys) as select_topp."""
    A = np.asarray(A, dtype=np.float64)
    k_sizes = np.asarray(k_sizes, dtype=np.int64)
    cq, ck = A.shape
    k = topk_count(k_sizes, rho)
    mask = np.zeros((cq, ck), dtype=bool)
    live = np.flatnonzero(k_sizes > 0)
    for i in range(cq):
        row = A[i]
        if not (row > 0).any():
            continue
        order = live[np.lexsort((live, -row[live]))]
        mask[i, order[:k]] = True
    counts = mask.sum(axis=1).astype(np.int32)
    cols = [np.flatnonzero(mask[i]).astype(np.int32) for i in range(cq)]
    keys = (mask * k_sizes[None, :]).sum(axis=1).astype(np.int64)
    return mask, counts, cols, keys


def sip_uniform(seed: int, head: int, i: int, j: int, ck: int) -> float:
    """Uniform draw in [0, 1) that decides whether row i samples key block j (select_sip).

    Reading (the page fixes no generator): the k-means++ counter stream of stream id 2, counter
    i * ck + j: 53 high bits of the first SplitMix64 output seeded with
    seed ^ (head << 32) ^ (2 << 24) ^ (i * ck + j), times 2^-53."""
    key = (seed ^ (head << 32) ^ (SIDE_SIP << 24) ^ (i * ck + j)) & _M64
    return (splitmix64_first(key) >> 11) * (2.0 ** -53)


def sip_probabilities(a, m):
    """Inclusion probabilities of one map row for sampling m blocks in expectation.

    AB-Attention page (SIP paragraph): blocks are sampled according to their estimated
    importance. Reading: probability proportional to importance, capped at 1,
    pi_j = min(1, kappa * a_j) over the blocks with a_j > 0 (others 0), with kappa chosen so that
    sum_j pi_j = m; when m reaches the number of positive blocks every one of them has pi = 1.
    Water filling: order the positive a descending (ties to the lower index); with the t largest
    capped at 1 the rest share m - t, kappa_t = (m - t) / (sum of the rest); the answer is the
    smallest t whose largest uncapped entry satisfies kappa_t * a <= 1.
    """
    a = np.asarray(a, dtype=np.float64)
    pi = np.zeros_like(a)
    pos = np.flatnonzero(a > 0)
    if pos.size == 0 or m <= 0:
        return pi
    if m >= pos.size:
        pi[pos] = 1.0
        return pi
    order = pos[np.lexsort((pos, -a[pos]))]
    vals = a[order]
    rest = np.cumsum(vals[::-1])[::-1]  # rest[t] = sum of vals[t:]
    for t in range(pos.size):
        kappa = (m - t) / rest[t]
        if kappa * vals[t] <= 1.0:
            break
    pi[order[:t]] = 1.0
    pi[order[t:]] = np.minimum(kappa * vals[t:], 1.0)
    return pi


def select_sip(A, k_sizes, rho, seed=0, head=0):
    """Sampling with inclusion-probability weighting of every map row (AB-Attention page, SIP
    paragraph: sample blocks by estimated importance instead of truncating, reweight each sampled
    block by the inverse of its inclusion probability).

    Readings: the expected number of sampled blocks per row is the top-k budget at ratio rho,
    m = topk_count(k_sizes, rho); empty key clusters have importance 0 (never sampled); block j of
    row i is kept iff sip_uniform(seed, head, i, j) < pi_ij; a kept block carries the log weight
    ln(1 / pi_ij). Returns (mask, counts, cols, keys, log_w, pi): the first four as select_topp,
    log_w [Cq, Ck] (0 where not kept) and the probabilities pi [Cq, Ck].
    """
    A = np.asarray(A, dtype=np.float64)
    k_sizes = np.asarray(k_sizes, dtype=np.int64)
    cq, ck = A.shape
    m = topk_count(k_sizes, rho)
    mask = np.zeros((cq, ck), dtype=bool)
    log_w = np.zeros((cq, ck))
    pi = np.zeros((cq, ck))
    for i in range(cq):
        a = np.where(k_sizes > 0, np.maximum(A[i], 0.0), 0.0)
        pi[i] = sip_probabilities(a, m)
        for j in np.flatnonzero(pi[i] > 0):
            if sip_uniform(seed, head, i, int(j), ck) < pi[i, j]:
                mask[i, j] = True
                log_w[i, j] = -math.log(pi[i, j])
    counts = mask.sum(axis=1).astype(np.int32)
    cols = [np.flatnonzero(mask[i]).astype(np.int32) for i in range(cq)]
    keys = (mask * k_sizes[None, :]).sum(axis=1).astype(np.int64)
    return mask, counts, cols, keys, log_w, pi


def merge_cost(n_q, keys, bm: int):
    """CTA-aligned cost of a query group (HyperVAttention page, abstract: clusters are processed in
    fixed-size tiles, so a group of n_q queries occupies ceil(n_q / bm) tiles, each running over
    every selected key): ceil(n_q / bm) * keys."""
    return -(-int(n_q) // bm) * int(keys)


def merge_clusters(q_sizes, cols, k_sizes, bm: int):
    """Tile-aware merging of query clusters by parallel agglomeration (HyperVAttention page,
    abstract: merging that lowers the CTA-aligned execution cost fills idle tile capacity and
    makes every merged query attend to the union of the selections).

    Reading (the page gives the idea only): groups start as the non-empty query clusters (empty ones
    stay alone and select nothing). A group G has n(G) queries, selection S(G) = union of its
    clusters' selections and cost merge_cost(n(G), L(S(G)), bm), L = total size of the key clusters.
    Each round every group proposes the partner with the largest positive gain
    cost(a) + cost(b) - cost(a u b) (ties to the lower index); pairs that propose each other merge
    into the lower index. The gain is symmetric, so the pair of largest gain always proposes itself
    and every round with a positive gain merges; the rounds stop when no pair gains.
    Returns (group, sel): group[i] = the lowest cluster index of i's group, sel[r] = the sorted
    union selection of the group with root r.
    """
    q_sizes = np.asarray(q_sizes, dtype=np.int64)
    k_sizes = np.asarray(k_sizes, dtype=np.int64)
    cq = q_sizes.size
    parent = np.arange(cq)
    n = {i: int(q_sizes[i]) for i in range(cq) if q_sizes[i] > 0}
    S = {i: set(int(j) for j in cols[i]) for i in n}

    def L(sel):
        return int(sum(k_sizes[j] for j in sel))

    def cost(i):
        return merge_cost(n[i], L(S[i]), bm)

    while True:
        roots = sorted(n)
        best = {}
        for a in roots:
            ba, bg = -1, 0
            for b in roots:
                if b == a:
                    continue
                g = cost(a) + cost(b) - merge_cost(n[a] + n[b], L(S[a] | S[b]), bm)
                if g > bg:
                    ba, bg = b, g
            best[a] = ba
        pairs = [(a, b) for a, b in best.items() if b > a and best.get(b) == a]
        if not pairs:
            break
        for a, b in pairs:
            n[a] += n.pop(b)
            S[a] |= S.pop(b)
            parent[parent == b] = a
    group = parent.copy()
    sel = {r: np.array(sorted(S.get(r, set())), dtype=np.int64) for r in set(group.tolist())}
    for i in range(cq):
        if q_sizes[i] == 0:
            sel[i] = np.array([], dtype=np.int64)
    return group, sel


def merged_order(q_perm, q_offsets, group, sel):
    """The merged groups as a query clustering: groups in increasing order of their lowest cluster,
    each group's queries cluster by cluster in increasing cluster order (each cluster's queries in
    their q_perm order). Returns (perm, offsets, cols) with cq slots: slot g < G holds the g-th
    group, slots G .. cq - 1 are empty."""
    q_perm = np.asarray(q_perm)
    q_offsets = np.asarray(q_offsets)
    cq = q_offsets.size - 1
    roots = sorted(set(np.asarray(group).tolist()))
    perm, offsets, cols = [], [0], [np.array([], dtype=np.int64) for _ in range(cq)]
    for g, r in enumerate(roots):
        for i in range(cq):
            if group[i] == r:
                perm.extend(q_perm[q_offsets[i]:q_offsets[i + 1]].tolist())
        offsets.append(len(perm))
        cols[g] = sel[r]
    offsets += [len(perm)] * (cq + 1 - len(offsets))
    return np.array(perm, dtype=np.int32), np.array(offsets, dtype=np.int32), cols


def key_runs(cols, k_offsets):
    """Key ranges in sorted-key positions that one query block attends to: selected clusters in
    ascending order, adjacent clusters merged into one run. Returns a list of (start, end)."""
    runs = []
    for j in cols:
        a, b = int(k_offsets[j]), int(k_offsets[j + 1])
        if a == b:
            continue
        if runs and runs[-1][1] == a:
            runs[-1] = (runs[-1][0], b)
        else:
            runs.append((a, b))
    return runs


# --------------------------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------------------------

def _attend(q, k, v, scale):
    s = scale * (q @ k.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return (e @ v) / l, (m + np.log(l))[:, 0]


def sparse_attention(Q, K, V, q_perm, q_offsets, k_perm, k_offsets, cols, scale, rows=None):
    """Attention of every query over the keys of the key clusters its query block selected.

    PARK abstract: attention is computed only within the retrieved blocks. Reading: the softmax
    is renormalised over the selected keys (no reweighting of dropped mass). Outputs are in the
    original token order: O [N, d] and the log-sum-exp LSE [N] of the scaled scores over the
    selected keys. ``rows`` limits the work to the given query blocks (other rows stay NaN).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n, d = Q.shape
    O = np.full((n, V.shape[1]), np.nan)
    lse = np.full(n, np.nan)
    cq = len(q_offsets) - 1
    for i in (range(cq) if rows is None else rows):
        t = np.asarray(q_perm[q_offsets[i]:q_offsets[i + 1]])
        if t.size == 0:
            continue
        u = [np.asarray(k_perm[k_offsets[j]:k_offsets[j + 1]]) for j in cols[i]]
        u = np.concatenate(u) if u else np.zeros(0, dtype=np.int64)
        if u.size == 0:
            O[t] = 0.0
            lse[t] = -np.inf
            continue
        O[t], lse[t] = _attend(Q[t], K[u], V[u], scale)
    return O, lse


def weighted_sparse_attention(Q, K, V, q_perm, q_offsets, k_perm, k_offsets, cols, log_w, scale, rows=None):
    """Attention over the selected blocks with block weights (AB-Attention page, SIP paragraph:
    sampled blocks are reweighted by the inverse of their inclusion probability, so that one sparse
    pass estimates dense attention).

    For a query t of block i with selected key blocks S and weights w_j = exp(log_w[i, j]):
        O_t = sum_{j in S} w_j sum_{k in j} e^{s q_t.k} v_k / sum_{j in S} w_j sum_{k in j} e^{s q_t.k},
    i.e. the logit of every key of block j gains ln w_j; LSE_t is the log of the denominator (an
    estimate of the dense log-sum-exp). With log_w = 0 this is sparse_attention.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    log_w = np.asarray(log_w, dtype=np.float64)
    n, d = Q.shape
    O = np.full((n, V.shape[1]), np.nan)
    lse = np.full(n, np.nan)
    cq = len(q_offsets) - 1
    for i in (range(cq) if rows is None else rows):
        t = np.asarray(q_perm[q_offsets[i]:q_offsets[i + 1]])
        if t.size == 0:
            continue
        u, b = [], []
        for j in cols[i]:
            keys = np.asarray(k_perm[k_offsets[j]:k_offsets[j + 1]])
            u.append(keys)
            b.append(np.full(keys.size, log_w[i, j]))
        u = np.concatenate(u) if u else np.zeros(0, dtype=np.int64)
        if u.size == 0:
            O[t] = 0.0
            lse[t] = -np.inf
            continue
        s = scale * (Q[t] @ K[u].T) + np.concatenate(b)[None, :]
        mx = s.max(axis=1, keepdims=True)
        e = np.exp(s - mx)
        den = e.sum(axis=1, keepdims=True)
        O[t] = (e @ V[u]) / den
        lse[t] = (mx + np.log(den))[:, 0]
    return O, lse


def dense_attention(Q, K, V, scale, rows=None, block=2048):
    """Full softmax attention; ``rows`` limits it to some query rows (others stay NaN)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n = Q.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows)
    O = np.full((n, V.shape[1]), np.nan)
    lse = np.full(n, np.nan)
    for a in range(0, rows.size, block):
        r = rows[a:a + block]
        O[r], lse[r] = _attend(Q[r], K, V, scale)
    return O, lse


def recall(lse_sparse, lse_dense):
    """Attention recall of each query: the share of its dense softmax mass that falls on the
    selected keys, exp(LSE_selected - LSE_dense) (PARK page, Table 1: mean, P05 and worst attention
    recall; reading: per query, then averaged per head)."""
    return np.exp(np.asarray(lse_sparse, dtype=np.float64) - np.asarray(lse_dense, dtype=np.float64))


def density(mask, q_sizes, k_sizes):
    """(block density, token density): selected (query block, key block) pairs over non-empty
    pairs, and selected query-key pairs over N^2 (the computed share of dense attention work)."""
    mask = np.asarray(mask, dtype=bool)
    q_sizes = np.asarray(q_sizes, dtype=np.float64)
    k_sizes = np.asarray(k_sizes, dtype=np.float64)
    ne = np.outer(q_sizes > 0, k_sizes > 0)
    blocks = mask.sum() / max(ne.sum(), 1)
    n = q_sizes.sum()
    tokens = (mask * np.outer(q_sizes, k_sizes)).sum() / (n * k_sizes.sum())
    return float(blocks), float(tokens)


# --------------------------------------------------------------------------------------------
# Retrieval diagnostics (PARK page, Tables 1, 4, 5 and Figure 4). CPU only.
# --------------------------------------------------------------------------------------------

def _block_sum(P, k_labels, ck):
    out = np.zeros((P.shape[0], ck))
    for j in range(ck):
        out[:, j] = P[:, k_labels == j].sum(axis=1)
    return out


def estimator_maps(Q, K, q_labels, k_labels, q_cent, k_cent, scale):
    """Per-query block distributions under the four query/key representations of Table 1/Table 4.

    Returns dict name -> [N, Ck] array, each row the distribution over key blocks that stands for
    one original query:
      FF (full query, full key): exact block mass of the dense softmax;
      CC: softmax over key centroids (size-weighted) of the query's centroid;
      CF: exact block mass of the query centroid's softmax over all keys;
      FC: softmax over key centroids (size-weighted) of the query itself (PAMA's per-query rows).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    ck = k_cent.shape[0]
    sizes = np.bincount(k_labels, minlength=ck)
    logn = np.where(sizes > 0, np.log(np.maximum(sizes, 1)), -np.inf)

    def softmax(z):
        z = z - z.max(axis=1, keepdims=True)
        e = np.exp(z)
        return e / e.sum(axis=1, keepdims=True)

    ff = _block_sum(softmax(scale * Q @ K.T), k_labels, ck)
    qc = np.asarray(q_cent, dtype=np.float64)[q_labels]
    kc = np.asarray(k_cent, dtype=np.float64)
    return {
        "FF": ff,
        "CC": softmax(scale * qc @ kc.T + logn[None, :]),
        "CF": _block_sum(softmax(scale * qc @ K.T), k_labels, ck),
        "FC": softmax(scale * Q @ kc.T + logn[None, :]),
    }


def estimator_block_maps(Q, K, q_perm, q_offsets, q_cent, k_perm, k_offsets, k_cent, scale):
    """Block maps [Cq, Ck] under the four query/key representations of Table 1 (PARK-p2): each query
    block's row is the mean over its queries of the per-query block distributions of
    estimator_maps, so FC is the PAMA map; the centroid-query rows (CC, CF) are the same for every
    query of a block. Centroids enter as given (the caller passes them as consumed). An empty query
    block gets a zero row."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    cq = len(q_offsets) - 1
    ck = len(k_offsets) - 1
    q_labels = np.empty(Q.shape[0], dtype=np.int64)
    for i in range(cq):
        q_labels[np.asarray(q_perm[q_offsets[i]:q_offsets[i + 1]])] = i
    k_labels = np.empty(K.shape[0], dtype=np.int64)
    for j in range(ck):
        k_labels[np.asarray(k_perm[k_offsets[j]:k_offsets[j + 1]])] = j
    rows = estimator_maps(Q, K, q_labels, k_labels, q_cent, k_cent, scale)
    out = {}
    for name, R in rows.items():
        A = np.zeros((cq, ck))
        for i in range(cq):
            t = np.asarray(q_perm[q_offsets[i]:q_offsets[i + 1]])
            if t.size:
                A[i] = R[t].mean(axis=0)
        out[name] = A
    return out


def tv_to_full(est, ff):
    """Mean over queries of the total-variation distance between two block distributions."""
    return float(0.5 * np.abs(np.asarray(est) - np.asarray(ff)).sum(axis=1).mean())


def raw_key_mse(K, k_labels, k_cent):
    """Mean over keys of ||k - c(k)||^2 (Table 5 "raw-key MSE"; normalisation is a reading)."""
    K = np.asarray(K, dtype=np.float64)
    d = K - np.asarray(k_cent, dtype=np.float64)[k_labels]
    return float((d * d).sum(axis=1).mean())


def qk_score_sq_error(Q, K, k_labels, k_cent):
    """Mean over (query, key) pairs of (q.k - q.c(k))^2 (Table 5 "QK-score squared error")."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    d = K - np.asarray(k_cent, dtype=np.float64)[k_labels]
    e = Q @ d.T
    return float((e * e).mean())


def centered_log_mass_error(Q, K, k_labels, k_cent, scale):
    """PARITY UNPINNED. Figure 4 names a "centered log-mass error" without defining it. Reading:
    per query and non-empty key block, the log of the exact unnormalised block mass minus the log
    of its centroid estimate n_j exp(s q.c_j), centred over blocks per query; mean square."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    kc = np.asarray(k_cent, dtype=np.float64)
    ck = kc.shape[0]
    sizes = np.bincount(k_labels, minlength=ck)
    live = sizes > 0
    s = scale * Q @ K.T
    m = s.max(axis=1, keepdims=True)
    true = np.log(_block_sum(np.exp(s - m), k_labels, ck)[:, live]) + m
    est = scale * Q @ kc[live].T + np.log(sizes[live])[None, :]
    e = true - est
    e -= e.mean(axis=1, keepdims=True)
    return float((e * e).mean())


# --------------------------------------------------------------------------------------------
# The whole path for one head
# --------------------------------------------------------------------------------------------

def retrieve(Q, K, cq, ck, iters, p, scale, seed=0, head=0, bf16=True, kmetric=QRKC,
             q_init=None, k_init=None):
    """Retrieval for one head: QRKC metric, both clusterings, PAMA map and top-p selection."""
    M = qrkc_metric(Q) if kmetric == QRKC else None
    Mr = round_f32(M) if M is not None else None
    qc = cluster(Q, cq, iters, EUCLID, None, seed, head, SIDE_Q, bf16, q_init)
    kc = cluster(K, ck, iters, kmetric, Mr, seed, head, SIDE_K, bf16, k_init)
    k_sizes = np.diff(kc["offsets"])
    k_hat = round_bf16(kc["centroids"]) if bf16 else kc["centroids"]
    A = pama(Q, qc["perm"], qc["offsets"], k_hat, k_sizes, scale)
    mask, counts, cols, keys = select_topp(A, k_sizes, p)
    return {"M": Mr, "q": qc, "k": kc, "map": A, "mask": mask, "counts": counts, "cols": cols,
            "keys": keys}


def forward(Q, K, V, cq, ck, iters, p, scale, seed=0, head=0, bf16=True, kmetric=QRKC):
    """Retrieval followed by block-sparse attention for one head (attention reads bf16 values)."""
    r = retrieve(Q, K, cq, ck, iters, p, scale, seed, head, bf16, kmetric)
    Qa, Ka, Va = (round_bf16(x) for x in (Q, K, V))
    O, lse = sparse_attention(Qa, Ka, Va, r["q"]["perm"], r["q"]["offsets"], r["k"]["perm"],
                              r["k"]["offsets"], r["cols"], scale)
    r["out"], r["lse"] = O, lse
    return r
