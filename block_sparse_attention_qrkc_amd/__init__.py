"""PARK block retrieval + block-sparse attention for MI355X (gfx950).

Thin Python layer over the C ABI of ``libpark.so`` (see ``include/park.h``). Functions take and
return torch tensors on the ROCm device and enqueue on the current stream; the computation runs
entirely in the library's HIP kernels.

Method: "PARK: Accurate Block Retrieval for Sparse Attention in Video Diffusion Transformers"
(Figure 2 caption and abstract): Euclidean K-means on queries, query-aware (QRKC) K-means on keys,
cluster-contiguous token order, the PAMA block-importance map, top-p selection (Table 1 caption)
and attention restricted to the selected blocks.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import (  # noqa: F401
    EXPORTED, LIB_PATH, PARK_ENTRY_MERGE, PARK_INIT_SUBSET, STATS_FIELDS, PARK_BF16, PARK_EHIP, PARK_EINVAL, PARK_ENTRY_CLUSTER_K, PARK_ENTRY_CLUSTER_Q,
    PARK_ENTRY_ESTIMATOR, PARK_ENTRY_FORWARD, PARK_ENTRY_METRIC, PARK_ENTRY_RETRIEVE_MAP, PARK_ENTRY_SELECT_TOPP,
    PARK_ENTRY_SPARSE_ATTN, PARK_ENTRY_SPARSE_ATTN_WEIGHTED, PARK_EST_CC, PARK_EST_CF, PARK_EST_FC, PARK_EST_FF,
    PARK_EUCLID, PARK_EUNSUPPORTED, PARK_EWORKSPACE, PARK_F32, PARK_INIT_KMEANSPP, PARK_INIT_WARM, PARK_OK,
    PARK_QRKC, PARK_SIDE_K, PARK_SIDE_Q, PARK_DEVSTATUS_SEED_TIMEOUT, ParkError, Workspace, lib, make_params, make_shape, park_forward_outputs,
    park_params, park_shape, workspace_bytes,
)
from ._lib import _check, _ptr, _stream, _ws

__all__ = [
    "park_qrkc_metric", "park_cluster", "park_cluster_subset", "park_retrieve_map", "park_estimator_map", "park_select_topp",
    "park_select_topk", "park_sparse_attn", "park_merge_clusters",
    "park_permute_rows", "park_unpermute_rows", "park_forward", "park_version", "ParkError", "lib",
]


def park_version() -> str:
    return lib().park_version().decode()


def park_qrkc_metric(q, out=None, ws=None, stream=None):
    """M_h = (1/n) sum_t q_t q_t^T per head, float32 [heads, d, d]."""
    sh = make_shape(q)
    M = out if out is not None else torch.empty(sh.heads, sh.d, sh.d, dtype=torch.float32, device=q.device)
    wp, wn = _ws(PARK_ENTRY_METRIC, sh, None, q.device, ws)
    _check(lib().park_qrkc_metric(ctypes.byref(sh), _ptr(q), _ptr(M), wp, wn, _stream(stream)))
    return M


def park_cluster(x, n_clusters, iters, metric=PARK_EUCLID, qmetric=None, init=PARK_INIT_KMEANSPP, seed=0,
                 side=PARK_SIDE_Q, centroids=None, status=None, ws=None, stream=None):
    """K-means of one token side. Returns dict(centroids, labels, perm, offsets).

    With ``init=PARK_INIT_WARM`` the given ``centroids`` [heads, C, d] float32 are the start (and are
    updated in place). ``status``: optional int32 device tensor of one element; PARK_DEVSTATUS_*
    bits are or-ed into it (never cleared)."""
    sh = make_shape(x)
    H, N, D = sh.heads, sh.n, sh.d
    dev = x.device
    if centroids is None:
        if init == PARK_INIT_WARM:
            raise ValueError("warm start needs centroids")
        centroids = torch.empty(H, n_clusters, D, dtype=torch.float32, device=dev)
    labels = torch.empty(H, N, dtype=torch.int32, device=dev) if iters > 0 else None
    perm = torch.empty(H, N, dtype=torch.int32, device=dev) if iters > 0 else None
    offsets = torch.empty(H, n_clusters + 1, dtype=torch.int32, device=dev) if iters > 0 else None
    prm = make_params(cq=n_clusters, ck=n_clusters, kmetric=metric)
    entry = PARK_ENTRY_CLUSTER_K if metric == PARK_QRKC else PARK_ENTRY_CLUSTER_Q
    wp, wn = _ws(entry, sh, prm, dev, ws)
    _check(lib().park_cluster(ctypes.byref(sh), _ptr(x), int(metric), _ptr(qmetric), int(n_clusters), int(iters),
                              int(init), int(seed) & ((1 << 64) - 1), int(side), _ptr(centroids), _ptr(labels),
                              _ptr(perm), _ptr(offsets), _ptr(status), wp, wn, _stream(stream)))
    return {"centroids": centroids, "labels": labels, "perm": perm, "offsets": offsets}


def park_cluster_subset(x, n_clusters, iters, stride, phase, centroids, labels, metric=PARK_EUCLID, qmetric=None,
                        ws=None, stream=None):
    """Subset update between anchor steps: re-assign the tokens phase, phase + stride, ... and update
    the centroids over all tokens. ``centroids`` [heads, C, d] float32 and ``labels`` [heads, n] int32
    hold the previous step's state and are updated in place. Returns dict(centroids, labels, perm,
    offsets)."""
    sh = make_shape(x)
    H, N = sh.heads, sh.n
    perm = torch.empty(H, N, dtype=torch.int32, device=x.device)
    offsets = torch.empty(H, n_clusters + 1, dtype=torch.int32, device=x.device)
    prm = make_params(cq=n_clusters, ck=n_clusters, kmetric=metric)
    entry = PARK_ENTRY_CLUSTER_K if metric == PARK_QRKC else PARK_ENTRY_CLUSTER_Q
    wp, wn = _ws(entry, sh, prm, x.device, ws)
    _check(lib().park_cluster_subset(ctypes.byref(sh), _ptr(x), int(metric), _ptr(qmetric), int(n_clusters),
                                     int(iters), int(stride), int(phase), _ptr(centroids), _ptr(labels), _ptr(perm),
                                     _ptr(offsets), wp, wn, _stream(stream)))
    return {"centroids": centroids, "labels": labels, "perm": perm, "offsets": offsets}


def park_retrieve_map(q, q_perm, q_offsets, k_centroids, k_offsets, scale=0.0, out=None, ws=None, stream=None):
    """PAMA map [heads, cq, ck] float32."""
    sh = make_shape(q)
    cq = q_offsets.shape[1] - 1
    ck = k_offsets.shape[1] - 1
    M = out if out is not None else torch.empty(sh.heads, cq, ck, dtype=torch.float32, device=q.device)
    prm = make_params(cq=cq, ck=ck)
    wp, wn = _ws(PARK_ENTRY_RETRIEVE_MAP, sh, prm, q.device, ws)
    _check(lib().park_retrieve_map(ctypes.byref(sh), _ptr(q), _ptr(q_perm), _ptr(q_offsets), cq, _ptr(k_centroids),
                                   _ptr(k_offsets), ck, float(scale), _ptr(M), wp, wn, _stream(stream)))
    return M


def park_select_topp(map, k_offsets, p, stream=None):
    """Top-p cut of every map row. Returns dict(mask, counts, cols, sel_keys)."""
    H, cq, ck = map.shape
    dev = map.device
    mask = torch.empty(H, cq, ck, dtype=torch.uint8, device=dev)
    counts = torch.empty(H, cq, dtype=torch.int32, device=dev)
    cols = torch.empty(H, cq, ck, dtype=torch.int32, device=dev)
    sel = torch.empty(H, cq, dtype=torch.int64, device=dev)
    _check(lib().park_select_topp(_ptr(map), H, cq, ck, _ptr(k_offsets), float(p), _ptr(mask), _ptr(counts),
                                  _ptr(cols), _ptr(sel), _stream(stream)))
    return {"mask": mask, "counts": counts, "cols": cols, "sel_keys": sel}


def park_select_topk(map, k_offsets, rho, stream=None):
    """Top-k cut of every map row at retrieval ratio rho. Returns dict(mask, counts, cols, sel_keys)."""
    H, cq, ck = map.shape
    dev = map.device
    mask = torch.empty(H, cq, ck, dtype=torch.uint8, device=dev)
    counts = torch.empty(H, cq, dtype=torch.int32, device=dev)
    cols = torch.empty(H, cq, ck, dtype=torch.int32, device=dev)
    sel = torch.empty(H, cq, dtype=torch.int64, device=dev)
    _check(lib().park_select_topk(_ptr(map), H, cq, ck, _ptr(k_offsets), float(rho), _ptr(mask), _ptr(counts),
                                  _ptr(cols), _ptr(sel), _stream(stream)))
    return {"mask": mask, "counts": counts, "cols": cols, "sel_keys": sel}


def park_select_sip(map, k_offsets, rho, seed=0, stream=None):
    """Sampling with inclusion-probability weighting of every map row, budget = the top-k count at
    ratio rho. Returns dict(mask, counts, cols, sel_keys, log_w)."""
    H, cq, ck = map.shape
    dev = map.device
    mask = torch.empty(H, cq, ck, dtype=torch.uint8, device=dev)
    counts = torch.empty(H, cq, dtype=torch.int32, device=dev)
    cols = torch.empty(H, cq, ck, dtype=torch.int32, device=dev)
    sel = torch.empty(H, cq, dtype=torch.int64, device=dev)
    log_w = torch.empty(H, cq, ck, dtype=torch.float32, device=dev)
    _check(lib().park_select_sip(_ptr(map), H, cq, ck, _ptr(k_offsets), float(rho), int(seed) & (2**64 - 1),
                                 _ptr(mask), _ptr(counts), _ptr(cols), _ptr(sel), _ptr(log_w), _stream(stream)))
    return {"mask": mask, "counts": counts, "cols": cols, "sel_keys": sel, "log_w": log_w}


def park_estimator_map(mode, k_offsets, q=None, k=None, q_perm=None, q_offsets=None, q_centroids=None, k_perm=None,
                       k_centroids=None, scale=0.0, out=None, ws=None, stream=None):
    """Block map [heads, cq, ck] float32 under a PARK_EST_* query/key representation (Table 1). The
    shape and dtype come from q (or k when q is not given); q_offsets is read in every mode."""
    ref = q if q is not None else k
    sh = make_shape(ref)
    cq = q_offsets.shape[1] - 1
    ck = k_offsets.shape[1] - 1
    M = out if out is not None else torch.empty(sh.heads, cq, ck, dtype=torch.float32, device=ref.device)
    prm = make_params(cq=cq, ck=ck)
    wp, wn = _ws(PARK_ENTRY_ESTIMATOR, sh, prm, ref.device, ws)
    _check(lib().park_estimator_map(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(q_perm), _ptr(q_offsets), cq,
                                    _ptr(q_centroids), _ptr(k_perm), _ptr(k_offsets), ck, _ptr(k_centroids),
                                    int(mode), float(scale), _ptr(M), wp, wn, _stream(stream)))
    return M


def park_sparse_attn(q, k, v, q_perm, q_offsets, k_perm, k_offsets, counts, cols, scale=0.0, out=None, lse=True,
                     ws=None, stream=None):
    """Attention over the selected blocks. Returns (out [heads, n, d], lse [heads, n] or None)."""
    sh = make_shape(q)
    cq = q_offsets.shape[1] - 1
    ck = k_offsets.shape[1] - 1
    o = out if out is not None else torch.empty_like(q)
    L = None
    if lse is True:
        L = torch.empty(sh.heads, sh.n, dtype=torch.float32, device=q.device)
    elif isinstance(lse, torch.Tensor):
        L = lse
    prm = make_params(cq=cq, ck=ck)
    wp, wn = _ws(PARK_ENTRY_SPARSE_ATTN, sh, prm, q.device, ws)
    _check(lib().park_sparse_attn(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(q_perm), _ptr(q_offsets), cq,
                                  _ptr(k_perm), _ptr(k_offsets), ck, _ptr(counts), _ptr(cols), float(scale), _ptr(o),
                                  _ptr(L), wp, wn, _stream(stream)))
    return o, L


def park_sparse_attn_weighted(q, k, v, q_perm, q_offsets, k_perm, k_offsets, counts, cols, log_w, scale=0.0,
                              out=None, lse=True, ws=None, stream=None):
    """Attention over the selected blocks, the logits of block j of row i raised by log_w[h, i, j].
    Returns (out [heads, n, d], lse [heads, n] or None)."""
    sh = make_shape(q)
    cq = q_offsets.shape[1] - 1
    ck = k_offsets.shape[1] - 1
    o = out if out is not None else torch.empty_like(q)
    L = None
    if lse is True:
        L = torch.empty(sh.heads, sh.n, dtype=torch.float32, device=q.device)
    elif isinstance(lse, torch.Tensor):
        L = lse
    prm = make_params(cq=cq, ck=ck)
    wp, wn = _ws(PARK_ENTRY_SPARSE_ATTN_WEIGHTED, sh, prm, q.device, ws)
    _check(lib().park_sparse_attn_weighted(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(q_perm),
                                           _ptr(q_offsets), cq, _ptr(k_perm), _ptr(k_offsets), ck, _ptr(counts),
                                           _ptr(cols), _ptr(log_w), float(scale), _ptr(o), _ptr(L), wp, wn,
                                           _stream(stream)))
    return o, L


def park_merge_clusters(q_perm, q_offsets, k_offsets, counts, cols, bm=384, ws=None, stream=None):
    """Tile-aware merging of the query clusters (CTA-aligned cost with bm-query tiles). Returns
    dict(group, q_perm, q_offsets, counts, cols): the merged groups as a query clustering with the
    same number of slots, ready for park_sparse_attn."""
    H, N = q_perm.shape
    cq = q_offsets.shape[1] - 1
    ck = k_offsets.shape[1] - 1
    dev = q_perm.device
    group = torch.empty(H, cq, dtype=torch.int32, device=dev)
    m_perm = torch.empty(H, N, dtype=torch.int32, device=dev)
    m_off = torch.empty(H, cq + 1, dtype=torch.int32, device=dev)
    m_cnt = torch.empty(H, cq, dtype=torch.int32, device=dev)
    m_cols = torch.zeros(H, cq, ck, dtype=torch.int32, device=dev)
    sh = park_shape(H, N, 128, PARK_BF16)
    prm = make_params(cq=cq, ck=ck)
    wp, wn = _ws(PARK_ENTRY_MERGE, sh, prm, dev, ws)
    _check(lib().park_merge_clusters(H, N, cq, ck, int(bm), _ptr(q_perm), _ptr(q_offsets), _ptr(k_offsets),
                                     _ptr(counts), _ptr(cols), _ptr(group), _ptr(m_perm), _ptr(m_off), _ptr(m_cnt),
                                     _ptr(m_cols), wp, wn, _stream(stream)))
    return {"group": group, "q_perm": m_perm, "q_offsets": m_off, "counts": m_cnt, "cols": m_cols}


def park_permute_rows(x, perm, out=None, stream=None):
    """out[h, p] = x[h, perm[h, p]]."""
    sh = make_shape(x)
    o = out if out is not None else torch.empty_like(x)
    _check(lib().park_permute_rows(ctypes.byref(sh), _ptr(x), _ptr(perm), _ptr(o), _stream(stream)))
    return o


def park_unpermute_rows(x, perm, out=None, stream=None):
    """out[h, perm[h, p]] = x[h, p]."""
    sh = make_shape(x)
    o = out if out is not None else torch.empty_like(x)
    _check(lib().park_unpermute_rows(ctypes.byref(sh), _ptr(x), _ptr(perm), _ptr(o), _stream(stream)))
    return o


_FWD_FIELDS = {
    "metric": lambda H, N, D, cq, ck: ((H, D, D), torch.float32),
    "q_labels": lambda H, N, D, cq, ck: ((H, N), torch.int32),
    "q_perm": lambda H, N, D, cq, ck: ((H, N), torch.int32),
    "q_offsets": lambda H, N, D, cq, ck: ((H, cq + 1), torch.int32),
    "k_labels": lambda H, N, D, cq, ck: ((H, N), torch.int32),
    "k_perm": lambda H, N, D, cq, ck: ((H, N), torch.int32),
    "k_offsets": lambda H, N, D, cq, ck: ((H, ck + 1), torch.int32),
    "map": lambda H, N, D, cq, ck: ((H, cq, ck), torch.float32),
    "mask": lambda H, N, D, cq, ck: ((H, cq, ck), torch.uint8),
    "counts": lambda H, N, D, cq, ck: ((H, cq), torch.int32),
    "cols": lambda H, N, D, cq, ck: ((H, cq, ck), torch.int32),
    "sel_keys": lambda H, N, D, cq, ck: ((H, cq), torch.int64),
    "lse": lambda H, N, D, cq, ck: ((H, N), torch.float32),
    "status": lambda H, N, D, cq, ck: ((1,), torch.int32),
    "stats": lambda H, N, D, cq, ck: ((8,), torch.int64),
}


def park_forward(q, k, v, cq, ck, iters, p, scale=0.0, seed=0, kmetric=PARK_QRKC, init=PARK_INIT_KMEANSPP,
                 q_centroids=None, k_centroids=None, outputs=(), out=None, ws=None, stream=None, subset=(1, 0),
                 q_labels=None, k_labels=None):
    """The whole path for one layer. ``outputs`` names intermediates to return (see
    park_forward_outputs); q_centroids / k_centroids are caller state for warm starts. With
    ``init=PARK_INIT_SUBSET``, ``subset`` = (stride, phase) and ``q_labels`` / ``k_labels`` (the
    previous step's labels, updated in place) are required. ``"stats"`` in ``outputs`` returns the
    park_stats totals as an int64 tensor (fields STATS_FIELDS)."""
    sh = make_shape(q)
    H, N, D = sh.heads, sh.n, sh.d
    dev = q.device
    if q_centroids is None:
        q_centroids = torch.empty(H, cq, D, dtype=torch.float32, device=dev)
    if k_centroids is None:
        k_centroids = torch.empty(H, ck, D, dtype=torch.float32, device=dev)
    o = out if out is not None else torch.empty_like(q)
    res = {}
    fo = park_forward_outputs()
    given = {"q_labels": q_labels, "k_labels": k_labels}
    for name, t in given.items():
        if t is not None:
            res[name] = t
            setattr(fo, name, t.data_ptr())
    for name in outputs:
        if given.get(name) is not None:
            continue
        shp, dt = _FWD_FIELDS[name](H, N, D, cq, ck)
        t = torch.zeros(shp, dtype=dt, device=dev) if name == "status" else torch.empty(shp, dtype=dt, device=dev)
        res[name] = t
        setattr(fo, name, t.data_ptr())
    prm = make_params(cq, ck, iters, p, scale, seed, kmetric, init, subset[0], subset[1])
    wp, wn = _ws(PARK_ENTRY_FORWARD, sh, prm, dev, ws)
    _check(lib().park_forward(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(o), ctypes.byref(prm),
                              _ptr(q_centroids), _ptr(k_centroids), ctypes.byref(fo), wp, wn, _stream(stream)))
    res.update(out=o, q_centroids=q_centroids, k_centroids=k_centroids)
    return res
