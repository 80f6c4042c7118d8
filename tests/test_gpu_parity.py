"""HIP path vs the fp64 oracle, stage by stage, on the same seeded inputs (lock-step: every oracle
stage is fed exactly what the GPU stage consumed). Sizes span several tiles with ragged tails."""
import numpy as np
import pytest
import torch

import block_sparse_attention_qrkc_amd as bsa
import oracle as O
from gpu_helpers import (ATTN_MAX_ABS, ATTN_MEAN_ABS, LSE_ABS, MAP_ABS, SMALL, TAU, attn_view, check_topp_rows,
                         cols_list, inputs, np_i, to64)

pytestmark = pytest.mark.gpu

WL = ["small", "small64", "tiny", "small32"]


def _bf(w):
    return w.dtype == "bf16"


@pytest.fixture(scope="module", params=WL)
def case(request):
    w = SMALL[request.param]
    Q, K, V = inputs(w)
    M = bsa.park_qrkc_metric(Q)
    torch.cuda.synchronize()
    print(f"\n[case] {w.name}: H={w.heads} N={w.n} d={w.d} {w.dtype} cq={w.cq} ck={w.ck}", flush=True)
    return w, Q, K, V, M


def test_qrkc_metric(case):
    w, Q, K, V, M = case
    Mg = to64(M)
    for h in range(w.heads):
        Mo = O.qrkc_metric(to64(Q[h]))
        rel = np.abs(Mg[h] - Mo).max() / np.abs(Mo).max()
        assert rel <= (2e-6 if _bf(w) else 1e-7), rel
        np.testing.assert_array_equal(Mg[h], Mg[h].T)


@pytest.mark.parametrize("side", ["q", "k"])
def test_kmeanspp_seeding(case, side):
    w, Q, K, V, M = case
    X = Q if side == "q" else K
    C = w.cq if side == "q" else w.ck
    metric = bsa.PARK_EUCLID if side == "q" else bsa.PARK_QRKC
    sd = bsa.PARK_SIDE_Q if side == "q" else bsa.PARK_SIDE_K
    res = bsa.park_cluster(X, C, 0, metric, M if side == "k" else None, seed=11, side=sd)
    cg = to64(res["centroids"])
    near = 0
    for h in range(w.heads):
        Mh = to64(M[h]) if side == "k" else None
        co, chosen, margins = O.kmeanspp(to64(X[h]), C, Mh, seed=11, head=h, side=sd, return_trace=True)
        diff = np.flatnonzero(np.any(cg[h] != co, axis=1))
        if diff.size:
            m = diff[0]
            assert margins[m] <= TAU, f"head {h}: seeding differs at step {m} (margin {margins[m]:.3g})"
            near += 1
    print(f"[kmeans++ {side}] near-ties: {near}")


@pytest.mark.parametrize("side", ["q", "k"])
def test_lloyd_lockstep(case, side):
    w, Q, K, V, M = case
    X = Q if side == "q" else K
    C = w.cq if side == "q" else w.ck
    metric = bsa.PARK_EUCLID if side == "q" else bsa.PARK_QRKC
    sd = bsa.PARK_SIDE_Q if side == "q" else bsa.PARK_SIDE_K
    Mp = M if side == "k" else None
    cent = bsa.park_cluster(X, C, 0, metric, Mp, seed=5, side=sd)["centroids"]
    Xs = [to64(X[h]) for h in range(w.heads)]
    xmax = max(np.abs(x).max() for x in Xs)
    near = 0
    for it in range(3):
        prev = to64(cent)
        res = bsa.park_cluster(X, C, 1, metric, Mp, init=bsa.PARK_INIT_WARM, side=sd, centroids=cent)
        lab, perm, off, new = np_i(res["labels"]), np_i(res["perm"]), np_i(res["offsets"]), to64(res["centroids"])
        for h in range(w.heads):
            Mh = to64(M[h]) if side == "k" else None
            g, b = O.consumed_centroids(prev[h], metric, Mh, bf16=_bf(w))
            n_near, bad = O.assign_near_tie(Xs[h], g, b, lab[h], TAU)
            assert bad.size == 0, f"iter {it} head {h}: {bad.size} labels differ beyond near-ties, e.g. {bad[:5]}"
            near += n_near
            po, oo = O.cluster_order(lab[h], C)
            np.testing.assert_array_equal(perm[h], po)
            np.testing.assert_array_equal(off[h], oo)
            co = O.update(Xs[h], lab[h], C, prev[h])
            err = np.abs(new[h] - co).max()
            assert err <= 1e-6 * xmax, err
    print(f"[lloyd {side}] assignment near-ties over 3 iterations: {near}")


@pytest.mark.parametrize("name", ["small", "small64"])
def test_fused_step_empty_cluster(name):
    """Euclidean bf16 sides with at most 128 clusters run the fused step (assignment and member sums
    in one pass). A centroid moved far from every point draws no members and keeps its value; the
    labels are the assignment against the consumed centroids (near-ties counted) and every other
    centroid is the fp64 mean of its members."""
    w = SMALL[name]
    Q, K, V = inputs(w)
    C = w.cq
    cent = bsa.park_cluster(Q, C, 0, bsa.PARK_EUCLID, seed=3, side=bsa.PARK_SIDE_Q)["centroids"]
    cent[:, 5] = 1.0e3
    prev = to64(cent)
    res = bsa.park_cluster(Q, C, 1, bsa.PARK_EUCLID, init=bsa.PARK_INIT_WARM, side=bsa.PARK_SIDE_Q, centroids=cent)
    lab, perm, off, new = np_i(res["labels"]), np_i(res["perm"]), np_i(res["offsets"]), to64(res["centroids"])
    near = 0
    for h in range(w.heads):
        x = to64(Q[h])
        assert not np.any(lab[h] == 5)
        np.testing.assert_array_equal(new[h][5], prev[h][5])
        g, b = O.consumed_centroids(prev[h], O.EUCLID, None, bf16=True)
        n_near, bad = O.assign_near_tie(x, g, b, lab[h], TAU)
        assert bad.size == 0, f"head {h}: {bad.size} labels differ beyond near-ties"
        near += n_near
        po, oo = O.cluster_order(lab[h], C)
        np.testing.assert_array_equal(perm[h], po)
        np.testing.assert_array_equal(off[h], oo)
        assert np.abs(new[h] - O.update(x, lab[h], C, prev[h])).max() <= 1e-6 * np.abs(x).max()
    print(f"[fused step {name}] near-ties: {near}")


def test_fused_step_full_tiles_and_128_clusters():
    """The fused step at its cluster limit (128 clusters: every 32-cluster tile of the assignment
    live) on 3000 tokens (a ragged last 128-token tile), where the first five tiles belong to one
    cluster (every bit of that cluster's per-tile membership mask set) and the other tokens spread
    over all clusters; labels, order and means against the oracle as in the test above."""
    g = torch.Generator().manual_seed(11)
    H, N, D, C = 2, 3000, 128, 128
    dirs = torch.randn(C, D, generator=g)
    dirs = dirs / dirs.norm(dim=1, keepdim=True) * 8.0
    cen = torch.randint(0, C, (H, N), generator=g)
    cen[:, :640] = 7
    Q = (dirs[cen] + 0.3 * torch.randn(H, N, D, generator=g)).to(torch.bfloat16).cuda().contiguous()
    cent = dirs.unsqueeze(0).repeat(H, 1, 1).float().cuda().contiguous()
    prev = to64(cent)
    res = bsa.park_cluster(Q, C, 1, bsa.PARK_EUCLID, init=bsa.PARK_INIT_WARM, side=bsa.PARK_SIDE_Q, centroids=cent)
    lab, perm, off, new = np_i(res["labels"]), np_i(res["perm"]), np_i(res["offsets"]), to64(res["centroids"])
    near = 0
    for h in range(H):
        x = to64(Q[h])
        assert np.all(lab[h][:640] == 7)
        assert len(np.unique(lab[h])) > 100
        gg, b = O.consumed_centroids(prev[h], O.EUCLID, None, bf16=True)
        n_near, bad = O.assign_near_tie(x, gg, b, lab[h], TAU)
        assert bad.size == 0, f"head {h}: {bad.size} labels differ beyond near-ties"
        near += n_near
        po, oo = O.cluster_order(lab[h], C)
        np.testing.assert_array_equal(perm[h], po)
        np.testing.assert_array_equal(off[h], oo)
        assert np.abs(new[h] - O.update(x, lab[h], C, prev[h])).max() <= 1e-6 * np.abs(x).max()
    print(f"[fused step, 128 clusters] near-ties: {near}")


@pytest.mark.parametrize("side", ["q", "k"])
@pytest.mark.parametrize("stride,phase", [(3, 1), (4, 0), (1, 0)])
def test_subset_update_lockstep(case, side, stride, phase):
    """Subset updates (hybrid clustering between anchor steps): the rows phase, phase + stride, ...
    are re-assigned against the consumed centroids (near-ties counted), every other row keeps its
    label bit for bit, the order is the stable sort of the labels, and the centroids are the fp64
    member means. The labels start from a clustering with some rows scrambled, a few of them
    outside [0, C) (taken as cluster 0)."""
    w, Q, K, V, M = case
    X = Q if side == "q" else K
    C = w.cq if side == "q" else w.ck
    metric = bsa.PARK_EUCLID if side == "q" else bsa.PARK_QRKC
    sd = bsa.PARK_SIDE_Q if side == "q" else bsa.PARK_SIDE_K
    Mp = M if side == "k" else None
    base = bsa.park_cluster(X, C, 2, metric, Mp, seed=7, side=sd)
    rng = np.random.default_rng(stride * 10 + phase)
    lab0 = np_i(base["labels"])
    scr = rng.random(lab0.shape) < 0.1
    lab0[scr] = rng.integers(0, C, int(scr.sum()))
    lab0[:, 5] = C + 3
    lab0[:, 11] = -2
    labels = torch.tensor(lab0, dtype=torch.int32, device="cuda")
    prev = base["centroids"].clone()
    res = bsa.park_cluster_subset(X, C, 1, stride, phase, base["centroids"], labels, metric, Mp)
    lab, perm, off, new = np_i(res["labels"]), np_i(res["perm"]), np_i(res["offsets"]), to64(res["centroids"])
    start = np.where((lab0 < 0) | (lab0 >= C), 0, lab0)
    rows = O.subset_rows(w.n, stride, phase)
    keep = np.setdiff1d(np.arange(w.n), rows)
    xmax = 0.0
    near = 0
    for h in range(w.heads):
        x = to64(X[h])
        xmax = max(xmax, np.abs(x).max())
        np.testing.assert_array_equal(lab[h][keep], start[h][keep])
        Mh = to64(M[h]) if side == "k" else None
        g, b = O.consumed_centroids(to64(prev[h]), metric, Mh, bf16=_bf(w))
        n_near, bad = O.assign_near_tie(x[rows], g, b, lab[h][rows], TAU)
        assert bad.size == 0, f"head {h}: {bad.size} subset labels differ beyond near-ties"
        near += n_near
        po, oo = O.cluster_order(lab[h], C)
        np.testing.assert_array_equal(perm[h], po)
        np.testing.assert_array_equal(off[h], oo)
        # the oracle's subset update from the same start (a near-tie would only move a centroid)
        lo, co = O.lloyd_subset(x, to64(prev[h]), start[h], 1, stride, phase, metric, Mh, bf16=_bf(w))
        if n_near == 0:
            np.testing.assert_array_equal(lab[h], lo)
        assert np.abs(new[h] - O.update(x, lab[h], C, to64(prev[h]))).max() <= 1e-6 * xmax
    print(f"[subset {side} stride={stride} phase={phase}] near-ties: {near}")


@pytest.fixture(scope="module")
def clustered(case):
    w, Q, K, V, M = case
    qc = bsa.park_cluster(Q, w.cq, 3, bsa.PARK_EUCLID, None, seed=1, side=bsa.PARK_SIDE_Q)
    kc = bsa.park_cluster(K, w.ck, 3, bsa.PARK_QRKC, M, seed=1, side=bsa.PARK_SIDE_K)
    return w, Q, K, V, M, qc, kc


def test_pama_map(clustered):
    w, Q, K, V, M, qc, kc = clustered
    A = bsa.park_retrieve_map(Q, qc["perm"], qc["offsets"], kc["centroids"], kc["offsets"])
    Ag = to64(A)
    for h in range(w.heads):
        kcent = to64(kc["centroids"][h])
        khat = O.round_bf16(kcent) if _bf(w) else kcent
        sizes = np.diff(np_i(kc["offsets"][h]))
        Ao = O.pama(to64(Q[h]), np_i(qc["perm"][h]), np_i(qc["offsets"][h]), khat, sizes, w.scale)
        err = np.abs(Ag[h] - Ao).max()
        assert err <= MAP_ABS, err
        live = np.diff(np_i(qc["offsets"][h])) > 0
        assert np.abs(Ag[h][live].sum(1) - 1).max() <= MAP_ABS
        assert np.all(Ag[h][~live] == 0)
        assert np.all(Ag[h][:, sizes == 0] == 0)


@pytest.mark.parametrize("p", [0.5, 0.9, 0.95, 1.0])
def test_select_topp(clustered, p):
    w, Q, K, V, M, qc, kc = clustered
    A = bsa.park_retrieve_map(Q, qc["perm"], qc["offsets"], kc["centroids"], kc["offsets"])
    sel = bsa.park_select_topp(A, kc["offsets"], p)
    Ag = to64(A)
    mask, counts, cols, keys = np_i(sel["mask"]), np_i(sel["counts"]), np_i(sel["cols"]), np_i(sel["sel_keys"])
    near = 0
    for h in range(w.heads):
        sizes = np.diff(np_i(kc["offsets"][h]))
        n_near, bad = check_topp_rows(Ag[h], sizes, p, counts[h], cols[h], keys[h])
        assert not bad, f"head {h} rows {bad}"
        near += n_near
        for i in range(w.cq):
            c = cols[h, i, :counts[h, i]]
            assert np.all(np.diff(c) > 0)
            assert np.array_equal(np.flatnonzero(mask[h, i]), c)
            assert keys[h, i] == sizes[c].sum()
            if Ag[h, i].sum() > 0 and p < 1:
                mass = Ag[h, i, c].sum()
                assert mass >= p - 1e-6  # P2: the kept mass reaches p
                assert mass - Ag[h, i, c].min() < p + 1e-6  # and the kept set is minimal
            if p >= 1 and Ag[h, i].sum() > 0:
                assert np.array_equal(c, np.flatnonzero(sizes > 0))
    print(f"[top-p {p}] near-ties: {near}")


@pytest.mark.parametrize("bm", [64, 384])
def test_merge_clusters(clustered, bm):
    """Tile-aware merging of the query clusters on the top-p selection: groups, merged order,
    offsets and union selections bit-exact against the oracle's merge; attention over the merged
    groups against the fp64 masked softmax over each group's union selection."""
    w, Q, K, V, M, qc, kc = clustered
    A = bsa.park_retrieve_map(Q, qc["perm"], qc["offsets"], kc["centroids"], kc["offsets"])
    sel = bsa.park_select_topp(A, kc["offsets"], w.p)
    mg = bsa.park_merge_clusters(qc["perm"], qc["offsets"], kc["offsets"], sel["counts"], sel["cols"], bm=bm)
    groups = 0
    for h in range(w.heads):
        qo = np_i(qc["offsets"][h])
        sizes = np.diff(np_i(kc["offsets"][h]))
        cl = cols_list(np_i(sel["counts"][h]), np_i(sel["cols"][h]))
        group, gsel = O.merge_clusters(np.diff(qo), cl, sizes, bm)
        perm, off, mcols = O.merged_order(np_i(qc["perm"][h]), qo, group, gsel)
        roots = sorted(set(group.tolist()))
        rank = {r: g for g, r in enumerate(roots)}
        np.testing.assert_array_equal(np_i(mg["group"][h]), [rank[r] for r in group])
        np.testing.assert_array_equal(np_i(mg["q_perm"][h]), perm)
        np.testing.assert_array_equal(np_i(mg["q_offsets"][h]), off)
        cnt = np_i(mg["counts"][h])
        for g in range(w.cq):
            np.testing.assert_array_equal(np_i(mg["cols"][h, g, :cnt[g]]), mcols[g])
        groups += len(roots)
    out, lse = bsa.park_sparse_attn(Q, K, V, mg["q_perm"], mg["q_offsets"], kc["perm"], kc["offsets"], mg["counts"],
                                    mg["cols"])
    worst, mean = _attn_check(w, Q, K, V, mg["q_perm"], mg["q_offsets"], kc["perm"], kc["offsets"], mg["counts"],
                              mg["cols"], out, lse)
    print(f"[merge bm={bm}] {w.heads * w.cq} clusters -> {groups} groups; attention max-abs {worst:.2e}")


def test_select_topp_hand_fixture():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "topp_hand.json")))
    A = torch.tensor(g["map"], dtype=torch.float32, device="cuda")[None].contiguous()
    ko = torch.tensor([np.concatenate([[0], np.cumsum(g["k_sizes"])]).tolist()], dtype=torch.int32, device="cuda")
    for case in g["cases"]:
        sel = bsa.park_select_topp(A, ko, case["p"])
        counts, cols, keys = np_i(sel["counts"])[0], np_i(sel["cols"])[0], np_i(sel["sel_keys"])[0]
        assert [cols[i, :counts[i]].tolist() for i in range(3)] == case["cols"]
        assert keys.tolist() == case["keys"]


def _attn_check(w, Q, K, V, qp, qo, kp, ko, counts, cols, out, lse, heads=None):
    worst, mean_acc, n = 0.0, 0.0, 0
    for h in (range(w.heads) if heads is None else heads):
        Oo, Lo = O.sparse_attention(attn_view(w, Q[h]), attn_view(w, K[h]), attn_view(w, V[h]), np_i(qp[h]),
                                    np_i(qo[h]), np_i(kp[h]), np_i(ko[h]), cols_list(np_i(counts[h]), np_i(cols[h])),
                                    w.scale)
        Og, Lg = to64(out[h]), to64(lse[h])
        e = np.abs(Og - Oo)
        worst = max(worst, e.max())
        mean_acc += e.sum()
        n += e.size
        fin = np.isfinite(Lo)
        np.testing.assert_array_equal(np.isfinite(Lg), fin)
        assert np.abs(Lg[fin] - Lo[fin]).max() <= LSE_ABS
    assert worst <= ATTN_MAX_ABS, worst
    assert mean_acc / n <= ATTN_MEAN_ABS, mean_acc / n
    return worst, mean_acc / n


@pytest.mark.parametrize("p", [0.9, 1.0])
def test_sparse_attention(clustered, p):
    w, Q, K, V, M, qc, kc = clustered
    A = bsa.park_retrieve_map(Q, qc["perm"], qc["offsets"], kc["centroids"], kc["offsets"])
    sel = bsa.park_select_topp(A, kc["offsets"], p)
    out, lse = bsa.park_sparse_attn(Q, K, V, qc["perm"], qc["offsets"], kc["perm"], kc["offsets"], sel["counts"],
                                    sel["cols"])
    worst, mean = _attn_check(w, Q, K, V, qc["perm"], qc["offsets"], kc["perm"], kc["offsets"], sel["counts"],
                              sel["cols"], out, lse)
    print(f"[attention p={p}] max-abs {worst:.2e} mean-abs {mean:.2e}")
    if p == 1.0:  # P3: top-p = 1 reproduces dense attention
        for h in range(w.heads):
            Od, Ld = O.dense_attention(attn_view(w, Q[h]), attn_view(w, K[h]), attn_view(w, V[h]), w.scale)
            e = np.abs(to64(out[h]) - Od)
            assert e.max() <= ATTN_MAX_ABS and e.mean() <= ATTN_MEAN_ABS
            assert np.abs(to64(lse[h]) - Ld).max() <= LSE_ABS


def test_sparse_attention_edge_selections():
    """Hand-built clusterings and selections: singleton and empty clusters, empty rows, runs that
    merge across adjacent clusters, and key clusters that are selected but empty."""
    w = SMALL["small"]
    rng = np.random.default_rng(3)
    Q, K, V = inputs(w)
    H, N = w.heads, w.n
    cq, ck = 37, 61
    qps, qos, kps, kos, cnts, colss = [], [], [], [], [], []
    for h in range(H):
        ql = rng.integers(0, cq, N)
        ql[ql == 5] = 6              # empty query cluster
        ql[:3] = 7                   # cluster 7 is small
        ql[ql == 7] = 8
        ql[100] = 7                  # singleton query cluster
        kl = rng.integers(0, ck, N)
        kl[kl == 9] = 10             # empty key cluster
        kl[kl == 11] = 12
        kl[200] = 11                 # singleton key cluster
        qp, qo = O.cluster_order(ql, cq)
        kp, ko = O.cluster_order(kl, ck)
        cols = np.zeros((cq, ck), dtype=np.int32)
        cnt = np.zeros(cq, dtype=np.int32)
        for i in range(cq):
            if i == 3:
                sel = np.array([], dtype=np.int64)        # a query cluster that selected nothing
            elif i == 4:
                sel = np.arange(ck)                       # everything, including the empty cluster
            elif i == 8:
                sel = np.array([9, 11])                   # an empty and a singleton key cluster
            else:
                sel = np.flatnonzero(rng.random(ck) < 0.3)
            cnt[i] = sel.size
            cols[i, :sel.size] = sel
        qps.append(qp); qos.append(qo); kps.append(kp); kos.append(ko); cnts.append(cnt); colss.append(cols)
    T = lambda a: torch.tensor(np.stack(a), dtype=torch.int32, device="cuda").contiguous()
    qp, qo, kp, ko, counts, cols = map(T, (qps, qos, kps, kos, cnts, colss))
    out, lse = bsa.park_sparse_attn(Q, K, V, qp, qo, kp, ko, counts, cols)
    _attn_check(w, Q, K, V, qp, qo, kp, ko, counts, cols, out, lse)
    # the cluster that selected nothing gets zero output and -inf log-sum-exp
    for h in range(H):
        rows = np_i(qp[h])[np_i(qo[h])[3]:np_i(qo[h])[4]]
        assert np.all(to64(out[h])[rows] == 0) and np.all(np.isneginf(to64(lse[h])[rows]))


def test_sparse_attention_many_clusters():
    """More query and key clusters than one 1024-thread block has threads (the per-head work order
    sorts 1500 clusters, several per thread), a few large query clusters spanning several 384-query
    work items among many tiny ones, and many clusters with equal selected key counts (ties)."""
    w = SMALL["small"]
    rng = np.random.default_rng(11)
    Q, K, V = inputs(w)
    H, N = w.heads, w.n
    cq, ck = 1500, 1100
    qps, qos, kps, kos, cnts, colss = [], [], [], [], [], []
    for h in range(H):
        ql = rng.integers(3, cq, N)
        big = rng.random(N) < 0.45
        ql[big] = rng.integers(0, 3, int(big.sum()))   # clusters 0..2 hold ~500 queries each
        kl = rng.integers(0, ck, N)
        qp, qo = O.cluster_order(ql, cq)
        kp, ko = O.cluster_order(kl, ck)
        cols = np.zeros((cq, ck), dtype=np.int32)
        cnt = np.zeros(cq, dtype=np.int32)
        for i in range(cq):
            sel = np.sort(rng.choice(ck, size=int(rng.integers(1, 40)), replace=False))
            cnt[i] = sel.size
            cols[i, :sel.size] = sel
        qps.append(qp); qos.append(qo); kps.append(kp); kos.append(ko); cnts.append(cnt); colss.append(cols)
    T = lambda a: torch.tensor(np.stack(a), dtype=torch.int32, device="cuda").contiguous()
    qp, qo, kp, ko, counts, cols = map(T, (qps, qos, kps, kos, cnts, colss))
    out, lse = bsa.park_sparse_attn(Q, K, V, qp, qo, kp, ko, counts, cols)
    _attn_check(w, Q, K, V, qp, qo, kp, ko, counts, cols, out, lse)


def test_sparse_attention_split_items():
    """Work items of at most 192 queries split their keys over two wave groups (each group one
    32-key half of every 64-key tile, merged at the end): query clusters just below, at and above
    that size and at the 384-query item boundary, against selections whose key counts fall just
    below, at and above the 32- and 64-key tile edges (a second group that meets no key included)."""
    w = SMALL["small"]
    rng = np.random.default_rng(5)
    Q, K, V = inputs(w)
    H, N = w.heads, w.n
    qsz = [1, 31, 32, 33, 64, 96, 160, 191, 192, 193, 250, 384, 385, 576]
    qsz.append(N - sum(qsz))
    ksz = [1, 31, 32, 33, 63, 64, 65, 97, 128, 129, 300]
    ksz.append(N - sum(ksz))
    cq, ck = len(qsz), len(ksz)
    combos = [[0, 2, 5], list(range(ck)), [1, 3], [4, 10]]
    qps, qos, kps, kos, cnts, colss = [], [], [], [], [], []
    for h in range(H):
        ql = rng.permutation(np.repeat(np.arange(cq), qsz))
        kl = rng.permutation(np.repeat(np.arange(ck), ksz))
        qp, qo = O.cluster_order(ql, cq)
        kp, ko = O.cluster_order(kl, ck)
        cols = np.zeros((cq, ck), dtype=np.int32)
        cnt = np.zeros(cq, dtype=np.int32)
        for i in range(cq):
            sel = np.array([(i + 5 * h) % 11]) if i < 11 else np.array(combos[i - 11])
            cnt[i] = sel.size
            cols[i, :sel.size] = np.sort(sel)
        qps.append(qp); qos.append(qo); kps.append(kp); kos.append(ko); cnts.append(cnt); colss.append(cols)
    T = lambda a: torch.tensor(np.stack(a), dtype=torch.int32, device="cuda").contiguous()
    qp, qo, kp, ko, counts, cols = map(T, (qps, qos, kps, kos, cnts, colss))
    out, lse = bsa.park_sparse_attn(Q, K, V, qp, qo, kp, ko, counts, cols)
    worst, mean = _attn_check(w, Q, K, V, qp, qo, kp, ko, counts, cols, out, lse)
    print(f"[attention split items] max-abs {worst:.2e} mean-abs {mean:.2e}")


def test_sparse_attention_repeatable():
    """Repeated launches give bitwise-identical outputs (each work item is computed by one work-group
    in a fixed order): thousands of work items, so that many work-groups start items at once, with
    unrelated matrix products between the launches; no oracle is needed for this property."""
    H, N, D, cq, ck = 8, 40000, 128, 160, 200
    g = torch.Generator(device="cuda").manual_seed(3)
    Q, K, V = (torch.randn(H, N, D, device="cuda", generator=g).to(torch.bfloat16) for _ in range(3))
    rng = np.random.default_rng(13)
    qps, qos, kps, kos, cnts, colss = [], [], [], [], [], []
    for h in range(H):
        qp, qo = O.cluster_order(rng.integers(0, cq, N), cq)
        kp, ko = O.cluster_order(rng.integers(0, ck, N), ck)
        cols = np.zeros((cq, ck), dtype=np.int32)
        cnt = rng.integers(1, ck // 2, cq).astype(np.int32)
        for i in range(cq):
            cols[i, :cnt[i]] = np.sort(rng.choice(ck, size=int(cnt[i]), replace=False))
        qps.append(qp); qos.append(qo); kps.append(kp); kos.append(ko); cnts.append(cnt); colss.append(cols)
    T = lambda a: torch.tensor(np.stack(a), dtype=torch.int32, device="cuda").contiguous()
    qp, qo, kp, ko, counts, cols = map(T, (qps, qos, kps, kos, cnts, colss))
    ref_out, ref_lse = bsa.park_sparse_attn(Q, K, V, qp, qo, kp, ko, counts, cols)
    a = torch.randn(2048, 2048, device="cuda", generator=g)
    for rep in range(6):
        _ = a @ a
        out, lse = bsa.park_sparse_attn(Q, K, V, qp, qo, kp, ko, counts, cols)
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), rep
    assert torch.isfinite(ref_out.float()).all() and torch.isfinite(ref_lse).all()


def test_pipeline_at_the_cluster_limit():
    """Both sides at the ABI's cluster limit (2048 query and 2048 key clusters over 4096 tokens, so
    most clusters hold one to a few tokens): k-means++ step by step, one Lloyd step of each side in
    lock-step, the map, the top-p rows and the attention (thousands of tiny work items) against the
    oracle."""
    w = SMALL["maxc"]
    Q, K, V = inputs(w)
    M = bsa.park_qrkc_metric(Q)
    res = {}
    for side, X, C, metric, sd, Mp in (("q", Q, w.cq, bsa.PARK_EUCLID, bsa.PARK_SIDE_Q, None),
                                       ("k", K, w.ck, bsa.PARK_QRKC, bsa.PARK_SIDE_K, M)):
        cent = bsa.park_cluster(X, C, 0, metric, Mp, seed=7, side=sd)["centroids"]
        x = to64(X[0])
        Mh = to64(Mp[0]) if Mp is not None else None
        co, chosen, margins = O.kmeanspp(x, C, Mh, seed=7, head=0, side=sd, return_trace=True)
        diff = np.flatnonzero(np.any(to64(cent)[0] != co, axis=1))
        if diff.size:
            assert margins[diff[0]] <= TAU, f"{side}: seeding differs at step {diff[0]}"
        prev = to64(cent)
        r = bsa.park_cluster(X, C, 1, metric, Mp, init=bsa.PARK_INIT_WARM, side=sd, centroids=cent)
        lab, perm, off = np_i(r["labels"]), np_i(r["perm"]), np_i(r["offsets"])
        g, b = O.consumed_centroids(prev[0], metric, Mh, bf16=True)
        _, bad = O.assign_near_tie(x, g, b, lab[0], TAU)
        assert bad.size == 0, f"{side}: {bad.size} labels differ beyond near-ties"
        po, oo = O.cluster_order(lab[0], C)
        np.testing.assert_array_equal(perm[0], po)
        np.testing.assert_array_equal(off[0], oo)
        assert np.abs(to64(r["centroids"])[0] - O.update(x, lab[0], C, prev[0])).max() <= 1e-6 * np.abs(x).max()
        res[side] = r
    qc, kc = res["q"], res["k"]
    A = bsa.park_retrieve_map(Q, qc["perm"], qc["offsets"], kc["centroids"], kc["offsets"])
    sizes = np.diff(np_i(kc["offsets"][0]))
    Ao = O.pama(to64(Q[0]), np_i(qc["perm"][0]), np_i(qc["offsets"][0]), O.round_bf16(to64(kc["centroids"][0])),
                sizes, w.scale)
    assert np.abs(to64(A)[0] - Ao).max() <= MAP_ABS
    sel = bsa.park_select_topp(A, kc["offsets"], w.p)
    _, bad = check_topp_rows(to64(A)[0], sizes, w.p, np_i(sel["counts"][0]), np_i(sel["cols"][0]),
                             np_i(sel["sel_keys"][0]))
    assert not bad, bad[:5]
    out, lse = bsa.park_sparse_attn(Q, K, V, qc["perm"], qc["offsets"], kc["perm"], kc["offsets"], sel["counts"],
                                    sel["cols"])
    worst, mean = _attn_check(w, Q, K, V, qc["perm"], qc["offsets"], kc["perm"], kc["offsets"], sel["counts"],
                              sel["cols"], out, lse)
    print(f"[cluster limit] attention max-abs {worst:.2e} mean-abs {mean:.2e}")


def test_many_heads():
    """1000 heads of 4096 tokens: more heads than the cooperative seeding can keep on the CUs, so each
    (head, side) is seeded by one work-group; seeding step by step, the forward's orders on every head,
    and map, top-p and attention of sampled heads against the oracle."""
    w = SMALL["many_heads"]
    Q, K, V = inputs(w)
    M = bsa.park_qrkc_metric(Q)
    heads = [0, 511, 999]
    for X, C, metric, sd, Mp in ((Q, w.cq, bsa.PARK_EUCLID, bsa.PARK_SIDE_Q, None),
                                 (K, w.ck, bsa.PARK_QRKC, bsa.PARK_SIDE_K, M)):
        cg = to64(bsa.park_cluster(X, C, 0, metric, Mp, seed=9, side=sd)["centroids"])
        for h in heads:
            co, _, margins = O.kmeanspp(to64(X[h]), C, to64(Mp[h]) if Mp is not None else None, seed=9, head=h,
                                        side=sd, return_trace=True)
            diff = np.flatnonzero(np.any(cg[h] != co, axis=1))
            if diff.size:
                assert margins[diff[0]] <= TAU, f"head {h}: seeding differs at step {diff[0]}"
    r = bsa.park_forward(Q, K, V, w.cq, w.ck, w.iters, w.p, seed=9, outputs=ALL_OUT)
    for side, C in (("q", w.cq), ("k", w.ck)):
        lab, perm, off = np_i(r[f"{side}_labels"]), np_i(r[f"{side}_perm"]), np_i(r[f"{side}_offsets"])
        for h in range(w.heads):
            po, oo = O.cluster_order(lab[h], C)
            np.testing.assert_array_equal(perm[h], po)
            np.testing.assert_array_equal(off[h], oo)
    for h in heads:
        sizes = np.diff(np_i(r["k_offsets"][h]))
        Ao = O.pama(to64(Q[h]), np_i(r["q_perm"][h]), np_i(r["q_offsets"][h]),
                    O.round_bf16(to64(r["k_centroids"][h])), sizes, w.scale)
        assert np.abs(to64(r["map"][h]) - Ao).max() <= MAP_ABS
        _, bad = check_topp_rows(to64(r["map"][h]), sizes, w.p, np_i(r["counts"][h]), np_i(r["cols"][h]),
                                 np_i(r["sel_keys"][h]))
        assert not bad
    _attn_check(w, Q, K, V, r["q_perm"], r["q_offsets"], r["k_perm"], r["k_offsets"], r["counts"], r["cols"],
                r["out"], r["lse"], heads=heads)
    assert torch.isfinite(r["out"].float()).all()


def test_permute_roundtrip(case):
    """P12: gather then scatter is the identity; the gather matches the permutation."""
    w, Q, K, V, M = case
    qc = bsa.park_cluster(Q, w.cq, 2, bsa.PARK_EUCLID, None, seed=2)
    Qp = bsa.park_permute_rows(Q, qc["perm"])
    back = bsa.park_unpermute_rows(Qp, qc["perm"])
    assert torch.equal(back, Q)
    for h in range(w.heads):
        assert torch.equal(Qp[h], Q[h][qc["perm"][h].long()])


ALL_OUT = ("metric", "q_labels", "q_perm", "q_offsets", "k_labels", "k_perm", "k_offsets", "map", "mask", "counts",
           "cols", "sel_keys", "lse")


def test_forward_matches_entry_points_and_oracle(case):
    w, Q, K, V, M = case
    r = bsa.park_forward(Q, K, V, w.cq, w.ck, w.iters, w.p, seed=3, outputs=ALL_OUT)
    # the fused entry equals the separate entry points, bit for bit
    qc = bsa.park_cluster(Q, w.cq, w.iters, bsa.PARK_EUCLID, None, seed=3, side=bsa.PARK_SIDE_Q)
    kc = bsa.park_cluster(K, w.ck, w.iters, bsa.PARK_QRKC, r["metric"], seed=3, side=bsa.PARK_SIDE_K)
    A = bsa.park_retrieve_map(Q, qc["perm"], qc["offsets"], kc["centroids"], kc["offsets"])
    sel = bsa.park_select_topp(A, kc["offsets"], w.p)
    out, lse = bsa.park_sparse_attn(Q, K, V, qc["perm"], qc["offsets"], kc["perm"], kc["offsets"], sel["counts"],
                                    sel["cols"])
    assert torch.equal(r["metric"], M)
    assert torch.equal(r["q_perm"], qc["perm"]) and torch.equal(r["k_perm"], kc["perm"])
    assert torch.equal(r["q_centroids"], qc["centroids"]) and torch.equal(r["k_centroids"], kc["centroids"])
    assert torch.equal(r["map"], A) and torch.equal(r["counts"], sel["counts"])
    assert torch.equal(r["out"], out) and torch.equal(r["lse"], lse)
    # lock-step oracle on the forward's own intermediates
    for h in range(w.heads):
        sizes = np.diff(np_i(r["k_offsets"][h]))
        kcent = to64(r["k_centroids"][h])
        Ao = O.pama(to64(Q[h]), np_i(r["q_perm"][h]), np_i(r["q_offsets"][h]),
                    O.round_bf16(kcent) if _bf(w) else kcent, sizes, w.scale)
        assert np.abs(to64(r["map"][h]) - Ao).max() <= MAP_ABS
        _, bad = check_topp_rows(to64(r["map"][h]), sizes, w.p, np_i(r["counts"][h]), np_i(r["cols"][h]),
                                 np_i(r["sel_keys"][h]))
        assert not bad
    _attn_check(w, Q, K, V, r["q_perm"], r["q_offsets"], r["k_perm"], r["k_offsets"], r["counts"], r["cols"],
                r["out"], r["lse"])
    # determinism: a second run is bitwise identical
    r2 = bsa.park_forward(Q, K, V, w.cq, w.ck, w.iters, w.p, seed=3, outputs=("map", "lse"))
    assert torch.equal(r2["out"], r["out"]) and torch.equal(r2["map"], r["map"]) and torch.equal(r2["lse"], r["lse"])


def test_forward_free_running_vs_oracle_tiny():
    """The tiny workload end to end against the oracle run on its own (no lock-step): labels agree
    up to near-tie cascades and the recall of both stays above the dense-mass bound."""
    w = SMALL["tiny"]
    Q, K, V = inputs(w)
    r = bsa.park_forward(Q, K, V, w.cq, w.ck, w.iters, w.p, seed=0, outputs=ALL_OUT)
    q, k, v = to64(Q[0]), to64(K[0]), to64(V[0])
    ro = O.forward(q, k, v, w.cq, w.ck, w.iters, w.p, w.scale, seed=0, bf16=False)
    agree_q = (np_i(r["q_labels"][0]) == ro["q"]["labels"]).mean()
    agree_k = (np_i(r["k_labels"][0]) == ro["k"]["labels"]).mean()
    _, ld = O.dense_attention(*(O.round_bf16(x) for x in (q, k, v)), w.scale)
    rec_g = O.recall(to64(r["lse"][0]), ld).mean()
    rec_o = O.recall(ro["lse"], ld).mean()
    print(f"[tiny free-running] label agreement q={agree_q:.4f} k={agree_k:.4f}; recall gpu={rec_g:.4f} "
          f"oracle={rec_o:.4f}")
    assert agree_q > 0.99 and agree_k > 0.99
    assert abs(rec_g - rec_o) < 0.01
    # p = 1: dense equivalence through the fused entry
    r1 = bsa.park_forward(Q, K, V, w.cq, w.ck, w.iters, 1.0, seed=0)
    Od, _ = O.dense_attention(*(O.round_bf16(x) for x in (q, k, v)), w.scale)
    e = np.abs(to64(r1["out"][0]) - Od)
    assert e.max() <= ATTN_MAX_ABS and e.mean() <= ATTN_MEAN_ABS


def test_seed_timeout_reaches_the_status_word():
    """A cooperative seeding exchange that gives up must not pass as success: the device status word
    carries PARK_DEVSTATUS_SEED_TIMEOUT. The failure is forced from the host (the launch starts with
    its failure flag raised, so every bounded wait gives up at once and each kernel ends normally)."""
    w = SMALL["small"]
    Q, K, V = inputs(w)
    M = bsa.park_qrkc_metric(Q)
    bit = bsa.PARK_DEVSTATUS_SEED_TIMEOUT
    ok = torch.zeros(1, dtype=torch.int32, device="cuda")
    ref = bsa.park_cluster(K, w.ck, 1, bsa.PARK_QRKC, M, seed=3, side=bsa.PARK_SIDE_K, status=ok)
    r_ok = bsa.park_forward(Q, K, V, w.cq, w.ck, 1, w.p, seed=3, outputs=("status",))
    torch.cuda.synchronize()
    assert int(ok.item()) == 0 and int(r_ok["status"].item()) == 0
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    bsa.lib().park_debug_force_seed_timeout(1)
    try:
        bsa.park_cluster(K, w.ck, 1, bsa.PARK_QRKC, M, seed=3, side=bsa.PARK_SIDE_K, status=st)
        r_bad = bsa.park_forward(Q, K, V, w.cq, w.ck, 1, w.p, seed=3, outputs=("status",))
        torch.cuda.synchronize()
    finally:
        bsa.lib().park_debug_force_seed_timeout(0)
    assert int(st.item()) & bit
    assert int(r_bad["status"].item()) & bit
    # the status word is or-ed into, never cleared: a later clean call leaves the bit set
    bsa.park_cluster(K, w.ck, 1, bsa.PARK_QRKC, M, seed=3, side=bsa.PARK_SIDE_K, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & bit
    # with the hook off again, a clean call is back to the reference result
    again = bsa.park_cluster(K, w.ck, 1, bsa.PARK_QRKC, M, seed=3, side=bsa.PARK_SIDE_K)
    torch.cuda.synchronize()
    assert torch.equal(again["labels"], ref["labels"]) and torch.equal(again["centroids"], ref["centroids"])
