"""Top-k selection and the four estimator block maps (PARK-p2 Tables 1 and 10) on the GPU against the
fp64 oracle, on the ragged bf16 case (2 heads, N = 3330, Cq = 24, Ck = 96) and the d = 64 case."""
import numpy as np
import pytest
import torch

import block_sparse_attention_qrkc_amd as bsa
import oracle as O
from gpu_helpers import MAP_ABS, SMALL, TAU, inputs, np_i, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", params=["small", "small64"])
def clustered(request):
    w = SMALL[request.param]
    Q, K, V = inputs(w)
    M = bsa.park_qrkc_metric(Q)
    qc = bsa.park_cluster(Q, w.cq, 3, bsa.PARK_EUCLID, None, seed=1, side=bsa.PARK_SIDE_Q)
    kc = bsa.park_cluster(K, w.ck, 3, bsa.PARK_QRKC, M, seed=1, side=bsa.PARK_SIDE_K)
    A = bsa.park_retrieve_map(Q, qc["perm"], qc["offsets"], kc["centroids"], kc["offsets"])
    torch.cuda.synchronize()
    print(f"\n[case] {w.name}: H={w.heads} N={w.n} d={w.d} cq={w.cq} ck={w.ck}", flush=True)
    return w, Q, K, V, qc, kc, A


@pytest.mark.parametrize("rho", [0.0, 0.05, 0.1, 0.5, 1.0])
def test_select_topk(clustered, rho):
    w, Q, K, V, qc, kc, A = clustered
    sel = bsa.park_select_topk(A, kc["offsets"], rho)
    Ag = to64(A)
    counts, cols, keys, mask = np_i(sel["counts"]), np_i(sel["cols"]), np_i(sel["sel_keys"]), np_i(sel["mask"])
    near = 0
    for h in range(w.heads):
        sizes = np.diff(np_i(kc["offsets"][h]))
        k = O.topk_count(sizes, rho)
        _, counts_o, cols_o, keys_o = O.select_topk(Ag[h], sizes, rho)
        for i in range(w.cq):
            cg = cols[h, i, :counts[h, i]]
            assert np.array_equal(np.flatnonzero(mask[h, i]), cg)
            assert np.all(np.diff(cg) > 0) and np.all(sizes[cg] > 0)
            assert counts[h, i] == counts_o[i] == (k if Ag[h, i].sum() > 0 else 0)
            assert keys[h, i] == sizes[cg].sum()
            if np.array_equal(cg, cols_o[i]):
                continue
            # a differing row is a near-tie: the blocks that differ tie in importance at the cut
            diff = np.setxor1d(cg, cols_o[i])
            kept = Ag[h, i, cols_o[i]]
            assert np.all(np.abs(Ag[h, i, diff] - kept.min()) <= TAU), (h, i)
            near += 1
    print(f"[top-k {rho}] near-ties: {near}")


def test_select_topk_hand_fixture():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "topk_hand.json")))
    A = torch.tensor(g["map"], dtype=torch.float32, device="cuda")[None].contiguous()
    ko = torch.tensor([np.concatenate([[0], np.cumsum(g["k_sizes"])]).tolist()], dtype=torch.int32, device="cuda")
    for case in g["cases"]:
        sel = bsa.park_select_topk(A, ko, case["rho"])
        counts, cols, keys = np_i(sel["counts"])[0], np_i(sel["cols"])[0], np_i(sel["sel_keys"])[0]
        assert [cols[i, :counts[i]].tolist() for i in range(len(g["map"]))] == case["cols"], case["rho"]
        assert keys.tolist() == case["keys"]


@pytest.mark.parametrize("mode", ["FC", "CC", "CF", "FF"])
def test_estimator_maps(clustered, mode):
    w, Q, K, V, qc, kc, A = clustered
    m = {"FC": bsa.PARK_EST_FC, "CC": bsa.PARK_EST_CC, "CF": bsa.PARK_EST_CF, "FF": bsa.PARK_EST_FF}[mode]
    E = bsa.park_estimator_map(m, kc["offsets"], q=Q, k=K, q_perm=qc["perm"], q_offsets=qc["offsets"],
                               q_centroids=qc["centroids"], k_perm=kc["perm"], k_centroids=kc["centroids"])
    if mode == "FC":  # the PAMA map itself
        assert torch.equal(E, A)
    Eg = to64(E)
    for h in range(w.heads):
        qp, qo = np_i(qc["perm"][h]), np_i(qc["offsets"][h])
        kp, ko = np_i(kc["perm"][h]), np_i(kc["offsets"][h])
        # centroids as consumed by the matrix cores
        qcent = O.round_bf16(to64(qc["centroids"][h]))
        kcent = O.round_bf16(to64(kc["centroids"][h]))
        Eo = O.estimator_block_maps(to64(Q[h]), to64(K[h]), qp, qo, qcent, kp, ko, kcent, w.scale)[mode]
        err = np.abs(Eg[h] - Eo).max()
        assert err <= MAP_ABS, (mode, h, err)
        live = np.diff(qo) > 0
        assert np.abs(Eg[h][live].sum(1) - 1).max() <= MAP_ABS
        assert np.all(Eg[h][~live] == 0) and np.all(Eg[h][:, np.diff(ko) == 0] == 0)
    print(f"[estimator {mode}] ok")


@pytest.mark.parametrize("name", ["small", "small64"])
def test_cf_map_many_clusters(name):
    """The CF map's key-split passes at cluster counts beyond one merge block (300 query clusters)
    and a key-cluster count that is not a multiple of a work-group's eight, with an empty query
    cluster (zero row) and an empty key cluster (zero column); centroids are arbitrary rows."""
    w = SMALL[name]
    rng = np.random.default_rng(5)
    Q, K, V = inputs(w)
    H, N, d = w.heads, w.n, w.d
    cq, ck = 300, 203
    qps, qos, kps, kos = [], [], [], []
    for h in range(H):
        ql = rng.integers(0, cq, N)
        ql[ql == 17] = 18            # empty query cluster
        kl = rng.integers(0, ck, N)
        kl[kl == 40] = 41            # empty key cluster
        qp, qo = O.cluster_order(ql, cq)
        kp, ko = O.cluster_order(kl, ck)
        qps.append(qp); qos.append(qo); kps.append(kp); kos.append(ko)
    T = lambda a: torch.tensor(np.stack(a), dtype=torch.int32, device="cuda").contiguous()
    qp, qo, kp, ko = map(T, (qps, qos, kps, kos))
    qcent = torch.tensor(rng.normal(0.0, 1.0, (H, cq, d)), dtype=torch.float32, device="cuda")
    kcent = torch.tensor(rng.normal(0.0, 1.0, (H, ck, d)), dtype=torch.float32, device="cuda")
    E = bsa.park_estimator_map(bsa.PARK_EST_CF, ko, q=Q, k=K, q_perm=qp, q_offsets=qo, q_centroids=qcent,
                               k_perm=kp, k_centroids=kcent)
    Eg = to64(E)
    for h in range(H):
        qcent64 = O.round_bf16(to64(qcent[h]))
        Eo = O.estimator_block_maps(to64(Q[h]), to64(K[h]), np_i(qp[h]), np_i(qo[h]), qcent64, np_i(kp[h]),
                                    np_i(ko[h]), O.round_bf16(to64(kcent[h])), w.scale)["CF"]
        err = np.abs(Eg[h] - Eo).max()
        assert err <= MAP_ABS, (h, err)
        assert np.all(Eg[h][17] == 0) and np.all(Eg[h][:, 40] == 0)
    print(f"[cf many clusters {name}] ok")
