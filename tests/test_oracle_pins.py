"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test ties one oracle step to something other than itself: a library routine, a closed form,
a brute-force enumeration on a tiny input, or a hand-worked fixture under tests/golden.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.spatial.distance as ssd
import scipy.special as ssp
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _blobs(rng, n, d, centres, spread=0.3, scale=5.0):
    c = rng.normal(size=(centres, d)) * scale
    lab = rng.integers(0, centres, n)
    return c[lab] + spread * rng.normal(size=(n, d)), lab


# ------------------------------------------------------------------------------------ RNG
def test_splitmix64_reference_outputs():
    for case in _golden("splitmix64.json")["cases"]:
        s = case["seed"]
        for want in case["outputs"]:
            s, out = O.splitmix64_next(s)
            assert out == int(want)


def test_kpp_uniform_is_first_output_scaled():
    # u_m = (first SplitMix64 output seeded with the stream key) >> 11, times 2^-53
    first = int(_golden("splitmix64.json")["cases"][1]["outputs"][0])
    assert O.kpp_uniform(0, 0, 0, 0) == (first >> 11) * 2.0 ** -53
    u = [O.kpp_uniform(7, h, s, m) for h in range(3) for s in range(2) for m in range(50)]
    assert all(0.0 <= x < 1.0 for x in u)
    assert len(set(u)) == len(u)


# ------------------------------------------------------------------------------------ rounding
def test_round_bf16_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(size=20000) * 10.0 ** rng.integers(-5, 5, 20000),
                        # exact halfway cases: low 16 bits 0x8000, both parities of the kept lsb
                        (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32).astype(np.float64),
                        -(np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32).astype(np.float64)])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_bf16(x), want)


def test_bf16_unit_roundoff_is_two_to_minus_eight():
    """bf16 keeps 8 significant bits, so round-to-nearest errs by up to a relative 2^-8 (the bound the
    attention's log-sum-exp tolerance is derived from): 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    and rounds to the even neighbour 1; just above it rounds up."""
    x = 1.0 + 2.0 ** -8
    assert O.round_bf16(x) == 1.0
    assert abs(O.round_bf16(x) - x) / x == 2.0 ** -8 / (1.0 + 2.0 ** -8)
    assert O.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -20) == 1.0 + 2.0 ** -7
    # no value is off by more than that
    v = np.random.default_rng(4).uniform(0.5, 4.0, 200000)
    assert (np.abs(O.round_bf16(v) - v) / v).max() <= 2.0 ** -8


def test_round_f32_known_neighbours_and_ties():
    """Nearest float32, ties to even, on values worked out from the binary expansions."""
    # 0.1 lies between the float32 values 13421772 * 2^-27 and 13421773 * 2^-27 and is nearer
    # the second (0.1 * 2^27 = 13421772.8)
    assert O.round_f32(0.1) == 13421773 * 2.0 ** -27 == 0.100000001490116119384765625
    assert O.round_f32(-0.1) == -13421773 * 2.0 ** -27
    # 1/3 * 2^25 = 11184810.67 -> 11184811 * 2^-25
    assert O.round_f32(1.0 / 3.0) == 11184811 * 2.0 ** -25
    # exact halfway cases: 1 + 2^-24 lies between 1 (even) and 1 + 2^-23 (odd) -> 1;
    # 1 + 3 * 2^-24 between 1 + 2^-23 (odd) and 1 + 2^-22 (even) -> 1 + 2^-22
    assert O.round_f32(1.0 + 2.0 ** -24) == 1.0
    assert O.round_f32(1.0 + 3 * 2.0 ** -24) == 1.0 + 2.0 ** -22
    # just above a halfway point rounds up
    assert O.round_f32(1.0 + 2.0 ** -24 + 2.0 ** -40) == 1.0 + 2.0 ** -23
    # values already in float32 are unchanged, including the largest finite one
    for v in (0.0, 1.5, -2.0 ** -149, (2.0 - 2.0 ** -23) * 2.0 ** 127):
        assert O.round_f32(v) == v
    # below half the smallest subnormal flushes to zero; above it rounds to 2^-149
    assert O.round_f32(2.0 ** -151) == 0.0
    assert O.round_f32(0.75 * 2.0 ** -149) == 2.0 ** -149


# ------------------------------------------------------------------------------------ metric
def test_qrkc_metric_is_mean_squared_qk_score_difference():
    """P9: sum_{t,u} (q.k - q.c)^2 / (N Nk) == sum_u (k-c)^T M (k-c) / Nk for M = qrkc_metric(Q)."""
    rng = np.random.default_rng(2)
    Q = rng.normal(size=(40, 6)) + 1.5  # non-zero mean: a centred covariance would fail
    K = rng.normal(size=(30, 6))
    Cn = rng.normal(size=(5, 6))
    lab = rng.integers(0, 5, 30)
    M = O.qrkc_metric(Q)
    lhs = O.qk_score_sq_error(Q, K, lab, Cn)
    rhs = np.mean([O.metric_distance(K[u:u + 1], Cn[lab[u]], M)[0] for u in range(30)])
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))
    # brute force over explicit pairs
    bf = np.mean([(Q[t] @ K[u] - Q[t] @ Cn[lab[u]]) ** 2 for t in range(40) for u in range(30)])
    assert abs(bf - lhs) <= 1e-10 * max(1.0, abs(bf))


def test_metric_distance_matches_scipy_mahalanobis():
    rng = np.random.default_rng(3)
    A = rng.normal(size=(7, 5))
    M = A.T @ A / 7
    P = rng.normal(size=(20, 5))
    c = rng.normal(size=5)
    want = ssd.cdist(P, c[None, :], "mahalanobis", VI=M)[:, 0] ** 2
    np.testing.assert_allclose(O.metric_distance(P, c, M), want, rtol=1e-12, atol=1e-12)
    want_e = ssd.cdist(P, c[None, :], "sqeuclidean")[:, 0]
    np.testing.assert_allclose(O.metric_distance(P, c), want_e, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------------------ init
def test_candidate_rows():
    np.testing.assert_array_equal(O.candidate_rows(10, 2), np.arange(10))
    r = O.candidate_rows(75600, 500)
    assert r.size == 4096 and r[0] == 0 and r[-1] == (4095 * 75600) // 4096
    assert O.candidate_rows(219600, 1000).size == 8000
    assert np.all(np.diff(r) > 0)


@pytest.mark.parametrize("case", _golden("kmeanspp_hand.json")["cases"], ids=lambda c: c["name"])
def test_kmeanspp_hand_worked(case):
    X = np.asarray(case["X"], dtype=np.float64)
    M = None if case["M"] is None else np.asarray(case["M"], dtype=np.float64)
    draws = case["draws"]
    cent, chosen, _ = O.kmeanspp(X, case["C"], M, draws=lambda m: draws[m], return_trace=True)
    np.testing.assert_array_equal(chosen, case["chosen"])
    np.testing.assert_array_equal(cent, np.asarray(case["centres"], dtype=np.float64))


def test_kmeanspp_c_equals_n_picks_every_point_once():
    """P11: with C = N distinct points every point is chosen exactly once."""
    X = np.random.default_rng(4).normal(size=(50, 3))
    _, chosen, _ = O.kmeanspp(X, 50, None, seed=3, return_trace=True)
    assert sorted(chosen.tolist()) == list(range(50))
    _, chosen, _ = O.kmeanspp(X, 50, O.qrkc_metric(X), seed=5, return_trace=True)
    assert sorted(chosen.tolist()) == list(range(50))


def test_kmeanspp_duplicates_fall_back_to_lowest_unchosen():
    X = np.zeros((6, 2))
    X[3] = 1.0
    _, chosen, _ = O.kmeanspp(X, 4, None, draws=lambda m: 0.0, return_trace=True)
    # first 0; then only row 3 has mass; then all D2 = 0 -> lowest unchosen rows 1
    assert chosen.tolist() == [0, 3, 1, 2]


def test_kmeanspp_sampling_frequencies_follow_d2():
    """Second centre is drawn with probability D^2 / sum D^2 (checked over many seeds)."""
    X = np.array([[0.0], [1.0], [2.0], [4.0]])
    counts = np.zeros(4)
    for s in range(4000):
        _, chosen, _ = O.kmeanspp(X, 2, None, draws=lambda m, s=s: 0.0 if m == 0 else O.kpp_uniform(s, 0, 0, 1),
                                  return_trace=True)
        counts[chosen[1]] += 1
    p = np.array([0, 1, 4, 16]) / 21.0
    assert np.all(np.abs(counts / 4000 - p) < 0.03)


# ------------------------------------------------------------------------------------ Lloyd
def _sk_lloyd(X, init, iters):
    from sklearn.cluster import KMeans
    km = KMeans(n_clusters=init.shape[0], init=init, n_init=1, max_iter=iters, tol=0.0, algorithm="lloyd")
    km.fit(X)
    return km.labels_, km.cluster_centers_


def test_assign_matches_scipy_argmin():
    rng = np.random.default_rng(5)
    X = rng.normal(size=(500, 8))
    C = rng.normal(size=(13, 8))
    g, b = O.consumed_centroids(C, O.EUCLID, None, bf16=False)
    d = ssd.cdist(X, O.round_f32(C), "sqeuclidean")
    np.testing.assert_array_equal(O.assign(X, g, b), np.argmin(d, axis=1))
    M = O.qrkc_metric(rng.normal(size=(60, 8)) + 0.5)
    g, b = O.consumed_centroids(C, O.QRKC, M, bf16=False)
    dm = ssd.cdist(X, O.round_f32(C), "mahalanobis", VI=M) ** 2
    srt = np.sort(dm, axis=1)
    clear = (srt[:, 1] - srt[:, 0]) > 1e-6 * (1 + srt[:, 0])
    assert clear.mean() > 0.95
    np.testing.assert_array_equal(O.assign(X, g, b)[clear], np.argmin(dm, axis=1)[clear])


def test_assign_near_tie_hand_worked():
    """The classifier that turns a differing GPU label into a near-tie or an error."""
    c = _golden("assign_near_tie_hand.json")
    X, g, b = (np.array(c[k], dtype=np.float64) for k in ("X", "g", "b"))
    np.testing.assert_array_equal(O.assign(X, g, b), c["argmin"])
    n_near, bad = O.assign_near_tie(X, g, b, np.array(c["labels_other"]), tau=c["tau"])
    assert n_near == c["near_ties"]
    np.testing.assert_array_equal(bad, c["bad_rows"])
    # identical labels: nothing to classify
    n_near, bad = O.assign_near_tie(X, g, b, np.array(c["argmin"]), tau=c["tau"])
    assert n_near == 0 and bad.size == 0
    # the band scales with tau: at tau = 0 both differing rows are errors, at 1e-4 both pass
    n_near, bad = O.assign_near_tie(X, g, b, np.array(c["labels_other"]), tau=0.0)
    assert n_near == 0 and list(bad) == [0, 1]
    n_near, bad = O.assign_near_tie(X, g, b, np.array(c["labels_other"]), tau=1e-4)
    assert n_near == 2 and bad.size == 0


def test_assign_ties_go_to_lowest_index():
    X = np.array([[0.0, 0.0], [1.0, 0.0]])
    C = np.array([[1.0, 1.0], [1.0, -1.0], [1.0, 1.0]])
    g, b = O.consumed_centroids(C, O.EUCLID, None, bf16=False)
    assert O.assign(X, g, b).tolist() == [0, 0]


def test_consumed_centroids_bf16_rules():
    rng = np.random.default_rng(6)
    C = rng.normal(size=(4, 8)).astype(np.float32).astype(np.float64)
    g, b = O.consumed_centroids(C, O.EUCLID, None, bf16=True)
    gt = torch.from_numpy(C.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(g, gt)
    np.testing.assert_array_equal(b, (gt * gt).sum(1).astype(np.float32).astype(np.float64))
    M = O.round_f32(O.qrkc_metric(rng.normal(size=(30, 8))))
    g, b = O.consumed_centroids(C, O.QRKC, M, bf16=True)
    y = C @ M  # M symmetric
    np.testing.assert_array_equal(g, torch.from_numpy(y.astype(np.float32)).to(torch.bfloat16).double().numpy())
    np.testing.assert_allclose(b, np.einsum("ij,jk,ik->i", C, M, C), rtol=1e-7)


def test_lloyd_euclid_matches_sklearn():
    rng = np.random.default_rng(7)
    X, _ = _blobs(rng, 600, 5, 8)
    init = X[rng.choice(600, 8, replace=False)]
    for iters in (1, 3, 30):
        lab, c = O.lloyd(X, init, iters, O.EUCLID, None, bf16=False)
        sl, sc = _sk_lloyd(X, O.round_f32(init), iters)
        np.testing.assert_allclose(c, sc, rtol=1e-6, atol=1e-6)
        if iters == 30:  # converged: sklearn's final relabel agrees with the last assignment
            np.testing.assert_array_equal(lab, sl)


def test_lloyd_qrkc_is_euclidean_kmeans_on_whitened_keys():
    """QRKC K-means == Euclidean K-means on y = L^T x with M = L L^T (library K-means)."""
    rng = np.random.default_rng(8)
    K, _ = _blobs(rng, 500, 4, 6, spread=0.4)
    Q = rng.normal(size=(200, 4)) * np.array([3.0, 1.0, 0.5, 0.2]) + 0.3
    M = O.round_f32(O.qrkc_metric(Q))
    L = np.linalg.cholesky(M)
    init = K[rng.choice(500, 6, replace=False)]
    lab, c = O.lloyd(K, init, 25, O.QRKC, M, bf16=False)
    sl, sc = _sk_lloyd(K @ L, O.round_f32(init) @ L, 25)
    np.testing.assert_array_equal(lab, sl)
    np.testing.assert_allclose(c, sc @ np.linalg.inv(L), rtol=1e-5, atol=1e-5)


def test_qrkc_equals_euclid_when_metric_is_isotropic():
    """P8: M = a*I (queries = scaled orthogonal rows) -> identical labels and centroids."""
    rng = np.random.default_rng(9)
    d = 8
    Q = np.vstack([np.eye(d) * 2.0, -np.eye(d) * 2.0])
    M = O.qrkc_metric(Q)
    np.testing.assert_allclose(M, np.eye(d) * 4.0 * 2 / (2 * d) * 1.0, atol=0)
    X, _ = _blobs(rng, 300, d, 5)
    # fp32 consumption: M = I/2 scales every b_j - 2 x.g_j by exactly 1/2
    ce = O.cluster(X, 5, 6, O.EUCLID, None, seed=1, side=O.SIDE_K, bf16=False)
    cm = O.cluster(X, 5, 6, O.QRKC, M, seed=1, side=O.SIDE_K, bf16=False)
    np.testing.assert_array_equal(ce["labels"], cm["labels"])
    np.testing.assert_array_equal(ce["centroids"], cm["centroids"])


def test_lloyd_objective_non_increasing():
    """P10: the K-means objective never rises from one iteration to the next (fp64 data)."""
    rng = np.random.default_rng(10)
    X = rng.normal(size=(800, 6))
    for metric, M in ((O.EUCLID, None), (O.QRKC, O.round_f32(O.qrkc_metric(rng.normal(size=(100, 6)) + 1)))):
        trace = []
        O.lloyd(X, X[:20], 12, metric, M, bf16=False, trace=trace)
        obj = []
        for lab, c in trace:
            obj.append(sum(O.metric_distance(X[lab == j], c[j], M).sum() for j in range(20)))
        assert all(b <= a * (1 + 1e-9) for a, b in zip(obj, obj[1:]))


def test_subset_update_hand_worked():
    c = _golden("subset_update_hand.json")
    X, init = np.array(c["X"]), np.array(c["init"])
    for case in c["cases"]:
        lab, cent = O.lloyd_subset(X, init, np.array(c["labels"]), case["iters"], case["stride"], case["phase"],
                                   bf16=False)
        np.testing.assert_array_equal(lab, case["labels"])
        np.testing.assert_allclose(cent, np.array(case["centroids"]), rtol=1e-7)  # centroids stored in fp32
    np.testing.assert_array_equal(O.subset_rows(10, 4, 1), [1, 5, 9])
    assert O.subset_rows(3, 4, 3).size == 0


@pytest.mark.parametrize("metric", [O.EUCLID, O.QRKC])
def test_subset_update_stride_one_is_lloyd_and_keeps_the_rest(metric):
    rng = np.random.default_rng(29)
    X, _ = _blobs(rng, 300, 6, 5, spread=1.0, scale=2.0)
    M = O.qrkc_metric(rng.normal(size=(50, 6)) + 0.5) if metric == O.QRKC else None
    init = X[rng.choice(300, 7, replace=False)]
    prev, _ = O.lloyd(X, init, 2, metric, M, bf16=True)
    # stride 1: every row is re-assigned, i.e. plain warm-started Lloyd iterations
    l1, c1 = O.lloyd_subset(X, init, prev, 3, 1, 0, metric, M, bf16=True)
    l2, c2 = O.lloyd(X, init, 3, metric, M, bf16=True)
    np.testing.assert_array_equal(l1, l2)
    np.testing.assert_array_equal(c1, c2)
    # stride 4: rows off the subset keep their labels, rows on it take the fp64 argmin, the
    # centroids are the member means, and the objective does not increase
    scrambled = rng.integers(0, 7, 300).astype(np.int32)
    c0 = O.update(X, scrambled, 7, O.round_f32(init))
    lab, cent = O.lloyd_subset(X, c0, scrambled, 1, 4, 3, metric, M, bf16=True)
    off = np.setdiff1d(np.arange(300), np.arange(3, 300, 4))
    np.testing.assert_array_equal(lab[off], scrambled[off])
    g, b = O.consumed_centroids(c0, metric, M, bf16=True)
    np.testing.assert_array_equal(lab[3::4], O.assign(X[3::4], g, b))
    np.testing.assert_array_equal(cent, O.update(X, lab, 7, c0))

    # without the bf16 rounding of the consumed centroids the re-assignment is exact, so the
    # objective cannot increase (the Lloyd argument, restricted to the re-assigned rows)
    def objective(lb, cc):
        return sum(O.metric_distance(X[lb == j], cc[j], M).sum() for j in range(7))
    lab32, cent32 = O.lloyd_subset(X, c0, scrambled, 2, 4, 3, metric, M, bf16=False)
    assert objective(lab32, cent32) <= objective(scrambled, c0) * (1 + 1e-12)


def test_update_keeps_empty_clusters():
    X = np.array([[1.0, 2.0], [3.0, 4.0]])
    prev = np.array([[9.0, 9.0], [0.0, 0.0], [5.0, -5.0]])
    c = O.update(X, np.array([1, 1]), 3, prev)
    np.testing.assert_array_equal(c, [[9.0, 9.0], [2.0, 3.0], [5.0, -5.0]])


def test_cluster_order_is_stable_argsort():
    rng = np.random.default_rng(11)
    lab = rng.integers(0, 17, 3000)
    lab[lab == 5] = 6  # an empty cluster
    perm, off = O.cluster_order(lab, 17)
    np.testing.assert_array_equal(perm, np.argsort(lab, kind="stable"))
    np.testing.assert_array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(lab, minlength=17))]))
    assert off[5] == off[6]


# ------------------------------------------------------------------------------------ PAMA
def test_pama_hand_worked():
    g = _golden("pama_hand.json")
    perm, off = O.cluster_order(np.array(g["q_labels"]), g["cq"])
    A = O.pama(np.array(g["Q"]), perm, off, np.array(g["k_cent"]), np.array(g["k_sizes"]), g["scale"])
    np.testing.assert_allclose(A, np.array(g["map"]), rtol=0, atol=1e-15)


def _toy_head(rng, n=120, d=8):
    Q = rng.normal(size=(n, d)) + 0.5
    K = rng.normal(size=(n, d)) + 0.5
    V = rng.normal(size=(n, d))
    return Q, K, V


def test_pama_rows_sum_to_one():
    """P1."""
    rng = np.random.default_rng(12)
    Q, K, _ = _toy_head(rng)
    ql = rng.integers(0, 7, 120)
    ql[ql == 3] = 4  # empty query block -> zero row
    kl = rng.integers(0, 9, 120)
    kl[kl == 2] = 1  # empty key block
    perm, off = O.cluster_order(ql, 7)
    kc = np.stack([K[kl == j].mean(0) if (kl == j).any() else np.zeros(8) for j in range(9)])
    A = O.pama(Q, perm, off, kc, np.bincount(kl, minlength=9), 0.35)
    live = np.diff(off) > 0
    np.testing.assert_allclose(A[live].sum(1), 1.0, atol=1e-12)
    assert np.all(A[~live] == 0) and np.all(A[:, 2] == 0)


def test_pama_singleton_key_clusters_equal_full_estimate():
    """P5: Ck = N singletons -> PAMA == exact block mass of the dense softmax (scipy softmax)."""
    rng = np.random.default_rng(13)
    Q, K, _ = _toy_head(rng, 60)
    ql = rng.integers(0, 5, 60)
    perm, off = O.cluster_order(ql, 5)
    s = 0.4
    A = O.pama(Q, perm, off, K, np.ones(60, dtype=np.int64), s)
    P = ssp.softmax(s * Q @ K.T, axis=1)
    for i in range(5):
        np.testing.assert_allclose(A[i], P[ql == i].mean(0), atol=1e-13)


def test_pama_singleton_queries_and_keys_is_each_query_softmax():
    """P6: Cq = Ck = N -> every map row is one query's own softmax over the keys."""
    rng = np.random.default_rng(14)
    Q, K, _ = _toy_head(rng, 40)
    ident = np.arange(40)
    A = O.pama(Q, ident, np.arange(41), K, np.ones(40, dtype=np.int64), 0.3)
    np.testing.assert_allclose(A, ssp.softmax(0.3 * Q @ K.T, axis=1), atol=1e-13)


def test_pama_size_weighting_exact_for_identical_keys():
    """P7: keys equal inside each cluster -> size-weighted centroid softmax equals the exact
    block mass (dropping the ln n term fails this)."""
    rng = np.random.default_rng(15)
    base = rng.normal(size=(6, 8))
    kl = np.repeat(np.arange(6), [1, 2, 3, 5, 8, 13])
    K = base[kl]
    Q = rng.normal(size=(30, 8))
    ql = rng.integers(0, 4, 30)
    perm, off = O.cluster_order(ql, 4)
    A = O.pama(Q, perm, off, base, np.bincount(kl), 0.5)
    P = ssp.softmax(0.5 * Q @ K.T, axis=1)
    FF = np.stack([P[:, kl == j].sum(1) for j in range(6)], axis=1)
    for i in range(4):
        np.testing.assert_allclose(A[i], FF[ql == i].mean(0), atol=1e-13)


# ------------------------------------------------------------------------------------ top-p
def test_topp_hand_worked():
    g = _golden("topp_hand.json")
    A = np.array(g["map"])
    ks = np.array(g["k_sizes"])
    for case in g["cases"]:
        mask, counts, cols, keys = O.select_topp(A, ks, case["p"])
        assert [c.tolist() for c in cols] == case["cols"], case["p"]
        assert keys.tolist() == case["keys"]
        assert counts.tolist() == [len(c) for c in case["cols"]]
        assert np.array_equal(mask, np.array([[j in c for j in range(5)] for c in case["cols"]]))


def test_topk_hand_worked():
    g = _golden("topk_hand.json")
    A = np.array(g["map"])
    ks = np.array(g["k_sizes"])
    for case in g["cases"]:
        assert O.topk_count(ks, case["rho"]) == case["k"]
        mask, counts, cols, keys = O.select_topk(A, ks, case["rho"])
        assert [c.tolist() for c in cols] == case["cols"], case["rho"]
        assert keys.tolist() == case["keys"]
        assert counts.tolist() == [len(c) for c in case["cols"]]


def test_topk_count_guards_rounding():
    assert O.topk_count([1] * 10, 0.3) == 3       # 0.3 * 10 is 3.0000000000000004 in fp64
    assert O.topk_count([1] * 500, 0.1) == 50
    assert O.topk_count([1] * 7, 0.1) == 1
    assert O.topk_count([0, 0], 0.5) == 0


def test_topk_is_max_mass_set_bruteforce():
    """The kept set has the largest importance among all k-subsets of non-empty blocks, and is the
    lexicographically smallest among the sets that tie with it."""
    rng = np.random.default_rng(4)
    for trial in range(40):
        ck = int(rng.integers(2, 8))
        sizes = rng.integers(0, 3, ck)
        if not (sizes > 0).any():
            sizes[0] = 1
        A = np.round(rng.random((3, ck)), 1)  # coarse values: ties happen
        A[:, sizes == 0] = 0.0
        rho = float(rng.choice([0.1, 0.3, 0.5, 0.7, 1.0]))
        k = O.topk_count(sizes, rho)
        live = [j for j in range(ck) if sizes[j] > 0]
        _, _, cols, _ = O.select_topk(A, sizes, rho)
        for i in range(3):
            if not (A[i] > 0).any():
                assert cols[i].size == 0
                continue
            best = max(itertools.combinations(live, k), key=lambda c: (sum(A[i, list(c)]), [-x for x in c]))
            assert cols[i].tolist() == sorted(best), (trial, i)


# ------------------------------------------------------------------------------------ SIP
def test_sip_probabilities_hand_worked():
    for case in _golden("sip_hand.json")["probabilities"]:
        pi = O.sip_probabilities(case["a"], case["m"])
        np.testing.assert_allclose(pi, case["pi"], rtol=0, atol=1e-15, err_msg=case["work"])


def test_sip_probabilities_match_bisection():
    """An independent solver: bisection on kappa of the monotone sum_j min(1, kappa a_j) - m."""
    rng = np.random.default_rng(21)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        a = rng.dirichlet(np.ones(n) * float(rng.choice([0.1, 0.5, 2.0])))
        a[rng.random(n) < 0.2] = 0.0
        npos = int((a > 0).sum())
        m = int(rng.integers(1, n + 2))
        pi = O.sip_probabilities(a, m)
        assert np.all((pi >= 0) & (pi <= 1)) and np.all(pi[a == 0] == 0), trial
        if npos == 0:
            continue
        if m >= npos:
            assert np.all(pi[a > 0] == 1), trial
            continue
        lo, hi = 0.0, 1.0 / a[a > 0].min()  # at hi every positive block is capped: the sum is npos > m
        for _ in range(200):
            mid = 0.5 * (lo + hi)
            if np.minimum(1.0, mid * a).sum() < m:
                lo = mid
            else:
                hi = mid
        np.testing.assert_allclose(pi, np.minimum(1.0, hi * a), rtol=0, atol=1e-12, err_msg=str(trial))
        assert abs(pi.sum() - m) < 1e-12, trial


def test_sip_inclusion_frequencies_match_probabilities():
    """Over many seeds block j of a row is kept with frequency pi_j (within 5 binomial sigma), kept
    blocks carry ln(1/pi), blocks with pi = 1 are always kept and empty clusters never."""
    A = np.array([[0.05, 0.6, 0.0, 0.25, 0.1, 0.0], [0.3, 0.3, 0.2, 0.1, 0.05, 0.05]])
    sizes = np.array([3, 2, 4, 1, 5, 0])
    rho = 0.5  # 5 non-empty clusters: m = ceil(2.5) = 3
    S = 3000
    hits = np.zeros_like(A)
    pi = None
    for seed in range(S):
        mask, counts, cols, keys, log_w, pi = O.select_sip(A, sizes, rho, seed=seed, head=3)
        hits += mask
        assert np.all(mask[:, 5] == 0) and np.all(mask[pi == 1.0])
        np.testing.assert_allclose(log_w[mask], -np.log(pi[mask]), rtol=0, atol=1e-15)
        assert np.all(log_w[~mask] == 0)
        assert keys.tolist() == [int(sizes[c].sum()) for c in cols]
    np.testing.assert_allclose(pi.sum(axis=1), [3.0, 3.0], atol=1e-12)
    freq = hits / S
    sigma = np.sqrt(pi * (1 - pi) / S)
    assert np.all(np.abs(freq - pi) <= 5 * sigma + 1e-12), (freq, pi)


def test_weighted_attention_hand_worked():
    g = _golden("sip_hand.json")["weighted_attention"]
    Q, K, V = (np.array(g[x]) for x in ("q", "k", "v"))
    out, lse = O.weighted_sparse_attention(Q, K, V, [0], [0, 1], [0, 1], [0, 1, 2], [np.array([0, 1])],
                                           np.log([g["w"]]), 1.0)
    np.testing.assert_allclose(out, g["out"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, g["lse"], rtol=0, atol=1e-15)


def test_sip_weighted_attention_is_unbiased_by_enumeration():
    """Summed over every inclusion pattern, weighted by its probability, the weighted numerator
    sum_j w_j sum_(k in j) e^(s q.k) v_k and denominator of each query equal the dense ones."""
    rng = np.random.default_rng(5)
    nq, n, d, ck = 7, 30, 8, 6
    Q, K, V = rng.normal(size=(nq, d)), rng.normal(size=(n, d)), rng.normal(size=(n, d))
    labels = np.concatenate([np.arange(ck), rng.integers(0, ck, n - ck)])
    k_perm = np.argsort(labels, kind="stable")
    k_off = np.concatenate([[0], np.cumsum(np.bincount(labels, minlength=ck))])
    a = np.array([0.55, 0.2, 0.1, 0.08, 0.05, 0.02])  # the first block is capped at m = 3
    pi = O.sip_probabilities(a, 3)
    assert pi[0] == 1.0 and np.all(pi[1:] < 1.0)
    scale = 0.4
    num = np.zeros((nq, d))
    den = np.zeros(nq)
    for pattern in itertools.product([False, True], repeat=ck):
        inc = np.array(pattern)
        prob = np.prod(np.where(inc, pi, 1.0 - pi))
        if prob == 0.0:
            continue
        log_w = np.where(inc, -np.log(pi), 0.0)[None, :]
        out, lse = O.weighted_sparse_attention(Q, K, V, np.arange(nq), [0, nq], k_perm, k_off,
                                               [np.flatnonzero(inc)], log_w, scale)
        e = np.exp(lse)
        num += prob * e[:, None] * out
        den += prob * e
    Od, lsed = O.dense_attention(Q, K, V, scale)
    np.testing.assert_allclose(den, np.exp(lsed), rtol=1e-12)
    np.testing.assert_allclose(num, np.exp(lsed)[:, None] * Od, rtol=1e-11, atol=1e-13)


def test_sip_full_budget_is_dense():
    """With the budget covering every block (rho = 1) every non-empty block is kept with weight 1
    and the weighted attention is dense attention."""
    rng = np.random.default_rng(8)
    n, d, cq, ck = 64, 8, 4, 5
    Q, K, V = rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, d))
    ql = rng.integers(0, cq, n)
    kl = np.concatenate([np.arange(ck), rng.integers(0, ck, n - ck)])
    qp, kp = np.argsort(ql, kind="stable"), np.argsort(kl, kind="stable")
    qo = np.concatenate([[0], np.cumsum(np.bincount(ql, minlength=cq))])
    ko = np.concatenate([[0], np.cumsum(np.bincount(kl, minlength=ck))])
    A = rng.dirichlet(np.ones(ck), size=cq)
    mask, counts, cols, keys, log_w, pi = O.select_sip(A, np.diff(ko), 1.0, seed=2)
    assert mask.all() and np.all(log_w == 0)
    out, lse = O.weighted_sparse_attention(Q, K, V, qp, qo, kp, ko, cols, log_w, 0.3)
    Od, lsed = O.dense_attention(Q, K, V, 0.3)
    np.testing.assert_allclose(out, Od, atol=1e-13)
    np.testing.assert_allclose(lse, lsed, atol=1e-13)


def test_topp_is_minimal_max_mass_set_bruteforce():
    """P2 by enumeration: the kept set reaches p, no smaller set does, and among sets of its size it
    has the largest mass (ties broken toward lower indices)."""
    rng = np.random.default_rng(16)
    for trial in range(300):
        ck = int(rng.integers(1, 7))
        row = rng.dirichlet(np.ones(ck) * 0.7)
        if trial % 5 == 0:
            row = np.round(row * 8) / 8  # exact ties and exact hits of p
            if row.sum() == 0:
                continue
            row = row / row.sum()
        p = float(rng.choice([0.3, 0.5, 0.75, 0.9, 0.95]))
        mask, _, cols, _ = O.select_topp(row[None, :], np.ones(ck, dtype=np.int64), p)
        sel = tuple(cols[0].tolist())
        best = None
        for k in range(1, ck + 1):
            cands = [c for c in itertools.combinations(range(ck), k) if row[list(c)].sum() >= p]
            if cands:
                top = max(row[list(c)].sum() for c in cands)
                best = [c for c in cands if row[list(c)].sum() == top]
                break
        if best is None:  # rounding: the whole row is below p
            assert sel == tuple(np.flatnonzero(row > 0))
            continue
        assert len(sel) == len(best[0])
        assert row[list(sel)].sum() == row[list(best[0])].sum()
        assert sel == min(best)  # lexicographically smallest among equal-mass sets


# ------------------------------------------------------------------------------------ attention
def _selection(rng, cq, ck, k_sizes, density=0.5):
    cols = []
    for _ in range(cq):
        c = np.flatnonzero((rng.random(ck) < density) & (k_sizes > 0))
        if c.size == 0:
            c = np.flatnonzero(k_sizes > 0)[:1]
        cols.append(c.astype(np.int32))
    return cols


def test_sparse_attention_matches_torch_sdpa_with_block_mask():
    rng = np.random.default_rng(17)
    n, d = 150, 16
    Q, K, V = (rng.normal(size=(n, d)) for _ in range(3))
    ql = rng.integers(0, 6, n)
    kl = rng.integers(0, 9, n)
    kl[kl == 4] = 5
    qp, qo = O.cluster_order(ql, 6)
    kp, ko = O.cluster_order(kl, 9)
    cols = _selection(rng, 6, 9, np.diff(ko))
    s = 0.3
    Os, lse = O.sparse_attention(Q, K, V, qp, qo, kp, ko, cols, s)
    allowed = np.zeros((n, n), dtype=bool)
    for t in range(n):
        allowed[t] = np.isin(kl, cols[ql[t]])
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
        attn_mask=torch.from_numpy(allowed)[None], scale=s)[0].numpy()
    np.testing.assert_allclose(Os, want, atol=1e-12)
    sc = torch.from_numpy(s * Q @ K.T).masked_fill(~torch.from_numpy(allowed), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(sc, dim=1).numpy(), atol=1e-12)


def test_dense_attention_matches_torch_sdpa():
    rng = np.random.default_rng(18)
    Q, K, V = (rng.normal(size=(70, 8)) for _ in range(3))
    Od, lse = O.dense_attention(Q, K, V, 0.25, block=16)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None], scale=0.25)[0].numpy()
    np.testing.assert_allclose(Od, want, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(torch.from_numpy(0.25 * Q @ K.T), 1).numpy(), atol=1e-12)


def test_p_one_sparse_equals_dense():
    """P3: top-p with p = 1 keeps all non-empty key clusters, so sparse == dense."""
    rng = np.random.default_rng(19)
    Q, K, V = _toy_head(rng, 100)
    r = O.retrieve(Q, K, 6, 10, 3, 1.0, 0.3, bf16=False)
    Os, ls = O.sparse_attention(Q, K, V, r["q"]["perm"], r["q"]["offsets"], r["k"]["perm"],
                                r["k"]["offsets"], r["cols"], 0.3)
    Od, ld = O.dense_attention(Q, K, V, 0.3)
    np.testing.assert_allclose(Os, Od, atol=1e-12)
    np.testing.assert_allclose(ls, ld, atol=1e-12)


def test_identity_values_return_the_masked_softmax():
    """P16: with V = I the attention output is the masked softmax matrix itself."""
    rng = np.random.default_rng(20)
    n = 64
    Q, K = rng.normal(size=(n, n)), rng.normal(size=(n, n))
    ql, kl = rng.integers(0, 4, n), rng.integers(0, 5, n)
    qp, qo = O.cluster_order(ql, 4)
    kp, ko = O.cluster_order(kl, 5)
    cols = _selection(rng, 4, 5, np.diff(ko))
    Os, _ = O.sparse_attention(Q, K, np.eye(n), qp, qo, kp, ko, cols, 0.125)
    for t in range(n):
        sel = np.isin(kl, cols[ql[t]])
        want = np.zeros(n)
        want[sel] = ssp.softmax(0.125 * Q[t] @ K[sel].T)
        np.testing.assert_allclose(Os[t], want, atol=1e-13)


def test_recall_from_lse_equals_bruteforce_softmax_mass():
    """P13: exp(LSE_sel - LSE_dense) == the dense softmax mass on the selected keys."""
    rng = np.random.default_rng(21)
    Q, K, V = _toy_head(rng, 90)
    ql, kl = rng.integers(0, 5, 90), rng.integers(0, 7, 90)
    qp, qo = O.cluster_order(ql, 5)
    kp, ko = O.cluster_order(kl, 7)
    cols = _selection(rng, 5, 7, np.diff(ko), 0.4)
    _, ls = O.sparse_attention(Q, K, V, qp, qo, kp, ko, cols, 0.3)
    _, ld = O.dense_attention(Q, K, V, 0.3)
    r = O.recall(ls, ld)
    P = ssp.softmax(0.3 * Q @ K.T, axis=1)
    want = np.array([P[t, np.isin(kl, cols[ql[t]])].sum() for t in range(90)])
    np.testing.assert_allclose(r, want, atol=1e-13)


def test_full_full_topp_recall_reaches_p():
    """P4 (Table 1 Full/Full rows: worst recall just above p): selecting blocks by the exact
    block mass gives every query block a mean recall >= p."""
    rng = np.random.default_rng(22)
    Q, K, V = _toy_head(rng, 200, 8)
    r = O.retrieve(Q, K, 8, 16, 4, 0.9, 0.35, bf16=False)
    ql, kl = r["q"]["labels"], r["k"]["labels"]
    est = O.estimator_maps(Q, K, ql, kl, r["q"]["centroids"], r["k"]["centroids"], 0.35)
    qp, qo = r["q"]["perm"], r["q"]["offsets"]
    A_ff = np.stack([est["FF"][qp[qo[i]:qo[i + 1]]].mean(0) if qo[i + 1] > qo[i] else np.zeros(16)
                     for i in range(8)])
    _, _, cols, _ = O.select_topp(A_ff, np.diff(r["k"]["offsets"]), 0.9)
    _, ls = O.sparse_attention(Q, K, V, qp, qo, r["k"]["perm"], r["k"]["offsets"], cols, 0.35)
    _, ld = O.dense_attention(Q, K, V, 0.35)
    rec = O.recall(ls, ld)
    for i in range(8):
        t = qp[qo[i]:qo[i + 1]]
        if t.size:
            assert rec[t].mean() >= 0.9 - 1e-12
    # and the FC (PAMA) rows are the per-query rows of the FC estimator, averaged
    A_fc = O.pama(Q, qp, qo, r["k"]["centroids"], np.diff(r["k"]["offsets"]), 0.35)
    for i in range(8):
        t = qp[qo[i]:qo[i + 1]]
        if t.size:
            np.testing.assert_allclose(A_fc[i], est["FC"][t].mean(0), atol=1e-13)


def test_merge_clusters_hand_worked():
    for c in _golden("merge_hand.json")["cases"]:
        group, sel = O.merge_clusters(c["q_sizes"], c["cols"], c["k_sizes"], c["bm"])
        np.testing.assert_array_equal(group, c["group"])
        assert {str(r): v.tolist() for r, v in sel.items()} == c["sel"]


def _merge_case(rng, cq=40, ck=60):
    q_sizes = rng.integers(0, 700, cq) * (rng.random(cq) < 0.9)
    k_sizes = rng.integers(0, 300, ck)
    cols = [np.sort(rng.choice(ck, size=int(rng.integers(0, ck // 2)), replace=False)) for _ in range(cq)]
    return q_sizes, k_sizes, cols


@pytest.mark.parametrize("bm", [1, 32, 384])
def test_merge_clusters_invariants(bm):
    """Every cluster lands in exactly one group under its lowest member; a group selects the union
    of its members' selections; the total cost does not increase; no two final groups gain by
    merging; with bm = 1 no merge can gain (n_a L_a + n_b L_b <= (n_a + n_b) L(union))."""
    rng = np.random.default_rng(bm)
    for _ in range(3):
        q_sizes, k_sizes, cols = _merge_case(rng)
        group, sel = O.merge_clusters(q_sizes, cols, k_sizes, bm)
        L = lambda s: int(k_sizes[np.asarray(list(s), dtype=np.int64)].sum()) if len(s) else 0
        roots = sorted(set(group.tolist()))
        assert all(group[r] == r and np.all(np.flatnonzero(group == r) >= r) for r in roots)
        total0 = sum(O.merge_cost(q_sizes[i], L(cols[i]), bm) for i in range(len(q_sizes)) if q_sizes[i] > 0)
        total = 0
        for r in roots:
            members = np.flatnonzero(group == r)
            union = set().union(*(set(cols[i].tolist()) for i in members)) if q_sizes[r] > 0 else set()
            assert sel[r].tolist() == sorted(union)
            total += O.merge_cost(q_sizes[members].sum(), L(union), bm)
        assert total <= total0
        if bm == 1:
            assert len(roots) == len(q_sizes)
        live = [r for r in roots if q_sizes[r] > 0]
        for a in live:
            for b in live:
                if a < b:
                    na, nb = q_sizes[group == a].sum(), q_sizes[group == b].sum()
                    g = (O.merge_cost(na, L(sel[a]), bm) + O.merge_cost(nb, L(sel[b]), bm)
                         - O.merge_cost(na + nb, L(set(sel[a].tolist()) | set(sel[b].tolist())), bm))
                    assert g <= 0, (a, b, g)


def test_merged_order_is_a_clustering():
    rng = np.random.default_rng(5)
    q_sizes, k_sizes, cols = _merge_case(rng)
    labels = np.repeat(np.arange(q_sizes.size), q_sizes)
    rng.shuffle(labels)
    q_perm, q_off = O.cluster_order(labels, q_sizes.size)
    group, sel = O.merge_clusters(q_sizes, cols, k_sizes, 384)
    perm, off, mcols = O.merged_order(q_perm, q_off, group, sel)
    np.testing.assert_array_equal(np.sort(perm), np.arange(labels.size))
    roots = sorted(set(group.tolist()))
    assert off[-1] == labels.size and np.all(np.diff(off) >= 0) and np.all(np.diff(off)[len(roots):] == 0)
    for g, r in enumerate(roots):
        members = np.flatnonzero(group == r)
        np.testing.assert_array_equal(perm[off[g]:off[g + 1]],
                                      np.concatenate([q_perm[q_off[i]:q_off[i + 1]] for i in members]))
        np.testing.assert_array_equal(mcols[g], sel[r])


def test_key_runs_merge_adjacent_clusters():
    off = np.array([0, 3, 3, 7, 9, 12])
    assert O.key_runs([0, 1, 2], off) == [(0, 7)]
    assert O.key_runs([0, 3, 4], off) == [(0, 3), (7, 12)]
    assert O.key_runs([1], off) == []


def test_density_definitions():
    mask = np.array([[1, 0], [1, 1]], dtype=bool)
    b, t = O.density(mask, [2, 3], [1, 4])
    assert b == 3 / 4
    assert t == (2 * 1 + 3 * 1 + 3 * 4) / 25


def _estimator_case(rng, n=48, d=6, cq=5, ck=7):
    Q = rng.normal(size=(n, d))
    K = rng.normal(size=(n, d))
    ql = rng.integers(0, cq, n)
    kl = rng.integers(0, ck, n)
    qp, qo = O.cluster_order(ql, cq)
    kp, ko = O.cluster_order(kl, ck)
    qc = np.stack([Q[ql == i].mean(0) if (ql == i).any() else np.zeros(d) for i in range(cq)])
    kc = np.stack([K[kl == j].mean(0) if (kl == j).any() else np.zeros(d) for j in range(ck)])
    return Q, K, qp, qo, qc, kp, ko, kc, np.diff(ko)


def test_estimator_block_maps_fc_is_pama_and_rows_are_distributions():
    rng = np.random.default_rng(8)
    Q, K, qp, qo, qc, kp, ko, kc, ks = _estimator_case(rng)
    m = O.estimator_block_maps(Q, K, qp, qo, qc, kp, ko, kc, 0.4)
    np.testing.assert_allclose(m["FC"], O.pama(Q, qp, qo, kc, ks, 0.4), atol=1e-13)
    live = np.diff(qo) > 0
    for name, A in m.items():
        np.testing.assert_allclose(A[live].sum(1), 1.0, atol=1e-12, err_msg=name)
        assert np.all(A[~live] == 0) and np.all(A[:, ks == 0] == 0), name


def test_estimator_block_maps_collapse_in_the_limits():
    """Singleton key blocks make key centroids exact (FC = FF, CC = CF); singleton query blocks make
    query centroids exact (CF = FF, CC = FC); identical keys in every block make the size-weighted
    key-centroid softmax exact (FC = FF, CC = CF)."""
    rng = np.random.default_rng(9)
    n, d = 24, 5
    Q = rng.normal(size=(n, d))
    K = rng.normal(size=(n, d))
    ql = rng.integers(0, 4, n)
    qp, qo = O.cluster_order(ql, 4)
    qc = np.stack([Q[ql == i].mean(0) for i in range(4)])
    kp, ko = O.cluster_order(np.arange(n), n)  # one key per block
    m = O.estimator_block_maps(Q, K, qp, qo, qc, kp, ko, K.copy(), 0.5)
    np.testing.assert_allclose(m["FC"], m["FF"], atol=1e-13)
    np.testing.assert_allclose(m["CC"], m["CF"], atol=1e-13)
    kl = rng.integers(0, 5, n)
    kp, ko = O.cluster_order(kl, 5)
    kc = np.stack([K[kl == j].mean(0) for j in range(5)])
    qp1, qo1 = O.cluster_order(np.arange(n), n)  # one query per block
    m = O.estimator_block_maps(Q, K, qp1, qo1, Q.copy(), kp, ko, kc, 0.5)
    np.testing.assert_allclose(m["CF"], m["FF"], atol=1e-13)
    np.testing.assert_allclose(m["CC"], m["FC"], atol=1e-13)
    base = rng.normal(size=(5, d))
    K2 = base[kl]  # every key equals its block's centroid
    m = O.estimator_block_maps(Q, K2, qp, qo, qc, kp, ko, base, 0.5)
    np.testing.assert_allclose(m["FC"], m["FF"], atol=1e-12)
    np.testing.assert_allclose(m["CC"], m["CF"], atol=1e-12)


def test_tv_to_full_hand_values():
    """Mean over rows of half the L1 distance (PARK page, Table 4: mean attention-weight TV)."""
    assert O.tv_to_full([[0.5, 0.5]], [[1.0, 0.0]]) == 0.5
    assert O.tv_to_full([[0.0, 1.0]], [[1.0, 0.0]]) == 1.0  # disjoint supports: the maximum
    # rows 0.5 and 0 -> mean 0.25
    assert O.tv_to_full([[0.5, 0.5], [1.0, 0.0]], [[1.0, 0.0], [1.0, 0.0]]) == 0.25
    # 0.5 * (0.3 + 0 + 0.3) = 0.3
    assert abs(O.tv_to_full([[0.2, 0.3, 0.5]], [[0.5, 0.3, 0.2]]) - 0.3) < 1e-15
    # symmetric
    a, b = [[0.1, 0.6, 0.3]], [[0.4, 0.4, 0.2]]
    assert O.tv_to_full(a, b) == O.tv_to_full(b, a)


def test_raw_key_mse_hand_value():
    """Mean over keys of the squared distance to the key's centroid (PARK page, Table 5)."""
    K = [[1.0, 2.0], [3.0, 5.0], [0.0, 0.0]]
    cent = [[2.0, 3.0], [1.0, -1.0]]
    # |(-1,-1)|^2 = 2, |(1,2)|^2 = 5, |(-1,1)|^2 = 2 -> mean 3
    assert O.raw_key_mse(K, np.array([0, 0, 1]), cent) == 3.0
    # labels index the centroids: swapping them changes the value
    # |(0,3)|^2 = 9, |(2,6)|^2 = 40, |(-2,-3)|^2 = 13 -> mean 62 / 3
    assert abs(O.raw_key_mse(K, np.array([1, 1, 0]), cent) - 62.0 / 3.0) < 1e-13


def test_tv_zero_for_full_and_estimators_are_distributions():
    rng = np.random.default_rng(23)
    Q, K, _ = _toy_head(rng, 80)
    r = O.retrieve(Q, K, 5, 8, 3, 0.9, 0.35, bf16=False)
    est = O.estimator_maps(Q, K, r["q"]["labels"], r["k"]["labels"], r["q"]["centroids"],
                           r["k"]["centroids"], 0.35)
    assert O.tv_to_full(est["FF"], est["FF"]) == 0.0
    for v in est.values():
        np.testing.assert_allclose(v.sum(1), 1.0, atol=1e-12)
