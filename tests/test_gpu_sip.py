"""Sampling with inclusion-probability weighting (AB-Attention page, SIP paragraph) and the
block-weighted attention on the GPU against the fp64 oracle, on the ragged bf16 cases (d = 128 and
d = 64) and the fp32 tiny workload."""
import json
import os

import numpy as np
import pytest
import torch

import block_sparse_attention_qrkc_amd as bsa
import oracle as O
from gpu_helpers import (ATTN_MAX_ABS, ATTN_MEAN_ABS, LSE_ABS, SMALL, attn_view, cols_list, inputs, np_i, to64)

pytestmark = pytest.mark.gpu

# a differing sampling decision is a near-tie when the draw lies this close to the probability
# (the probabilities differ between the two sides only by fp64 summation order)
U_TIE = 1e-9
# kept log weights: fp32 rounding of ln(1/pi) on top of fp64 probabilities
LOGW_ABS = 1e-6


@pytest.fixture(scope="module", params=["small", "small64", "tiny"])
def clustered(request):
    w = SMALL[request.param]
    Q, K, V = inputs(w)
    M = bsa.park_qrkc_metric(Q)
    qc = bsa.park_cluster(Q, w.cq, 3, bsa.PARK_EUCLID, None, seed=1, side=bsa.PARK_SIDE_Q)
    kc = bsa.park_cluster(K, w.ck, 3, bsa.PARK_QRKC, M, seed=1, side=bsa.PARK_SIDE_K)
    A = bsa.park_retrieve_map(Q, qc["perm"], qc["offsets"], kc["centroids"], kc["offsets"])
    torch.cuda.synchronize()
    print(f"\n[case] {w.name}: H={w.heads} N={w.n} d={w.d} {w.dtype} cq={w.cq} ck={w.ck}", flush=True)
    return w, Q, K, V, qc, kc, A


def _check_sip(A64, sizes, rho, seed, head, counts, cols, mask, keys, log_w):
    """One head of a GPU SIP selection against the oracle fed the same map. Returns near-ties."""
    mask_o, counts_o, cols_o, keys_o, log_w_o, pi = O.select_sip(A64, sizes, rho, seed=seed, head=head)
    cq, ck = A64.shape
    near = 0
    for i in range(cq):
        cg = cols[i, :counts[i]]
        assert np.array_equal(np.flatnonzero(mask[i]), cg)
        assert np.all(np.diff(cg) > 0) and np.all(sizes[cg] > 0)
        assert keys[i] == sizes[cg].sum()
        for j in np.setxor1d(cg, cols_o[i]):
            u = O.sip_uniform(seed, head, i, int(j), ck)
            assert abs(u - pi[i, j]) <= U_TIE, (i, j, u, pi[i, j])
            near += 1
        both = np.intersect1d(cg, cols_o[i])
        np.testing.assert_allclose(log_w[i, both], log_w_o[i, both], rtol=0, atol=LOGW_ABS)
        assert np.all(log_w[i, ~mask[i].astype(bool)] == 0)
        assert np.all(pi[i, cg] > 0)
    return near


@pytest.mark.parametrize("rho", [0.05, 0.1, 0.3, 1.0])
def test_select_sip(clustered, rho):
    w, Q, K, V, qc, kc, A = clustered
    seed = 11
    sel = bsa.park_select_sip(A, kc["offsets"], rho, seed=seed)
    Ag = to64(A)
    counts, cols, mask = np_i(sel["counts"]), np_i(sel["cols"]), np_i(sel["mask"])
    keys, log_w = np_i(sel["sel_keys"]), to64(sel["log_w"])
    near = 0
    for h in range(w.heads):
        sizes = np.diff(np_i(kc["offsets"][h]))
        near += _check_sip(Ag[h], sizes, rho, seed, h, counts[h], cols[h], mask[h], keys[h], log_w[h])
        if rho == 1.0:  # the budget covers every block: all non-empty blocks with weight 1
            live = np.diff(np_i(qc["offsets"][h])) > 0
            assert np.all(mask[h][live] == (sizes > 0)[None, :]) and np.all(log_w[h] == 0)
    print(f"[sip {rho}] near-ties: {near}")


def test_select_sip_hand_probabilities():
    """The hand-worked inclusion probabilities: a kept block's weight is 1/pi, and blocks with pi = 1
    are always kept (budget m = ceil(rho * C_ne) with rho = m / C_ne)."""
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "sip_hand.json")))
    for case in g["probabilities"]:
        a = np.array(case["a"])
        ck = a.size
        A = torch.tensor(a[None, None, :], dtype=torch.float32, device="cuda").contiguous()
        ko = torch.arange(ck + 1, dtype=torch.int32, device="cuda")[None].contiguous()
        want = np.array(case["pi"])
        for seed in range(20):
            sel = bsa.park_select_sip(A, ko, case["m"] / ck, seed=seed)
            m = np_i(sel["mask"])[0, 0].astype(bool)
            lw = to64(sel["log_w"])[0, 0]
            assert np.all(m[want == 1.0]) and not np.any(m[want == 0.0]), case["work"]
            np.testing.assert_allclose(np.exp(-lw[m]), want[m], rtol=1e-6, err_msg=case["work"])


def test_select_sip_budget_in_expectation(clustered):
    """Kept blocks per row average to the budget m over seeds and rows (5 sigma of the sum of
    independent Bernoulli draws)."""
    w, Q, K, V, qc, kc, A = clustered
    rho = 0.1
    Ag = to64(A)
    tot, want, var = 0.0, 0.0, 0.0
    for seed in range(40):
        counts = np_i(bsa.park_select_sip(A, kc["offsets"], rho, seed=seed)["counts"])
        tot += counts.sum()
    for h in range(w.heads):
        sizes = np.diff(np_i(kc["offsets"][h]))
        _, _, _, _, _, pi = O.select_sip(Ag[h], sizes, rho, seed=0, head=h)
        want += 40 * pi.sum()
        var += 40 * (pi * (1 - pi)).sum()
    assert abs(tot - want) <= 5 * np.sqrt(var) + 1e-9, (tot, want, var)


def _weighted_check(w, Q, K, V, qc, kc, counts, cols, log_w, out, lse):
    worst, acc, n = 0.0, 0.0, 0
    for h in range(w.heads):
        Oo, Lo = O.weighted_sparse_attention(attn_view(w, Q[h]), attn_view(w, K[h]), attn_view(w, V[h]),
                                             np_i(qc["perm"][h]), np_i(qc["offsets"][h]), np_i(kc["perm"][h]),
                                             np_i(kc["offsets"][h]), cols_list(np_i(counts[h]), np_i(cols[h])),
                                             to64(log_w[h]), w.scale)
        Og, Lg = to64(out[h]), to64(lse[h])
        e = np.abs(Og - Oo)
        worst = max(worst, e.max())
        acc += e.sum()
        n += e.size
        fin = np.isfinite(Lo)
        np.testing.assert_array_equal(np.isfinite(Lg), fin)
        assert np.abs(Lg[fin] - Lo[fin]).max() <= LSE_ABS
    assert worst <= ATTN_MAX_ABS, worst
    assert acc / n <= ATTN_MEAN_ABS, acc / n
    return worst, acc / n


@pytest.mark.parametrize("rho", [0.1, 0.3])
def test_weighted_attention_sip(clustered, rho):
    w, Q, K, V, qc, kc, A = clustered
    sel = bsa.park_select_sip(A, kc["offsets"], rho, seed=5)
    out, lse = bsa.park_sparse_attn_weighted(Q, K, V, qc["perm"], qc["offsets"], kc["perm"], kc["offsets"],
                                             sel["counts"], sel["cols"], sel["log_w"])
    worst, mean = _weighted_check(w, Q, K, V, qc, kc, sel["counts"], sel["cols"], sel["log_w"], out, lse)
    print(f"[weighted attention rho={rho}] max-abs {worst:.2e} mean-abs {mean:.2e}")


def test_weighted_attention_arbitrary_weights(clustered):
    """Log weights of both signs and up to 30 in magnitude on a top-p selection."""
    w, Q, K, V, qc, kc, A = clustered
    sel = bsa.park_select_topp(A, kc["offsets"], 0.9)
    g = torch.Generator().manual_seed(9)
    log_w = ((torch.rand(A.shape, generator=g) - 0.5) * 60).to(torch.float32).cuda().contiguous()
    out, lse = bsa.park_sparse_attn_weighted(Q, K, V, qc["perm"], qc["offsets"], kc["perm"], kc["offsets"],
                                             sel["counts"], sel["cols"], log_w)
    _weighted_check(w, Q, K, V, qc, kc, sel["counts"], sel["cols"], log_w, out, lse)


def test_weighted_attention_zero_weights_is_sparse_attention(clustered):
    """log w = 0 adds +0.0 to every score: the weighted kernel reproduces park_sparse_attn bit for bit."""
    w, Q, K, V, qc, kc, A = clustered
    sel = bsa.park_select_topp(A, kc["offsets"], 0.9)
    zero = torch.zeros_like(A)
    o1, l1 = bsa.park_sparse_attn(Q, K, V, qc["perm"], qc["offsets"], kc["perm"], kc["offsets"], sel["counts"],
                                  sel["cols"])
    o2, l2 = bsa.park_sparse_attn_weighted(Q, K, V, qc["perm"], qc["offsets"], kc["perm"], kc["offsets"],
                                           sel["counts"], sel["cols"], zero)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
