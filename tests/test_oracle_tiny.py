"""The oracle end to end on the tiny workload (1 head, N = 2048, d = 64, fp32, Cq = 16, Ck = 32)."""
import time

import numpy as np
import pytest

import oracle as O
import synth


@pytest.fixture(scope="module")
def tiny():
    w = synth.WORKLOADS["tiny"]
    Q, K, V = synth.make_qkv(w, seed=0)
    return w, Q[0].double().numpy(), K[0].double().numpy(), V[0].double().numpy()


def test_tiny_forward_invariants(tiny):
    w, Q, K, V = tiny
    t0 = time.time()
    r = O.forward(Q, K, V, w.cq, w.ck, w.iters, w.p, w.scale, seed=0, bf16=False)
    assert time.time() - t0 < 60
    qs, ks = np.diff(r["q"]["offsets"]), np.diff(r["k"]["offsets"])
    assert qs.sum() == w.n and ks.sum() == w.n
    live = qs > 0
    np.testing.assert_allclose(r["map"][live].sum(1), 1.0, atol=1e-12)  # P1
    # P2: selected mass >= p and minimal
    for i in np.flatnonzero(live):
        sel = r["map"][i, r["cols"][i]]
        assert sel.sum() >= w.p
        assert sel.sum() - sel.min() < w.p
    # centroids are the exact member means (last update after the last assignment)
    for j in range(w.ck):
        rows = K[r["k"]["labels"] == j]
        if rows.size:
            np.testing.assert_allclose(r["k"]["centroids"][j], rows.mean(0), rtol=0, atol=1e-6)
    Qa, Ka, Va = (O.round_bf16(x) for x in (Q, K, V))
    _, ld = O.dense_attention(Qa, Ka, Va, w.scale)
    rec = O.recall(r["lse"], ld)
    assert np.all(rec <= 1 + 1e-12)
    assert rec.mean() > 0.8


def test_tiny_p_one_is_dense(tiny):
    """P3 on the tiny workload: p = 1.0 reproduces dense attention."""
    w, Q, K, V = tiny
    r = O.forward(Q, K, V, w.cq, w.ck, w.iters, 1.0, w.scale, seed=0, bf16=False)
    Od, ld = O.dense_attention(*(O.round_bf16(x) for x in (Q, K, V)), w.scale)
    np.testing.assert_allclose(r["out"], Od, atol=1e-12)
    np.testing.assert_allclose(r["lse"], ld, atol=1e-12)


def test_tiny_directional_relations(tiny, capsys):
    """P14 (reported, not failed): the pages' directions on real models (Table 1 recall FC > CC;
    Table 4 TV FC < CF < CC; Table 5 QRKC lowers QK-score error and raises raw-key MSE)."""
    w, Q, K, V = tiny
    M = O.round_f32(O.qrkc_metric(Q))
    qc = O.cluster(Q, w.cq, w.iters, O.EUCLID, None, 0, 0, O.SIDE_Q, bf16=False)
    ke = O.cluster(K, w.ck, w.iters, O.EUCLID, None, 0, 0, O.SIDE_K, bf16=False)
    km = O.cluster(K, w.ck, w.iters, O.QRKC, M, 0, 0, O.SIDE_K, bf16=False)
    est = O.estimator_maps(Q, K, qc["labels"], ke["labels"], qc["centroids"], ke["centroids"], w.scale)
    tv = {k: O.tv_to_full(v, est["FF"]) for k, v in est.items()}
    mse = (O.raw_key_mse(K, ke["labels"], ke["centroids"]), O.raw_key_mse(K, km["labels"], km["centroids"]))
    qke = (O.qk_score_sq_error(Q, K, ke["labels"], ke["centroids"]),
           O.qk_score_sq_error(Q, K, km["labels"], km["centroids"]))
    with capsys.disabled():
        print(f"\n[tiny] TV FF={tv['FF']:.4f} FC={tv['FC']:.4f} CF={tv['CF']:.4f} CC={tv['CC']:.4f}; "
              f"raw-key MSE euclid={mse[0]:.3f} qrkc={mse[1]:.3f}; QK err euclid={qke[0]:.3f} qrkc={qke[1]:.3f}")
    assert tv["FF"] == 0.0
