"""Benchmark of the PARK path on one MI355X: retrieval + block-sparse attention per layer.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wan] [--no-cpu] [--no-stages]
python bench.py --sweep        # p x Ck grid on the Wan-shaped layer (one JSON document)
python bench.py --schedule     # the long clip's 10-step schedule: warm / subset / reuse between anchors
python bench.py --estimators   # FC / CC / CF / FF block maps: recall and density of top-p / top-k
python bench.py --sip          # top-k truncation vs SIP sampling with inverse-probability weights
python bench.py --merge        # tile-aware merging of query clusters: attention time, recall, density
python bench.py --ablation     # QRKC against Euclidean key clustering (the "w/o QRKC" row)

A step is one park_forward call (QRKC metric, seeded K-means on queries and keys, PAMA map, top-p,
block-sparse attention) over one synthetic layer already resident in HBM. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

import synth

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "retrieval+sparse-attn ms/layer; effective TFLOP/s & MFMA % at N=75,600, p=0.9"


def _events():
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_call(fn, reps, warmup=1):
    """Mean ms of fn() over `reps` calls, timed with HIP events on the current stream."""
    for _ in range(warmup):
        fn()
    a, b = _events()
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def cpu_baseline(w, Q, K, V, seed):
    """The oracle as it stands on a bounded sample of the workload, scaled to ms per layer, with the
    per-stage split.

    Sample: the whole retrieval of heads 0-3 (metric, both seedings and clusterings, PAMA, top-p,
    each stage timed; the oracle's own retrieval steps called one by one) and the sparse attention
    of the first `na` query clusters of head 0; scaled by heads and by query clusters respectively."""
    import oracle as O
    nh = min(4, w.heads)
    st = {"metric": 0.0, "cluster_q": 0.0, "cluster_k": 0.0, "pama": 0.0, "select": 0.0}
    bf = w.dtype == "bf16"

    def timed(key, fn):
        t0 = time.perf_counter()
        out = fn()
        st[key] += time.perf_counter() - t0
        return out

    r = None
    for hh in range(nh):
        qh, kh = (x[hh].to(torch.float64).cpu().numpy() for x in (Q, K))
        Mr = timed("metric", lambda: O.round_f32(O.qrkc_metric(qh)))
        qc = timed("cluster_q", lambda: O.cluster(qh, w.cq, w.iters, O.EUCLID, None, seed, hh, O.SIDE_Q, bf))
        kc = timed("cluster_k", lambda: O.cluster(kh, w.ck, w.iters, O.QRKC, Mr, seed, hh, O.SIDE_K, bf))
        ks = np.diff(kc["offsets"])
        khat = O.round_bf16(kc["centroids"]) if bf else kc["centroids"]
        A = timed("pama", lambda: O.pama(qh, qc["perm"], qc["offsets"], khat, ks, w.scale))
        sel = timed("select", lambda: O.select_topp(A, ks, w.p))
        if hh == 0:
            r = {"q": qc, "k": kc, "cols": sel[2]}
    t_ret = sum(st.values()) / nh
    q, k, v = (x[0].to(torch.float64).cpu().numpy() for x in (Q, K, V))
    na = 50
    qp, qo = r["q"]["perm"], r["q"]["offsets"]
    rows = [i for i in range(w.cq) if qo[i + 1] > qo[i]][:na]
    t0 = time.perf_counter()
    O.sparse_attention(q, k, v, qp, qo, r["k"]["perm"], r["k"]["offsets"], r["cols"], w.scale, rows=rows)
    t_att = time.perf_counter() - t0
    n_live = sum(1 for i in range(w.cq) if qo[i + 1] > qo[i])
    att_ms = 1e3 * t_att * (n_live / max(len(rows), 1)) * w.heads
    stages = {key: round(1e3 * val / nh * w.heads, 1) for key, val in st.items()}
    stages["sparse_attn"] = round(att_ms, 1)
    ms = 1e3 * t_ret * w.heads + att_ms
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = max((p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"), default=None)
    except Exception:
        pass
    return {"value": ms, "unit": "ms/layer", "cores": cores, "kind": "oracle", "stages_ms": stages,
            "cpu_count": os.cpu_count(), "blas_threads": blas,
            "sample": f"retrieval of heads 0-{nh - 1} ({t_ret:.1f} s per head) x {w.heads} heads + sparse attention "
                      f"of {len(rows)} of {n_live} query clusters of head 0 ({t_att:.1f} s) scaled to all clusters "
                      f"and heads"}


def kernel_only(args, w, Q, K, V, step, bsa, ws, log):
    r = step()
    torch.cuda.synchronize()
    if args.kernel_only == "sparse_attn":
        out = torch.empty_like(Q)
        lse = torch.empty(w.heads, w.n, dtype=torch.float32, device=Q.device)
        fn = lambda: bsa.park_sparse_attn(Q, K, V, r["q_perm"], r["q_offsets"], r["k_perm"], r["k_offsets"],
                                          r["counts"], r["cols"], out=out, lse=lse, ws=ws)
    elif args.kernel_only == "assign":
        fn = lambda: bsa.park_cluster(K, w.ck, 1, bsa.PARK_QRKC, r["metric"], init=bsa.PARK_INIT_WARM,
                                      side=bsa.PARK_SIDE_K, centroids=r["k_centroids"].clone(), ws=ws)
    else:
        A = torch.empty(w.heads, w.cq, w.ck, dtype=torch.float32, device=Q.device)
        kc = r["k_centroids"]
        fn = lambda: bsa.park_retrieve_map(Q, r["q_perm"], r["q_offsets"], kc, r["k_offsets"], out=A, ws=ws)
    for _ in range(args.steps):
        fn()
    torch.cuda.synchronize()
    src = torch.empty(1 << 30, dtype=torch.uint8, device=Q.device)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"ran {args.kernel_only} x{args.steps} and a 1 GiB copy")


PROFILE_PMC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "sparse_attn_bf16_wan_pmc.md")
ATTN_SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "block_sparse_attention_qrkc_amd", "csrc",
                        "attn.hip")


def measured_traffic():
    """HBM bytes per attention launch from the committed counter summary, if it was taken on the
    attention source as it is now (else None)."""
    import hashlib
    import re
    try:
        txt = open(PROFILE_PMC).read()
        sha = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    m = re.search(r"traffic_bytes_per_launch = ([0-9.eE+]+) \(attn.hip sha256 prefix ([0-9a-f]+)\)", txt)
    if m and m.group(2) == sha:
        return float(m.group(1))
    return None


def ceilings(dev):
    """Measured ceilings on this GPU: a large bf16 GEMM (vendor library) and a device copy."""
    a = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    ms = time_call(lambda: torch.mm(a, b), 10, warmup=3)
    gemm = 2 * 8192 ** 3 / (ms * 1e9)
    del a, b
    src = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    ms = time_call(lambda: dst.copy_(src), 10, warmup=2)
    copy = 2 * (1 << 31) / (ms * 1e6)
    del src, dst
    torch.cuda.empty_cache()
    return {"gemm_bf16_tflops": round(gemm, 1), "copy_gbs": round(copy, 1)}


def topp_near_ties(A, k_offsets, counts, p, tau=1e-5):
    """Top-p rows whose cut is close to a decision boundary: `sum` counts rows where the kept prefix,
    or the prefix one shorter, sums to within tau of p; `order` counts rows where the last kept and
    the first dropped importances agree to a relative tau (an order two correct implementations may
    resolve differently). Either kind may legitimately differ between implementations."""
    if p >= 1.0:
        return {"rows": 0, "sum": 0, "order": 0, "tau": tau}
    A = A.double().cpu().numpy()
    ko = k_offsets.cpu().numpy()
    cnt = counts.cpu().numpy().astype(np.int64)
    rows = n_sum = n_order = 0
    for h in range(A.shape[0]):
        live = np.diff(ko[h]) > 0
        v = -np.sort(-np.maximum(A[h][:, live], 0.0), axis=1)
        cum = np.cumsum(v, axis=1)
        for i in range(A.shape[1]):
            k = int(cnt[h, i])
            if k <= 0 or k > v.shape[1]:
                continue
            rows += 1
            n_sum += int(abs(cum[i, k - 1] - p) <= tau or (k >= 2 and abs(cum[i, k - 2] - p) <= tau))
            n_order += int(k < v.shape[1] and v[i, k - 1] - v[i, k] <= tau * v[i, k - 1])
    return {"rows": rows, "sum": n_sum, "order": n_order, "tau": tau}


def selection_stats(w, r):
    """Token density, computed and padded FLOPs of one layer's selection."""
    qsz = torch.diff(r["q_offsets"], dim=1).to(torch.float64)
    ksel = r["sel_keys"].to(torch.float64)
    computed = 4.0 * w.d * float((qsz * ksel).sum())
    # the kernel runs whole 32-query blocks and whole 32-key tiles (64 for d = 64)
    bn = 64 if w.d == 64 else 32
    padded = 4.0 * w.d * float((torch.ceil(qsz / 32) * 32 * torch.ceil(ksel / bn) * bn).sum())
    dense = 4.0 * w.d * w.n * w.n * w.heads
    return computed, padded, dense


def run_sweep(args, bsa, w0, dev, log):
    """p x Ck grid on the Wan-shaped layer: density, recall, retrieval and attention ms."""
    out = {"sweep": "p x ck on " + w0.name, "points": []}
    Q, K, V = synth.make_qkv(w0, seed=args.seed, device=dev)
    ws = bsa.Workspace()
    for ck in synth.SWEEP_CK:
        M = bsa.park_qrkc_metric(Q, ws=ws)
        qc = bsa.park_cluster(Q, w0.cq, w0.iters, bsa.PARK_EUCLID, None, seed=args.seed, side=bsa.PARK_SIDE_Q, ws=ws)
        kc = bsa.park_cluster(K, ck, w0.iters, bsa.PARK_QRKC, M, seed=args.seed, side=bsa.PARK_SIDE_K, ws=ws)
        A = bsa.park_retrieve_map(Q, qc["perm"], qc["offsets"], kc["centroids"], kc["offsets"], ws=ws)
        t_ret = (time_call(lambda: bsa.park_cluster(K, ck, w0.iters, bsa.PARK_QRKC, M, seed=args.seed,
                                                    side=bsa.PARK_SIDE_K, ws=ws), 1)
                 + time_call(lambda: bsa.park_cluster(Q, w0.cq, w0.iters, bsa.PARK_EUCLID, None, seed=args.seed,
                                                      side=bsa.PARK_SIDE_Q, ws=ws), 1)
                 + time_call(lambda: bsa.park_retrieve_map(Q, qc["perm"], qc["offsets"], kc["centroids"],
                                                          kc["offsets"], out=A, ws=ws), 1))
        args_attn = (Q, K, V, qc["perm"], qc["offsets"], kc["perm"], kc["offsets"])
        dsel = bsa.park_select_topp(A, kc["offsets"], 1.0)
        _, lse_d = bsa.park_sparse_attn(*args_attn, dsel["counts"], dsel["cols"], ws=ws)
        for p in synth.SWEEP_P:
            sel = bsa.park_select_topp(A, kc["offsets"], p)
            out_t = torch.empty_like(Q)
            lse = torch.empty(w0.heads, w0.n, dtype=torch.float32, device=dev)
            t_att = time_call(lambda: bsa.park_sparse_attn(*args_attn, sel["counts"], sel["cols"], out=out_t,
                                                           lse=lse, ws=ws), 2)
            rec = torch.exp(lse.double() - lse_d.double()).mean(dim=1).cpu().numpy()
            r = {"q_offsets": qc["offsets"], "sel_keys": sel["sel_keys"]}
            computed, padded, dense = selection_stats(w0, r)
            pt = {"p": p, "ck": ck, "token_density": round(computed / dense, 5), "sparse_attn_ms": round(t_att, 3),
                  "retrieval_ms": round(t_ret, 3), "computed_tflops": round(computed / (t_att * 1e9), 1),
                  "padded_over_computed": round(padded / max(computed, 1.0), 4),
                  "recall": {"mean": round(float(rec.mean()), 4), "worst": round(float(rec.min()), 4)}}
            out["points"].append(pt)
            log(f"sweep {pt}")
    print(json.dumps(out), flush=True)


def run_schedule(args, bsa, w, dev, log):
    """The long clip's denoising schedule (PARK-p2 Table 9: how often the retrieval is recomputed).
    Inputs drift every step. Full K-means (k-means++ and ``iters`` iterations) at the anchor steps;
    three policies between anchors, each carrying its own state from the last anchor:
    * warm: warm start from the previous centroids with ``warm_iters`` iterations over every token;
    * subset: hybrid clustering (HyperVAttention page, abstract): ``warm_iters`` subset updates of
      every fourth token (phase = step mod 4) from the previous centroids and labels;
    * reuse: the anchor's clustering and block selection are kept; the step runs the attention only.
    Each step reports ms, token density and recall (from the kernel's log-sum-exp against dense
    attention of the same step)."""
    Q, K, V, Qm, Km = synth.make_qkv(w, seed=args.seed, device=dev, keep_fp32=True)
    ws = bsa.Workspace()
    stride = 4
    outs = ("q_perm", "q_offsets", "k_perm", "k_offsets", "counts", "cols", "sel_keys", "lse", "stats")
    shape_c = lambda c: torch.empty(w.heads, c, w.d, dtype=torch.float32, device=dev)
    st = {k: {"qc": shape_c(w.cq), "kc": shape_c(w.ck),
              "ql": torch.zeros(w.heads, w.n, dtype=torch.int32, device=dev),
              "kl": torch.zeros(w.heads, w.n, dtype=torch.int32, device=dev)} for k in ("warm", "subset")}
    cols_all = torch.arange(w.ck, dtype=torch.int32, device=dev).expand(w.heads, w.cq, w.ck).contiguous()
    cnt_all = torch.full((w.heads, w.cq), w.ck, dtype=torch.int32, device=dev)

    def timed(fn, state=None):
        """fn() twice from the same state (a warm-up call, then the timed one); returns (result, ms)."""
        saved = {k: v.clone() for k, v in state.items()} if state else None
        fn()
        torch.cuda.synchronize()
        if saved:
            for k, v in saved.items():
                state[k].copy_(v)
        a, b = _events()
        a.record()
        r = fn()
        b.record()
        torch.cuda.synchronize()
        return r, a.elapsed_time(b)

    def quality(r, ld, ms):
        rec = torch.exp(r["lse"] - ld).mean(dim=1)
        stats = dict(zip(bsa.STATS_FIELDS, r["stats"].tolist()))
        return {"ms": round(ms, 3), "token_density": round(stats["pairs"] / (w.heads * w.n * w.n), 5),
                "recall_mean": round(rec.mean().item(), 4), "recall_worst": round(rec.min().item(), 4)}

    steps, kept = [], None
    for t in range(w.steps):
        if t > 0:
            Q.copy_(synth.drift_step(w, Qm, args.seed, t, 0))
            K.copy_(synth.drift_step(w, Km, args.seed, t, 1))
        full = t in w.anchors
        entry = {"step": t, "full_kmeans": full}
        if full:
            s0 = st["warm"]
            r, ms = timed(lambda: bsa.park_forward(Q, K, V, w.cq, w.ck, w.iters, w.p, seed=args.seed,
                                                   q_centroids=s0["qc"], k_centroids=s0["kc"], q_labels=s0["ql"],
                                                   k_labels=s0["kl"], outputs=outs, ws=ws), s0)
            for k in ("qc", "kc", "ql", "kl"):
                st["subset"][k].copy_(s0[k])
            kept = {k: r[k].clone() for k in ("q_perm", "q_offsets", "k_perm", "k_offsets", "counts", "cols")}
            _, ld = bsa.park_sparse_attn(Q, K, V, r["q_perm"], r["q_offsets"], r["k_perm"], r["k_offsets"], cnt_all,
                                         cols_all, ws=ws)
            q = quality(r, ld, ms)
            entry.update(warm=q, subset=dict(q), reuse=dict(q))
        else:
            for name, init, sub in (("warm", bsa.PARK_INIT_WARM, (1, 0)),
                                    ("subset", bsa.PARK_INIT_SUBSET, (stride, t % stride))):
                s0 = st[name]
                r, ms = timed(lambda: bsa.park_forward(Q, K, V, w.cq, w.ck, w.warm_iters, w.p, seed=args.seed,
                                                       init=init, subset=sub, q_centroids=s0["qc"],
                                                       k_centroids=s0["kc"], q_labels=s0["ql"], k_labels=s0["kl"],
                                                       outputs=outs, ws=ws), s0)
                _, ld = bsa.park_sparse_attn(Q, K, V, r["q_perm"], r["q_offsets"], r["k_perm"], r["k_offsets"],
                                             cnt_all, cols_all, ws=ws)
                entry[name] = quality(r, ld, ms)
            fa = lambda: bsa.park_sparse_attn(Q, K, V, kept["q_perm"], kept["q_offsets"], kept["k_perm"],
                                              kept["k_offsets"], kept["counts"], kept["cols"], ws=ws)
            (_, lr), ms = timed(fa)
            _, ld = bsa.park_sparse_attn(Q, K, V, kept["q_perm"], kept["q_offsets"], kept["k_perm"],
                                         kept["k_offsets"], cnt_all, cols_all, ws=ws)
            qsz = torch.diff(kept["q_offsets"], dim=1).double()
            ksz = torch.diff(kept["k_offsets"], dim=1).double()
            # cols is row-padded: entries past counts are not written, so they are masked before lookup
            valid = torch.arange(w.ck, device=dev)[None, None, :] < kept["counts"][:, :, None]
            idx = torch.where(valid, kept["cols"].long(), torch.zeros_like(kept["cols"], dtype=torch.long))
            keys = (torch.gather(ksz, 1, idx.view(w.heads, -1)).view(w.heads, w.cq, w.ck) * valid).sum(-1)
            pairs = float((qsz * keys).sum())
            rr = torch.exp(lr - ld).mean(dim=1)
            entry["reuse"] = {"ms": round(ms, 3), "token_density": round(pairs / (w.heads * w.n * w.n), 5),
                              "recall_mean": round(rr.mean().item(), 4), "recall_worst": round(rr.min().item(), 4)}
        steps.append(entry)
        log(f"schedule {entry}")
    pol = ("warm", "subset", "reuse")
    tot = {k: round(sum(x[k]["ms"] for x in steps), 3) for k in pol}
    print(json.dumps({"schedule": w.name, "heads": w.heads, "n": w.n, "cq": w.cq, "ck": w.ck, "p": w.p,
                      "anchors": list(w.anchors), "warm_iters": w.warm_iters, "subset_stride": stride,
                      "steps": steps, "total_ms": tot,
                      "ms_per_step": {k: round(v / len(steps), 3) for k, v in tot.items()}}), flush=True)


def run_merge(args, bsa, w, dev, log):
    """Tile-aware merging of query clusters (HyperVAttention page, abstract) on one layer: the top-p
    selection's attention as is, and after merging the query clusters under the CTA-aligned cost with
    the attention's 384-query work items (and, for comparison, 32-query tiles): groups, work items,
    token density (computed pairs), recall against dense attention, merge and attention ms."""
    Q, K, V = synth.make_qkv(w, seed=args.seed, device=dev)
    ws = bsa.Workspace()
    r = bsa.park_forward(Q, K, V, w.cq, w.ck, w.iters, w.p, seed=args.seed,
                         outputs=("q_perm", "q_offsets", "k_perm", "k_offsets", "counts", "cols", "sel_keys",
                                  "stats"), ws=ws)
    cols_all = torch.arange(w.ck, dtype=torch.int32, device=dev).expand(w.heads, w.cq, w.ck).contiguous()
    cnt_all = torch.full((w.heads, w.cq), w.ck, dtype=torch.int32, device=dev)
    _, ld = bsa.park_sparse_attn(Q, K, V, r["q_perm"], r["q_offsets"], r["k_perm"], r["k_offsets"], cnt_all,
                                 cols_all, ws=ws)
    ksz = torch.diff(r["k_offsets"], dim=1).double()

    def measure(qp, qo, counts, cols):
        o, lse = bsa.park_sparse_attn(Q, K, V, qp, qo, r["k_perm"], r["k_offsets"], counts, cols, ws=ws)
        ms = time_call(lambda: bsa.park_sparse_attn(Q, K, V, qp, qo, r["k_perm"], r["k_offsets"], counts, cols,
                                                    out=o, lse=lse, ws=ws), 3)
        rec = torch.exp(lse - ld).mean(dim=1).double()
        qsz = torch.diff(qo, dim=1).double()
        # cols is row-padded: entries past counts are not written, so they are masked before any lookup
        valid = torch.arange(w.ck, device=dev)[None, None, :] < counts[:, :, None]
        idx = torch.where(valid, cols.long(), torch.zeros_like(cols, dtype=torch.long))
        keys = (torch.gather(ksz, 1, idx.view(w.heads, -1)).view(w.heads, w.cq, w.ck) * valid).sum(-1)
        pairs = float((qsz * keys).sum())
        items = int(((qsz + 383) // 384).sum())
        return {"attn_ms": round(ms, 3), "token_density": round(pairs / (w.heads * w.n * w.n), 5),
                "computed_tflops": round(4 * w.d * pairs / (ms * 1e9), 1), "work_items": items,
                "groups": int((qsz > 0).sum()),
                "recall_mean": round(float(rec.mean()), 4), "recall_p05": round(float(torch.quantile(rec, 0.05)), 4),
                "recall_worst": round(float(rec.min()), 4)}

    out = {"merge": w.name, "heads": w.heads, "n": w.n, "cq": w.cq, "ck": w.ck, "p": w.p,
           "base": measure(r["q_perm"], r["q_offsets"], r["counts"], r["cols"])}
    log(f"merge base {out['base']}")
    for bm in (384, 32):
        mg = bsa.park_merge_clusters(r["q_perm"], r["q_offsets"], r["k_offsets"], r["counts"], r["cols"], bm=bm, ws=ws)
        ms = time_call(lambda: bsa.park_merge_clusters(r["q_perm"], r["q_offsets"], r["k_offsets"], r["counts"],
                                                       r["cols"], bm=bm, ws=ws), 3)
        pt = measure(mg["q_perm"], mg["q_offsets"], mg["counts"], mg["cols"])
        pt["merge_ms"] = round(ms, 3)
        out[f"merged_bm{bm}"] = pt
        log(f"merge bm={bm} {pt}")
    print(json.dumps(out), flush=True)


def run_ablation(args, bsa, w, dev, log):
    """QRKC against Euclidean key clustering (PARK-p2 Table 3 ablation rows, Table 5) on one layer:
    for each key metric, the recall of the top-p selection (mean, P05, worst over heads), token and
    block density at p, and on one sampled head (head 0) the QK-score squared error
    mean_{t,u} (q_t.k_u - q_t.c(u))^2 over 4096 sampled queries and the raw-key squared error
    mean_u |k_u - c(u)|^2 (c(u) = the key's cluster centroid)."""
    Q, K, V = synth.make_qkv(w, seed=args.seed, device=dev)
    ws = bsa.Workspace()
    cols_all = torch.arange(w.ck, dtype=torch.int32, device=dev).expand(w.heads, w.cq, w.ck).contiguous()
    cnt_all = torch.full((w.heads, w.cq), w.ck, dtype=torch.int32, device=dev)
    out = {"ablation": w.name, "heads": w.heads, "n": w.n, "cq": w.cq, "ck": w.ck, "p": w.p, "metrics": {}}
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed + 77)
    tq = torch.randperm(w.n, generator=g, device=dev)[:4096]
    for name, km in (("qrkc", bsa.PARK_QRKC), ("euclid", bsa.PARK_EUCLID)):
        r = bsa.park_forward(Q, K, V, w.cq, w.ck, w.iters, w.p, seed=args.seed, kmetric=km,
                             outputs=("q_perm", "q_offsets", "k_perm", "k_offsets", "k_labels", "lse", "stats"),
                             ws=ws)
        ms = time_call(lambda: bsa.park_forward(Q, K, V, w.cq, w.ck, w.iters, w.p, seed=args.seed, kmetric=km,
                                                ws=ws), 2)
        _, ld = bsa.park_sparse_attn(Q, K, V, r["q_perm"], r["q_offsets"], r["k_perm"], r["k_offsets"], cnt_all,
                                     cols_all, ws=ws)
        rec = torch.exp(r["lse"] - ld).mean(dim=1).double()
        stats = dict(zip(bsa.STATS_FIELDS, r["stats"].tolist()))
        k0 = K[0].double()
        c0 = r["k_centroids"][0].double()[r["k_labels"][0].long()]
        diff = k0 - c0
        qk = Q[0].double()[tq] @ diff.T
        entry = {"forward_ms": round(ms, 3),
                 "recall_mean": round(float(rec.mean()), 4), "recall_p05": round(float(torch.quantile(rec, 0.05)), 4),
                 "recall_worst": round(float(rec.min()), 4),
                 "token_density": round(stats["pairs"] / (w.heads * w.n * w.n), 5),
                 "block_density": round(stats["blocks"] / stats["live_blocks"], 5),
                 "qk_score_sq_error_head0": round(float((qk * qk).mean()), 4),
                 "raw_key_sq_error_head0": round(float((diff * diff).sum(1).mean()), 4)}
        out["metrics"][name] = entry
        log(f"ablation {name} {entry}")
    print(json.dumps(out), flush=True)


def run_estimators(args, bsa, w, dev, log):
    """Retrieval quality under the four query/key representations of PARK-p2 Table 1 (FC = PAMA, CC,
    CF, FF) on one synthetic layer: top-p (p of the workload) and top-k at rho = 0.1 (Table 10)
    selections from each block map, attention over them, and the recall of every head
    (exp(LSE_selected - LSE_dense) averaged over its queries); mean, P05 and worst over heads, block
    and token density, the block-map total variation to FF, and the time of each map."""
    Q, K, V = synth.make_qkv(w, seed=args.seed, device=dev)
    ws = bsa.Workspace()
    r = bsa.park_forward(Q, K, V, w.cq, w.ck, w.iters, w.p, seed=args.seed,
                         outputs=("q_perm", "q_offsets", "k_perm", "k_offsets", "map"), ws=ws)
    cols_all = torch.arange(w.ck, dtype=torch.int32, device=dev).expand(w.heads, w.cq, w.ck).contiguous()
    cnt_all = torch.full((w.heads, w.cq), w.ck, dtype=torch.int32, device=dev)
    _, ld = bsa.park_sparse_attn(Q, K, V, r["q_perm"], r["q_offsets"], r["k_perm"], r["k_offsets"], cnt_all,
                                 cols_all, ws=ws)
    modes = {"FC": bsa.PARK_EST_FC, "CC": bsa.PARK_EST_CC, "CF": bsa.PARK_EST_CF, "FF": bsa.PARK_EST_FF}
    kw = dict(q=Q, k=K, q_perm=r["q_perm"], q_offsets=r["q_offsets"], q_centroids=r["q_centroids"],
              k_perm=r["k_perm"], k_centroids=r["k_centroids"], ws=ws)
    maps, out = {}, {"estimators": w.name, "heads": w.heads, "n": w.n, "cq": w.cq, "ck": w.ck, "p": w.p,
                     "rho": 0.1, "modes": {}}
    for name, m in modes.items():
        E = bsa.park_estimator_map(m, r["k_offsets"], **kw)
        maps[name] = E
        ms = time_call(lambda: bsa.park_estimator_map(m, r["k_offsets"], out=E, **kw), 1)
        out["modes"][name] = {"map_ms": round(ms, 3)}
    live = torch.diff(r["q_offsets"].long(), dim=1) > 0
    for name, E in maps.items():
        entry = out["modes"][name]
        tv = 0.5 * (E - maps["FF"]).abs().sum(-1)
        entry["tv_to_ff"] = round(float(tv[live].mean()), 5)
        for label, sel in (("top_p", bsa.park_select_topp(E, r["k_offsets"], w.p)),
                           ("top_k", bsa.park_select_topk(E, r["k_offsets"], 0.1))):
            _, lse = bsa.park_sparse_attn(Q, K, V, r["q_perm"], r["q_offsets"], r["k_perm"], r["k_offsets"],
                                          sel["counts"], sel["cols"], ws=ws)
            head = torch.exp(lse - ld).mean(dim=1).double().cpu()
            q = torch.diff(r["q_offsets"], dim=1).double()
            pairs = (live.sum(1) * (torch.diff(r["k_offsets"], dim=1) > 0).sum(1)).double().sum()
            blocks = float(sel["counts"].double().sum() / pairs)
            tokens = float((q * sel["sel_keys"].double()).sum()) / (w.n * w.n * w.heads)
            entry[label] = {"recall_mean": round(float(head.mean()), 4),
                            "recall_p05": round(float(torch.quantile(head, 0.05)), 4),
                            "recall_worst": round(float(head.min()), 4),
                            "block_density": round(blocks, 4), "token_density": round(tokens, 4)}
        log(f"estimator {name} {entry}")
    print(json.dumps(out), flush=True)


def run_sip(args, bsa, w, dev, log):
    """Top-k truncation against sampling with inclusion-probability weighting (AB-Attention page, SIP
    paragraph) at the same budget on one synthetic layer: for each ratio rho, top-k keeps the k
    most important blocks of every PAMA row; SIP samples k blocks in expectation with
    probabilities proportional to importance (capped at 1) and reweights them by 1/pi. Reported per
    selection: the mean over queries of the relative L2 error of the attention output against dense
    attention, the mean |LSE - LSE_dense| (top-k's LSE is the log of the kept mass, SIP's estimates
    the dense one), the recall of the selected keys (dense softmax mass they hold), token density
    and the attention time; SIP figures are averaged over three seeds."""
    Q, K, V = synth.make_qkv(w, seed=args.seed, device=dev)
    ws = bsa.Workspace()
    r = bsa.park_forward(Q, K, V, w.cq, w.ck, w.iters, w.p, seed=args.seed,
                         outputs=("q_perm", "q_offsets", "k_perm", "k_offsets", "map"), ws=ws)
    geo = (r["q_perm"], r["q_offsets"], r["k_perm"], r["k_offsets"])
    cols_all = torch.arange(w.ck, dtype=torch.int32, device=dev).expand(w.heads, w.cq, w.ck).contiguous()
    cnt_all = torch.full((w.heads, w.cq), w.ck, dtype=torch.int32, device=dev)
    od, ld = bsa.park_sparse_attn(Q, K, V, *geo, cnt_all, cols_all, ws=ws)
    odn = od.float().norm(dim=-1)
    qsz = torch.diff(r["q_offsets"], dim=1).double()
    out = {"sip": w.name, "heads": w.heads, "n": w.n, "cq": w.cq, "ck": w.ck, "points": []}

    def stats(o, lse, sel, ms):
        err = ((o.float() - od.float()).norm(dim=-1) / odn.clamp_min(1e-30)).mean()
        fin = torch.isfinite(lse)
        lerr = torch.where(fin, (lse - ld).abs(), torch.zeros_like(lse)).sum() / fin.sum()
        _, lsel = bsa.park_sparse_attn(Q, K, V, *geo, sel["counts"], sel["cols"], ws=ws)
        rec = torch.exp(lsel - ld).mean()
        tokens = float((qsz * sel["sel_keys"].double()).sum()) / (w.n * w.n * w.heads)
        return {"out_rel_err": float(err), "lse_abs_err": float(lerr), "recall": float(rec),
                "token_density": tokens, "attn_ms": ms, "unselected_queries": int((~fin).sum())}

    for rho in (0.05, 0.1, 0.2):
        sel = bsa.park_select_topk(r["map"], r["k_offsets"], rho)
        o, lse = bsa.park_sparse_attn(Q, K, V, *geo, sel["counts"], sel["cols"], ws=ws)
        ms = time_call(lambda: bsa.park_sparse_attn(Q, K, V, *geo, sel["counts"], sel["cols"], out=o, lse=lse, ws=ws), 3)
        top = stats(o, lse, sel, ms)
        runs = []
        for seed in range(3):
            ss = bsa.park_select_sip(r["map"], r["k_offsets"], rho, seed=seed)
            o, lse = bsa.park_sparse_attn_weighted(Q, K, V, *geo, ss["counts"], ss["cols"], ss["log_w"], ws=ws)
            ms = time_call(lambda: bsa.park_sparse_attn_weighted(Q, K, V, *geo, ss["counts"], ss["cols"], ss["log_w"],
                                                                 out=o, lse=lse, ws=ws), 3)
            runs.append(stats(o, lse, ss, ms))
        sip = {k: sum(x[k] for x in runs) / len(runs) for k in runs[0]}
        sel_ms = time_call(lambda: bsa.park_select_sip(r["map"], r["k_offsets"], rho, seed=0), 3)
        pt = {"rho": rho, "top_k": {k: round(v, 5) for k, v in top.items()},
              "sip": {k: round(v, 5) for k, v in sip.items()}, "sip_select_ms": round(sel_ms, 3)}
        out["points"].append(pt)
        log(f"sip {pt}")
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-stages", action="store_true", help="skip the per-stage breakdown")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured GEMM / copy ceilings")
    ap.add_argument("--sweep", action="store_true", help="p x Ck grid on the Wan-shaped layer (own JSON document)")
    ap.add_argument("--estimators", action="store_true",
                    help="FC / CC / CF / FF block maps: recall and density of their top-p and top-k selections")
    ap.add_argument("--sip", action="store_true",
                    help="top-k truncation vs SIP sampling with inverse-probability weights at equal budgets")
    ap.add_argument("--schedule", action="store_true",
                    help="the long clip's multi-step schedule: warm / subset / reuse between anchors (own JSON)")
    ap.add_argument("--merge", action="store_true",
                    help="tile-aware merging of query clusters: attention time, recall and density (own JSON)")
    ap.add_argument("--ablation", action="store_true",
                    help="QRKC against Euclidean key clustering: recall, density, QK-score error (own JSON)")
    ap.add_argument("--kernel-only", choices=["sparse_attn", "assign", "pama"], default=None,
                    help="profiling aid: prepare one layer, then launch only this stage --steps times, followed "
                         "by a 1 GiB device copy (reference for byte counters); prints no JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}); "
              "heads shard across GPUs with no exchange inside the path, so per-GPU throughput is the N=1 figure.",
              file=sys.stderr)
        sys.exit(2)

    import block_sparse_attention_qrkc_amd as bsa

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log = lambda msg: print(f"[bench] {msg}", file=sys.stderr, flush=True)
    if args.sweep:
        run_sweep(args, bsa, synth.WORKLOADS["wan"], dev, log)
        return
    if args.estimators:
        run_estimators(args, bsa, w, dev, log)
        return
    if args.schedule:
        run_schedule(args, bsa, synth.WORKLOADS["long"], dev, log)
        return
    if args.sip:
        run_sip(args, bsa, w, dev, log)
        return
    if args.merge:
        run_merge(args, bsa, w, dev, log)
        return
    if args.ablation:
        run_ablation(args, bsa, w, dev, log)
        return
    Q, K, V = synth.make_qkv(w, seed=args.seed, device=dev)
    torch.cuda.synchronize()
    log(f"inputs ready: {w.name} H={w.heads} N={w.n} d={w.d}")
    ws = bsa.Workspace()
    qcent = torch.empty(w.heads, w.cq, w.d, dtype=torch.float32, device=dev)
    kcent = torch.empty(w.heads, w.ck, w.d, dtype=torch.float32, device=dev)
    outs = ("q_perm", "q_offsets", "k_perm", "k_offsets", "counts", "cols", "sel_keys", "lse", "map", "metric",
            "stats")
    if args.kernel_only:
        outs = outs + ("k_labels",)

    def step():
        return bsa.park_forward(Q, K, V, w.cq, w.ck, w.iters, w.p, seed=args.seed, q_centroids=qcent,
                                k_centroids=kcent, outputs=outs, ws=ws)

    if args.kernel_only:
        kernel_only(args, w, Q, K, V, step, bsa, ws, log)
        return
    for _ in range(args.warmup):
        r = step()
    torch.cuda.synchronize()
    log("warmup done")
    t0 = time.perf_counter()
    evs = [_events() for _ in range(args.steps)]
    a, b = _events()
    a.record()
    for k in range(args.steps):
        evs[k][0].record()
        r = step()
        evs[k][1].record()
    b.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_step = a.elapsed_time(b) / args.steps
    per = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (median {per[len(per) // 2]:.3f}, min {per[0]:.3f})")

    # selection statistics of the last step (park_stats, written by the library on the device)
    n = w.n
    stats = dict(zip(bsa.STATS_FIELDS, r["stats"].tolist()))
    computed_flops = 4.0 * w.d * stats["pairs"]
    padded_flops = 4.0 * w.d * stats["padded_pairs"]
    dense_flops = 4.0 * w.d * w.n * w.n * w.heads
    density = computed_flops / dense_flops

    res = {"metric": METRIC, "value": round(ms_step, 3), "unit": "ms/layer", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": False, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
           "config": {"workload": w.name, "heads": w.heads, "n": n, "d": w.d, "cq": w.cq, "ck": w.ck,
                      "iters": w.iters, "p": w.p, "grid": list(w.grid)}}
    res["host_wall_ms_per_step"] = round(wall, 3)
    res["step_ms_median"] = round(per[len(per) // 2], 3)
    res["step_ms_min"] = round(per[0], 3)
    res["token_density"] = round(density, 5)
    res["padded_over_computed_flops"] = round(padded_flops / computed_flops, 4)
    res["work_items"] = stats["work_items"]

    if not args.no_stages:
        M = r["metric"]
        st = {}
        st["metric"] = time_call(lambda: bsa.park_qrkc_metric(Q, out=M, ws=ws), 3)
        st["cluster_q"] = time_call(lambda: bsa.park_cluster(Q, w.cq, w.iters, bsa.PARK_EUCLID, None, seed=args.seed,
                                                             side=bsa.PARK_SIDE_Q, ws=ws), 2)
        st["cluster_k"] = time_call(lambda: bsa.park_cluster(K, w.ck, w.iters, bsa.PARK_QRKC, M, seed=args.seed,
                                                             side=bsa.PARK_SIDE_K, ws=ws), 2)
        qc = bsa.park_cluster(Q, w.cq, w.iters, bsa.PARK_EUCLID, None, seed=args.seed, side=bsa.PARK_SIDE_Q, ws=ws)
        kc = bsa.park_cluster(K, w.ck, w.iters, bsa.PARK_QRKC, M, seed=args.seed, side=bsa.PARK_SIDE_K, ws=ws)
        A = bsa.park_retrieve_map(Q, qc["perm"], qc["offsets"], kc["centroids"], kc["offsets"], ws=ws)
        st["pama"] = time_call(lambda: bsa.park_retrieve_map(Q, qc["perm"], qc["offsets"], kc["centroids"],
                                                             kc["offsets"], out=A, ws=ws), 5)
        sel = bsa.park_select_topp(A, kc["offsets"], w.p)
        st["select"] = time_call(lambda: bsa.park_select_topp(A, kc["offsets"], w.p), 5)
        out = torch.empty_like(Q)
        lse = torch.empty(w.heads, n, dtype=torch.float32, device=dev)
        args_attn = (Q, K, V, qc["perm"], qc["offsets"], kc["perm"], kc["offsets"])
        st["sparse_attn"] = time_call(lambda: bsa.park_sparse_attn(*args_attn, sel["counts"], sel["cols"], out=out,
                                                                   lse=lse, ws=ws), 3)
        dsel = bsa.park_select_topp(A, kc["offsets"], 1.0)
        lse_d = torch.empty_like(lse)
        st["dense_attn"] = time_call(lambda: bsa.park_sparse_attn(*args_attn, dsel["counts"], dsel["cols"], out=out,
                                                                  lse=lse_d, ws=ws), 2)
        bsa.park_sparse_attn(*args_attn, sel["counts"], sel["cols"], out=out, lse=lse, ws=ws)
        torch.cuda.synchronize()
        rec = torch.exp(lse.double() - lse_d.double()).mean(dim=1).cpu().numpy()
        qsz2 = torch.diff(qc["offsets"], dim=1).to(torch.float64)
        flops_sel = 4.0 * w.d * float((qsz2 * sel["sel_keys"].to(torch.float64)).sum())
        retrieval = st["metric"] + st["cluster_q"] + st["cluster_k"] + st["pama"] + st["select"]
        res["stages_ms"] = {k: round(v, 3) for k, v in st.items()}
        res["retrieval_ms"] = round(retrieval, 3)
        res["sparse_attn_ms"] = round(st["sparse_attn"], 3)
        res["dense_attn_ms"] = round(st["dense_attn"], 3)
        res["retrieval_over_dense"] = round(retrieval / st["dense_attn"], 4)
        # the same ratio against dense attention at the bf16 matrix-core peak (the ideal kernel)
        res["retrieval_over_dense_at_peak"] = round(retrieval / (dense_flops / (PEAK_BF16_TFLOPS * 1e9)), 4)
        res["block_density"] = round(stats["blocks"] / stats["live_blocks"], 5)
        res["effective_tflops_dense_equiv"] = round(dense_flops / (ms_step * 1e9), 2)
        res["computed_tflops"] = round(computed_flops / (ms_step * 1e9), 2)
        res["mfma_frac_whole_path"] = round(computed_flops / (ms_step * 1e9) / PEAK_BF16_TFLOPS, 4)
        res["dense_attn_tflops"] = round(dense_flops / (st["dense_attn"] * 1e9), 2)
        res["recall"] = {"mean": round(float(rec.mean()), 4), "p05": round(float(np.percentile(rec, 5)), 4),
                         "worst": round(float(rec.min()), 4)}
        res["near_ties"] = topp_near_ties(A, kc["offsets"], sel["counts"], w.p)
        ach = flops_sel / (st["sparse_attn"] * 1e9)
        log(f"stages: {res['stages_ms']}")
        traffic = measured_traffic() if w.name == "wan" else None
        res["roofline"] = {"kernel": "sparse_attn_bf16", "bound": "mfma", "achieved": round(ach, 2),
                           "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                           "traffic": traffic,
                           "work": f"4*d*sum_i n_q(i)*L(i) = {flops_sel / 1e12:.3f} TFLOP per launch",
                           "traffic_note": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated) from "
                                           "profiles/sparse_attn_bf16_wan_pmc.md; null when the kernel source changed"}
        if not args.no_ceilings:
            res["ceilings"] = ceilings(dev)
            res["roofline"]["frac_of_measured_gemm"] = round(ach / res["ceilings"]["gemm_bf16_tflops"], 4)

    if not args.no_cpu:
        log("cpu baseline (oracle sample)")
        res["cpu_baseline"] = cpu_baseline(w, Q, K, V, args.seed)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
