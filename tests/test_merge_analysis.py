"""Tile-aware merging on a full Wan-shaped head, computed with the oracle only (CPU): the work-item
capacity the attention pays for against the useful (query, key) pairs, before and after merging
the query clusters (HyperVAttention page, abstract: merging fills idle tile capacity and the merged
queries attend to the union of the selections).

Two costs of a query group with n queries and L selected keys:
  * the CTA-aligned cost of the page, ceil(n / 384) * 384 * L (work items of 384 queries);
  * the cost the attention kernel pays: a work item of 384 queries runs 12 waves of 32 queries,
    three per SIMD, and lasts as long as its busiest SIMD, so an item holding a waves costs
    ceil(a / 4) / 3 of a full one (its waves are dealt to the four SIMDs in turn).
The test prints both excesses over the useful pairs sum n * L and checks that merging under the
page's cost does not raise it, that every query keeps at least its own keys, and that the union
selections never lose recall mass (the selections only grow)."""
import numpy as np
import pytest

import oracle as O
import synth


def _simd_cost(n, L, bm=384, wave=32):
    items = -(-n // bm)
    full, rest = divmod(n, bm)
    a = -(-rest // wave)
    return (full + (-(-a // 4) / 3.0 if rest else 0.0)) * bm * L, items


@pytest.mark.slow
def test_merge_capacity_on_a_wan_head():
    w = synth.WORKLOADS["wan"]
    Q, K, V = synth.make_qkv(w, seed=0, heads=1)
    q, k = Q[0].double().numpy(), K[0].double().numpy()
    r = O.retrieve(q, k, w.cq, w.ck, w.iters, w.p, w.scale, seed=0, head=0)
    qs = np.diff(r["q"]["offsets"]).astype(np.int64)
    ks = np.diff(r["k"]["offsets"]).astype(np.int64)
    L = np.array([ks[c].sum() for c in r["cols"]], dtype=np.int64)
    useful = float((qs * L).sum())
    cta0 = float(sum(O.merge_cost(n, l, 384) * 384 for n, l in zip(qs, L) if n > 0))
    simd0 = float(sum(_simd_cost(n, l)[0] for n, l in zip(qs, L) if n > 0))
    group, sel = O.merge_clusters(qs, r["cols"], ks, 384)
    roots = sorted(set(group.tolist()))
    gn = {g: int(qs[group == g].sum()) for g in roots}
    gL = {g: int(ks[sel[g]].sum()) for g in roots}
    useful1 = float(sum(gn[g] * gL[g] for g in roots))
    cta1 = float(sum(O.merge_cost(gn[g], gL[g], 384) * 384 for g in roots if gn[g] > 0))
    simd1 = float(sum(_simd_cost(gn[g], gL[g])[0] for g in roots if gn[g] > 0))
    items0 = sum(-(-n // 384) for n in qs)
    items1 = sum(-(-gn[g] // 384) for g in roots)
    print(f"\n[merge analysis, Wan head 0] {int((qs > 0).sum())} query clusters -> {sum(1 for g in roots if gn[g])} "
          f"groups; work items {items0} -> {items1}; selected pairs {useful:.4g} -> {useful1:.4g} "
          f"(+{100 * (useful1 / useful - 1):.1f} %)")
    print(f"[merge analysis] CTA-aligned capacity over the original useful pairs: {100 * (cta0 / useful - 1):.1f} % -> "
          f"{100 * (cta1 / useful - 1):.1f} %; kernel (busiest-SIMD) cost: {100 * (simd0 / useful - 1):.1f} % -> "
          f"{100 * (simd1 / useful - 1):.1f} %")
    assert cta1 <= cta0
    # every query keeps at least the keys it selected before (recall can only grow)
    for i in range(w.cq):
        if qs[i]:
            assert set(r["cols"][i].tolist()) <= set(sel[group[i]].tolist())
    assert useful1 >= useful
