"""park_sparse_attn_noalloc (the attention with its scratch in a static device array, for callers
that cannot allocate) against park_sparse_attn with a caller workspace: two calls in a row, the
second on a smaller input, each bit-identical to the workspace entry (the same kernels run)."""
import ctypes

import pytest
import torch

import block_sparse_attention_qrkc_amd as bsa
import synth
from block_sparse_attention_qrkc_amd._lib import _ptr, _stream, lib
from gpu_helpers import SMALL

pytestmark = pytest.mark.gpu


def _noalloc(Q, K, V, r):
    sh = bsa.make_shape(Q)
    cq = r["q_offsets"].shape[1] - 1
    ck = r["k_offsets"].shape[1] - 1
    out = torch.empty_like(Q)
    lse = torch.empty(sh.heads, sh.n, dtype=torch.float32, device=Q.device)
    st = lib().park_sparse_attn_noalloc(ctypes.byref(sh), _ptr(Q), _ptr(K), _ptr(V), _ptr(r["q_perm"]),
                                        _ptr(r["q_offsets"]), cq, _ptr(r["k_perm"]), _ptr(r["k_offsets"]), ck,
                                        _ptr(r["counts"]), _ptr(r["cols"]), 0.0, _ptr(out), _ptr(lse), _stream())
    assert st == bsa.PARK_OK, lib().park_last_error().decode()
    return out, lse


@pytest.mark.parametrize("order", [("wan", "small")])
def test_noalloc_matches_the_workspace_entry(order):
    outs = ("q_perm", "q_offsets", "k_perm", "k_offsets", "counts", "cols")
    for name in order:
        w = synth.WORKLOADS[name] if name in synth.WORKLOADS else SMALL[name]
        print(f"\n[no-alloc] {w.name}: H={w.heads} N={w.n} cq={w.cq} ck={w.ck}", flush=True)
        Q, K, V = synth.make_qkv(w, seed=1, device="cuda")
        r = bsa.park_forward(Q, K, V, w.cq, w.ck, w.iters, w.p, seed=1, outputs=outs)
        ref_out, ref_lse = bsa.park_sparse_attn(Q, K, V, r["q_perm"], r["q_offsets"], r["k_perm"], r["k_offsets"],
                                                r["counts"], r["cols"])
        got_out, got_lse = _noalloc(Q, K, V, r)
        torch.cuda.synchronize()
        assert torch.equal(got_out, ref_out)
        assert torch.equal(got_lse, ref_lse)
        del Q, K, V, r, ref_out, ref_lse, got_out, got_lse
        torch.cuda.empty_cache()


def test_noalloc_replayed_from_a_graph():
    """The allocation-free attention captured once in a HIP graph (through torch) and replayed: every
    replay, with eager work and a synchronisation before it, equals the eager workspace entry bit for
    bit; after V changes in place, a replay equals the eager entry on the new V."""
    w = SMALL["small"]
    outs = ("q_perm", "q_offsets", "k_perm", "k_offsets", "counts", "cols")
    Q, K, V = synth.make_qkv(w, seed=2, device="cuda")
    r = bsa.park_forward(Q, K, V, w.cq, w.ck, w.iters, w.p, seed=2, outputs=outs)
    args = (r["q_perm"], r["q_offsets"], r["k_perm"], r["k_offsets"], r["counts"], r["cols"])
    ref_out, ref_lse = bsa.park_sparse_attn(Q, K, V, *args)
    sh = bsa.make_shape(Q)
    cq, ck = r["q_offsets"].shape[1] - 1, r["k_offsets"].shape[1] - 1
    out = torch.empty_like(Q)
    lse = torch.empty(sh.heads, sh.n, dtype=torch.float32, device=Q.device)

    def call():
        st = lib().park_sparse_attn_noalloc(ctypes.byref(sh), _ptr(Q), _ptr(K), _ptr(V), _ptr(r["q_perm"]),
                                            _ptr(r["q_offsets"]), cq, _ptr(r["k_perm"]), _ptr(r["k_offsets"]), ck,
                                            _ptr(r["counts"]), _ptr(r["cols"]), 0.0, _ptr(out), _ptr(lse), _stream())
        assert st == bsa.PARK_OK, lib().park_last_error().decode()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # first call outside the capture (sets up the scratch address)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), rep
    V.mul_(2)
    ref2_out, ref2_lse = bsa.park_sparse_attn(Q, K, V, *args)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, ref2_out) and torch.equal(lse, ref2_lse)
