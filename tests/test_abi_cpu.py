"""The C ABI library on the CPU: it loads, exports every declared entry point, and rejects bad
arguments on the host (before any HIP call, so no GPU is needed)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "park.h")


@pytest.fixture(scope="module")
def L():
    from block_sparse_attention_qrkc_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from block_sparse_attention_qrkc_amd import build
        build.build(verbose=False)
    return _lib


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:park_status|size_t|const char\*|void)\s+(park_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("park_cluster", "park_retrieve_map", "park_select_topp", "park_sparse_attn", "park_forward",
              "park_qrkc_metric", "park_workspace_bytes", "park_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    lib = L.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(park_\w+)$", out, re.M))
    for n in _declared():
        assert n in exported, n
        assert hasattr(lib, n)
    assert set(L.EXPORTED) == set(_declared())
    assert lib.park_version().decode().startswith("park-mi355x")


def test_library_has_no_unresolved_symbols_of_its_own():
    """Every kernel launch stub and helper is defined in the library (a kernel whose host pass was
    dropped shows up as an undefined park:: symbol and the library would fail to load)."""
    from block_sparse_attention_qrkc_amd import _lib
    out = subprocess.run(["nm", "-D", "--undefined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    assert not [ln for ln in out.splitlines() if "park" in ln]
    ctypes.CDLL(_lib.LIB_PATH)


def test_status_strings(L):
    lib = L.lib()
    assert lib.park_status_string(0) == b"PARK_OK"
    assert lib.park_status_string(3) == b"PARK_EWORKSPACE"
    assert lib.park_status_string(99) == b"PARK_UNKNOWN"


FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: validation fails first
MIS = ctypes.c_void_p((1 << 20) + 4)  # misaligned for 16-byte data
ODD = ctypes.c_void_p((1 << 20) + 2)  # misaligned for 4-byte words


def _shape(L, H=2, N=1000, d=128, dt=1):
    return L.park_shape(H, N, d, dt)


def _status(L, fn, *args):
    lib = L.lib()
    st = getattr(lib, fn)(*args)
    return st, lib.park_last_error().decode()


def test_validation_errors(L):
    sh = _shape(L)
    bp = ctypes.byref
    # unsupported head dimension / dtype
    st, msg = _status(L, "park_qrkc_metric", bp(_shape(L, d=96)), FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == L.PARK_EUNSUPPORTED and "d must be" in msg
    st, _ = _status(L, "park_qrkc_metric", bp(_shape(L, dt=7)), FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == L.PARK_EUNSUPPORTED
    # null / misaligned tensors
    st, msg = _status(L, "park_qrkc_metric", bp(sh), None, FAKE, FAKE, 1 << 30, None)
    assert st == L.PARK_EINVAL and "q is NULL" in msg
    st, msg = _status(L, "park_qrkc_metric", bp(sh), MIS, FAKE, FAKE, 1 << 30, None)
    assert st == L.PARK_EINVAL and "aligned" in msg
    # workspace too small
    st, msg = _status(L, "park_qrkc_metric", bp(sh), FAKE, FAKE, FAKE, 16, None)
    assert st == L.PARK_EWORKSPACE and "workspace too small" in msg
    # clusters out of range
    st, msg = _status(L, "park_cluster", bp(sh), FAKE, 0, None, 0, 3, 0, 0, 0, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert st == L.PARK_EINVAL and "n_clusters" in msg
    st, _ = _status(L, "park_cluster", bp(sh), FAKE, 0, None, 1001, 3, 0, 0, 0, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert st == L.PARK_EINVAL
    st, _ = _status(L, "park_cluster", bp(sh), FAKE, 0, None, 4096, 3, 0, 0, 0, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert st == L.PARK_EINVAL
    # QRKC without a metric
    st, msg = _status(L, "park_cluster", bp(sh), FAKE, 1, None, 8, 3, 0, 0, 1, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert st == L.PARK_EINVAL and "qmetric" in msg
    # bad init / side / iters
    st, _ = _status(L, "park_cluster", bp(sh), FAKE, 0, None, 8, 3, 5, 0, 0, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert st == L.PARK_EINVAL
    st, _ = _status(L, "park_cluster", bp(sh), FAKE, 0, None, 8, 3, 0, 0, 2, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert st == L.PARK_EINVAL
    st, _ = _status(L, "park_cluster", bp(sh), FAKE, 0, None, 8, -1, 0, 0, 0, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert st == L.PARK_EINVAL
    # the optional status word must be aligned
    st, msg = _status(L, "park_cluster", bp(sh), FAKE, 0, None, 8, 2, 0, 0, 0, FAKE, FAKE, FAKE, FAKE, ODD, FAKE,
                      1 << 40, None)
    assert st == L.PARK_EINVAL and "status" in msg
    # labels required when iterating
    st, msg = _status(L, "park_cluster", bp(sh), FAKE, 0, None, 8, 2, 0, 0, 0, FAKE, None, FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert st == L.PARK_EINVAL and "labels" in msg
    # top-p outside (0, 1]
    for p in (0.0, -0.1, 1.5, float("nan")):
        st, _ = _status(L, "park_select_topp", FAKE, 2, 10, 20, FAKE, p, FAKE, FAKE, FAKE, FAKE, None)
        assert st == L.PARK_EINVAL, p
    st, _ = _status(L, "park_select_topp", FAKE, 2, 10, 4000, FAKE, 0.9, FAKE, FAKE, FAKE, FAKE, None)
    assert st == L.PARK_EINVAL
    # top-k ratio outside [0, 1]
    for rho in (-0.1, 1.5, float("nan")):
        st, _ = _status(L, "park_select_topk", FAKE, 2, 10, 20, FAKE, rho, FAKE, FAKE, FAKE, FAKE, None)
        assert st == L.PARK_EINVAL, rho
    # SIP: ratio outside [0, 1], log weights required
    for rho in (-0.1, 1.5, float("nan")):
        st, _ = _status(L, "park_select_sip", FAKE, 2, 10, 20, FAKE, rho, 7, FAKE, FAKE, FAKE, FAKE, FAKE, None)
        assert st == L.PARK_EINVAL, rho
    st, msg = _status(L, "park_select_sip", FAKE, 2, 10, 20, FAKE, 0.1, 7, FAKE, FAKE, FAKE, FAKE, None, None)
    assert st == L.PARK_EINVAL and "log_w" in msg
    # estimator maps: unknown mode; centroid and full-key modes need bf16 data; missing inputs
    st, msg = _status(L, "park_estimator_map", bp(sh), FAKE, FAKE, FAKE, FAKE, 10, FAKE, FAKE, FAKE, 20, FAKE, 9,
                      0.0, FAKE, FAKE, 1 << 40, None)
    assert st == L.PARK_EINVAL and "mode" in msg
    sh32 = L.park_shape(2, 100, 64, L.PARK_F32)
    st, _ = _status(L, "park_estimator_map", bp(sh32), FAKE, FAKE, FAKE, FAKE, 10, FAKE, FAKE, FAKE, 20, FAKE,
                    L.PARK_EST_FF, 0.0, FAKE, FAKE, 1 << 40, None)
    assert st == L.PARK_EUNSUPPORTED
    shb = L.park_shape(2, 100, 64, L.PARK_BF16)
    st, msg = _status(L, "park_estimator_map", bp(shb), FAKE, None, FAKE, FAKE, 10, FAKE, FAKE, FAKE, 20, FAKE,
                      L.PARK_EST_FF, 0.0, FAKE, FAKE, 1 << 40, None)
    assert st == L.PARK_EINVAL and msg.startswith("k")
    st, msg = _status(L, "park_estimator_map", bp(shb), None, None, None, FAKE, 10, None, None, FAKE, 20, FAKE,
                      L.PARK_EST_CC, 0.0, FAKE, FAKE, 1 << 40, None)
    assert st == L.PARK_EINVAL and "q_centroids" in msg
    # sparse attention: null selection, small workspace
    st, msg = _status(L, "park_sparse_attn", bp(sh), FAKE, FAKE, FAKE, FAKE, FAKE, 10, FAKE, FAKE, 20, None, FAKE,
                      0.0, FAKE, None, FAKE, 1 << 40, None)
    assert st == L.PARK_EINVAL and "counts" in msg
    st, msg = _status(L, "park_sparse_attn", bp(sh), FAKE, FAKE, FAKE, FAKE, FAKE, 10, FAKE, FAKE, 20, FAKE, FAKE,
                      0.0, FAKE, None, FAKE, 8, None)
    assert st == L.PARK_EWORKSPACE
    # weighted attention: log weights required; a workspace one byte short is refused
    st, msg = _status(L, "park_sparse_attn_weighted", bp(sh), FAKE, FAKE, FAKE, FAKE, FAKE, 10, FAKE, FAKE, 20, FAKE,
                      FAKE, None, 0.0, FAKE, None, FAKE, 1 << 40, None)
    assert st == L.PARK_EINVAL and "log_w" in msg
    prm = L.make_params(10, 20, 1, 0.9)
    need = L.workspace_bytes(L.PARK_ENTRY_SPARSE_ATTN_WEIGHTED, sh, prm)
    st, _ = _status(L, "park_sparse_attn_weighted", bp(sh), FAKE, FAKE, FAKE, FAKE, FAKE, 10, FAKE, FAKE, 20, FAKE,
                    FAKE, FAKE, 0.0, FAKE, None, FAKE, need - 1, None)
    assert st == L.PARK_EWORKSPACE
    # forward: iters must be >= 1, p in range
    prm = L.make_params(10, 20, 0, 0.9)
    st, msg = _status(L, "park_forward", bp(sh), FAKE, FAKE, FAKE, FAKE, bp(prm), FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert st == L.PARK_EINVAL and "iters" in msg
    prm = L.make_params(10, 20, 3, 0.0)
    st, _ = _status(L, "park_forward", bp(sh), FAKE, FAKE, FAKE, FAKE, bp(prm), FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert st == L.PARK_EINVAL
    # the allocation-free attention refuses a shape whose scratch would exceed its 96 MiB (checked
    # before any pointer is touched or anything is enqueued)
    big = L.park_shape(40, 219600, 128, 1)
    st, msg = _status(L, "park_sparse_attn_noalloc", bp(big), FAKE, FAKE, FAKE, FAKE, FAKE, 1000, FAKE, FAKE, 2000,
                      FAKE, FAKE, 0.0, FAKE, None, None)
    assert st == L.PARK_EWORKSPACE and "scratch" in msg
    # permutation: in place is rejected
    st, msg = _status(L, "park_permute_rows", bp(sh), FAKE, FAKE, FAKE, None)
    assert st == L.PARK_EINVAL and "overlap" in msg


def test_workspace_bytes(L):
    wan = L.park_shape(40, 75600, 128, 1)
    prm = L.make_params(100, 500, 10, 0.9)
    fwd = L.workspace_bytes(L.PARK_ENTRY_FORWARD, wan, prm)
    assert fwd > 0
    # the forward workspace holds at least the per-token int arrays and the map
    assert fwd >= 40 * 75600 * 4 * 4 + 40 * 100 * 500 * 4
    assert L.workspace_bytes(L.PARK_ENTRY_METRIC, wan) > 0
    assert L.workspace_bytes(L.PARK_ENTRY_FORWARD, L.park_shape(40, 75600, 96, 1), prm) == 0
    assert L.workspace_bytes(L.PARK_ENTRY_FORWARD, wan, L.make_params(100, 500, 0, 0.9)) == 0
    assert L.workspace_bytes(L.PARK_ENTRY_CLUSTER_K, wan, prm) > L.workspace_bytes(L.PARK_ENTRY_CLUSTER_Q, wan, prm)
    # the attention keeps per (head, query cluster) at most ck runs of its selected keys (three ints
    # each), so its workspace scales with the selection's own size [heads, cq, ck], not with n
    attn = L.workspace_bytes(L.PARK_ENTRY_SPARSE_ATTN, wan, prm)
    assert attn <= 40 * 100 * (3 * 500 + 4 + 3) * 4 + 40 * (2 * 100 + 1) * 4 + 40 * 64 + 1024
    assert L.workspace_bytes(L.PARK_ENTRY_SPARSE_ATTN_WEIGHTED, wan, prm) == attn
    assert L.workspace_bytes(L.PARK_ENTRY_SPARSE_ATTN, L.park_shape(40, 219600, 128, 1), prm) == attn
    # the long clip's whole forward pass fits in 2 GB of workspace (the per-token int arrays, the
    # candidate products of the seeding, the map, sort and map partials)
    long_fwd = L.workspace_bytes(L.PARK_ENTRY_FORWARD, L.park_shape(40, 219600, 128, 1),
                                 L.make_params(200, 1000, 10, 0.9))
    assert 0 < long_fwd <= 2 * 1024 ** 3, long_fwd
    print(f"workspace: Wan attention {attn / 2**20:.1f} MiB, long-clip forward {long_fwd / 2**30:.2f} GiB")
