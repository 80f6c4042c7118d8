"""ctypes binding of ``libpark.so`` (the C ABI in ``include/park.h``).

Argument marshalling only: torch tensors supply device memory and the current HIP stream; every
step of the computation runs in the library's HIP kernels. There is no CPU fallback: if the built
library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpark.so")

PARK_OK, PARK_EINVAL, PARK_EUNSUPPORTED, PARK_EWORKSPACE, PARK_EHIP = range(5)
PARK_F32, PARK_BF16 = 0, 1
PARK_EUCLID, PARK_QRKC = 0, 1
PARK_INIT_KMEANSPP, PARK_INIT_WARM, PARK_INIT_SUBSET = 0, 1, 2
PARK_SIDE_Q, PARK_SIDE_K = 0, 1
PARK_EST_FC, PARK_EST_CC, PARK_EST_CF, PARK_EST_FF = range(4)
(PARK_ENTRY_METRIC, PARK_ENTRY_CLUSTER_Q, PARK_ENTRY_CLUSTER_K, PARK_ENTRY_RETRIEVE_MAP,
 PARK_ENTRY_SELECT_TOPP, PARK_ENTRY_SPARSE_ATTN, PARK_ENTRY_FORWARD, PARK_ENTRY_ESTIMATOR,
 PARK_ENTRY_SPARSE_ATTN_WEIGHTED, PARK_ENTRY_MERGE) = range(10)
PARK_DEVSTATUS_SEED_TIMEOUT = 1

EXPORTED = [
    "park_workspace_bytes", "park_status_string", "park_last_error", "park_version",
    "park_qrkc_metric", "park_cluster", "park_retrieve_map", "park_estimator_map", "park_select_topp",
    "park_select_topk", "park_select_sip", "park_sparse_attn", "park_sparse_attn_weighted",
    "park_permute_rows", "park_unpermute_rows", "park_forward", "park_debug_force_seed_timeout",
    "park_cluster_subset", "park_merge_clusters", "park_sparse_attn_noalloc",
]


class ParkError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_STATUS = {PARK_OK: "PARK_OK", PARK_EINVAL: "PARK_EINVAL", PARK_EUNSUPPORTED: "PARK_EUNSUPPORTED",
           PARK_EWORKSPACE: "PARK_EWORKSPACE", PARK_EHIP: "PARK_EHIP"}


class park_shape(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int64), ("n", ctypes.c_int64), ("d", ctypes.c_int64), ("dtype", ctypes.c_int32)]


class park_params(ctypes.Structure):
    _fields_ = [("cq", ctypes.c_int32), ("ck", ctypes.c_int32), ("iters", ctypes.c_int32), ("p", ctypes.c_double),
                ("scale", ctypes.c_float), ("seed", ctypes.c_uint64), ("kmetric", ctypes.c_int32),
                ("init", ctypes.c_int32), ("subset_stride", ctypes.c_int32), ("subset_phase", ctypes.c_int32)]


class park_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("pairs", "padded_pairs", "blocks", "live_blocks", "work_items",
                                              "tokens", "reserved0", "reserved1")]


STATS_FIELDS = ("pairs", "padded_pairs", "blocks", "live_blocks", "work_items", "tokens")


_P = ctypes.c_void_p


class park_forward_outputs(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("metric", "q_labels", "q_perm", "q_offsets", "k_labels", "k_perm", "k_offsets",
                                  "map", "mask", "counts", "cols", "sel_keys", "lse",
                                  "status", "stats")]


_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """Load libpark.so (built by ``python -m block_sparse_attention_qrkc_amd.build``)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m block_sparse_attention_qrkc_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, u64, f32, f64, sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float,
                                       ctypes.c_double, ctypes.c_size_t)
        SP = ctypes.POINTER(park_shape)
        PP = ctypes.POINTER(park_params)
        sig = {
            "park_workspace_bytes": (sz, [i32, SP, PP]),
            "park_status_string": (ctypes.c_char_p, [i32]),
            "park_last_error": (ctypes.c_char_p, []),
            "park_version": (ctypes.c_char_p, []),
            "park_qrkc_metric": (i32, [SP, _P, _P, _P, sz, _P]),
            "park_cluster": (i32, [SP, _P, i32, _P, i32, i32, i32, u64, i32, _P, _P, _P, _P, _P, _P, sz, _P]),
            "park_debug_force_seed_timeout": (None, [i32]),
            "park_cluster_subset": (i32, [SP, _P, i32, _P, i32, i32, i32, i32, _P, _P, _P, _P, _P, sz, _P]),
            "park_merge_clusters": (i32, [i64, i64, i32, i32, i32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, sz,
                                          _P]),
            "park_retrieve_map": (i32, [SP, _P, _P, _P, i32, _P, _P, i32, f32, _P, _P, sz, _P]),
            "park_estimator_map": (i32, [SP, _P, _P, _P, _P, i32, _P, _P, _P, i32, _P, i32, f32, _P, _P, sz, _P]),
            "park_select_topp": (i32, [_P, i64, i32, i32, _P, f64, _P, _P, _P, _P, _P]),
            "park_select_topk": (i32, [_P, i64, i32, i32, _P, f64, _P, _P, _P, _P, _P]),
            "park_select_sip": (i32, [_P, i64, i32, i32, _P, f64, u64, _P, _P, _P, _P, _P, _P]),
            "park_sparse_attn": (i32, [SP, _P, _P, _P, _P, _P, i32, _P, _P, i32, _P, _P, f32, _P, _P, _P, sz, _P]),
            "park_sparse_attn_weighted": (i32, [SP, _P, _P, _P, _P, _P, i32, _P, _P, i32, _P, _P, _P, f32, _P, _P, _P,
                                                sz, _P]),
            "park_sparse_attn_noalloc": (i32, [SP, _P, _P, _P, _P, _P, i32, _P, _P, i32, _P, _P, f32, _P, _P, _P]),
            "park_permute_rows": (i32, [SP, _P, _P, _P, _P]),
            "park_unpermute_rows": (i32, [SP, _P, _P, _P, _P]),
            "park_forward": (i32, [SP, _P, _P, _P, _P, PP, _P, _P, ctypes.POINTER(park_forward_outputs), _P, sz,
                                   _P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
        return L


def _check(status: int):
    if status != PARK_OK:
        raise ParkError(status, lib().park_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_shape(x: torch.Tensor) -> park_shape:
    if x.dim() != 3 or not x.is_contiguous():
        raise ValueError("expected a contiguous [heads, n, d] tensor")
    if x.dtype == torch.bfloat16:
        dt = PARK_BF16
    elif x.dtype == torch.float32:
        dt = PARK_F32
    else:
        raise ValueError("dtype must be bfloat16 or float32")
    return park_shape(x.shape[0], x.shape[1], x.shape[2], dt)


def make_params(cq=1, ck=1, iters=1, p=0.9, scale=0.0, seed=0, kmetric=PARK_QRKC, init=PARK_INIT_KMEANSPP,
                subset_stride=1, subset_phase=0):
    return park_params(int(cq), int(ck), int(iters), float(p), float(scale), int(seed) & ((1 << 64) - 1),
                       int(kmetric), int(init), int(subset_stride), int(subset_phase))


class Workspace:
    """Device workspace reused across calls (grown on demand)."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes: int, device) -> torch.Tensor | None:
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != torch.device(device):
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        return self.buf


_WS = Workspace()


def workspace_bytes(entry: int, shape: park_shape, params: park_params | None = None) -> int:
    return int(lib().park_workspace_bytes(entry, ctypes.byref(shape), ctypes.byref(params) if params else None))


def _ws(entry, shape, params, device, ws):
    n = workspace_bytes(entry, shape, params)
    buf = (ws or _WS).get(n, device)
    return _ptr(buf), (buf.numel() if buf is not None else 0)
