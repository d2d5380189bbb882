"""ctypes binding to libmil_ssm.so: argument marshalling only.

Every step of the layer runs in the HIP library; this module passes device pointers,
sizes and the current HIP stream, and turns status codes into exceptions.  If the
library has not been built the import of `lib()` fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmil_ssm.so")

MIL_OK, MIL_E_INVALID, MIL_E_ALIGN, MIL_E_ORDER, MIL_E_UNSUPPORTED, MIL_E_HIP, MIL_E_WORKSPACE = range(7)
MIL_F32, MIL_BF16 = 0, 1
MIL_PREFILL_CONTINUE = 1
MIL_COMMIT_MATERIALIZE = 1
MIL_DEVERR_ACCEPT = 1
MIL_DEVERR_TREE = 2
MIL_DEVERR_SCAN = 4
MIL_KMAX_LIMIT = 16
PHASE_UNINIT, PHASE_READY, PHASE_VERIFIED = 0, 1, 2

# every function the header declares
EXPORTS = [
    "mil_status_string", "mil_ssm_supported", "mil_ssm_cache_layout", "mil_ssm_cache_bytes",
    "mil_ssm_cache_init", "mil_ssm_cache_attach", "mil_ssm_prefill_workspace_bytes", "mil_ssm_prefill", "mil_ssm_verify",
    "mil_ssm_commit", "mil_ssm_cache_status", "mil_ssm_cache_phase", "mil_ssm_cache_trace",
    "mil_ssm_greedy_workspace_bytes", "mil_ssm_commit_greedy", "mil_ssm_project_workspace_bytes", "mil_ssm_project",
    "mil_ssm_verify_tree", "mil_ssm_commit_tree", "mil_ssm_prefill_kernels", "mil_ssm_commit_greedy_noalloc",
    "mil_ssm_commit_layers",
]
MIL_COMMIT_LAYERS_MAX = 32
MIL_GREEDY_NOALLOC_MAX_ROWS = 512
TRACE = {"off": 0, "verify": 1, "fold": 2, "commit": 3, "prefill_state": 4, "prefill_pass": 5, "prefill_out": 6,
         "accept": 7, "prefill_scan": 8}


class MilError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("nheads", ctypes.c_int32), ("headdim", ctypes.c_int32),
                ("dstate", ctypes.c_int32), ("ngroups", ctypes.c_int32)]


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("bytes", "state_off", "state_head_stride", "pend_x_off",
                                              "pend_B_off", "pend_dt_off", "pos_off", "pending_off",
                                              "err_off", "scan_off", "append_off")]


class CacheDesc(ctypes.Structure):
    _fields_ = [("opaque", ctypes.c_uint64 * 24)]


_lib = None


def lib():
    """The loaded library.  Raises if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m speculative_decode_amd.build` "
                          "(or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, u32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_uint32
    dims_p, lay_p, cache_p = ctypes.POINTER(Dims), ctypes.POINTER(Layout), ctypes.POINTER(CacheDesc)
    sigs = {
        "mil_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "mil_ssm_supported": ([dims_p, i32], ctypes.c_int),
        "mil_ssm_cache_layout": ([dims_p, i32, i32, lay_p], ctypes.c_int),
        "mil_ssm_cache_bytes": ([dims_p, i32, i32], sz),
        "mil_ssm_cache_init": ([cache_p, dims_p, i32, i32, vp, sz, vp], ctypes.c_int),
        "mil_ssm_cache_attach": ([cache_p, dims_p, i32, i32, vp, sz], ctypes.c_int),
        "mil_ssm_prefill_workspace_bytes": ([dims_p, i32, i32, i32], sz),
        "mil_ssm_prefill": ([cache_p, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, u32, vp],
                            ctypes.c_int),
        "mil_ssm_verify": ([cache_p, i32, vp, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
        "mil_ssm_commit": ([cache_p, i32, vp, vp, vp, vp, vp, vp, u32, vp], ctypes.c_int),
        "mil_ssm_cache_status": ([cache_p, ctypes.POINTER(i32), i32, vp], ctypes.c_int),
        "mil_ssm_cache_phase": ([cache_p], ctypes.c_int),
        "mil_ssm_cache_trace": ([cache_p, i32, vp, vp], ctypes.c_int),
        "mil_ssm_greedy_workspace_bytes": ([dims_p, i32, i32], sz),
        "mil_ssm_commit_greedy": ([cache_p, i32, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, u32, vp],
                                  ctypes.c_int),
        "mil_ssm_commit_greedy_noalloc": ([cache_p, i32, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, u32, vp],
                                          ctypes.c_int),
        "mil_ssm_project_workspace_bytes": ([dims_p, i32, i32], sz),
        "mil_ssm_verify_tree": ([cache_p, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
        "mil_ssm_prefill_kernels": ([cache_p, i32, i32, i32], ctypes.c_int),
        "mil_ssm_commit_tree": ([cache_p, i32, vp, vp, vp, vp, vp, vp, vp, u32, vp], ctypes.c_int),
        "mil_ssm_commit_layers": ([ctypes.POINTER(cache_p), i32, i32, vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                   ctypes.POINTER(vp), vp], ctypes.c_int),
        "mil_ssm_project": ([dims_p, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, sz, vp],
                            ctypes.c_int),
    }
    for name, (args, res) in sigs.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def status_string(status: int) -> str:
    try:
        return lib().mil_status_string(status).decode()
    except ImportError:  # pragma: no cover
        return "unknown"


def check(status: int, what: str) -> None:
    if status != MIL_OK:
        raise MilError(status, what)
