"""ctypes loader for libcpattn.so: argument marshalling only.

``torch`` is imported before the library is opened so that the library's
``libamdhip64.so.7`` resolves to the HIP runtime torch already loaded (one
runtime per process: stream handles from torch are then valid in the
library).  A missing library is an error: there is no fallback path.
"""

import ctypes
import os

import torch  # noqa: F401  (must precede loading the HIP library)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcpattn.so")

OK = 0
EINVAL = -1
EUNSUPPORTED = -2
ENOWORKSPACE = -3
EHIP = -4

CONTIGUOUS = 0
ZIGZAG = 1
BF16 = 0
FP32 = 1

OPT_MERGE = 1
OPT_SERIALIZE = 2
OPT_RECV = 3
OPT_POISON = 4
OPT_STEP_TIMING = 5
OPT_RECV_BLOCKS = 6
OPT_GRAPH = 7
OPT_KSPLIT = 8
OPT_COUNTERS = 9
OPT_BWD_KEYS = 10
OPT_LOCKSTEP = 12
OPT_FUSED_RING = 13
OPT_BWD_FUSED = 14

NOALLOC_SCRATCH_BYTES = 128 << 20  # CP_ATTN_NOALLOC_SCRATCH_BYTES

_c_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64

# name -> (restype, argtypes); mirrors include/cp_attn.h
SIGNATURES = {
    "cp_attn_plan": (ctypes.c_int, [_i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.POINTER(_c_p)]),
    "cp_attn_plan_destroy": (ctypes.c_int, [_c_p]),
    "cp_attn_set_dtype": (ctypes.c_int, [_c_p, ctypes.c_int]),
    "cp_attn_set_option": (ctypes.c_int, [_c_p, ctypes.c_int, ctypes.c_int]),
    "cp_attn_workspace_bytes": (ctypes.c_int, [_c_p, ctypes.POINTER(_i64)]),
    "cp_attn_ring_wait_timeouts": (ctypes.c_int, [_c_p, ctypes.POINTER(_i32)]),
    "cp_attn_fused_ring_active": (ctypes.c_int, [_c_p, ctypes.POINTER(_i32)]),
    "cp_attn_set_workspace": (ctypes.c_int, [_c_p, _c_p, _i64]),
    "cp_attn_set_streams": (ctypes.c_int, [_c_p, _c_p, _c_p]),
    "cp_attn_set_documents": (ctypes.c_int, [_c_p, ctypes.POINTER(_i64), _i64]),
    "cp_attn_rank_forward": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, ctypes.c_int, _c_p]),
    "cp_attn_rank_forward_noalloc": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, ctypes.c_int, _c_p]),
    "cp_attn_full_forward": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p]),
    "cp_attn_ulysses_a2a": (ctypes.c_int, [_c_p, _c_p, _c_p, ctypes.c_int, _c_p]),
    "cp_attn_ulysses_forward": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p]),
    "cp_attn_rank_backward": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, ctypes.c_int,
                                             _c_p]),
    "cp_attn_full_backward": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p]),
    "cp_attn_local_rows": (ctypes.c_int, [_c_p, ctypes.POINTER(_i64)]),
    "cp_attn_rank_chunks": (ctypes.c_int, [_c_p, ctypes.c_int, ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "cp_attn_rank_valid_rows": (ctypes.c_int, [_c_p, ctypes.c_int, ctypes.POINTER(_i64)]),
    "cp_attn_step_source": (ctypes.c_int, [_c_p, ctypes.c_int, ctypes.c_int, ctypes.POINTER(_i32)]),
    "cp_attn_step_segments": (ctypes.c_int, [_c_p, ctypes.c_int, ctypes.c_int, ctypes.POINTER(_i64),
                                             ctypes.POINTER(_i32)]),
    "cp_attn_valid_work": (ctypes.c_int, [_c_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "cp_attn_layout_gather": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p]),
    "cp_attn_layout_scatter": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p]),
    "cp_attn_lse_merge": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _i64, ctypes.c_int, ctypes.c_int, _c_p]),
    "cp_attn_last_step_times": (ctypes.c_int, [_c_p, ctypes.POINTER(ctypes.c_float), ctypes.c_int]),
    "cp_attn_allgather_forward": (ctypes.c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, ctypes.c_int, _c_p]),
    "cp_attn_last_tile_counts": (ctypes.c_int, [_c_p, ctypes.POINTER(ctypes.c_int64), ctypes.c_int,
                                                ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]),
    "cp_attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "cp_attn_last_error": (ctypes.c_char_p, []),
}

_lib = None


class CpAttnError(RuntimeError):
    def __init__(self, status, func, detail):
        self.status = status
        super().__init__(f"{func} failed: status {status} ({detail})")


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m ring_context_parallelism_amd.build`")
        h = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def check(status, func):
    if status != OK:
        detail = lib().cp_attn_last_error().decode(errors="replace") or lib().cp_attn_status_string(status).decode()
        raise CpAttnError(status, func, detail)
    return status
