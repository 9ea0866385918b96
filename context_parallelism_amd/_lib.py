"""ctypes binding of libcpattn.so: the C ABI of include/cpattn.h, same names.

Argument marshalling only. The library is loaded from this package
directory (built in-tree by ``context_parallelism_amd.build``); if it is
missing, loading raises -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_int32, c_int64, c_size_t, c_uint32, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcpattn.so")

CP_OK = 0
CP_EINVAL = -1
CP_ENOSPC = -2
CP_EUNSUPPORTED = -3
CP_EHIP = -4
CP_DTYPE_F32 = 0
CP_DTYPE_BF16 = 1
CP_MAX_CP_SIZE = 32
CP_SPLIT_HEAD_TAIL = 0
CP_SPLIT_CONTIGUOUS = 1
CP_SCHED_AUTO = 0
CP_SCHED_ROW_TILE = 1
CP_SCHED_PER_STEP = 2
CP_NOALLOC_SCRATCH_BYTES = 16 << 20

# (name, restype, argtypes) for every entry point declared in include/cpattn.h
_P32 = POINTER(c_int32)
_P64 = POINTER(c_int64)
SIGNATURES = [
    ("cp_partition_index", c_int32,
     [c_int64, _P32, _P32, c_int32, c_int32, c_int32, _P32, c_int64, _P64, _P32]),
    ("cp_pair_counts", c_int32, [c_int64, _P32, _P32, c_int32, c_int32, c_int32, _P64, _P64]),
    ("cp_attn_rank_workspace_size", c_int32,
     [c_int64, _P32, _P32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
      POINTER(c_size_t)]),
    ("cp_attn_rank_plan_stats", c_int32,
     [c_int64, _P32, _P32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
      _P64, _P64, _P64, _P64, _P64]),
    ("cp_attn_rank_fwd", c_int32,
     [c_void_p, c_void_p, c_void_p, c_int32, c_int64, _P32, _P32, c_int32, c_int32, c_int32,
      c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    ("cp_attn_rank_fwd_timed", c_int32,
     [c_void_p, c_void_p, c_void_p, c_int32, c_int64, _P32, _P32, c_int32, c_int32, c_int32,
      c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p, POINTER(c_void_p)]),
    ("cp_attn_rank_fwd_noalloc", c_int32,
     [c_void_p, c_void_p, c_void_p, c_int32, c_int64, _P32, _P32, c_int32, c_int32, c_int32,
      c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
    ("cp_gather_rows", c_int32, [c_void_p, c_int32, c_int64, c_int64, c_void_p, c_int64, c_void_p, c_void_p]),
    ("cp_lse_merge", c_int32,
     [c_void_p, c_void_p, c_void_p, c_int32, c_int64, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
    ("cp_partition_index_ex", c_int32,
     [c_int64, _P32, _P32, c_int32, c_int32, c_int32, c_int32, _P32, c_int64, _P64, _P32]),
    ("cp_pair_counts_ex", c_int32, [c_int64, _P32, _P32, c_int32, c_int32, c_int32, c_int32, _P64, _P64]),
    ("cp_attn_rank_workspace_size_ex", c_int32,
     [c_int64, _P32, _P32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
      c_int32, POINTER(c_size_t)]),
    ("cp_attn_rank_plan_stats_ex", c_int32,
     [c_int64, _P32, _P32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
      _P64, _P64, _P64, _P64, _P64]),
    ("cp_attn_rank_fwd_ex", c_int32,
     [c_void_p, c_void_p, c_void_p, c_int32, c_int64, _P32, _P32, c_int32, c_int32, c_int32, c_int32,
      c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p,
      POINTER(c_void_p)]),
    ("cp_attn_rank_bwd_workspace_size", c_int32,
     [c_int64, _P32, _P32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
      POINTER(c_size_t)]),
    ("cp_attn_rank_bwd", c_int32,
     [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int64, _P32, _P32, c_int32,
      c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
      c_size_t, c_void_p]),
    ("cp_status_string", c_char_p, [c_int32]),
]

_lib = None


class CpError(RuntimeError):
    """A non-zero cp_status from the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {cp_status_string(status)} (status {status})")


def load() -> ctypes.CDLL:
    """Load libcpattn.so once and attach the C signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python context_parallelism_amd/build.py` "
                "(there is no fallback implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int, where: str) -> None:
    if status != CP_OK:
        raise CpError(status, where)


def cp_status_string(status: int) -> str:
    return load().cp_status_string(status).decode()


def _fn(name):
    def call(*args):
        return getattr(load(), name)(*args)

    call.__name__ = name
    call.__doc__ = f"Direct call of the C entry point {name} (see include/cpattn.h)."
    return call


cp_partition_index = _fn("cp_partition_index")
cp_pair_counts = _fn("cp_pair_counts")
cp_attn_rank_workspace_size = _fn("cp_attn_rank_workspace_size")
cp_attn_rank_plan_stats = _fn("cp_attn_rank_plan_stats")
cp_attn_rank_fwd = _fn("cp_attn_rank_fwd")
cp_attn_rank_fwd_timed = _fn("cp_attn_rank_fwd_timed")
cp_attn_rank_fwd_noalloc = _fn("cp_attn_rank_fwd_noalloc")
cp_gather_rows = _fn("cp_gather_rows")
cp_lse_merge = _fn("cp_lse_merge")
cp_partition_index_ex = _fn("cp_partition_index_ex")
cp_pair_counts_ex = _fn("cp_pair_counts_ex")
cp_attn_rank_workspace_size_ex = _fn("cp_attn_rank_workspace_size_ex")
cp_attn_rank_plan_stats_ex = _fn("cp_attn_rank_plan_stats_ex")
cp_attn_rank_fwd_ex = _fn("cp_attn_rank_fwd_ex")
cp_attn_rank_bwd_workspace_size = _fn("cp_attn_rank_bwd_workspace_size")
cp_attn_rank_bwd = _fn("cp_attn_rank_bwd")
