"""ctypes loader for ``libdcpmla.so`` (the C ABI declared in ``include/dcpmla.h``).

Argument marshalling only.  There is no fallback: if the library is missing,
importing this module raises, so nothing can silently run another path.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdcpmla.so")

KV_BF16 = 0
KV_FP8_E4M3 = 1
BOUNDARY_CAUSAL = 0
BOUNDARY_BLOCK = 1
Q_SPLIT = 0
Q_FP8 = 1
P_SPLIT = 0
P_FP8 = 1

OK = 0
E_INVALID = -1
E_ALIAS = -2
E_WORKSPACE = -3
E_UNSUPPORTED = -4
E_HIP = -5
E_SCRATCH = -6

ERR_CTX_LT_QLEN = 1
ERR_TABLE_CAPACITY = 2
ERR_LOCAL_PAGES = 4
ERR_BLOCK_ID = 8
ERR_PAGE_RANGE = 16
ERR_TOKEN = 32
ERR_KERNARG = 64


class Geom(ctypes.Structure):
    _fields_ = [
        ("dcp_world", ctypes.c_int32),
        ("interleave", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("qlen", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_local_pages", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("groups", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("row_boundary", ctypes.c_int32),
        ("q_format", ctypes.c_int32),
        ("p_format", ctypes.c_int32),
    ]


class Meta(ctypes.Structure):
    _fields_ = [
        ("row_local_len", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("last_page_len", ctypes.c_void_p),
        ("err", ctypes.c_void_p),
        ("work", ctypes.c_void_p),
    ]


_P = ctypes.c_void_p
_G = ctypes.POINTER(Geom)
_M = ctypes.POINTER(Meta)
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F = ctypes.c_float

#: every entry point of include/dcpmla.h with (restype, argtypes)
class DeviceInfo(ctypes.Structure):
    """Mirror of ``dcpmla_device_info``."""
    _fields_ = [("compute_units", ctypes.c_int32), ("clock_khz", ctypes.c_int32),
                ("memory_clock_khz", ctypes.c_int32), ("memory_bus_bits", ctypes.c_int32),
                ("lds_bytes_per_block", ctypes.c_int64), ("arch", ctypes.c_char * 64)]


SIGNATURES = {
    "dcpmla_validate": (ctypes.c_int, [_G]),
    "dcpmla_subpage_size": (_I32, [_I32]),
    "dcpmla_work_ints": (_I64, [_G]),
    "dcpmla_workspace_bytes": (_I64, [_G]),
    "dcpmla_write_kv": (ctypes.c_int, [_G, _I32, _I64, _P, _P, _P, _P, _P, _P, _P, _P]),
    "dcpmla_build_metadata": (ctypes.c_int, [_G, _I32, _P, _P, _M, _P]),
    "dcpmla_partial_attention": (ctypes.c_int, [_G, _P, _P, _F, _F, _M, _P, _I64, _P, _P, _P]),
    "dcpmla_merge_segments": (ctypes.c_int, [_G, _M, _P, _I64, _P, _P, _P]),
    "dcpmla_rank_attention": (ctypes.c_int, [_G, _P, _P, _F, _F, _M, _P, _I64, _P, _P, _P]),
    "dcpmla_rank_attention_static": (ctypes.c_int, [_G, _P, _P, _F, _F, _M, _P, _P, _P]),
    "dcpmla_static_scratch_bytes": (_I64, []),
    "dcpmla_merge_ranks": (ctypes.c_int, [_I32, _I64, _P, _P, _P, _P, _P]),
    "dcpmla_merge_segments_dense": (ctypes.c_int, [_I64, _I32, _P, _P, _P, _P, _P]),
    "dcpmla_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "dcpmla_get_device_info": (ctypes.c_int, [_I32, ctypes.c_void_p]),
    "dcpmla_a2a_message_elems": (_I64, [_I32]),
    "dcpmla_split_q": (ctypes.c_int, [_I64, _P, _P, _P, _P]),
    "dcpmla_split_q_bytes": (ctypes.c_int64, [_I64]),
    "dcpmla_partial_attention_split": (ctypes.c_int, [_G, _P, _P, _P, _F, _F, _M, _P, _I64, _P, _P, _P]),
    "dcpmla_a2a_pack": (ctypes.c_int, [_I32, _I64, _I32, _I32, _P, _P, _P, _P]),
    "dcpmla_a2a_combine": (ctypes.c_int, [_I32, _I64, _I32, _I32, _P, _P, _P, _P]),
    "dcpmla_project_heads": (ctypes.c_int, [_I64, _I32, _I32, _P, _P, _P, _P]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m decode_context_parallelism_amd.build` "
            "(hipcc for gfx950) first")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def strerror(status: int) -> str:
    return lib.dcpmla_strerror(int(status)).decode()
