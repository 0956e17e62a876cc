"""ctypes loader for the HIP library and the C structs of include/ep_mi355x.h.

There is no fallback: if the library is not built, loading raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (load torch's HIP runtime first so the library binds to it)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libep_mi355x.so")

EP_OK = 0
EP_EINVAL = 1
EP_ENOTSUP = 2
EP_EHIP = 3
EP_EWORKSPACE = 4
EP_ESCRATCH = 5

EP_MAX_TOPK = 32
EP_MAX_KEYS = 1024
EP_LAYOUT_SCRATCH_BYTES = 9 << 18

EP_STATUS_INVALID_IDS = 0
EP_STATUS_ROWS_EXPERT = 1
EP_STATUS_ROWS_GROUP = 2
EP_STATUS_LIST_OVERFLOW = 3
EP_STATUS_COMBINE_OOB = 4
EP_STATUS_EXPERT_LIST_OVERFLOW = 5
EP_STATUS_SELECTIONS = 6
EP_STATUS_DISPATCH_OVERFLOW = 7
EP_STATUS_GENERATION = 8
EP_STATUS_STALE = 9
EP_STATUS_WORDS = 16

EP_FLAG_ZERO_PADDING = 1
EP_FLAG_GATHER_ROWS = 2
EP_FLAG_PACKED_WEIGHTS = 4

EP_FORMAT_BF16 = 0
EP_FORMAT_FP8_PACKED = 1
EP_ROWS_EXPERT = 0
EP_ROWS_GROUP = 1
EP_COMBINE_FLAT = 0
EP_COMBINE_GROUPED = 1

EXPORTS = (
    "ep_fp8_row_bytes",
    "ep_layout_workspace_bytes",
    "ep_layout",
    "ep_layout_noalloc",
    "ep_dispatch",
    "ep_combine",
    "ep_expert_gemm",
    "ep_expert_weights_packed_bytes",
    "ep_pack_expert_weights",
    "ep_strerror",
)


class Problem(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int64),
        ("hidden", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("num_groups", ctypes.c_int32),
        ("expert_alignment", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


class LayoutStruct(ctypes.Structure):
    _fields_ = [
        ("counts", ctypes.c_void_p),
        ("offsets", ctypes.c_void_p),
        ("slot", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
        ("group_counts", ctypes.c_void_p),
        ("group_offsets", ctypes.c_void_p),
        ("grow", ctypes.c_void_p),
        ("row_src", ctypes.c_void_p),
        ("row_topk_idx", ctypes.c_void_p),
        ("row_topk_weights", ctypes.c_void_p),
        ("row_capacity", ctypes.c_int64),
        ("expert_row_src", ctypes.c_void_p),
        ("expert_row_capacity", ctypes.c_int64),
        ("recv_stats", ctypes.c_void_p),
        ("generation", ctypes.c_uint32),
    ]


class EPError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with code {code}: {msg}")
        self.code = code


_LIB = None


def lib(path: str | None = None) -> ctypes.CDLL:
    """Load (once) and type the library's exports.  Raises if it is missing."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"HIP library {p} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`"
        )
    L = ctypes.CDLL(p)
    P = ctypes.POINTER(Problem)
    LS = ctypes.POINTER(LayoutStruct)
    vp = ctypes.c_void_p
    L.ep_fp8_row_bytes.argtypes = [ctypes.c_int32]
    L.ep_fp8_row_bytes.restype = ctypes.c_int64
    L.ep_layout_workspace_bytes.argtypes = [P]
    L.ep_layout_workspace_bytes.restype = ctypes.c_size_t
    L.ep_layout.argtypes = [P, vp, vp, LS, vp, ctypes.c_size_t, vp]
    L.ep_layout.restype = ctypes.c_int
    L.ep_layout_noalloc.argtypes = [P, vp, vp, LS, vp]
    L.ep_layout_noalloc.restype = ctypes.c_int
    L.ep_dispatch.argtypes = [P, LS, vp, vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp]
    L.ep_dispatch.restype = ctypes.c_int
    L.ep_combine.argtypes = [P, LS, vp, vp, vp, ctypes.c_int64, vp, vp, vp, ctypes.c_int32, vp]
    L.ep_combine.restype = ctypes.c_int
    L.ep_expert_gemm.argtypes = [P, LS, vp, ctypes.c_int64, vp, ctypes.c_int32, vp, ctypes.c_int64, vp]
    L.ep_expert_gemm.restype = ctypes.c_int
    L.ep_expert_weights_packed_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    L.ep_expert_weights_packed_bytes.restype = ctypes.c_int64
    L.ep_pack_expert_weights.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp]
    L.ep_pack_expert_weights.restype = ctypes.c_int
    L.ep_strerror.argtypes = [ctypes.c_int]
    L.ep_strerror.restype = ctypes.c_char_p
    if path is None:
        _LIB = L
    return L


def check(fn: str, code: int) -> None:
    if code != EP_OK:
        raise EPError(fn, code, lib().ep_strerror(code).decode())
