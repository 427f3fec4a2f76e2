"""ctypes declarations of libmoe's C ABI (include/moe.h).

The library is loaded after torch so that it binds to the HIP runtime torch
already loaded (both carry the soname libamdhip64.so.7): device pointers and
hipStream_t handles then mean the same thing on both sides.  A missing
library is an error; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

c_i32 = ctypes.c_int32
c_ptr = ctypes.c_void_p

MOE_F32 = 0
MOE_BF16 = 1
NOALLOC_SCRATCH_BYTES = 128 << 20  # MOE_NOALLOC_SCRATCH_BYTES

STATUS = {
    0: "MOE_OK",
    1: "MOE_ERR_INVALID_ARG",
    2: "MOE_ERR_NULL_PTR",
    3: "MOE_ERR_WORKSPACE_TOO_SMALL",
    4: "MOE_ERR_UNSUPPORTED",
    5: "MOE_ERR_HIP",
}

EXPORTED = [
    "moe_status_string", "moe_query", "moe_workspace_size", "moe_dispatch_carve", "moe_route", "moe_permute",
    "moe_ffn_gate_up", "moe_ffn_gate_up_gather", "moe_ffn_down", "moe_grouped_ffn", "moe_combine",
    "moe_forward", "moe_ffn_gate_up_fp8", "moe_ffn_down_fp8", "moe_forward_fp8", "moe_pack_blocked16",
    "moe_forward_noalloc",
]


class MoeShape(ctypes.Structure):
    _fields_ = [("T", c_i32), ("d", c_i32), ("E", c_i32), ("k", c_i32), ("F", c_i32),
                ("capacity", c_i32), ("dtype", c_i32), ("tile_rows", c_i32), ("weight_layout", c_i32)]


class MoeSizes(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("tile_rows", c_i32), ("max_tiles", c_i32),
                ("n_passes", c_i32), ("count_blocks", c_i32), ("dispatch_bytes", ctypes.c_size_t),
                ("permute_ws_bytes", ctypes.c_size_t), ("forward_ws_bytes", ctypes.c_size_t)]


DISPATCH_ARRAYS = ["counts", "offsets", "spill_counts", "spill_offsets", "row_of", "token_of",
                   "tile_off", "tile_map", "n_tiles", "err_flags", "kpart"]


class MoeDispatch(ctypes.Structure):
    _fields_ = [(n, c_ptr) for n in DISPATCH_ARRAYS] + [("tile_rows", c_i32), ("max_tiles", c_i32)]


class MoeForwardViews(ctypes.Structure):
    _fields_ = [("disp", MoeDispatch), ("topk_ids", c_ptr), ("topk_w", c_ptr), ("x_perm", c_ptr),
                ("h", c_ptr), ("y_perm", c_ptr)]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg}")
        self.status = status


_lib = None
_lock = threading.Lock()


def _declare(lib):
    P = ctypes.POINTER
    S = P(MoeShape)
    D = P(MoeDispatch)
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    sig = {
        "moe_query": [S, P(MoeSizes)],
        "moe_workspace_size": [S, P(ctypes.c_size_t)],
        "moe_dispatch_carve": [S, c_ptr, ctypes.c_size_t, D],
        "moe_route": [S, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr],
        "moe_permute": [S, c_ptr, c_ptr, D, c_ptr, c_ptr, ctypes.c_size_t, c_ptr],
        "moe_ffn_gate_up": [S, c_ptr, c_ptr, c_ptr, D, ctypes.c_int, c_ptr, c_ptr],
        "moe_ffn_gate_up_gather": [S, c_ptr, c_ptr, c_ptr, D, ctypes.c_int, c_ptr, c_ptr],
        "moe_ffn_down": [S, c_ptr, c_ptr, D, ctypes.c_int, c_ptr, c_ptr],
        "moe_grouped_ffn": [S, c_ptr, c_ptr, c_ptr, c_ptr, D, c_ptr, c_ptr, c_ptr],
        "moe_combine": [S, c_ptr, c_ptr, D, c_ptr, c_ptr],
        "moe_forward": [S, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr,
                        ctypes.c_size_t, P(MoeForwardViews), c_ptr],
        "moe_ffn_gate_up_fp8": [S, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, D, ctypes.c_int, c_ptr, c_ptr],
        "moe_ffn_down_fp8": [S, c_ptr, c_ptr, c_ptr, D, ctypes.c_int, c_ptr, c_ptr],
        "moe_forward_fp8": [S, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr,
                            c_ptr, c_ptr, ctypes.c_size_t, P(MoeForwardViews), c_ptr],
        "moe_pack_blocked16": [c_ptr, c_ptr, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, c_ptr],
        "moe_forward_noalloc": [S, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr,
                                P(MoeForwardViews), c_ptr],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int


def lib():
    """The loaded libmoe (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                import torch  # noqa: F401  (binds libmoe to torch's HIP runtime)
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with `python -m grouped_gemm_gemv_amd.build`")
                l = ctypes.CDLL(LIB_PATH)
                _declare(l)
                _lib = l
    return _lib


def check(fn: str, status: int):
    if status != 0:
        msg = lib().moe_status_string(status).decode()
        raise MoeError(fn, status, msg)
