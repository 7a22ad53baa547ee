"""ctypes view of libh2o.so (the C ABI declared in include/h2o.h).

There is no fallback: if the library is missing or fails to load, importing
this module raises ImportError.  Build it with
``python h2o_sparse_attention_amd/build.py``.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int32, c_int64, c_size_t, c_void_p

# H2O_LIB_PATH loads another build of the same library (for instance the host-sanitizer
# build that the CPU tests make); by default the in-tree build.
LIB_PATH = os.environ.get("H2O_LIB_PATH") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "lib", "libh2o.so")

H2O_OK = 0
H2O_ERR_INVALID_ARG = -1
H2O_ERR_UNSUPPORTED = -2
H2O_ERR_CAPACITY = -3
H2O_ERR_WORKSPACE = -4
H2O_ERR_HIP = -5
STATUS_NAMES = {0: "H2O_OK", -1: "H2O_ERR_INVALID_ARG", -2: "H2O_ERR_UNSUPPORTED",
                -3: "H2O_ERR_CAPACITY", -4: "H2O_ERR_WORKSPACE", -5: "H2O_ERR_HIP"}

H2O_F32, H2O_BF16 = 0, 1
H2O_SCORE_H2O, H2O_SCORE_H2O_NORM = 0, 1
KERNEL_IDS = {"attn": 0, "colsum": 1, "update": 2, "select": 3, "insert": 4, "decode": 5,
              "decode_finish": 6, "backward": 7}

# Every function include/h2o.h declares, with its ctypes signature.
EXPORTS = {}


class Dims(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("capacity", c_int32), ("recent_window", c_int32),
                ("dtype", c_int32)]


class CacheStruct(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("pos", c_void_p), ("score", c_void_p),
                ("n_valid", c_int32)]


_SIGNATURES = {
    "h2o_workspace_bytes": (c_size_t, [POINTER(Dims), c_int32]),
    "h2o_chunk_attn": (c_int32, [POINTER(Dims), POINTER(CacheStruct), c_int64, c_int32, c_float,
                                 c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_size_t, c_void_p]),
    "h2o_update_scores": (c_int32, [POINTER(Dims), POINTER(CacheStruct), c_void_p, c_void_p]),
    "h2o_evict_and_insert": (c_int32, [POINTER(Dims), POINTER(CacheStruct), c_int64, c_int32,
                                       c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_size_t, c_void_p]),
    "h2o_update_evict_and_insert": (c_int32, [POINTER(Dims), POINTER(CacheStruct), c_void_p,
                                              c_int64, c_int32, c_int32, c_void_p, c_void_p,
                                              c_void_p, c_void_p, c_void_p]),
    "h2o_evict_and_insert_lastrec": (c_int32, [POINTER(Dims), POINTER(CacheStruct), c_int64,
                                               c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                               c_void_p]),
    "h2o_chunk_step": (c_int32, [POINTER(Dims), POINTER(CacheStruct), c_int64, c_int32, c_float,
                                 c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "h2o_select_slots": (c_int32, [POINTER(Dims), POINTER(CacheStruct), c_int64, c_int32,
                                   c_int32, c_void_p, c_void_p]),
    "h2o_buffer_attn": (c_int32, [POINTER(Dims), POINTER(CacheStruct), c_int64, c_int32, c_float,
                                  c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "h2o_insert": (c_int32, [POINTER(Dims), POINTER(CacheStruct), c_int64, c_int32, c_void_p,
                             c_void_p, c_void_p, c_void_p, c_void_p]),
    "h2o_backward_workspace_bytes": (c_size_t, [POINTER(Dims), c_int32]),
    "h2o_chunk_attn_backward": (c_int32, [POINTER(Dims), POINTER(CacheStruct), c_int64, c_int32,
                                          c_float] + [c_void_p] * 12 + [c_size_t, c_void_p]),
    "h2o_noalloc_scratch_bytes": (c_size_t, []),
    "h2o_chunk_attn_noalloc": (c_int32, [POINTER(Dims), POINTER(CacheStruct), c_int64, c_int32,
                                         c_float, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_void_p]),
    "h2o_last_error": (c_char_p, []),
    "h2o_abi_version": (c_int32, []),
    "h2o_kernel_timer_start": (c_int32, [c_int32, c_int32]),
    "h2o_kernel_timer_stop": (c_int32, [c_int32, POINTER(c_double), POINTER(c_int64)]),
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"libh2o.so not found at {path}; build it with "
                          "`python h2o_sparse_attention_amd/build.py`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
        EXPORTS[name] = fn
    return lib


lib = load()


class H2OError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def check(status: int) -> None:
    if status != H2O_OK:
        raise H2OError(status, lib.h2o_last_error().decode())
