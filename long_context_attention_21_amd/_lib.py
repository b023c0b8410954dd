"""ctypes loader for libcsa_mi355x.so (the C ABI of include/csa.h).

There is no fallback: if the library is missing or cannot be loaded, every
call raises.  Build it with ``python -m long_context_attention_21_amd.build``.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa_mi355x.so")

CSA_OK = 0
CSA_INVALID_ARG = -1
CSA_UNSUPPORTED = -2
CSA_WORKSPACE_TOO_SMALL = -3
CSA_HIP_ERROR = -4

FMT_BF16 = 0
FMT_MXFP4 = 1
FMT_FP8_ROPE_BF16 = 2
FMT_NVFP4 = 3
FMT_FP8 = 4
FMT_BF16_ROPED = 5

EXPORTS = ("csa_compress", "csa_cache_append", "csa_index_topk", "csa_index_topk_workspace_bytes",
           "csa_index_topk_noalloc",
           "csa_attend", "csa_attend_workspace_bytes", "csa_index_attend", "hca_attend", "csa_project_in",
           "csa_project_qidx", "csa_project_out", "csa_rope_rows", "csa_last_error", "csa_version")


class CsaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("status %d: %s" % (status, msg))
        self.status = status


_lib = None


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("HIP library %s is not built (python -m long_context_attention_21_amd.build)"
                           % LIB_PATH)
    L = C.CDLL(LIB_PATH)
    P, i32, i64, f32, sz = C.c_void_p, C.c_int, C.c_int64, C.c_float, C.c_size_t
    L.csa_compress.argtypes = [P, P, P, P, P, P, P, i32, i32, i64, i32, i32, i32, i32, i32, f32,
                               P, P, P, i32, P, P, i32, P]
    L.csa_cache_append.argtypes = [P, P, P, i32, i64, P, P, P, P, P, i32, P, i32, i32, i32, f32, P, P, P, i32,
                                   P, P, i32, i32, P]
    L.csa_index_topk.argtypes = [P, P, P, P, P, i32, i32, i32, i64, i32, i32, i32, i32, i32, P, P,
                                 sz, P, P]
    L.csa_index_topk_noalloc.argtypes = [P, P, P, P, P, i32, i32, i32, i64, i32, i32, i32, i32, i32, P, P, P]
    L.csa_index_topk_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i32]
    L.csa_index_topk_workspace_bytes.restype = sz
    L.csa_attend.argtypes = [P, i32, i32, i64, i32, i32, P, P, P, i32, i32, i32, P, i32, P, i64, i32,
                             i32, i32, P, P, i32, f32, P, P, sz, P]
    L.csa_index_attend.argtypes = [P, P, P, P, P, i32, i32, i32, i32, P, P,
                                   P, i32, i32, P, P, P, i32, P, i64, i32, i32, i32, P, P, i32, f32, P,
                                   i32, i32, i64, i32, i32, i32, P, P, P]
    L.csa_attend_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.csa_attend_workspace_bytes.restype = sz
    L.hca_attend.argtypes = [P, i32, i32, i64, i32, i32, P, i32, i32, P, i64, i32, i32, i32, P, i32, f32,
                             P, P]
    L.csa_rope_rows.argtypes = [P, i32, i32, i64, i32, f32, P, P]
    L.csa_project_in.argtypes = [P, i32, i32, P, i32, i32, i32, i32, i32, i32, P, i32, P, P, P, P, P, P, P, P, P]
    L.csa_project_qidx.argtypes = [P, i32, i32, P, i32, P, P, P, P]
    L.csa_project_out.argtypes = [P, i32, i32, i32, i32, P, i32, P, P]
    for f in ("csa_compress", "csa_cache_append", "csa_index_topk", "csa_index_topk_noalloc", "csa_attend",
              "csa_index_attend",
              "hca_attend", "csa_project_in", "csa_project_qidx", "csa_project_out", "csa_rope_rows",
              "csa_version"):
        getattr(L, f).restype = i32
    L.csa_last_error.restype = C.c_char_p
    L.csa_last_error.argtypes = []
    _lib = L
    return L


def check(status):
    if status != CSA_OK:
        raise CsaError(status, lib().csa_last_error().decode())
    return status
