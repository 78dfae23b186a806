"""ctypes loader for libcce.so and the C ABI's prototypes (include/cce.h).

Loading fails loudly if the library has not been built: there is no
fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcce.so")

CCE_OK, CCE_EINVAL, CCE_EUNSUPPORTED, CCE_EWORKSPACE, CCE_EHIP = range(5)
CCE_F32, CCE_BF16 = 0, 1
CCE_MAX_RANKS = 64
CCE_FLAG_SERIAL = 0x1
CCE_FLAG_GELU = 0x2
CCE_FLAG_COPY_DMA = 0x4
CCE_FLAG_FUSED_PERMUTE = 0x8
CCE_FLAG_BIDIRECTIONAL = 0x10
CCE_FLAG_FINE_GRAINED = 0x20
CCE_FLAG_ONE_CHAIN = 0x40
CCE_NOALLOC_SCRATCH_BYTES = 64 << 20

AG_MODES = {"lhs_rows": 0, "rhs_cols": 1, "lhs_cols": 2, "rhs_rows": 3, "lhs_batch": 4}
RS_MODES = {"slice_lhs_rows": 0, "slice_rhs_cols": 1}


class cce_mat(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("ld", ctypes.c_int64)]


class cce_prof_record(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("iter", ctypes.c_int32), ("ms", ctypes.c_float),
                ("flops", ctypes.c_double), ("bytes", ctypes.c_double)]


class CceError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func}: status {status} ({detail})")


_lib = None

_P = ctypes.c_void_p
_PP = ctypes.POINTER(ctypes.c_void_p)
_I = ctypes.c_int
_U32 = ctypes.c_uint32
_U64 = ctypes.c_uint64
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

PROTOTYPES = {
    "cce_status_string": (ctypes.c_char_p, [_I]),
    "cce_last_error": (ctypes.c_char_p, []),
    "cce_version": (ctypes.c_char_p, []),
    "cce_ctx_create": (_I, [_I, ctypes.POINTER(_P)]),
    "cce_ctx_destroy": (_I, [_P]),
    "cce_ctx_set_profiling": (_I, [_P, _I]),
    "cce_ctx_read_profile": (_I, [_P, _I, ctypes.POINTER(cce_prof_record), ctypes.POINTER(_I)]),
    "cce_ctx_check_signals": (_I, [_P, _P]),
    "cce_ctx_set_copy_stream": (_I, [_P, _P]),
    "cce_debug_signal_giveup": (_I, [_I]),
    "cce_shard_schedule": (_I, [_I, _I, ctypes.POINTER(ctypes.c_int32)]),
    "cce_looped_allgather_einsum_workspace": (_I, [_I, _I, _I, _I, cce_mat, cce_mat,
                                                   ctypes.POINTER(_SZ)]),
    "cce_looped_allgather_einsum": (_I, [_P, _I, _I, _I, _I, _PP, cce_mat, _PP, cce_mat, _PP,
                                         cce_mat, _P, _SZ, _U32, _P]),
    "cce_looped_einsum_reducescatter_workspace": (_I, [_I, _I, _I, cce_mat, ctypes.POINTER(_SZ)]),
    "cce_looped_einsum_reducescatter": (_I, [_P, _I, _I, _I, _I, _I, _PP, cce_mat, _PP, cce_mat,
                                             _PP, cce_mat, _P, _SZ, _U32, _P]),
    "cce_looped_einsum_reducescatter_epilogue": (_I, [_P, _I, _I, _I, _I, _PP, cce_mat, _PP,
                                                      cce_mat, _P, _PP, _I64, ctypes.c_double,
                                                      _U64, _U64, ctypes.POINTER(ctypes.c_int64),
                                                      _I64, _I64, _PP, cce_mat, _P, _SZ, _U32,
                                                      _P]),
    "cce_looped_einsum_reducescatter_epilogue_noalloc": (_I, [_P, _I, _I, _I, _I, _PP, cce_mat,
                                                              _PP, cce_mat, _P, _PP, _I64,
                                                              ctypes.c_double, _U64, _U64,
                                                              ctypes.POINTER(ctypes.c_int64),
                                                              _I64, _I64, _PP, cce_mat, _U32,
                                                              _P]),
    "cce_grouped_gemm": (_I, [_P, _I, _I, _I, _PP, cce_mat, _PP, cce_mat, _PP, cce_mat, _U32, _P]),
    "cce_fused_reduce_epilogue": (_I, [_P, _I, _I, _PP, cce_mat, _P, _I, _P, _I, _I64,
                                       ctypes.c_double, _U64, _U64, _I64, _I64, _I64, _P, _I,
                                       _I64, _P, _U32, _P]),
    "cce_fused_reduce_epilogue_batched": (_I, [_P, _I, _I, _I, _PP, cce_mat, _P, _I, _PP, _I,
                                               _I64, ctypes.c_double, _U64, _U64,
                                               ctypes.POINTER(ctypes.c_int64), _I64, _I64, _PP,
                                               _I, _I64, _PP, _U32, _P]),
    "cce_fused_allreduce_epilogue": (_I, [_P, _I, _I, _PP, cce_mat, _P, _I, _P, _I, _I64,
                                          ctypes.c_double, _U64, _U64, _I64, _I64, _I64, _PP, _I,
                                          _I64, _P, _U32, _P]),
    "cce_overlap_beneficial": (_I, [ctypes.c_double] * 4),
    "cce_overlap_choose": (_I, [ctypes.c_double] * 5),
    "cce_describe_plan": (_I, [_I, _I, _I, _I, _U32, ctypes.c_char_p, _SZ, ctypes.POINTER(_SZ)]),
    "cce_debug_fail_op": (_I, [_I]),
}


def lib():
    """Load libcce.so once.  torch is imported first so that the library
    binds to the HIP runtime torch already loaded."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m collective_overlap_amd.build` "
            "(there is no fallback implementation)")
    import torch  # noqa: F401  (loads torch's libamdhip64 first)
    L = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in PROTOTYPES.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def check(status: int, func: str):
    if status != CCE_OK:
        L = lib()
        raise CceError(status, func, L.cce_last_error().decode())


def ptr_array(ptrs) -> ctypes.Array:
    arr = (ctypes.c_void_p * max(1, len(ptrs)))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return arr
