"""ctypes loader and signatures of libsas.so (the C ABI declared in include/sas.h).

Loading fails loudly when the library has not been built: there is no other
implementation behind these entry points.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsas.so")

SAS_OK, SAS_ERR_NULL, SAS_ERR_SHAPE, SAS_ERR_UNSUPPORTED, SAS_ERR_WORKSPACE, SAS_ERR_HIP = 0, -1, -2, -3, -4, -5
SAS_F32, SAS_BF16 = 0, 1
SAS_SEL_GROUP, SAS_SEL_HEAD = 0, 1
SAS_REPS_POOLED, SAS_REPS_GIST = 0, 1
SAS_MAX_BATCH = 64
SAS_DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20

STATUS_NAMES = {0: "SAS_OK", -1: "SAS_ERR_NULL", -2: "SAS_ERR_SHAPE", -3: "SAS_ERR_UNSUPPORTED",
                -4: "SAS_ERR_WORKSPACE", -5: "SAS_ERR_HIP"}

EXPORTED = ("sas_num_qblocks", "sas_required_kcap", "sas_block_reps", "sas_block_reps_update",
            "sas_block_scores_workspace",
            "sas_block_scores", "sas_topk_select", "sas_select_decode_workspace", "sas_select_decode",
            "sas_sparse_prefill", "sas_sparse_decode_workspace", "sas_sparse_decode", "sas_hssa_select_workspace",
            "sas_hssa_select_decode", "sas_hssa_decode_workspace", "sas_hssa_decode", "sas_block_reps_paged",
            "sas_sparse_decode_paged", "sas_sparse_prefill_paged", "sas_sparse_prefill_backward_workspace",
            "sas_sparse_prefill_backward", "sas_sparse_prefill_lse", "sas_sparse_decode_noalloc", "sas_last_error")


class Problem(C.Structure):
    _fields_ = [("batch", C.c_int32), ("hq", C.c_int32), ("hkv", C.c_int32), ("head_dim", C.c_int32),
                ("block", C.c_int32), ("dtype", C.c_int32), ("max_len", C.c_int32),
                ("seq_lens", C.POINTER(C.c_int32)), ("seq_lens_device", C.c_int32)]


class Budget(C.Structure):
    _fields_ = [("k_fixed", C.c_int32), ("frac_num", C.c_int32), ("frac_den", C.c_int32),
                ("count_current", C.c_int32), ("force_sink", C.c_int32), ("gate", C.c_int32),
                ("coverage", C.c_float), ("shared_heads", C.c_int32), ("sqrt_num", C.c_int32),
                ("sqrt_den", C.c_int32)]


_P = C.POINTER(Problem)
_B = C.POINTER(Budget)
_I64_3 = C.POINTER(C.c_int64)
_VP = C.c_void_p
_I32P = C.c_void_p

_SIGS = {
    "sas_num_qblocks": (C.c_int32, [C.c_int32, C.c_int32]),
    "sas_required_kcap": (C.c_int32, [_P, C.c_int32, C.POINTER(C.c_int32), _B]),
    "sas_block_reps": (C.c_int, [_P, _VP, _I64_3, _VP, _I64_3, _VP]),
    "sas_block_reps_update": (C.c_int, [_P, _VP, _I64_3, _VP, _I64_3, C.POINTER(C.c_int32), _VP]),
    "sas_block_scores_workspace": (C.c_size_t, [_P, C.c_int32, C.c_int32]),
    "sas_block_scores": (C.c_int, [_P, _VP, _I64_3, C.c_int32, C.POINTER(C.c_int32), _VP, C.c_int32, _I64_3,
                                   C.c_int32, C.c_float, _VP, C.c_int64, _VP, C.c_size_t, _VP]),
    "sas_topk_select": (C.c_int, [_P, _VP, C.c_int64, C.c_int32, C.POINTER(C.c_int32), C.c_int32, _B, C.c_int32,
                                  _VP, _VP, _VP, _VP]),
    "sas_select_decode_workspace": (C.c_size_t, [_P]),
    "sas_select_decode": (C.c_int, [_P, _VP, _I64_3, _VP, C.c_int32, _I64_3, C.c_int32, C.c_float, _B, C.c_int32,
                                    _VP, C.c_int64, _VP, _VP, _VP, _VP, C.c_size_t, _VP]),
    "sas_sparse_prefill": (C.c_int, [_P, _VP, _I64_3, _VP, _VP, _I64_3, C.c_int32, C.POINTER(C.c_int32), C.c_int32,
                                     _VP, _VP, _VP, C.c_int32, C.c_float, _VP, _I64_3, _VP]),
    "sas_sparse_decode_workspace": (C.c_size_t, [_P, C.c_int32, C.c_int32, C.c_int32]),
    "sas_sparse_decode": (C.c_int, [_P, _VP, _I64_3, _VP, _VP, _I64_3, _VP, _VP, _I64_3, C.c_int32, _VP, _VP, _VP,
                                    C.c_int32, C.c_float, _VP, _I64_3, _VP, C.c_size_t, _VP]),
    "sas_sparse_decode_noalloc": (C.c_int, [_P, _VP, _I64_3, _VP, _VP, _I64_3, _VP, _VP, _I64_3, C.c_int32, _VP,
                                            _VP, _VP, C.c_int32, C.c_float, _VP, _I64_3, _VP]),
    "sas_hssa_select_workspace": (C.c_size_t, [_P, C.c_int32, C.c_int32, C.c_int32]),
    "sas_hssa_select_decode": (C.c_int, [_P, _VP, _I64_3, _VP, _I64_3, _VP, _I64_3, C.c_int32, C.c_int32, C.c_int32,
                                         C.c_int32, C.c_float, C.c_int32, C.c_int32, _VP, _VP, _VP, _VP, _VP,
                                         C.c_size_t, _VP]),
    "sas_hssa_decode_workspace": (C.c_size_t, [_P, C.c_int32, C.c_int32, C.c_int32, C.c_int32]),
    "sas_hssa_decode": (C.c_int, [_P, _VP, _I64_3, _VP, _VP, _I64_3, _VP, _VP, _I64_3, _VP, _VP, _I64_3, C.c_int32,
                                  C.c_int32, _VP, _VP, C.c_int32, _VP, C.c_int32, C.c_float, _VP, _I64_3, _VP,
                                  C.c_size_t, _VP]),
    "sas_block_reps_paged": (C.c_int, [_P, _VP, _I64_3, _VP, C.c_int64, _VP, _I64_3, C.POINTER(C.c_int32), _VP]),
    "sas_sparse_decode_paged": (C.c_int, [_P, _VP, _I64_3, _VP, _VP, _I64_3, _VP, C.c_int64, C.c_int32, _VP, _VP,
                                          _VP, C.c_int32, C.c_float, _VP, _I64_3, _VP, C.c_size_t, _VP]),
    "sas_sparse_prefill_paged": (C.c_int, [_P, _VP, _I64_3, _VP, _VP, _I64_3, _VP, C.c_int64, C.c_int32,
                                           C.POINTER(C.c_int32), C.c_int32, _VP, _VP, _VP, C.c_int32, C.c_float, _VP,
                                           _I64_3, _VP]),
    "sas_sparse_prefill_backward_workspace": (C.c_size_t, [_P, C.c_int32, C.c_int32, C.c_int32, C.c_int32]),
    "sas_sparse_prefill_backward": (C.c_int, [_P, _VP, _I64_3, _VP, _VP, _I64_3, C.c_int32, C.POINTER(C.c_int32),
                                              C.c_int32, _VP, _VP, _VP, C.c_int32, C.c_float, _VP, _VP, _I64_3, _VP,
                                              _VP, _I64_3, _VP, _VP, _I64_3, _VP, _VP, _VP, _I64_3, _VP, C.c_size_t,
                                              _VP]),
    "sas_sparse_prefill_lse": (C.c_int, [_P, _VP, _I64_3, _VP, _VP, _I64_3, C.c_int32, C.POINTER(C.c_int32),
                                         C.c_int32, _VP, _VP, _VP, C.c_int32, C.c_float, _VP, _I64_3, _VP, _VP]),
    "sas_last_error": (C.c_char_p, []),
}

_lib = None


def load() -> C.CDLL:
    """Load libsas.so (once).  Raises if it is missing: build it with build_lib.build()."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m top_block_sparse_gist_amd.build_lib`")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class SasError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != SAS_OK:
        msg = load().sas_last_error().decode(errors="replace")
        raise SasError(status, where, msg)


def i64x(vals) -> C.Array:
    arr = (C.c_int64 * len(vals))(*[int(v) for v in vals])
    return arr


def i32x(vals) -> C.Array:
    return (C.c_int32 * len(vals))(*[int(v) for v in vals])
