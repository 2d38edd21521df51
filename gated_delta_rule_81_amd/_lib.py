"""ctypes loader for ``libkda.so`` (the C ABI of include/kda.h).

The library is built in-tree by ``python -m gated_delta_rule_81_amd.build``.
There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_OK = 0
KDA_DTYPE_F32 = 0
KDA_DTYPE_BF16 = 1
KDA_SCRATCH_BYTES = 64 << 20  # include/kda.h: fixed scratch of the no-allocation entry point

STATUS = {
    0: "KDA_OK", -1: "KDA_ERR_NULL", -2: "KDA_ERR_SHAPE", -3: "KDA_ERR_UNSUPPORTED",
    -4: "KDA_ERR_ALIGN", -5: "KDA_ERR_ALIAS", -6: "KDA_ERR_DEVICE", -7: "KDA_ERR_LAUNCH",
    -8: "KDA_ERR_SCRATCH",
}

# Exported symbols and their C signatures, in include/kda.h order.
_vp, _fp, _i32, _i64 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
SIGNATURES = {
    "kda_chunk_fwd": ([_vp, _vp, _vp, _fp, _fp, _fp, _vp, _vp, _fp,
                       _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp], ctypes.c_int),
    "kda_chunk_fwd_snapshots": ([_vp, _vp, _vp, _fp, _fp, _fp, _vp, _vp, _fp, _fp,
                                 _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                 _vp], ctypes.c_int),
    "kda_chunk_fwd_scalar_gate": ([_vp, _vp, _vp, _fp, _fp, _fp, _vp, _vp, _fp,
                                   _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp], ctypes.c_int),
    "kda_chunk_fwd_segmented": ([_vp, _vp, _vp, _fp, _fp, _fp, _vp, _fp,
                                 _i32, _i32, _i32, _i32, _i32, _i32, _vp, _i64, _vp],
                                ctypes.c_int),
    "kda_chunk_fwd_segmented_workspace_size": ([_i32, _i32, _i32, _i32], _i64),
    "kda_chunk_fwd_segmented_noalloc": ([_vp, _vp, _vp, _fp, _fp, _fp, _vp, _fp,
                                         _i32, _i32, _i32, _i32, _i32, _i32, _vp],
                                        ctypes.c_int),
    "kda_chunk_bwd": ([_vp, _vp, _vp, _fp, _fp, _fp, _vp, _vp, _fp, _vp, _vp, _vp, _fp, _fp,
                       _fp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _i64, _vp],
                      ctypes.c_int),
    "kda_chunk_bwd_workspace_size": ([_i32, _i32, _i32, _i32], _i64),
    "kda_decode_step_scalar_gate": ([_vp, _vp, _vp, _fp, _fp, _fp, _vp,
                                     _i32, _i32, _i32, _i32, _i32, _vp], ctypes.c_int),
    "kda_decode_step": ([_vp, _vp, _vp, _fp, _fp, _fp, _vp,
                         _i32, _i32, _i32, _i32, _i32, _vp], ctypes.c_int),
    "kda_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "kda_abi_version": ([], ctypes.c_int),
}

_lib = None


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().kda_status_string(status).decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg})")


def lib():
    """Load ``libkda.so`` once.  torch is imported first so that the library
    binds to the HIP runtime torch already loaded (both carry the soname
    libamdhip64.so.7); streams and pointers are then shared with torch."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m gated_delta_rule_81_amd.build`")
        import torch  # noqa: F401
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def check(status: int, where: str) -> None:
    if status != KDA_OK:
        raise KdaError(status, where)
