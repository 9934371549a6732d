"""ctypes view of the C ABI declared in include/mla.h."""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

c_int32, c_int64, c_void_p, c_size_t = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t

MLA_F32, MLA_BF16, MLA_E4M3 = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 64 << 20     # MLA_NOALLOC_SCRATCH_BYTES

STATUS = {0: "MLA_OK", -1: "MLA_ERR_NULL", -2: "MLA_ERR_SHAPE", -3: "MLA_ERR_DTYPE",
          -4: "MLA_ERR_WORKSPACE", -5: "MLA_ERR_UNSUPPORTED", -6: "MLA_ERR_HIP"}

# every symbol include/mla.h declares, with (restype, argtypes)
SIGNATURES = {
    "mla_absorb_q": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "mla_cache_append": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int64,
                                   c_void_p, c_void_p, c_void_p]),
    "mla_absorb_q_append": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_void_p, c_void_p,
                                      c_void_p]),
    "mla_kv_project_workspace_bytes": (c_size_t, [c_void_p, c_int32, c_int32]),
    "mla_kv_project_append": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_int64, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "mla_probe_stream_read": (c_int32, [c_void_p, c_size_t, c_void_p, c_void_p]),
    "mla_probe_mfma_bf16": (c_int32, [c_int32, c_int32, c_void_p, c_void_p]),
    "mla_decode_workspace_bytes": (c_size_t, [c_void_p, c_int32, c_int32]),
    "mla_decode": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                             c_int32, c_void_p, c_size_t, c_void_p, c_void_p, c_void_p]),
    "mla_decode_window": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                    c_void_p, c_int32, c_void_p, c_size_t, c_void_p, c_void_p, c_void_p]),
    "mla_decode_noalloc": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                     c_void_p, c_int32, c_void_p, c_void_p, c_void_p]),
    "mla_decode_multi_workspace_bytes": (c_size_t, [c_void_p, c_int32, c_int32, c_int32]),
    "mla_decode_multi": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                   c_void_p, c_void_p, c_int32, c_void_p, c_size_t, c_void_p, c_void_p, c_void_p]),
    "mla_up_v": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "mla_status_string": (ctypes.c_char_p, [c_int32]),
    "mla_last_hip_error": (c_int32, []),
    "mla_abi_version": (c_int32, []),
}


class Dims(ctypes.Structure):
    """Mirror of struct mla_dims (40 bytes)."""
    _fields_ = [("n_heads", c_int32), ("d_head", c_int32), ("d_latent", c_int32), ("d_rope", c_int32),
                ("block_size", c_int32), ("act_dtype", c_int32), ("kv_dtype", c_int32),
                ("softmax_scale", ctypes.c_float), ("rope_base", ctypes.c_double)]


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0):
        self.status = status
        msg = f"{where}: {STATUS.get(status, status)}"
        if hip_error:
            msg += f" (hipError {hip_error})"
        super().__init__(msg)


_LIB = None


def lib(path: str | None = None):
    """Load the built library; raises if it has not been built."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"MLA HIP library not found at {p}; build it with __graft_entry__.build()")
    L = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    if path is None:
        _LIB = L
    return L


def check(status: int, where: str):
    if status != 0:
        raise MLAError(status, where, lib().mla_last_hip_error() if status == -6 else 0)
