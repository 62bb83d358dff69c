"""ctypes binding of libswa.so (argument marshalling only).

Every function here forwards to the C ABI declared in include/swa.h under the
same name.  There is no other implementation: if libswa.so is missing the
import of the library raises, on CPU and GPU machines alike.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libswa.so")

SWA_OK = 0
SWA_ERR_INVALID_ARG = -1
SWA_ERR_UNSUPPORTED = -2
SWA_ERR_HIP = -3
SWA_F32 = 0
SWA_BF16 = 1

# every symbol include/swa.h declares
EXPORTS = (
    "swa_prefill_workspace_bytes", "swa_rope_keys", "swa_prefill", "swa_cache_append", "swa_prefill_append",
    "swa_decode_workspace_bytes",
    "swa_decode", "swa_decode_step", "swa_decode_step_noalloc", "swa_decode_default_splits", "swa_prefill_dilated_workspace_bytes",
    "swa_prefill_dilated", "swa_prefill_global_workspace_bytes", "swa_prefill_global", "swa_backward_workspace_bytes", "swa_backward", "swa_status_str", "swa_last_error",
    "swa_abi_version",
)


class SwaDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32),
        ("s", ctypes.c_int32), ("r", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float), ("rope_base", ctypes.c_float),
    ]


class SwaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s (status %d)" % (message, status))
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libswa.so (built in-tree by sliding_window_attention_sink_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libswa.so is not built (%s); run python -m sliding_window_attention_sink_amd.build"
                          % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    dp = ctypes.POINTER(SwaDesc)
    lib.swa_prefill_workspace_bytes.argtypes = [dp, i64]
    lib.swa_prefill_workspace_bytes.restype = sz
    lib.swa_rope_keys.argtypes = [dp, vp, i64, i64, vp, vp]
    lib.swa_rope_keys.restype = ctypes.c_int
    lib.swa_prefill.argtypes = [dp, vp, vp, vp, vp, i64, vp, vp, i64, vp, sz, vp]
    lib.swa_prefill.restype = ctypes.c_int
    lib.swa_cache_append.argtypes = [dp, vp, vp, i64, i64, vp, vp, vp]
    lib.swa_cache_append.restype = ctypes.c_int
    lib.swa_prefill_append.argtypes = [dp, vp, vp, vp, vp, i64, vp, vp, i64, vp, vp, vp]
    lib.swa_prefill_append.restype = ctypes.c_int
    lib.swa_decode_workspace_bytes.argtypes = [dp, i32]
    lib.swa_decode_workspace_bytes.restype = sz
    lib.swa_decode.argtypes = [dp, vp, vp, vp, i64, vp, i32, vp, sz, vp]
    lib.swa_decode.restype = ctypes.c_int
    lib.swa_decode_step.argtypes = [dp, vp, vp, vp, vp, vp, i64, vp, i32, vp, sz, vp]
    lib.swa_decode_step.restype = ctypes.c_int
    lib.swa_decode_step_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, i64, vp, i32, vp]
    lib.swa_decode_step_noalloc.restype = ctypes.c_int
    lib.swa_prefill_dilated_workspace_bytes.argtypes = [dp, i64, i32]
    lib.swa_prefill_dilated_workspace_bytes.restype = sz
    lib.swa_prefill_dilated.argtypes = [dp, i32, vp, vp, vp, vp, i64, vp, sz, vp]
    lib.swa_prefill_dilated.restype = ctypes.c_int
    lib.swa_prefill_global_workspace_bytes.argtypes = [dp, i64, i32]
    lib.swa_prefill_global_workspace_bytes.restype = sz
    lib.swa_prefill_global.argtypes = [dp, vp, vp, vp, vp, i64, ctypes.POINTER(ctypes.c_int32), i32, vp, sz, vp]
    lib.swa_prefill_global.restype = ctypes.c_int
    lib.swa_backward_workspace_bytes.argtypes = [dp, i64]
    lib.swa_backward_workspace_bytes.restype = sz
    lib.swa_backward.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, sz, vp]
    lib.swa_backward.restype = ctypes.c_int
    lib.swa_decode_default_splits.argtypes = [dp]
    lib.swa_decode_default_splits.restype = i32
    lib.swa_status_str.argtypes = [ctypes.c_int]
    lib.swa_status_str.restype = ctypes.c_char_p
    lib.swa_last_error.argtypes = []
    lib.swa_last_error.restype = ctypes.c_char_p
    lib.swa_abi_version.argtypes = []
    lib.swa_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != SWA_OK:
        lib = load()
        raise SwaError(status, lib.swa_last_error().decode() or lib.swa_status_str(status).decode())


# ---- same-name wrappers over raw addresses (ints or None) -----------------
def swa_prefill_workspace_bytes(desc: SwaDesc, L: int) -> int:
    return load().swa_prefill_workspace_bytes(ctypes.byref(desc), L)


def swa_rope_keys(desc, k, n, pos0, k_rot, stream) -> int:
    return load().swa_rope_keys(ctypes.byref(desc), k, n, pos0, k_rot, stream)


def swa_prefill(desc, q, k, v, o, L, k_cache, v_cache, pos0, workspace, workspace_bytes, stream) -> int:
    return load().swa_prefill(ctypes.byref(desc), q, k, v, o, L, k_cache, v_cache, pos0, workspace,
                              workspace_bytes, stream)


def swa_cache_append(desc, k_new, v_new, n, pos0, k_cache, v_cache, stream) -> int:
    return load().swa_cache_append(ctypes.byref(desc), k_new, v_new, n, pos0, k_cache, v_cache, stream)


def swa_prefill_append(desc, q, k, v, o, L, k_cache, v_cache, pos0, k_next, v_next, stream) -> int:
    return load().swa_prefill_append(ctypes.byref(desc), q, k, v, o, L, k_cache, v_cache, pos0, k_next, v_next,
                                     stream)


def swa_decode_workspace_bytes(desc: SwaDesc, n_split: int) -> int:
    return load().swa_decode_workspace_bytes(ctypes.byref(desc), n_split)


def swa_decode_default_splits(desc: SwaDesc) -> int:
    return load().swa_decode_default_splits(ctypes.byref(desc))


def swa_decode(desc, q, k_cache, v_cache, T, o, n_split, workspace, workspace_bytes, stream) -> int:
    return load().swa_decode(ctypes.byref(desc), q, k_cache, v_cache, T, o, n_split, workspace,
                             workspace_bytes, stream)


def swa_decode_step(desc, q, k_new, v_new, k_cache, v_cache, T, o, n_split, workspace, workspace_bytes,
                    stream) -> int:
    return load().swa_decode_step(ctypes.byref(desc), q, k_new, v_new, k_cache, v_cache, T, o, n_split, workspace,
                                  workspace_bytes, stream)


def swa_decode_step_noalloc(desc, q, k_new, v_new, k_cache, v_cache, T, o, n_split, stream) -> int:
    return load().swa_decode_step_noalloc(ctypes.byref(desc), q, k_new, v_new, k_cache, v_cache, T, o, n_split,
                                          stream)


NOALLOC_SCRATCH_BYTES = 8 << 20   # SWA_NOALLOC_SCRATCH_BYTES of include/swa.h


def swa_prefill_dilated_workspace_bytes(desc: SwaDesc, L: int, dilation: int) -> int:
    return load().swa_prefill_dilated_workspace_bytes(ctypes.byref(desc), L, dilation)


def swa_prefill_dilated(desc, dilation, q, k, v, o, L, workspace, workspace_bytes, stream) -> int:
    return load().swa_prefill_dilated(ctypes.byref(desc), dilation, q, k, v, o, L, workspace, workspace_bytes, stream)


MAX_GLOBALS = 64   # SWA_MAX_GLOBALS of include/swa.h


def swa_prefill_global_workspace_bytes(desc: SwaDesc, L: int, ng: int) -> int:
    return load().swa_prefill_global_workspace_bytes(ctypes.byref(desc), L, ng)


def swa_prefill_global(desc, q, k, v, o, L, globals_, ng, workspace, workspace_bytes, stream) -> int:
    """globals_: a sequence of host positions (ints) or None."""
    arr = None
    if globals_ is not None:
        arr = (ctypes.c_int32 * max(1, len(globals_)))(*[int(x) for x in globals_])
    return load().swa_prefill_global(ctypes.byref(desc), q, k, v, o, L, arr, ng, workspace, workspace_bytes, stream)


def swa_backward_workspace_bytes(desc: SwaDesc, L: int) -> int:
    return load().swa_backward_workspace_bytes(ctypes.byref(desc), L)


def swa_backward(desc, q, k, v, o, dout, dq, dk, dv, L, workspace, workspace_bytes, stream) -> int:
    return load().swa_backward(ctypes.byref(desc), q, k, v, o, dout, dq, dk, dv, L, workspace, workspace_bytes,
                               stream)


def swa_status_str(status: int) -> str:
    return load().swa_status_str(status).decode()


def swa_last_error() -> str:
    return load().swa_last_error().decode()


def swa_abi_version() -> int:
    return load().swa_abi_version()
