"""ctypes view of libgemma_attn.so (declarations mirror include/gemma_attn.h)."""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgemma_attn.so")

GA_BF16, GA_F32 = 0, 1
GA_CACHE_NATIVE, GA_CACHE_INT8, GA_CACHE_PREROTATED = 0, 1, 2
STATUS = {0: "GA_OK", 1: "GA_EINVAL", 2: "GA_EUNSUPPORTED", 3: "GA_EWORKSPACE", 4: "GA_EHIP"}


class GaLayer(ctypes.Structure):
    _fields_ = [
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("kv_shared", ctypes.c_int32),
        ("rope_theta", ctypes.c_float),
        ("rope_fraction", ctypes.c_float),
        ("norm_eps", ctypes.c_float),
        ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("cache_format", ctypes.c_int32),
    ]


class GemmaAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_P = ctypes.c_void_p
_I = ctypes.c_int32
_Z = ctypes.c_size_t
_LP = ctypes.POINTER(GaLayer)

SIGNATURES = {
    "gemma_attn_prefill_workspace_size": (_Z, [_LP, _I, _I]),
    "gemma_attn_prefill": (_I, [_LP, _I, _I, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _Z, _P]),
    "kv_append": (_I, [_LP, _I, _P, _P, _P, _P, _P, _P, _I, _P]),
    "gemma_attn_prefill_chunk_workspace_size": (_Z, [_LP, _I, _I, _I]),
    "gemma_attn_prefill_chunk": (_I, [_LP, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _Z, _P]),
    "gemma_attn_decode_workspace_size": (_Z, [_LP, _I, _I]),
    "gemma_attn_decode": (_I, [_LP, _I, _P, _P, _P, _P, _I, _P, _I, _P, _P, _Z, _P]),
    "gemma_attn_decode_multi_workspace_size": (_Z, [_LP, _I, _I, _I]),
    "gemma_attn_decode_multi": (_I, [_LP, _I, _I, _P, _P, _P, _P, _I, _P, _I, _P, _P, _Z, _P]),
    "gemma_attn_decode_noalloc": (_I, [_LP, _I, _P, _P, _P, _P, _I, _P, _I, _P, _P]),
    "gemma_attn_cache_bytes": (_Z, [_LP, _I, _I]),
    "gemma_attn_last_error": (ctypes.c_char_p, []),
    "gemma_attn_calibrate_mfma": (_I, [_P, _I, _I, _I, _P, _P]),
    "gemma_attn_calibrate_stream": (_I, [_P, _Z, _I, _P, _P]),
    "gemma_attn_version": (ctypes.c_char_p, []),
    "gemma_attn_profile_enable": (None, [ctypes.c_int]),
    "gemma_attn_profile_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                                ctypes.POINTER(ctypes.c_int)]),
    "gemma_attn_profile_reset": (None, []),
}

_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m global_gqa_rope_amd.build` "
                           "(the attention path runs only in the HIP library)")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def check(status: int) -> None:
    if status != 0:
        msg = load().gemma_attn_last_error().decode(errors="replace")
        raise GemmaAttnError(status, msg)
