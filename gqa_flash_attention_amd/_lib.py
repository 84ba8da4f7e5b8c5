"""ctypes view of libgqa_attn.so, the C ABI declared in include/gqa_attn.h.

Loading fails loudly if the library has not been built: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import threading

LIB_NAME = "libgqa_attn.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

OK = 0
ERR_NULL = -1
ERR_DIM = -2
ERR_UNSUPPORTED = -3
ERR_HIP = -4
ERR_WORKSPACE = -5

_c_int = ctypes.c_int
_c_float = ctypes.c_float
_c_size_t = ctypes.c_size_t
_ptr = ctypes.c_void_p

# name -> (restype, argtypes), in the order of include/gqa_attn.h
SIGNATURES = {
    "gqa_attn_prefill": (_c_int, [_ptr, _ptr, _ptr, _ptr, _c_int, _c_int, _c_int, _c_int, _c_int,
                                  _c_float, _c_int, _ptr]),
    "gqa_attn_prefill_form": (_c_int, [_ptr, _ptr, _ptr, _ptr, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_float, _c_int, _c_int, _c_int, _ptr]),
    "gqa_attn_prefill_tiles": (_c_int, [_ptr, _ptr, _ptr, _ptr, _c_int, _c_int, _c_int, _c_int, _c_int,
                                        _c_float, _c_int, _c_int, _c_int, _c_int, _ptr]),
    "gqa_attn_prefill_plan": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int,
                                       ctypes.POINTER(_c_int), ctypes.POINTER(_c_int), ctypes.POINTER(_c_int)]),
    "gqa_attn_decode": (_c_int, [_ptr, _ptr, _ptr, _ptr, _ptr, _c_int, _c_int, _c_int, _c_int, _c_int,
                                 _c_float, _ptr]),
    "gqa_attn_decode_plan": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int,
                                      ctypes.POINTER(_c_int), ctypes.POINTER(_c_int)]),
    "gqa_attn_decode_workspace_bytes": (_c_size_t, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "gqa_attn_decode_noalloc": (_c_int, [_ptr, _ptr, _ptr, _ptr, _ptr, _c_int, _c_int, _c_int, _c_int, _c_int,
                                         _c_float, _ptr]),
    "gqa_attn_decode_ws": (_c_int, [_ptr, _ptr, _ptr, _ptr, _ptr, _c_int, _c_int, _c_int, _c_int, _c_int,
                                    _c_float, _c_int, _ptr, _c_size_t, _ptr]),
    "gqa_attn_decode_partials": (_c_int, [_ptr, _ptr, _ptr, _ptr, _c_int, _c_int, _c_int, _c_int, _c_int,
                                          _c_float, _c_int, _ptr, _c_size_t, _ptr]),
    "gqa_attn_decode_combine": (_c_int, [_ptr, _c_size_t, _ptr, _c_int, _c_int, _c_int, _c_int, _ptr]),
    "gqa_attn_probe_hbm_read": (_c_int, [_ptr, _c_size_t, _c_int, _ptr, _c_size_t, _ptr]),
    "gqa_attn_probe_mfma_bf16": (_c_int, [_c_int, ctypes.c_uint32, _c_int, _ptr, _c_size_t, _ptr,
                                          _c_size_t, _ptr]),
    "gqa_attn_strerror": (ctypes.c_char_p, [_c_int]),
    "gqa_attn_last_error": (ctypes.c_char_p, []),
    "gqa_attn_release": (None, []),
    "gqa_attn_version": (_c_int, []),
}

_lock = threading.Lock()
_lib = None


class GqaAttnError(RuntimeError):
    """A nonzero return code from the C ABI."""

    def __init__(self, code: int, where: str):
        self.code = code
        lib = get()
        msg = lib.gqa_attn_strerror(code).decode()
        if code == ERR_HIP:
            msg += ": " + lib.gqa_attn_last_error().decode()
        super().__init__(f"{where}: error {code}: {msg}")


def get(path: str | None = None) -> ctypes.CDLL:
    """The loaded library (loaded once). Raises if it is missing."""
    global _lib
    with _lock:
        if _lib is None:
            p = path or LIB_PATH
            if not os.path.exists(p):
                raise RuntimeError(
                    f"{p} is missing: build it with `python -m gqa_flash_attention_amd.build` "
                    "(there is no fallback implementation)")
            lib = ctypes.CDLL(p)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
        return _lib


def check(code: int, where: str) -> None:
    if code != OK:
        raise GqaAttnError(code, where)
