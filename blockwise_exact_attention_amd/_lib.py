"""ctypes loader for libattn.so: argument and return types of every C entry
point declared in include/attn.h.  Loading fails loudly when the library has
not been built; there is no fallback."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_OK = 0
ATTN_ERR_NULL = 1
ATTN_ERR_SHAPE = 2
ATTN_ERR_UNSUPPORTED = 3
ATTN_ERR_HIP = 4
ATTN_ERR_WORKSPACE = 5
ATTN_ERR_ALIAS = 6
ATTN_ERR_ALIGN = 7

ATTN_F32 = 0
ATTN_BF16 = 1

ATTN_RING_MAX_CHUNKS = 16
ATTN_BWD_STATIC_MAX_WORKSPACE = 64 << 20

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_ll = ctypes.c_longlong
_sz = ctypes.c_size_t

SIGNATURES = {
    "attn_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i,
                      _i, _i, _ll, _ll, _vp, _i]),
    "attn_fwd_acc": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i,
                          _i, _i, _ll, _ll, _vp, _i]),
    "attn_fwd_ring": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i,
                           _f, _i, _i, _i, _ll, _vp, _i]),
    "attn_fwd_kernel_name": (ctypes.c_char_p, [_i, _i, _i, _i, _i, _i, _f, _i, _i, _i, _ll,
                                               _ll, _i, _i]),
    "attn_merge": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "attn_hbm_copy": (_i, [_vp, _vp, _ll, _vp]),
    "attn_acc_init": (_i, [_vp, _vp, _i, _i, _i, _i, _vp]),
    "attn_acc_cast": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "attn_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i,
                      _i, _i, _i, _f, _i, _i, _i, _ll, _ll, _vp, _sz, _vp, _i]),
    "attn_bwd_acc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i,
                          _i, _i, _i, _f, _i, _i, _i, _ll, _ll, _vp, _sz, _vp, _i]),
    "attn_bwd_prepare_bytes": (_sz, [_i, _i, _i]),
    "attn_bwd_prepare": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _sz, _vp, _i]),
    "attn_bwd_acc_prepared": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i,
                                   _i, _i, _i, _i, _f, _i, _i, _i, _ll, _ll, _vp, _sz,
                                   _vp, _i]),
    "attn_bwd_ring": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _i, _i,
                           _i, _i, _i, _f, _i, _i, _i, _ll, _vp, _sz, _vp, _i]),
    "attn_bwd_static": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i,
                             _i, _i, _i, _f, _i, _i, _i, _ll, _ll, _vp, _i]),
    "attn_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "attn_status_string": (ctypes.c_char_p, [_i]),
}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = status_string(status) if _lib is not None else str(status)
        super().__init__(f"{fn} failed with status {status}: {msg}")


def lib():
    """The loaded libattn.so (built by blockwise_exact_attention_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m blockwise_exact_attention_amd.build` (hipcc, gfx950)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status):
    return lib().attn_status_string(int(status)).decode()


def check(fn, status):
    if status != ATTN_OK:
        raise AttnError(fn, status)
