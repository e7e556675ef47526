"""ctypes declarations of the C ABI in include/kda.h (libkda.so, built in-tree).

Loading fails loudly when the library is missing: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkda.so")

(KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, KDA_ERR_HIP,
 KDA_ERR_SCRATCH) = range(6)
KDA_F32, KDA_BF16 = 0, 1
GATES = {"standard": 0, "safe": 1, "none": 2}
KDA_GATE_PER_HEAD = 16

_c_int, _c_float, _vp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p

# name -> (restype, argtypes), in the order of include/kda.h
SIGNATURES = {
    "kda_status_string": (ctypes.c_char_p, [_c_int]),
    "kda_version": (_c_int, []),
    "kda_gate": (_c_int, [_vp, _vp, _vp, _c_int, _c_float, _c_int, _c_int, _c_int, _c_int,
                          _c_int, _vp, _vp]),
    "kda_chunk_fwd_workspace_bytes": (ctypes.c_size_t, [_c_int] * 7 + [_c_int]),
    "kda_chunk_fwd": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _vp, _vp, _vp, _c_int, _c_float, _vp,
                               _vp, _vp] + [_c_int] * 7 + [_vp, ctypes.c_size_t, _vp]),
    "kda_recurrent_step": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _vp, _vp, _vp, _c_int, _c_float,
                                    _vp, _vp] + [_c_int] * 5 + [_vp]),
    "kda_recurrent_fwd": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _vp, _vp, _vp, _c_int, _c_float,
                                   _vp, _vp, _vp] + [_c_int] * 6 + [_vp]),
    "kda_chunk_fwd_split_workspace_bytes": (ctypes.c_size_t, [_c_int] * 7),
    "kda_chunk_fwd_split": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _vp, _vp, _vp, _c_int, _c_float,
                                     _vp, _vp, _vp, _vp] + [_c_int] * 7
                            + [_vp, ctypes.c_size_t, _vp]),
    "kda_chunk_fwd_split_noalloc": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _vp, _vp, _vp, _c_int,
                                             _c_float, _vp, _vp, _vp, _vp] + [_c_int] * 7
                                    + [_vp]),
    "kda_bwd_workspace_bytes": (ctypes.c_size_t, [_c_int] * 6),
    "kda_bwd": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _vp, _vp, _vp, _c_int, _c_float, _vp,
                         _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp] + [_c_int] * 6
                + [_vp, ctypes.c_size_t, _vp]),
}

_lib = None


class KDAError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed: %s" % (fn, msg))
        self.status = status


def load(path: str = LIB_PATH):
    """Load libkda.so once (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libkda.so not found at %s: build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(fn_name: str, status: int):
    if status != KDA_OK:
        msg = load().kda_status_string(status).decode()
        raise KDAError(fn_name, status, msg)
