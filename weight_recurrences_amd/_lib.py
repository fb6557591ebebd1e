"""ctypes loader for ``liblinattn.so`` (the C ABI declared in include/linattn.h).

Loading fails loudly when the shared library has not been built: there is no
CPU fallback anywhere in this package.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "liblinattn.so")
HEADER = os.path.join(ROOT, "include", "linattn.h")

F32, BF16 = 0, 1
FMAP_DPFP, FMAP_POLY2 = 1, 2  # linattn_fmap_t
STATUS = {
    0: "LINATTN_OK", 1: "LINATTN_ERR_NULL", 2: "LINATTN_ERR_SHAPE", 3: "LINATTN_ERR_DTYPE",
    4: "LINATTN_ERR_UNSUPPORTED", 5: "LINATTN_ERR_ALIGN", 6: "LINATTN_ERR_ALIAS",
    7: "LINATTN_ERR_WORKSPACE", 8: "LINATTN_ERR_HIP",
}

_lock = threading.Lock()
_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t

SIGNATURES = {
    "linattn_causal_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "linattn_causal_fwd": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "linattn_causal_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "linattn_causal_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "linattn_noncausal_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "linattn_noncausal_fwd": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "linattn_noncausal_fwd_noalloc": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "linattn_decode_step": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "deltanet_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "deltanet_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "deltanet_decode_step": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "softmax_decode_step": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "linattn_fmap_dim": (_i, [_i, _i, _i]),
    "linattn_fmap_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "linattn_fmap_fwd": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i,
                              _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "linattn_status_str": (ctypes.c_char_p, [_i]),
    "linattn_abi_version": (_i, []),
}


class LinAttnError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = int(status)
        super().__init__(f"{where}: {STATUS.get(self.status, 'LINATTN_ERR_UNKNOWN')} ({self.status})")


def header_functions() -> list[str]:
    """Names of the functions include/linattn.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted({n for n in names if n.startswith(("linattn_", "deltanet_", "softmax_"))})


def load():
    """Load liblinattn.so once and attach the C signatures."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"{LIB_PATH} is missing: build the HIP library first "
                    "(python -m weight_recurrences_amd.build)")
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def check(status: int, where: str) -> None:
    if status != 0:
        raise LinAttnError(status, where)
