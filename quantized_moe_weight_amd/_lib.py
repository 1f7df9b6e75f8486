"""ctypes loader for the gfx950 decode library (libpqmoe.so).

The shared library is built in-tree by :func:`quantized_moe_weight_amd.build.build`.
Importing this module never falls back to anything: a missing or unloadable
library raises immediately.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpqmoe.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "pq.h")

_c_int, _c_size, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes); every pointer is passed as void*
SIGNATURES = {
    "pq_quantize_fp8": (_c_int, [_vp, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "pq_quantize_q4": (_c_int, [_vp, _c_int, _c_int, _vp, _vp, _vp]),
    "pq_gemv_fp8_workspace": (_c_size, [_c_int, _c_int, _c_int, _c_int]),
    "pq_gemv_fp8": (_c_int, [_vp, _c_int, _c_int, _vp, _vp, _c_int, _c_int, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "pq_gemm_fp8_workspace": (_c_size, [_c_int, _c_int, _c_int, _c_int]),
    "pq_gemm_fp8": (_c_int, [_vp, _c_int, _c_int, _vp, _vp, _c_int, _c_int, _vp, _vp, _c_size, _vp]),
    "pq_gemm_fp8_prequant": (_c_int, [_vp, _vp, _c_int, _c_int, _vp, _vp, _c_int, _c_int, _vp, _vp]),
    "pq_gemv_q4_workspace": (_c_size, [_c_int, _c_int, _c_int, _c_int]),
    "pq_gemv_q4": (_c_int, [_vp, _c_int, _c_int, _vp, _vp, _c_int, _c_int, _vp, _vp, _c_size, _vp]),
    "pq_gemv_q4_group": (_c_int, [_vp, _c_int, _c_int, _vp, _vp]),
    "moe_decode_layer_workspace": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "moe_decode_layer": (_c_int, [_vp, _c_int, _c_int, _vp, _vp, _vp, _c_int, _c_int, _c_int,
                                  _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "moe_decode_layer_ex": (_c_int, [_vp, _c_int, _c_int, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int,
                                     _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _c_size, _vp]),
    "moe_decode_layer_noalloc": (_c_int, [_vp, _c_int, _c_int, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int,
                                          _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                          _vp, _vp]),
    "pq_workspace_init": (_c_int, [_vp, _c_size, _vp]),
    "pq_workspace_check": (_c_int, [_vp, _vp]),
    "pq_strerror": (ctypes.c_char_p, [_c_int]),
    "pq_last_hip_error": (_c_int, []),
    "pq_launches_per_call": (_c_int, [ctypes.c_char_p]),
    "moe_decode_layer_config": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "pq_stream_probe": (_c_int, [_vp, _c_size, _vp, _vp]),
}



class Q4Linear(ctypes.Structure):
    """pq_q4_linear of include/pq.h."""
    _fields_ = [("x", _vp), ("w", _vp), ("w_scale", _vp), ("y", _vp),
                ("K", _c_int), ("N", _c_int), ("epi", _c_int)]


_lib = None


def header_functions(path: str = HEADER) -> list[str]:
    """Names of the functions declared in include/pq.h."""
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library once and attach signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with quantized_moe_weight_amd.build.build() "
                           "(the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
