"""ctypes loader of libmxfp4moe.so with the argument types of every C entry point.

The library is required: importing the binding without it raises, there is no fallback path.
"""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MXFP4MOE_LIB", os.path.join(_PKG, "libmxfp4moe.so"))

c_i32, c_i64, c_u32, c_sz, c_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_void_p


class MoeDims(ctypes.Structure):
    _fields_ = [("E", c_i32), ("H", c_i32), ("I", c_i32), ("has_bias", c_i32)]


_SIGS = {
    "mxfp4_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "mxfp4_version": (c_u32, []),
    "mxfp4_quantize": (ctypes.c_int, [c_p, c_i64, c_i64, c_i64, c_p, c_p, c_p, c_p]),
    "mxfp4_tiled_scale_bytes": (c_sz, [c_i64, c_i64]),
    "nvfp4_quantize": (ctypes.c_int, [c_p, c_i64, c_i64, c_i64, ctypes.c_float, c_p, c_p, c_p, c_p]),
    "nvfp4_tiled_scale_bytes": (c_sz, [c_i64, c_i64]),
    "mxfp4_repack_bytes": (c_sz, [ctypes.POINTER(MoeDims), c_u32]),
    "mxfp4_repack_offsets": (ctypes.c_int, [ctypes.POINTER(MoeDims), c_u32, ctypes.POINTER(c_sz)]),
    "mxfp4_repack_weights": (ctypes.c_int, [ctypes.POINTER(MoeDims), c_p, c_p, c_p, c_p, c_p, c_p, c_i32, c_u32, c_p,
                                            c_sz, c_p]),
    "mxfp4_unpack_weights": (ctypes.c_int, [ctypes.POINTER(MoeDims), c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p]),
    "mxfp4_check_packed": (ctypes.c_int, [ctypes.POINTER(MoeDims), c_p, c_p]),
    "mxfp4_linear_pack_bytes": (c_sz, [c_i64, c_i64, c_i32]),
    "mxfp4_linear_pack": (ctypes.c_int, [c_i64, c_i64, c_p, c_p, c_p, c_i32, c_p, c_sz, c_p]),
    "mxfp4_linear_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64]),
    "mxfp4_linear_forward": (ctypes.c_int, [c_p, c_i64, c_i64, c_i32, c_p, c_i64, c_i64, c_p, c_p, c_sz, c_p]),
    "moe_mxfp4_route_workspace_bytes": (c_sz, [c_i64, c_i32, c_i32]),
    "moe_mxfp4_route": (ctypes.c_int, [c_p, c_i64, c_i32, c_i32, c_i32, c_p, c_p, c_p, c_p, c_p, c_sz, c_p]),
    "moe_mxfp4_workspace_bytes": (c_sz, [ctypes.POINTER(MoeDims), c_i64, c_i32]),
    "moe_mxfp4_forward": (ctypes.c_int, [ctypes.POINTER(MoeDims), c_p, c_p, c_i64, c_i64, c_p, c_i32, c_i32, c_p, c_p,
                                         c_p, c_p, c_sz, c_p]),
    "moe_mxfp4_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(MoeDims), c_p, c_p, c_i64, c_i64, c_p, c_i32, c_i32,
                                                 c_p, c_p, c_p, c_p]),
    "moe_mxfp4_forward_act": (ctypes.c_int, [ctypes.POINTER(MoeDims), c_i32, c_p, c_p, c_i64, c_i64, c_p, c_i32,
                                             c_i32, c_p, c_p, c_p, c_p, c_sz, c_p]),
    "moe_mxfp4_forward_profiled": (ctypes.c_int, [ctypes.POINTER(MoeDims), c_i32, c_p, c_p, c_i64, c_i64, c_p, c_i32,
                                                  c_i32, c_p, c_p, c_p, c_p, c_sz, c_p, ctypes.POINTER(c_p), c_i32]),
}

EXPORTED = tuple(_SIGS)

_lib = None


def lib():
    """The loaded library (loaded on first use).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmxfp4moe.so not found at {LIB_PATH}; run __graft_entry__.build() "
                               "(or python mixed_precision_moe_amd/build_lib.py) first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class Mxfp4Error(RuntimeError):
    def __init__(self, fn, status):
        msg = lib().mxfp4_status_str(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def check(fn, status):
    if status != 0:
        raise Mxfp4Error(fn, status)
