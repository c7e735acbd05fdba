"""ctypes loader for libmoe_mi355x.so (the C ABI in include/moe.h)."""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_mi355x.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe.h")

# constants mirrored from include/moe.h (checked against the header in the CPU tests)
MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_ERR_SCRATCH = -5
MOE_DISPATCH_NOALLOC_SCRATCH = 8 << 20
MOE_F32, MOE_BF16, MOE_E4M3 = 0, 1, 2
MOE_BWD_AU_SAVED = 1
MOE_ROUTE_LOGITS_IN = 1
MOE_FFN_UP, MOE_FFN_DOWN, MOE_FFN_ALL = 1, 2, 3
MOE_ROUTE_BLOCK = 64
MOE_FP8_TILE = 128
MOE_OP_ROUTE, MOE_OP_DISPATCH, MOE_OP_EXPERT_FFN, MOE_OP_COMBINE = 1, 2, 3, 4
MOE_OP_ROUTE_BACKWARD, MOE_OP_EXPERT_FFN_BACKWARD = 5, 6


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("G", ctypes.c_int32), ("M", ctypes.c_int32), ("k", ctypes.c_int32),
                ("group_topk", ctypes.c_int32), ("d_ff", ctypes.c_int32)]


class MoeFfnExtra(ctypes.Structure):
    """moe_ffn_extra: one more expert-FFN group with buffers of its own."""
    _fields_ = [("rows", ctypes.c_int64), ("x", ctypes.c_void_p), ("x_scale", ctypes.c_void_p),
                ("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("w2_scale", ctypes.c_void_p), ("h", ctypes.c_void_p), ("h_scale", ctypes.c_void_p),
                ("y", ctypes.c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


_P = ctypes.c_void_p
_F32 = ctypes.c_float
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_INT = ctypes.c_int

SIGNATURES = {
    "moe_abi_version": (_INT, []),
    "moe_status_str": (ctypes.c_char_p, [_INT]),
    "moe_workspace_size": (_SZ, [_INT, ctypes.POINTER(MoeShape), _INT]),
    "moe_route": (_INT, [ctypes.POINTER(MoeShape), _P, _INT, _P, _P, _P, _P, _P, _P, _P, _INT, _P, _SZ, _P]),
    "moe_dispatch": (_INT, [ctypes.POINTER(MoeShape), _P, _P, _I32, _I32, _P, _INT, _INT,
                            _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_expert_ffn": (_INT, [_I32, _P, _I64, _I32, _I32, _INT, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                              _INT, ctypes.POINTER(MoeFfnExtra), _P, _SZ, _P]),
    "moe_dispatch_noalloc": (_INT, [ctypes.POINTER(MoeShape), _P, _P, _I32, _I32, _P, _INT, _INT,
                                    _P, _P, _P, _P, _P, _P, _P]),
    "moe_combine": (_INT, [ctypes.POINTER(MoeShape), _P, _P, _P, _INT, _P, _P, _INT, _INT, _P]),
    "moe_quantize_blocks_e4m3": (_INT, [_I64, _I32, _I32, _P, _P, _P, _P]),
    "moe_quantize_rows_e4m3": (_INT, [_I64, _I32, _P, _P, _P, _P]),
    "moe_bias_update": (_INT, [_I64, _I32, _P, _F32, _P, _P, _P]),
    "moe_route_hash": (_INT, [ctypes.POINTER(MoeShape), _P, ctypes.c_uint64, _P, _P, _P, _P, _P]),
    "moe_combine_backward": (_INT, [ctypes.POINTER(MoeShape), _P, _P, _P, _INT, _P, _INT, _P, _P, _P]),
    "moe_expert_ffn_backward": (_INT, [_I32, _P, _I64, _I32, _I32, _INT, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       _P, _INT, _P, _SZ, _P]),
    "moe_expert_ffn_train": (_INT, [_I32, _P, _I64, _I32, _I32, _INT, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_dispatch_backward": (_INT, [ctypes.POINTER(MoeShape), _P, _P, _INT, _P, _P, _INT, _P]),
    "moe_route_backward": (_INT, [ctypes.POINTER(MoeShape), _P, _INT, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                  ctypes.c_size_t, _P]),
}

_lib = None


def header_functions(path: str = HEADER):
    """Names of the functions include/moe.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", text, flags=re.M)))


def load():
    """Load the library (the in-tree build, or the file MOE_MI355X_LIB names);
    raises if it is missing (no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("MOE_MI355X_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m moe_expert_routing_sqrt_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(fn_name: str, status: int):
    if status != MOE_OK:
        msg = load().moe_status_str(status).decode()
        raise MoeError(fn_name, status, msg)
