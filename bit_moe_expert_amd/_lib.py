"""ctypes view of ``libmoe4.so`` (declared in ``include/moe4.h``).

Loading fails loudly when the library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe4.so")

MOE4_OK = 0
MOE4_ERR_INVALID_ARG = 1
MOE4_ERR_UNSUPPORTED = 2
MOE4_ERR_WORKSPACE = 3
MOE4_ERR_HIP = 4
STATUS_NAMES = {0: "MOE4_OK", 1: "MOE4_ERR_INVALID_ARG", 2: "MOE4_ERR_UNSUPPORTED",
                3: "MOE4_ERR_WORKSPACE", 4: "MOE4_ERR_HIP"}


class Shape(Structure):
    _fields_ = [("T", c_int32), ("H", c_int32), ("E", c_int32), ("k", c_int32),
                ("I", c_int32), ("n_shared", c_int32), ("eps", c_float)]


MOE4_NOALLOC_SCRATCH_BYTES = 64 << 20
MOE4_W4_CANONICAL = 1
MOE4_W4_TILED = 2


class W4(Structure):
    _fields_ = [("packed", c_void_p), ("scales", c_void_p), ("tscale", c_void_p), ("layout", c_int32)]


_SHAPE = POINTER(Shape)
_W4 = POINTER(W4)

# name -> (restype, argtypes); every function include/moe4.h declares
SIGNATURES = {
    "moe4_abi_version": (c_int, []),
    "moe4_last_error": (c_char_p, []),
    "moe4_prepack_w4": (c_int, [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                c_void_p]),
    "moe4_permute_workspace_bytes": (c_size_t, [_SHAPE]),
    "moe4_layer_workspace_bytes": (c_size_t, [_SHAPE]),
    "moe4_route": (c_int, [_SHAPE, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe4_permute": (c_int, [_SHAPE, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                             c_void_p]),
    "moe4_expert_ffn": (c_int, [_SHAPE, c_void_p, c_void_p, c_void_p, _W4, _W4, c_void_p, c_void_p,
                                c_void_p]),
    "moe4_expert_up": (c_int, [_SHAPE, c_void_p, c_void_p, c_void_p, _W4, c_void_p, c_void_p]),
    "moe4_act_f16": (c_int, [c_int64, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe4_expert_up_f16": (c_int, [_SHAPE, c_void_p, c_void_p, c_void_p, c_void_p, _W4, c_void_p, c_void_p]),
    "moe4_expert_down": (c_int, [_SHAPE, c_void_p, c_void_p, _W4, c_void_p, c_void_p]),
    "moe4_combine_norm": (c_int, [_SHAPE, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe4_layer": (c_int, [_SHAPE, c_void_p, c_void_p, c_void_p, _W4, _W4, _W4, _W4, c_void_p,
                           c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                           c_void_p]),
    "moe4_layer_noalloc": (c_int, [_SHAPE, c_void_p, c_void_p, c_void_p, _W4, _W4, _W4, _W4, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe4_layer_side": (c_int, [_SHAPE, c_void_p, c_void_p, c_void_p, _W4, _W4, _W4, _W4, c_void_p,
                                c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe4_quant_mxfp8": (c_int, [c_int64, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe4_w4a8_workspace_bytes": (c_size_t, [_SHAPE]),
    "moe4_expert_ffn_w4a8": (c_int, [_SHAPE, c_void_p, c_void_p, c_void_p, _W4, _W4, c_void_p, c_void_p,
                                     c_void_p, c_size_t, c_void_p]),
    "moe4_expert_up_w4a8": (c_int, [_SHAPE, c_void_p, c_void_p, c_void_p, c_void_p, _W4, c_void_p, c_void_p,
                                    c_void_p, c_void_p]),
    "moe4_expert_down_w4a8": (c_int, [_SHAPE, c_void_p, c_void_p, c_void_p, _W4, c_void_p, c_void_p]),
    "moe4_layer_w4a8": (c_int, [_SHAPE, c_void_p, c_void_p, c_void_p, _W4, _W4, _W4, _W4, c_void_p,
                                c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                c_void_p]),
    "moe4_add_rmsnorm": (c_int, [c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_float, c_void_p,
                                 c_void_p, c_void_p]),
    "moe4_group_rmsnorm": (c_int, [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_float, c_void_p,
                                   c_void_p]),
}

ABI_VERSION = 2
_lib = None


class Moe4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libmoe4.so (once) and attach the prototypes."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m bit_moe_expert_amd.build` "
            "(there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.moe4_abi_version() != ABI_VERSION:
        raise ImportError(f"libmoe4 ABI {lib.moe4_abi_version()} != {ABI_VERSION}")
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != MOE4_OK:
        msg = load().moe4_last_error().decode(errors="replace")
        raise Moe4Error(status, msg)
