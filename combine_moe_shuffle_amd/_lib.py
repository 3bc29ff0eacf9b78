"""Loads libmoe_shuffle.so (built in-tree by combine_moe_shuffle_amd.build)
and declares the C ABI of include/moe_shuffle.h for ctypes.

The launching entry points are called through the _moe_fastcall extension
when it is built (one compiled call that parses plain ints and floats, no
per-argument ctypes conversion), else through ctypes; both call the same
library. There is no fallback beyond that: if the library is missing, every
op raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_shuffle.so")
# MOE_ABI_VERSION of include/moe_shuffle.h that SIGNATURES describes
ABI_VERSION = 3

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_u32 = ctypes.c_uint32
_f32 = ctypes.c_float
_status = ctypes.c_int

# name -> (restype, argtypes), in the header's order
SIGNATURES = {
    "moe_abi_version": (ctypes.c_int, []),
    "moe_status_str": (ctypes.c_char_p, [_status]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_shuffle_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "moe_shuffle": (_status, [_p, _i64, _i64, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p,
                              _sz, _p]),
    "moe_shuffle_noalloc": (_status, [_p, _i64, _i64, _i32, _i32, _i32, _p, _p, _p, _p, _p,
                                      _p]),
    "moe_gather_scale_workspace_bytes": (_sz, [_i32, _i32]),
    "moe_gather_scale": (_status, [_p, _i32, _i32, _p, _p, _i32, _p, _i64, _i64, _i32, _p,
                                   _p, _p, _sz, _p]),
    "moe_gather_scale_by_token": (_status, [_p, _i32, _i32, _p, _i32, _p, _i32, _p, _i64,
                                            _i64, _i32, _p, _p, _p]),
    "moe_gather_scale_quant": (_status, [_p, _i32, _i32, _p, _p, _i32, _p, _i64, _i64, _i32,
                                         _p, _p, _p, _p, _p]),
    "moe_scatter_add_workspace_bytes": (_sz, [_i32, _i32]),
    "moe_scatter_add": (_status, [_p, _i32, _p, _p, _i32, _i32, _p, _p, _sz, _p]),
    "moe_scatter_add_by_token": (_status, [_p, _i32, _p, _p, _i32, _i32, _i32, _p, _p]),
    "moe_scatter_add_padded_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "moe_scatter_add_padded": (_status, [_p, _i32, _i32, _p, _i32, _p, _p, _i32, _i32, _p, _sz,
                                         _p]),
    "moe_scatter_add_padded_by_token": (_status, [_p, _i32, _i32, _p, _i32, _p, _i32, _p, _i32,
                                                  _i32, _p]),
    "moe_shuffling_workspace_bytes": (_sz, [_i32, _i32, _i64]),
    "moe_combine_shuffling": (_status, [_p, _i64, _p, _i64, _i32, _p, _i32, _i32, _i32, _i32,
                                        _i64, _p, _p, _sz, _p]),
    "moe_split_shuffling": (_status, [_p, _i64, _p, _i64, _i32, _p, _i32, _i32, _i32, _i32,
                                      _i64, _p, _p, _sz, _p]),
    "moe_mxfp8_scale_bytes": (_sz, [_i32, _i32, _u32]),
    "moe_finalize_rmsnorm": (_status, [_p, _i64, _p, _p, _p, _p, _f32, _i32, _i32, _i32, _u32,
                                       _p, _p, _p, _p]),
    "moe_finalize_mhc": (_status, [_p, _i64, _p, _p, _p, _p, _p, _p, _p, _p, _f32, _i32, _i32,
                                   _i32, _i32, _u32, _p, _p, _p, _p, _p]),
    "moe_convert_check": (_status, [_p, _i64, _p, _p, _p]),
    "moe_launch_floor_threads": (_i32, [_i32, _i32]),
    "moe_launch_floor": (_status, [_i32, _i32, _i32, _p, _p, _p]),
    "moe_stream_probe": (_status, [_i32, _i32, _i32, _i64, _p, _p, _p]),
}

STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED",
          3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_HIP"}


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None
_fast = None
_fast_tried = False


def fast():
    """The compiled fast-call module, or None when it is not built."""
    global _fast, _fast_tried
    if not _fast_tried:
        _fast_tried = True
        try:
            from . import _moe_fastcall
            _fast = _moe_fastcall
        except ImportError:
            _fast = None
    return _fast


_fns = {}


def fn(name: str):
    """The callable for a status-returning entry point: pointers as ints
    (0 for NULL), sizes as ints, floats as floats, the stream handle as an
    int."""
    f = _fns.get(name)
    if f is None:
        lib = load()  # also checks the library's ABI version
        mod = fast()
        f = getattr(mod, name) if mod is not None else getattr(lib, name)
        _fns[name] = f
    return f


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m combine_moe_shuffle_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.moe_abi_version() != ABI_VERSION:
        raise ImportError(
            f"{LIB_PATH} implements ABI {lib.moe_abi_version()}, the binding expects "
            f"{ABI_VERSION}: rebuild it with `python -m combine_moe_shuffle_amd.build`")
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != 0:
        mod = fast()
        msg = (mod.last_error() if mod is not None
               else load().moe_last_error().decode(errors="replace"))
        raise MoeError(status, msg)
