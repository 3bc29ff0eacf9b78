"""CPU oracle for the MoE dispatch/combine path (test infrastructure only).

The arithmetic lives in ``oracle.c`` (plain single-threaded C, binary32 IEEE
operations, no FMA contraction). This module only loads the shared object and
marshals numpy arrays. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it; the product library never does.

bf16 tensors are passed as ``np.uint16`` bit patterns, FP8 E4M3FN and UE8M0 as
``np.uint8`` codes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` next to it."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_f32p = ctypes.POINTER(ctypes.c_float)
_ll = ctypes.c_longlong
_int = ctypes.c_int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_to_f32.restype = ctypes.c_float
    lib.orc_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.orc_f32_to_bf16.restype = ctypes.c_uint16
    lib.orc_f32_to_e4m3.argtypes = [ctypes.c_float]
    lib.orc_f32_to_e4m3.restype = ctypes.c_uint8
    lib.orc_e4m3_to_f32.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_to_f32.restype = ctypes.c_float
    lib.orc_ue8m0_from_amax.argtypes = [ctypes.c_float]
    lib.orc_ue8m0_from_amax.restype = ctypes.c_uint8
    lib.orc_f32_to_bf16_array.argtypes = [_f32p, _u16p, _ll]
    lib.orc_f32_to_e4m3_array.argtypes = [_f32p, _u8p, _ll]
    lib.orc_ue8m0_array.argtypes = [_f32p, _u8p, _ll]
    lib.orc_topk.argtypes = [_f32p, _ll, _ll, _int, _int, _int, _i32p]
    lib.orc_shuffle.argtypes = [_f32p, _ll, _ll, _int, _int, _int, _int, _ll,
                                _i32p, _i32p, _i32p, _i32p]
    lib.orc_gather_scale.argtypes = [_u16p, _int, _int, _i32p, _i32p, _int,
                                     _f32p, _ll, _ll, _int, _int, _ll, _u16p]
    lib.orc_gather_scale_quant.argtypes = [_u16p, _int, _int, _i32p, _i32p,
                                           _int, _f32p, _ll, _ll, _int, _f32p,
                                           _int, _ll, _u8p, _f32p]
    lib.orc_scatter_add.argtypes = [_u16p, _int, _u16p, _i32p, _int, _int, _int,
                                    _ll]
    lib.orc_mxfp8_scale_bytes.argtypes = [_int, _int, _int]
    lib.orc_mxfp8_scale_bytes.restype = _ll
    lib.orc_mxfp8_swizzle_offset.argtypes = [_int, _int, _int]
    lib.orc_mxfp8_swizzle_offset.restype = _ll
    lib.orc_mxfp8_swizzle.argtypes = [_u8p, _int, _int, _u8p]
    lib.orc_finalize_rmsnorm.argtypes = [_u16p, _ll, ctypes.c_void_p, _i32p, _u16p,
                                         _u16p, ctypes.c_float, _int, _int,
                                         _int, ctypes.c_uint, _u16p, _u8p, _u8p]
    lib.orc_finalize_mhc.argtypes = [_u16p, _ll, ctypes.c_void_p, _i32p, _u16p, _u16p,
                                     _f32p, _f32p, _f32p, _u16p, ctypes.c_float, _int, _int,
                                     _int, _int, ctypes.c_uint, _u16p, _u16p, _u8p, _u8p]
    lib.orc_mxfp8_quantize.argtypes = [_u16p, _int, _int, _u8p, _u8p]
    lib.orc_shuffling.argtypes = [_int, _u16p, _ll, _u16p, _ll, _int, _i32p, _int, _int,
                                  _int, _int, _ll, _i32p]
    lib.orc_scatter_add_padded.argtypes = [_u16p, _int, _u16p, _int, _int, _i32p,
                                           _int, _i32p, _int]
    for name in ("orc_topk", "orc_shuffle", "orc_gather_scale",
                 "orc_gather_scale_quant", "orc_scatter_add",
                 "orc_finalize_rmsnorm", "orc_finalize_mhc", "orc_mxfp8_quantize",
                 "orc_scatter_add_padded", "orc_shuffling", "orc_mxfp8_swizzle"):
        getattr(lib, name).restype = _int
    _lib = lib
    return lib


def _p(arr, ctype):
    if arr is None:
        return None
    assert arr.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return arr.ctypes.data_as(ctype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (rc={rc})")


def _opt(count):
    """(given?, value) of an optional valid count."""
    return (0, 0) if count is None else (1, int(count))


def _scores_view(scores):
    """(pointer to the first element, stride_t, stride_e) of a 2-D fp32 view;
    strides are in elements, so transposed or sliced views pass through."""
    assert scores.dtype == np.float32 and scores.ndim == 2
    st, se = (s // 4 for s in scores.strides)
    return ctypes.cast(scores.ctypes.data, _f32p), st, se


# ---------------------------------------------------------------- encoders
def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (upper half of a binary32)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(f: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, dtype=np.uint16)
    _load().orc_f32_to_bf16_array(_p(f, _f32p), _p(out, _u16p), f.size)
    return out


def f32_to_e4m3(f: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, dtype=np.uint8)
    _load().orc_f32_to_e4m3_array(_p(f, _f32p), _p(out, _u8p), f.size)
    return out


def e4m3_to_f32(c: np.ndarray) -> np.ndarray:
    lib = _load()
    c = np.ascontiguousarray(c, dtype=np.uint8)
    table = np.array([lib.orc_e4m3_to_f32(i) for i in range(256)], np.float32)
    return table[c]


def ue8m0_from_amax(amax: np.ndarray) -> np.ndarray:
    amax = np.ascontiguousarray(amax, dtype=np.float32)
    out = np.empty(amax.shape, dtype=np.uint8)
    _load().orc_ue8m0_array(_p(amax, _f32p), _p(out, _u8p), amax.size)
    return out


# ---------------------------------------------------------------- stages
def topk(scores: np.ndarray, K: int) -> np.ndarray:
    base, st, se = _scores_view(scores)
    T, E = scores.shape
    sel = np.empty((T, K), dtype=np.int32)
    _check(_load().orc_topk(base, st, se, T, E, K, _p(sel, _i32p)), "topk")
    return sel


def shuffle(scores: np.ndarray, K: int, valid_token_count: int | None = None):
    """Returns (counts[E+1], expert_indices[a], token_indices[a], row_of_pair[T,K])."""
    base, st, se = _scores_view(scores)
    T, E = scores.shape
    a = T * K
    counts = np.empty(E + 1, dtype=np.int32)
    ei = np.empty(a, dtype=np.int32)
    ti = np.empty(a, dtype=np.int32)
    rop = np.empty((T, K), dtype=np.int32)
    has, vtc = _opt(valid_token_count)
    _check(_load().orc_shuffle(base, st, se, T, E, K, has, vtc,
                               _p(counts, _i32p), _p(ei, _i32p), _p(ti, _i32p),
                               _p(rop, _i32p)), "shuffle")
    return counts, ei, ti, rop


def gather_scale(x, token_indices, expert_indices, scores, valid_rows=None,
                 out=None):
    """x: uint16 (T,D) bf16 bits. Rows >= valid_rows of ``out`` are untouched."""
    T, D = x.shape
    a = token_indices.shape[0]
    base, st, se = _scores_view(scores)
    if out is None:
        out = np.zeros((a, D), dtype=np.uint16)
    has, vr = _opt(valid_rows)
    _check(_load().orc_gather_scale(
        _p(x, _u16p), T, D, _p(token_indices, _i32p), _p(expert_indices, _i32p),
        a, base, st, se, scores.shape[1], has, vr,
        _p(out, _u16p)), "gather_scale")
    return out


def gather_scale_quant(x, token_indices, expert_indices, scores, scale_ub=None,
                       valid_rows=None, out=None, out_scale=None):
    T, D = x.shape
    a = token_indices.shape[0]
    base, st, se = _scores_view(scores)
    if out is None:
        out = np.zeros((a, D), dtype=np.uint8)
    if out_scale is None:
        out_scale = np.zeros(a, dtype=np.float32)
    ub = None if scale_ub is None else np.array([scale_ub], dtype=np.float32)
    has, vr = _opt(valid_rows)
    _check(_load().orc_gather_scale_quant(
        _p(x, _u16p), T, D, _p(token_indices, _i32p), _p(expert_indices, _i32p),
        a, base, st, se, scores.shape[1], _p(ub, _f32p),
        has, vr, _p(out, _u8p), _p(out_scale, _f32p)), "gather_scale_quant")
    return out, out_scale


def scatter_add(out_tokens, in_tokens, token_indices, valid_rows=None):
    """In place on ``out_tokens`` (uint16 (T,D)); also returns it."""
    T, D = out_tokens.shape
    a = in_tokens.shape[0]
    has, vr = _opt(valid_rows)
    _check(_load().orc_scatter_add(_p(out_tokens, _u16p), T, _p(in_tokens, _u16p),
                                   _p(token_indices, _i32p), a, D, has, vr),
           "scatter_add")
    return out_tokens


def scatter_add_padded(out_tokens, in_tokens, token_counts, token_indices):
    """In place on out_tokens (uint16 (T,D)); in_tokens uint16 (EP, T_K, D)."""
    T, D = out_tokens.shape
    EP, T_K, D2 = in_tokens.shape
    assert D2 == D
    counts = np.ascontiguousarray(token_counts, dtype=np.int32)
    ti = np.ascontiguousarray(token_indices, dtype=np.int32)
    _check(_load().orc_scatter_add_padded(_p(out_tokens, _u16p), T, _p(in_tokens, _u16p), EP,
                                          T_K, _p(counts, _i32p), counts.size, _p(ti, _i32p),
                                          D), "scatter_add_padded")
    return out_tokens


def finalize_rmsnorm(y, expert_weights, row_of_pair, shared, gamma, eps,
                     flags=0, mxfp8=False):
    """Returns out (T,D) uint16, and (codes (T,D) uint8, scales) when
    ``mxfp8``; scales are (T, D/32) row-major, or with flags bit 2 the
    swizzled byte buffer. expert_weights: fp32 (T,K), or uint16 bf16 bits
    with flags bit 1."""
    T, K = row_of_pair.shape
    rows, D = y.shape
    w = np.ascontiguousarray(expert_weights)
    assert w.dtype == (np.uint16 if flags & 2 else np.float32)
    out = np.empty((T, D), dtype=np.uint16)
    codes = np.empty((T, D), dtype=np.uint8) if mxfp8 else None
    if mxfp8 and flags & 4:
        scales = np.empty(mxfp8_scale_bytes(T, D, True), dtype=np.uint8)
    else:
        scales = np.empty((T, D // 32), dtype=np.uint8) if mxfp8 else None
    _check(_load().orc_finalize_rmsnorm(
        _p(y, _u16p), rows, w.ctypes.data, _p(row_of_pair, _i32p),
        _p(shared, _u16p), _p(gamma, _u16p), float(eps), T, K, D, int(flags),
        _p(out, _u16p), _p(codes, _u8p), _p(scales, _u8p)), "finalize_rmsnorm")
    return (out, codes, scales) if mxfp8 else out


def finalize_mhc(y, expert_weights, row_of_pair, shared, residual, post, comb, pre,
                 gamma, eps, flags=0, mxfp8=False):
    """mHC finalize: returns (residual_out (T,hc,D) uint16, out (T,D) uint16 or
    None, codes, scales). ``pre`` None: residual only (out, codes and scales
    are None). residual (T,hc,D) bf16 bits; post and pre (T,hc) fp32; comb
    (T,hc,hc) fp32 indexed [source, target]. Weights and flags as in
    finalize_rmsnorm."""
    T, K = row_of_pair.shape
    rows, D = y.shape
    hc = residual.shape[1]
    assert residual.shape == (T, hc, D)
    w = np.ascontiguousarray(expert_weights)
    assert w.dtype == (np.uint16 if flags & 2 else np.float32)
    post = np.ascontiguousarray(post, dtype=np.float32).reshape(T, hc)
    comb = np.ascontiguousarray(comb, dtype=np.float32).reshape(T, hc, hc)
    if pre is not None:
        pre = np.ascontiguousarray(pre, dtype=np.float32).reshape(T, hc)
    res_out = np.empty((T, hc, D), dtype=np.uint16)
    out = np.empty((T, D), dtype=np.uint16) if pre is not None else None
    codes = scales = None
    if mxfp8:
        codes = np.empty((T, D), dtype=np.uint8)
        scales = (np.empty(mxfp8_scale_bytes(T, D, True), dtype=np.uint8) if flags & 4
                  else np.empty((T, D // 32), dtype=np.uint8))
    _check(_load().orc_finalize_mhc(
        _p(y, _u16p), rows, w.ctypes.data, _p(row_of_pair, _i32p), _p(shared, _u16p),
        _p(np.ascontiguousarray(residual), _u16p), _p(post, _f32p), _p(comb, _f32p),
        _p(pre, _f32p), _p(gamma, _u16p), float(eps), T, K, D, hc, int(flags),
        _p(res_out, _u16p), _p(out, _u16p), _p(codes, _u8p), _p(scales, _u8p)),
        "finalize_mhc")
    return res_out, out, codes, scales


def mxfp8_scale_bytes(M: int, D: int, swizzled: bool) -> int:
    return int(_load().orc_mxfp8_scale_bytes(M, D, int(bool(swizzled))))


def mxfp8_swizzle(rowmajor: np.ndarray) -> np.ndarray:
    """(M, cols) uint8 scales -> the swizzled 128x4 byte buffer."""
    rowmajor = np.ascontiguousarray(rowmajor, dtype=np.uint8)
    M, cols = rowmajor.shape
    out = np.empty(mxfp8_scale_bytes(M, 32 * cols, True), dtype=np.uint8)
    _check(_load().orc_mxfp8_swizzle(_p(rowmajor, _u8p), M, cols, _p(out, _u8p)), "swizzle")
    return out


def mxfp8_swizzle_offset(m: int, k: int, cols: int) -> int:
    return int(_load().orc_mxfp8_swizzle_offset(m, k, cols))


def mxfp8_quantize(o_bits: np.ndarray):
    """MXFP8 of bf16 rows (uint16 (rows, D), D % 32 == 0): (codes, scales)."""
    o_bits = np.ascontiguousarray(o_bits, dtype=np.uint16)
    rows, D = o_bits.shape
    codes = np.empty((rows, D), dtype=np.uint8)
    scales = np.empty((rows, D // 32), dtype=np.uint8)
    _check(_load().orc_mxfp8_quantize(_p(o_bits, _u16p), rows, D, _p(codes, _u8p),
                                      _p(scales, _u8p)), "mxfp8_quantize")
    return codes, scales


def _shuffling(inverse, in_rows_arr, counts, c_lo, c_hi, rank_stride, out):
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    EP, C = counts.shape
    oc = np.zeros(c_hi - c_lo + 1, dtype=np.int32)
    _check(_load().orc_shuffling(int(inverse), _p(in_rows_arr, _u16p), in_rows_arr.shape[0],
                                 _p(out, _u16p), out.shape[0], in_rows_arr.shape[1],
                                 _p(counts, _i32p), EP, C, c_lo, c_hi,
                                 -1 if rank_stride is None else int(rank_stride),
                                 _p(oc, _i32p)), "shuffling")
    return out, oc


def combine_shuffling(tokens, counts, c_lo=None, c_hi=None, rank_stride=None, out=None):
    """tokens uint16 (rows, D) grouped by (rank, column); counts (EP, C).
    Returns (out rows in expert-major order of columns [c_lo, c_hi),
    out_counts [n_local + 1]). rank_stride None = packed rank chunks."""
    EP, C = np.asarray(counts).shape
    c_lo = 0 if c_lo is None else c_lo
    c_hi = C if c_hi is None else c_hi
    if out is None:
        out = np.zeros_like(tokens)
    return _shuffling(0, np.ascontiguousarray(tokens), counts, c_lo, c_hi, rank_stride, out)


def split_shuffling(tokens, counts, c_lo=None, c_hi=None, rank_stride=None, out=None):
    """Inverse of combine_shuffling: rows in expert-major order back to their
    (rank, column) positions in ``out`` (other rows of out untouched)."""
    EP, C = np.asarray(counts).shape
    c_lo = 0 if c_lo is None else c_lo
    c_hi = C if c_hi is None else c_hi
    if out is None:
        out = np.zeros_like(tokens)
    return _shuffling(1, np.ascontiguousarray(tokens), counts, c_lo, c_hi, rank_stride, out)[0]
