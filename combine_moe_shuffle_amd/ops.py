"""torch-tensor bindings of the C ABI (include/moe_shuffle.h).

Argument marshalling only: every function checks dtypes, shapes, devices and
contiguity (ValueError), allocates outputs and workspaces with torch, and
calls the library on torch's current HIP stream. All the work runs in the
library's gfx950 kernels; there is no CPU path.

prepare(op, ...) runs an op once with its checks and returns a callable that
repeats its library calls on the same buffers (for loops that call one op on
fixed buffers every step).

bf16 tensors are torch.bfloat16; FP8 codes and UE8M0 scales are torch.uint8.
Device-side counts (valid_token_count, valid_rows) are int32 tensors of one
element on the same device, read by the kernels (no host sync).
"""
from __future__ import annotations

import threading

import torch

from . import _lib


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_get_device = getattr(torch._C, "_cuda_getDevice", None)


def _stream(device):
    """The current stream of the current device, as a raw handle. The library
    launches on the current HIP device, so the tensors must live there."""
    cur = _get_device() if _get_device is not None else torch.cuda.current_device()
    if device.index is not None and device.index != cur:
        raise ValueError(f"the tensors are on {device} but the current device is cuda:{cur}")
    if _raw_stream is not None:
        return _raw_stream(cur)
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t):
    if t is None:
        return 0
    keep = getattr(_rec, "tensors", None)
    if keep is not None:
        keep.append(t)  # a prepared call points into it: keep it
    return t.data_ptr()


def _need(t, name, dtype, ndim=None, device=None):
    """t is a GPU tensor of dtype (and ndim dimensions, on device, when given);
    else ValueError. The common case costs three tensor queries."""
    try:
        d = t.get_device()
        if (t.dtype == dtype and (ndim is None or t.dim() == ndim) and d >= 0
                and (device is None or device.index is None or d == device.index)):
            return
    except AttributeError:
        pass
    _need_explain(t, name, dtype, ndim, device)


def _need_explain(t, name, dtype, ndim, device):
    """Raises the ValueError that says which requirement of _need t fails."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    raise ValueError(f"{name} is not a usable tensor")


def _contig(t, name):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _scalar_i32(t, name, device):
    if t is None:
        return None
    _need(t, name, torch.int32, device=device)
    if t.numel() != 1:
        raise ValueError(f"{name} must hold one element")
    return t


def _out(t, name, dtype, shape, device):
    """An output tensor: the caller's, checked (dtype, device, contiguity and
    exact shape, so no kernel writes past its end), or a new one."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _need(t, name, dtype, len(shape), device)
    _contig(t, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _workspace(workspace, need, device):
    """The workspace tensor (allocated when None) and its size in bytes. A
    caller's workspace must be a contiguous tensor on the same GPU; the
    library checks its size and alignment."""
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    elif not isinstance(workspace, torch.Tensor):
        raise ValueError("workspace must be a tensor")
    else:
        if not workspace.is_cuda or workspace.device != device:
            raise ValueError(f"workspace must be on {device}")
        _contig(workspace, "workspace")
    return workspace, workspace.numel() * workspace.element_size()


def _scores(scores, device):
    _need(scores, "scores", torch.float32, 2, device)
    return scores.stride(0), scores.stride(1)


# ---------------------------------------------------------------- calls
# per thread: while prepare() runs an op, .calls collects its library calls and
# .tensors every tensor whose address they take (other threads are unaffected)
_rec = threading.local()


def _call(name, *args):
    """One status-returning library call; its last argument is the stream."""
    f = _lib.fn(name)
    calls = getattr(_rec, "calls", None)
    if calls is not None:
        calls.append((f, args[:-1]))
    _lib.check(f(*args))


class Prepared:
    """An op's library calls with their arguments checked and converted once
    (see prepare). Calling it makes the same calls again on the current stream
    and returns the op's result (the same tensors, rewritten)."""

    def __init__(self, calls, device, result, keep):
        self._calls = tuple(calls)
        self._device = device
        self._result = result
        self._keep = keep  # every tensor the calls point into stays alive

    def __call__(self):
        stream = _stream(self._device)
        for f, args in self._calls:
            _lib.check(f(*args, stream))
        return self._result


def prepare(op, *args, **kwargs):
    """Runs ``op(*args, **kwargs)`` once, with all its checks, and records the
    library calls it makes; returns a Prepared that repeats exactly those calls
    (same device pointers, sizes and flags, the then-current stream) without
    the Python-side checks and allocations. For a loop that calls one op on the
    same buffers every step (a decode step). The Prepared holds references to
    the arguments and the result; the caller must not resize them or replace
    their storage. Device-side counts are read by the kernels at each call, as
    in the op itself."""
    if getattr(_rec, "calls", None) is not None:
        raise RuntimeError("prepare() does not nest")
    calls, keep = [], []
    _rec.calls, _rec.tensors = calls, keep
    try:
        result = op(*args, **kwargs)
    finally:
        _rec.calls = _rec.tensors = None
    if not calls:
        raise ValueError("the op made no library call (an empty input?)")
    if not keep:
        raise ValueError("the op's library calls point into no tensor")
    device = next((t.device for t in keep if t.is_cuda), keep[0].device)
    return Prepared(calls, device, result, (keep, args, kwargs, result))


# ---------------------------------------------------------------- shuffle
def _shuffle_outputs(out, T, E, K, row_of_pair, device):
    """The four shuffle outputs: the caller's (checked) or new tensors."""
    if out is None:
        counts = torch.empty(E + 1, dtype=torch.int32, device=device)
        ei = torch.empty(T * K, dtype=torch.int32, device=device)
        ti = torch.empty(T * K, dtype=torch.int32, device=device)
        rop = torch.empty((T, K), dtype=torch.int32, device=device) if row_of_pair else None
        return counts, ei, ti, rop
    counts, ei, ti, rop = out
    for t, n, numel in ((counts, "counts", E + 1), (ei, "expert_indices", T * K),
                        (ti, "token_indices", T * K)):
        _need(t, n, torch.int32, device=device)
        _contig(t, n)
        if t.numel() != numel:
            raise ValueError(f"{n} must have {numel} elements")
    if rop is not None:
        _need(rop, "row_of_pair", torch.int32, device=device)
        _contig(rop, "row_of_pair")
        if rop.numel() != T * K:
            raise ValueError(f"row_of_pair must have {T * K} elements")
    return counts, ei, ti, rop


def moe_shuffle(scores, K, valid_token_count=None, *, row_of_pair=True, workspace=None,
                out=None):
    """Top-k routing + stable counting sort of (token, expert) pairs by expert.

    Returns (counts[E+1], expert_indices[T*K], token_indices[T*K],
    row_of_pair[T, K] or None); counts[E] is the valid row count V. ``out``
    may supply those four tensors (row_of_pair may be None)."""
    device = scores.device
    st, se = _scores(scores, device)
    T, E = scores.shape
    vtc = _scalar_i32(valid_token_count, "valid_token_count", device)
    lib = _lib.load()
    counts, ei, ti, rop = _shuffle_outputs(out, T, E, K, row_of_pair, device)
    workspace, nbytes = _workspace(workspace, lib.moe_shuffle_workspace_bytes(T, E, K), device)
    _call("moe_shuffle", _ptr(scores), st, se, T, E, K, _ptr(vtc), _ptr(counts),
          _ptr(ei), _ptr(ti), _ptr(rop), _ptr(workspace), nbytes, _stream(device))
    return counts, ei, ti, rop


def moe_shuffle_noalloc(scores, K, valid_token_count=None, *, row_of_pair=True, out=None):
    """moe_shuffle through the entry point that allocates nothing: its
    workspace is the library's static per-GPU scratch. With ``out`` given the
    call allocates nothing here either. Calls on one GPU share that scratch,
    so they must be ordered (one stream)."""
    device = scores.device
    st, se = _scores(scores, device)
    T, E = scores.shape
    vtc = _scalar_i32(valid_token_count, "valid_token_count", device)
    counts, ei, ti, rop = _shuffle_outputs(out, T, E, K, row_of_pair, device)
    _call("moe_shuffle_noalloc", _ptr(scores), st, se, T, E, K, _ptr(vtc), _ptr(counts),
          _ptr(ei), _ptr(ti), _ptr(rop), _stream(device))
    return counts, ei, ti, rop


# ---------------------------------------------------------------- dispatch
def _gather_common(x, expert_indices, scores, valid_rows):
    device = x.device
    _need(x, "x", torch.bfloat16, 2, device)
    _contig(x, "x")
    _need(expert_indices, "expert_indices", torch.int32, 1, device)
    _contig(expert_indices, "expert_indices")
    st, se = _scores(scores, device)
    if scores.shape[0] != x.shape[0]:
        raise ValueError("scores must be (T, E) with T = x.shape[0]")
    return device, st, se, _scalar_i32(valid_rows, "valid_rows", device)


def moe_gather_scale(x, token_indices, expert_indices, scores, valid_rows=None, out=None,
                     workspace=None, row_order=False):
    """out[i] = bf16(x[token_indices[i]] * scores[t, expert_indices[i]]) for
    i < valid_rows; other rows of ``out`` are left as they are.

    By default the rows are visited token by token, reading each x row once:
    up to 1024 rows each token's rows are found directly, beyond that through
    a list of each token's rows built in ``workspace`` (allocated when None,
    as the library requires it either way); ``row_order=True`` visits them
    row by row with no workspace. All give the same bits."""
    device, st, se, vr = _gather_common(x, expert_indices, scores, valid_rows)
    _need(token_indices, "token_indices", torch.int32, 1, device)
    _contig(token_indices, "token_indices")
    a = token_indices.numel()
    if expert_indices.numel() != a:
        raise ValueError("token_indices and expert_indices must have the same length")
    T, D = x.shape
    out = _out(out, "out", torch.bfloat16, (a, D), device)
    nbytes = 0
    if not row_order:
        workspace, nbytes = _workspace(
            workspace, _lib.load().moe_gather_scale_workspace_bytes(T, a), device)
    else:
        workspace = None
    _call("moe_gather_scale",
        _ptr(x), T, D, _ptr(token_indices), _ptr(expert_indices), a, _ptr(scores), st, se,
        scores.shape[1], _ptr(vr), _ptr(out), _ptr(workspace), nbytes, _stream(device))
    return out


def moe_gather_scale_by_token(x, row_of_pair, expert_indices, scores, valid_rows=None,
                              out=None):
    """moe_gather_scale's output, visiting tokens through the inverse map."""
    device, st, se, vr = _gather_common(x, expert_indices, scores, valid_rows)
    _need(row_of_pair, "row_of_pair", torch.int32, 2, device)
    _contig(row_of_pair, "row_of_pair")
    T, D = x.shape
    if row_of_pair.shape[0] != T:
        raise ValueError("row_of_pair must be (T, K)")
    K = row_of_pair.shape[1]
    a = expert_indices.numel()
    out = _out(out, "out", torch.bfloat16, (a, D), device)
    _call("moe_gather_scale_by_token",
        _ptr(x), T, D, _ptr(row_of_pair), K, _ptr(expert_indices), a, _ptr(scores), st, se,
        scores.shape[1], _ptr(vr), _ptr(out), _stream(device))
    return out


def moe_gather_scale_quant(x, token_indices, expert_indices, scores, scale_ub=None,
                           valid_rows=None, out=None, out_scale=None):
    """FP8 E4M3 rowwise dispatch. Returns (codes (a, D) uint8, scale (a,) fp32)."""
    device, st, se, vr = _gather_common(x, expert_indices, scores, valid_rows)
    _need(token_indices, "token_indices", torch.int32, 1, device)
    _contig(token_indices, "token_indices")
    a = token_indices.numel()
    T, D = x.shape
    if scale_ub is not None:
        _need(scale_ub, "scale_ub", torch.float32, device=device)
        if scale_ub.numel() != 1:
            raise ValueError("scale_ub must hold one element")
    out = _out(out, "out", torch.uint8, (a, D), device)
    out_scale = _out(out_scale, "out_scale", torch.float32, (a,), device)
    _call("moe_gather_scale_quant",
        _ptr(x), T, D, _ptr(token_indices), _ptr(expert_indices), a, _ptr(scores), st, se,
        scores.shape[1], _ptr(scale_ub), _ptr(vr), _ptr(out), _ptr(out_scale), _stream(device))
    return out, out_scale


# ---------------------------------------------------------------- combine
def _scatter_common(out_tokens, in_tokens, valid_rows):
    device = out_tokens.device
    _need(out_tokens, "out_tokens", torch.bfloat16, 2, device)
    _need(in_tokens, "in_tokens", torch.bfloat16, 2, device)
    _contig(out_tokens, "out_tokens")
    _contig(in_tokens, "in_tokens")
    if out_tokens.shape[1] != in_tokens.shape[1]:
        raise ValueError("out_tokens and in_tokens must have the same D")
    return device, _scalar_i32(valid_rows, "valid_rows", device)


def moe_scatter_add(out_tokens, in_tokens, token_indices, valid_rows=None, workspace=None):
    """In place: out[t] = bf16(f32(out[t]) + sum of its valid rows, ascending)."""
    device, vr = _scatter_common(out_tokens, in_tokens, valid_rows)
    _need(token_indices, "token_indices", torch.int32, 1, device)
    _contig(token_indices, "token_indices")
    T, D = out_tokens.shape
    a = in_tokens.shape[0]
    if token_indices.numel() != a:
        raise ValueError("token_indices must have in_tokens.shape[0] entries")
    lib = _lib.load()
    workspace, nbytes = _workspace(workspace, lib.moe_scatter_add_workspace_bytes(T, a), device)
    _call("moe_scatter_add", _ptr(out_tokens), T, _ptr(in_tokens), _ptr(token_indices),
          a, D, _ptr(vr), _ptr(workspace), nbytes, _stream(device))
    return out_tokens


def moe_scatter_add_by_token(out_tokens, in_tokens, row_of_pair, valid_rows=None):
    """moe_scatter_add's result, reading each token's rows from the inverse map."""
    device, vr = _scatter_common(out_tokens, in_tokens, valid_rows)
    _need(row_of_pair, "row_of_pair", torch.int32, 2, device)
    _contig(row_of_pair, "row_of_pair")
    T, D = out_tokens.shape
    if row_of_pair.shape[0] != T:
        raise ValueError("row_of_pair must be (T, K)")
    _call("moe_scatter_add_by_token",
        _ptr(out_tokens), T, _ptr(in_tokens), _ptr(row_of_pair), row_of_pair.shape[1],
        in_tokens.shape[0], D, _ptr(vr), _stream(device))
    return out_tokens


def moe_scatter_add_padded(in_tokens, token_counts, token_indices, out_tokens, workspace=None):
    """Static-shape expert-parallel combine: in_tokens (EP, T_K, D); rows of
    expert e come from rank e // (E // EP). In place on out_tokens (T, D)."""
    device = out_tokens.device
    _need(in_tokens, "in_tokens", torch.bfloat16, 3, device)
    _need(out_tokens, "out_tokens", torch.bfloat16, 2, device)
    _need(token_counts, "token_counts", torch.int32, 1, device)
    _need(token_indices, "token_indices", torch.int32, 1, device)
    for t, n in ((in_tokens, "in_tokens"), (out_tokens, "out_tokens"),
                 (token_counts, "token_counts"), (token_indices, "token_indices")):
        _contig(t, n)
    EP, T_K, D = in_tokens.shape
    T = out_tokens.shape[0]
    E = token_counts.numel()
    if out_tokens.shape[1] != D or token_indices.numel() != T_K:
        raise ValueError("shapes must be in (EP, T_K, D), token_indices (T_K,), out (T, D)")
    lib = _lib.load()
    workspace, nbytes = _workspace(
        workspace, lib.moe_scatter_add_padded_workspace_bytes(T, T_K, E), device)
    _call("moe_scatter_add_padded", _ptr(in_tokens), EP, T_K, _ptr(token_counts), E,
          _ptr(token_indices), _ptr(out_tokens), T, D, _ptr(workspace), nbytes,
          _stream(device))
    return out_tokens


def moe_scatter_add_padded_by_token(in_tokens, token_counts, row_of_pair, out_tokens):
    """moe_scatter_add_padded's result, reading each token's rows from the
    inverse map row_of_pair (T, K) instead of building row lists: no
    workspace. In place on out_tokens (T, D)."""
    device = out_tokens.device
    _need(in_tokens, "in_tokens", torch.bfloat16, 3, device)
    _need(out_tokens, "out_tokens", torch.bfloat16, 2, device)
    _need(token_counts, "token_counts", torch.int32, 1, device)
    _need(row_of_pair, "row_of_pair", torch.int32, 2, device)
    for t, n in ((in_tokens, "in_tokens"), (out_tokens, "out_tokens"),
                 (token_counts, "token_counts"), (row_of_pair, "row_of_pair")):
        _contig(t, n)
    EP, T_K, D = in_tokens.shape
    T = out_tokens.shape[0]
    if out_tokens.shape[1] != D or row_of_pair.shape[0] != T:
        raise ValueError("shapes must be in (EP, T_K, D), row_of_pair (T, K), out (T, D)")
    _call("moe_scatter_add_padded_by_token", _ptr(in_tokens), EP, T_K, _ptr(token_counts),
          token_counts.numel(), _ptr(row_of_pair), row_of_pair.shape[1], _ptr(out_tokens), T, D,
          _stream(device))
    return out_tokens


def _shuffling(name, tokens, counts, c_lo, c_hi, rank_stride, out, out_rows, with_counts,
               workspace):
    device = tokens.device
    _need(tokens, "tokens", torch.bfloat16, 2, device)
    _contig(tokens, "tokens")
    _need(counts, "counts", torch.int32, 2, device)
    _contig(counts, "counts")
    EP, C = counts.shape
    c_lo = 0 if c_lo is None else c_lo
    c_hi = C if c_hi is None else c_hi
    D = tokens.shape[1]
    if out is None:
        out = torch.empty((tokens.shape[0] if out_rows is None else out_rows, D),
                          dtype=torch.bfloat16, device=device)
    else:  # any number of rows (rows past its end are skipped), D columns
        _need(out, "out", torch.bfloat16, 2, device)
        _contig(out, "out")
        if out.shape[1] != D:
            raise ValueError(f"out must have D = {D} columns, got {out.shape[1]}")
    oc = torch.empty(c_hi - c_lo + 1, dtype=torch.int32, device=device) if with_counts else None
    lib = _lib.load()
    em_rows = out.shape[0] if name == "moe_combine_shuffling" else tokens.shape[0]
    workspace, nbytes = _workspace(
        workspace, lib.moe_shuffling_workspace_bytes(EP, c_hi - c_lo, em_rows), device)
    _call(name,
        _ptr(tokens), tokens.shape[0], _ptr(out), out.shape[0], D, _ptr(counts), EP, C, c_lo,
        c_hi, -1 if rank_stride is None else int(rank_stride), _ptr(oc), _ptr(workspace),
        nbytes, _stream(device))
    return out, oc


def moe_combine_shuffling(tokens, counts, c_lo=None, c_hi=None, rank_stride=None, out=None,
                          out_rows=None, workspace=None):
    """Re-sort rows grouped by (rank, expert column) into expert-major order of
    the local columns [c_lo, c_hi). counts (EP, C) int32; rank_stride None =
    packed rank chunks. Returns (out, out_counts[n_local + 1])."""
    return _shuffling("moe_combine_shuffling", tokens, counts, c_lo, c_hi, rank_stride, out,
                      out_rows, True, workspace)


def moe_split_shuffling(tokens, counts, c_lo=None, c_hi=None, rank_stride=None, out=None,
                        out_rows=None, workspace=None):
    """Inverse of moe_combine_shuffling: expert-major rows back to their
    (rank, column) positions in ``out`` (other rows are not written)."""
    return _shuffling("moe_split_shuffling", tokens, counts, c_lo, c_hi, rank_stride, out,
                      out_rows, False, workspace)[0]


# ---------------------------------------------------------------- finalize
BF16_SQUARES = 1
BF16_WEIGHTS = 2
MX_SWIZZLED = 4


def _finalize_common(y_permuted, expert_weights, row_of_pair, shared, gamma, flags, mxfp8,
                     scale_layout):
    """Checks of the finalize inputs shared by both finalize entry points;
    returns (flags, T, K, rows, D)."""
    device = y_permuted.device
    _need(y_permuted, "y_permuted", torch.bfloat16, 2, device)
    if expert_weights.dtype == torch.bfloat16:
        flags |= BF16_WEIGHTS
        _need(expert_weights, "expert_weights", torch.bfloat16, 2, device)
    else:
        _need(expert_weights, "expert_weights", torch.float32, 2, device)
    _need(row_of_pair, "row_of_pair", torch.int32, 2, device)
    for t, n in ((y_permuted, "y_permuted"), (expert_weights, "expert_weights"),
                 (row_of_pair, "row_of_pair")):
        _contig(t, n)
    if scale_layout not in ("rowmajor", "swizzled"):
        raise ValueError("scale_layout must be 'rowmajor' or 'swizzled'")
    if scale_layout == "swizzled":
        if not mxfp8:
            raise ValueError("the swizzled scale layout needs mxfp8=True")
        flags |= MX_SWIZZLED
    T, K = row_of_pair.shape
    rows, D = y_permuted.shape
    if tuple(expert_weights.shape) != (T, K):
        raise ValueError("expert_weights must be (T, K) like row_of_pair")
    if gamma is not None:
        _need(gamma, "gamma", torch.bfloat16, 1, device)
        _contig(gamma, "gamma")
        if gamma.numel() != D:
            raise ValueError("gamma must have D entries")
    if shared is not None:
        _need(shared, "shared", torch.bfloat16, 2, device)
        _contig(shared, "shared")
        if tuple(shared.shape) != (T, D):
            raise ValueError("shared must be (T, D)")
    return flags, T, K, rows, D


def _mx_outputs(T, D, flags, device, codes=None, scales=None):
    """MXFP8 output buffers: the caller's (checked) or new ones."""
    nbytes = _lib.load().moe_mxfp8_scale_bytes(T, D, flags)
    if codes is None:
        codes = torch.empty((T, D), dtype=torch.uint8, device=device)
    if scales is None:
        shape = (nbytes,) if flags & MX_SWIZZLED else (T, D // 32)
        scales = torch.empty(shape, dtype=torch.uint8, device=device)
    for t, n, numel in ((codes, "mx_codes", T * D), (scales, "mx_scales", nbytes)):
        _need(t, n, torch.uint8, None, device)
        _contig(t, n)
        if t.numel() < numel:
            raise ValueError(f"{n} needs {numel} bytes")
    return codes, scales


def moe_finalize_rmsnorm(y_permuted, expert_weights, row_of_pair, shared, gamma, eps,
                         flags=0, out=None, mxfp8=False, scale_layout="rowmajor",
                         mx_codes=None, mx_scales=None):
    """Weighted top-k reduction + shared add + RMSNorm (+ MXFP8).

    expert_weights may be fp32 or bf16 (the bf16-weight flag is set from the
    dtype). scale_layout "rowmajor" gives scales (T, D/32); "swizzled" gives
    the 128x4-tiled byte buffer with zeroed padding rows. Returns out (T, D)
    bf16, or (out, codes (T, D) uint8, scales uint8) with ``mxfp8``
    (written into mx_codes / mx_scales when given)."""
    if gamma is None:
        raise ValueError("gamma is required")
    flags, T, K, rows, D = _finalize_common(y_permuted, expert_weights, row_of_pair, shared,
                                            gamma, flags, mxfp8, scale_layout)
    device = y_permuted.device
    out = _out(out, "out", torch.bfloat16, (T, D), device)
    codes, scales = (_mx_outputs(T, D, flags, device, mx_codes, mx_scales) if mxfp8
                     else (None, None))
    _call("moe_finalize_rmsnorm",
        _ptr(y_permuted), rows, _ptr(expert_weights), _ptr(row_of_pair), _ptr(shared),
        _ptr(gamma), float(eps), T, K, D, int(flags), _ptr(out), _ptr(codes), _ptr(scales),
        _stream(device))
    return (out, codes, scales) if mxfp8 else out


def moe_finalize_mhc(y_permuted, expert_weights, row_of_pair, shared, residual, post, comb,
                     pre, gamma, eps, flags=0, residual_out=None, out=None, mxfp8=False,
                     scale_layout="rowmajor", mx_codes=None, mx_scales=None):
    """The finalize of a hyper-connection layer: routed sum h, mHC post-mix
    of the hc residual streams, pre-mix collapse, RMSNorm (+ MXFP8).

    residual (T, hc, D) bf16; post (T, hc) or (T, hc, 1) fp32; comb (T, hc, hc)
    fp32 indexed [source, target]; pre (T, hc) fp32, or None for residual
    only (then gamma is ignored and no layer input is produced). Returns
    (residual_out (T, hc, D) bf16, out (T, D) bf16 or None), plus codes and
    scales with ``mxfp8``."""
    if pre is None and mxfp8:
        raise ValueError("residual-only mode has no layer input to quantise")
    flags, T, K, rows, D = _finalize_common(y_permuted, expert_weights, row_of_pair, shared,
                                            gamma if pre is not None else None, flags, mxfp8,
                                            scale_layout)
    device = y_permuted.device
    _need(residual, "residual", torch.bfloat16, 3, device)
    _contig(residual, "residual")
    hc = residual.shape[1]
    if tuple(residual.shape) != (T, hc, D):
        raise ValueError("residual must be (T, hc, D)")
    for t, n, numel in ((post, "post", T * hc), (comb, "comb", T * hc * hc),
                        (pre, "pre", T * hc)):
        if t is None:
            continue
        _need(t, n, torch.float32, None, device)
        _contig(t, n)
        if t.numel() != numel or t.shape[0] != T:
            raise ValueError(f"{n} has the wrong shape")
    if pre is not None and gamma is None:
        raise ValueError("gamma is required with pre")
    residual_out = _out(residual_out, "residual_out", torch.bfloat16, (T, hc, D), device)
    if residual_out.numel() and residual_out.data_ptr() == residual.data_ptr():
        raise ValueError("residual_out must not alias residual")
    out = _out(out, "out", torch.bfloat16, (T, D), device) if pre is not None else None
    codes, scales = (_mx_outputs(T, D, flags, device, mx_codes, mx_scales) if mxfp8
                     else (None, None))
    _call("moe_finalize_mhc",
        _ptr(y_permuted), rows, _ptr(expert_weights), _ptr(row_of_pair), _ptr(shared),
        _ptr(residual), _ptr(post), _ptr(comb), _ptr(pre),
        _ptr(gamma) if pre is not None else 0, float(eps), T, K, D, hc, int(flags),
        _ptr(residual_out), _ptr(out), _ptr(codes), _ptr(scales), _stream(device))
    return (residual_out, out, codes, scales) if mxfp8 else (residual_out, out)


def moe_convert_check(values):
    """The kernels' device conversions of fp32 values: (bf16 bits as int16
    tensor, E4M3 codes of the +-448-clamped values as uint8)."""
    _need(values, "values", torch.float32, 1)
    _contig(values, "values")
    n = values.numel()
    bf = torch.empty(n, dtype=torch.int16, device=values.device)
    e4 = torch.empty(n, dtype=torch.uint8, device=values.device)
    _call("moe_convert_check", _ptr(values), n, _ptr(bf), _ptr(e4), _stream(values.device))
    return bf, e4


def moe_launch_floor(kind, T, D, src=None, dst=None, device=None):
    """A kernel with the finalize's launch shape for (T, D) that does nothing
    (kind 0) or two dependent 16-byte loads and a store per thread (kind 1):
    latency floors to time beside the finalize. For kind 1, ``src`` is an
    int32 tensor of 4 * n values (n = T * threads; the first of every 4 is an
    element index) and ``dst`` an int32 tensor of n; both made when None."""
    lib = _lib.load()
    threads = lib.moe_launch_floor_threads(T, D)
    if threads <= 0:
        raise ValueError(f"no finalize launch shape for T={T}, D={D}")
    n = T * threads
    device = device or (src.device if src is not None else torch.device("cuda", 0))
    if kind == 1:
        if src is None:
            src = torch.randint(0, n, (n, 4), dtype=torch.int32, device=device)
        if dst is None:
            dst = torch.empty(n, dtype=torch.int32, device=device)
        for t, nm, numel in ((src, "src", 4 * n), (dst, "dst", n)):
            _need(t, nm, torch.int32, device=device)
            _contig(t, nm)
            if t.numel() != numel:
                raise ValueError(f"{nm} must have {numel} elements")
    elif dst is None:
        dst = torch.empty(1, dtype=torch.int32, device=device)  # not written
    _call("moe_launch_floor", kind, T, D, _ptr(src if kind == 1 else None), _ptr(dst),
          _stream(device))
    return dst


def moe_stream_probe(R, W, units, src=None, dst=None, device=None, layout=0):
    """A plain contiguous stream of ``units`` waves, each reading R KiB and
    writing W KiB (each uint32 word written the wrapping sum of the R words
    at its position, xor the index of the destination KiB). layout 0: wave u
    reads R consecutive KiB of ``src`` and writes W consecutive KiB of
    ``dst``; layout 1: ``src`` holds R streams and ``dst`` W streams of
    ``units`` KiB, wave u reads and writes KiB u of each. Timed with a
    streaming kernel's read and write bytes it gives a reference rate for
    that mix. ``src`` is a uint8 tensor of at least units * R KiB, ``dst`` of
    at least units * W KiB; each is made when None. Returns dst."""
    device = device or (src.device if src is not None else torch.device("cuda", 0))
    if src is None:
        src = torch.zeros(units * R * 1024, dtype=torch.uint8, device=device)
    if dst is None:
        dst = torch.empty(units * W * 1024, dtype=torch.uint8, device=device)
    for t, nm, need in ((src, "src", units * R * 1024), (dst, "dst", units * W * 1024)):
        _need(t, nm, torch.uint8, device=device)
        _contig(t, nm)
        if t.numel() < need:
            raise ValueError(f"{nm} must hold at least {need} bytes (has {t.numel()})")
    _call("moe_stream_probe", layout, R, W, units, _ptr(src), _ptr(dst), _stream(device))
    return dst


# The pages' names for the same operations
gather_scale_dense_tokens = moe_gather_scale
gather_scale_quant_dense_tokens = moe_gather_scale_quant
scatter_add_dense_tokens = moe_scatter_add
scatter_add_padded_tokens = moe_scatter_add_padded
combine_shuffling = moe_combine_shuffling
split_shuffling = moe_split_shuffling
