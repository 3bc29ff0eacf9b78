"""The C ABI library on the CPU: it loads, exports every entry point the header
declares (with the binding's signature table covering each), and rejects bad
arguments on the host with the documented status before any HIP call (so
these calls run without a GPU). No compute call is made here."""
import ctypes
import os
import re

import pytest

from combine_moe_shuffle_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_shuffle.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x10000  # a 256-byte aligned non-NULL address; never dereferenced here


def _gpu_visible():
    import torch
    return torch.cuda.device_count() > 0


# The rejection tests pass fake device addresses that the host checks must
# refuse. Where a GPU is visible a wrong check would launch a kernel on them,
# so there these tests are skipped (they are host logic; the CPU runs them).
host_only = pytest.mark.skipif(_gpu_visible(), reason="fake device addresses: host-only")


def _declared():
    text = open(HEADER).read()
    return re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from combine_moe_shuffle_amd import build
        build.build()
    return _lib.load()


def test_header_declares_the_path(lib):
    names = set(_declared())
    for n in ("moe_shuffle", "moe_gather_scale", "moe_gather_scale_quant",
              "moe_scatter_add", "moe_finalize_rmsnorm"):
        assert n in names


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = _declared()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n                # exported by the .so
        assert n in _lib.SIGNATURES, n           # declared to ctypes


def test_signature_table_arity_matches_header(lib):
    text = open(HEADER).read()
    for name, (_, args) in _lib.SIGNATURES.items():
        m = re.search(rf"\b{name}\s*\(([^)]*)\)", text, re.S)
        assert m, name
        params = [p for p in m.group(1).split(",") if p.strip() not in ("", "void")]
        assert len(params) == len(args), (name, len(params), len(args))


def test_abi_version_and_status_strings(lib):
    assert lib.moe_abi_version() == 3
    assert lib.moe_status_str(0) == b"MOE_OK"
    assert lib.moe_status_str(3) == b"MOE_ERR_WORKSPACE"


def test_workspace_sizes(lib):
    # shuffle: T*K pair words + E*nblk histogram words, each region 256-aligned;
    # nblk = ceil(T/32), or ceil(T/16) for up to 128 tokens
    assert lib.moe_shuffle_workspace_bytes(8192, 256, 8) == 8192 * 8 * 4 + 256 * 256 * 4
    assert lib.moe_shuffle_workspace_bytes(65, 3, 2) == 768 + 256
    assert lib.moe_shuffle_workspace_bytes(100, 256, 8) == 3328 + 256 * 7 * 4
    assert lib.moe_shuffle_workspace_bytes(129, 256, 8) == 4352 + 256 * 5 * 4  # 4128 aligned
    assert lib.moe_shuffle_workspace_bytes(-1, 3, 2) == 0
    # scatter: (T+1) starts + a list entries, then (a <= 131072 rows, at most
    # 2048 ranges of 128 tokens) a (row, token) pairs and two [range][chunk of
    # 1024 rows] int matrices, else a slots
    assert lib.moe_scatter_add_workspace_bytes(8192, 65536) == (33024 + 262144 + 524288 +
                                                               2 * 64 * 64 * 4)
    assert lib.moe_scatter_add_workspace_bytes(1000, 200000) == (4096 + 800000 + 800000)


def _err(lib):
    return lib.moe_last_error().decode()


@host_only
def test_stream_probe_rejects(lib):
    f = lib.moe_stream_probe
    assert f(2, 1, 1, 4, FAKE, FAKE + (1 << 20), None) == INVALID
    assert "layout" in _err(lib)
    assert f(0, 0, 1, 4, FAKE, FAKE + (1 << 20), None) == INVALID
    assert "R must be" in _err(lib)
    assert f(1, 33, 1, 4, FAKE, FAKE + (1 << 20), None) == INVALID
    assert f(0, 1, 0, 4, FAKE, FAKE + (1 << 20), None) == INVALID
    assert "W must be" in _err(lib)
    assert f(1, 1, 33, 4, FAKE, FAKE + (1 << 20), None) == INVALID
    assert f(0, 1, 1, -1, FAKE, FAKE + (1 << 20), None) == INVALID
    assert f(0, 1, 1, 1 << 31, FAKE, FAKE + (1 << 20), None) == INVALID
    assert f(0, 1, 1, 4, None, FAKE, None) == INVALID
    assert f(1, 1, 1, 4, FAKE + 8, FAKE + (1 << 20), None) == INVALID
    assert "aligned" in _err(lib)
    # 4 waves of 2 KiB read from FAKE reach FAKE + 8 KiB: a dst inside overlaps
    assert f(0, 2, 1, 4, FAKE, FAKE + 8192 - 1024, None) == INVALID
    assert "overlap" in _err(lib)
    assert f(1, 1, 2, 4, FAKE + 8192 - 1024, FAKE, None) == INVALID
    # nothing to do: OK without touching anything
    assert f(0, 1, 1, 0, None, None, None) == OK


@host_only
def test_shuffle_rejects(lib):
    f = lib.moe_shuffle
    # K > E
    assert f(FAKE, 8, 1, 4, 8, 9, None, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == INVALID
    assert "K must be" in _err(lib)
    # E too large
    assert f(FAKE, 2048, 1, 4, 2048, 8, None, FAKE, FAKE, FAKE, None, FAKE, 1 << 20,
             None) == UNSUPPORTED
    # K too large
    assert f(FAKE, 128, 1, 4, 128, 65, None, FAKE, FAKE, FAKE, None, FAKE, 1 << 20,
             None) == UNSUPPORTED
    # workspace too small / NULL
    assert f(FAKE, 8, 1, 64, 8, 2, None, FAKE, FAKE, FAKE, None, FAKE, 16, None) == WORKSPACE
    assert f(FAKE, 8, 1, 64, 8, 2, None, FAKE, FAKE, FAKE, None, None, 1 << 20,
             None) == WORKSPACE
    # NULL scores, NULL counts, negative stride, misaligned workspace
    assert f(None, 8, 1, 64, 8, 2, None, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == INVALID
    assert f(FAKE, 8, 1, 64, 8, 2, None, None, FAKE, FAKE, None, FAKE, 1 << 20, None) == INVALID
    assert f(FAKE, -8, 1, 64, 8, 2, None, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == INVALID
    assert f(FAKE, 8, 1, 64, 8, 2, None, FAKE, FAKE, FAKE, None, FAKE + 4, 1 << 20,
             None) == INVALID
    # T*K overflow
    assert f(FAKE, 64, 1, 1 << 30, 64, 8, None, FAKE, FAKE, FAKE, None, FAKE, 1 << 20,
             None) == INVALID


@host_only
def test_shuffle_noalloc_rejects(lib):
    f = lib.moe_shuffle_noalloc
    # the workspace the sizes need exceeds the static scratch: refused before
    # any HIP call
    assert f(FAKE, 256, 1, 1 << 20, 256, 8, None, FAKE, FAKE, FAKE, None, None) == WORKSPACE
    assert "scratch" in _err(lib)
    # the shuffle's own checks come first
    assert f(FAKE, 8, 1, 4, 8, 9, None, FAKE, FAKE, FAKE, None, None) == INVALID
    assert f(FAKE, 2048, 1, 4, 2048, 8, None, FAKE, FAKE, FAKE, None, None) == UNSUPPORTED
    assert f(FAKE, 8, 1, 64, 8, 2, None, None, FAKE, FAKE, None, None) == INVALID


@host_only
def test_gather_rejects(lib):
    g = lib.moe_gather_scale
    # D % 8
    assert g(FAKE, 4, 12, FAKE, FAKE, 8, FAKE, 4, 1, 4, None, FAKE, None, 0, None) == INVALID
    assert "multiple of 8" in _err(lib)
    assert g(FAKE + 8, 4, 16, FAKE, FAKE, 8, FAKE, 4, 1, 4, None, FAKE, None, 0, None) == INVALID
    assert g(FAKE, 4, 16, None, FAKE, 8, FAKE, 4, 1, 4, None, FAKE, None, 0, None) == INVALID
    # E
    assert g(FAKE, 4, 16, FAKE, FAKE, 8, FAKE, 4, 1, 0, None, FAKE, None, 0, None) == INVALID
    assert g(FAKE, 4, 16, FAKE, FAKE, -1, FAKE, 4, 1, 4, None, FAKE, None, 0, None) == INVALID
    # nothing to do: OK without touching anything
    assert g(None, 0, 16, None, None, 0, None, 4, 1, 4, None, None, None, 0, None) == OK
    assert g(None, 4, 0, None, None, 8, None, 4, 1, 4, None, None, None, 0, None) == OK
    need = lib.moe_gather_scale_workspace_bytes(4, 8)
    assert need == lib.moe_scatter_add_workspace_bytes(4, 8)
    assert g(FAKE, 4, 16, FAKE, FAKE, 8, FAKE, 4, 1, 4, None, FAKE, FAKE, need - 1,
             None) == WORKSPACE
    assert g(FAKE, 4, 16, FAKE, FAKE, 8, FAKE, 4, 1, 4, None, FAKE, FAKE + 4, need,
             None) == INVALID  # workspace alignment
    bt = lib.moe_gather_scale_by_token
    assert bt(FAKE, 4, 16, FAKE, 0, FAKE, 8, FAKE, 4, 1, 4, None, FAKE, None) == INVALID
    assert bt(FAKE, 4, 16, FAKE, 65, FAKE, 8, FAKE, 4, 1, 4, None, FAKE, None) == INVALID
    q = lib.moe_gather_scale_quant
    assert q(FAKE, 4, 16, FAKE, FAKE, 8, FAKE, 4, 1, 4, None, None, FAKE, None,
             None) == INVALID  # out_scale NULL
    assert q(FAKE, 4, 1 << 17, FAKE, FAKE, 8, FAKE, 4, 1, 4, None, None, FAKE, FAKE,
             None) == UNSUPPORTED
    assert q(FAKE, 4, 16, FAKE, FAKE, 8, FAKE, 4, 1, 4, FAKE + 2, None, FAKE, FAKE,
             None) == INVALID  # misaligned scale_ub


@host_only
def test_scatter_rejects(lib):
    s = lib.moe_scatter_add
    assert s(FAKE, 8, FAKE, FAKE, 16, 64, None, FAKE, 16, None) == WORKSPACE
    assert s(FAKE, 8, FAKE, None, 16, 64, None, FAKE, 1 << 20, None) == INVALID
    assert s(FAKE, 8, FAKE, FAKE, 16, 60, None, FAKE, 1 << 20, None) == INVALID
    assert s(FAKE, 8, FAKE + 16, FAKE, 16, 64, None, FAKE + 8, 1 << 20, None) == INVALID
    assert s(None, 8, None, None, 0, 64, None, None, 0, None) == OK       # a == 0
    b = lib.moe_scatter_add_by_token
    assert b(FAKE, 8, FAKE, None, 2, 16, 64, None, None) == INVALID
    assert b(FAKE, 8, FAKE, FAKE, 0, 16, 64, None, None) == INVALID


@host_only
def test_scatter_padded_rejects(lib):
    p = lib.moe_scatter_add_padded
    ws = 1 << 22
    assert p(FAKE, 3, 64, FAKE, 8, FAKE, FAKE, 16, 64, FAKE, ws, None) == INVALID   # E % EP
    assert p(FAKE, 2, 64, FAKE, 2048, FAKE, FAKE, 16, 64, FAKE, ws, None) == UNSUPPORTED
    assert p(FAKE, 2, 64, FAKE, 8, FAKE, FAKE, 16, 60, FAKE, ws, None) == INVALID   # D % 8
    assert p(FAKE, 2, 64, None, 8, FAKE, FAKE, 16, 64, FAKE, ws, None) == INVALID
    assert p(FAKE, 2, 64, FAKE, 8, FAKE, FAKE, 16, 64, FAKE, 8, None) == WORKSPACE
    assert p(FAKE, 1 << 10, 1 << 22, FAKE, 1 << 10, FAKE, FAKE, 16, 64, FAKE, ws,
             None) == INVALID                                                     # EP*T_K
    assert p(None, 2, 0, None, 8, None, None, 16, 64, None, 0, None) == OK        # T_K == 0
    # expert prefix, starts, list, (row, token) pairs, two 1x1 matrices
    assert lib.moe_scatter_add_padded_workspace_bytes(16, 64, 8) == 256 + 256 + 256 + 512 + \
        2 * 256


@host_only
def test_scatter_padded_by_token_rejects(lib):
    p = lib.moe_scatter_add_padded_by_token
    # (in, EP, T_K, counts, E, row_of_pair, K, out, T, D, stream)
    assert p(FAKE, 3, 64, FAKE, 8, FAKE, 2, FAKE, 16, 64, None) == INVALID        # E % EP
    assert p(FAKE, 2, 64, FAKE, 2048, FAKE, 2, FAKE, 16, 64, None) == UNSUPPORTED
    assert p(FAKE, 2, 64, FAKE, 8, FAKE, 0, FAKE, 16, 64, None) == INVALID        # K
    assert "K must be" in _err(lib)
    assert p(FAKE, 2, 64, FAKE, 8, FAKE, 65, FAKE, 16, 64, None) == INVALID
    assert p(FAKE, 2, 64, FAKE, 8, FAKE, 2, FAKE, 16, 60, None) == INVALID        # D % 8
    assert p(FAKE, 2, 64, None, 8, FAKE, 2, FAKE, 16, 64, None) == INVALID
    assert p(FAKE, 2, 64, FAKE, 8, None, 2, FAKE, 16, 64, None) == INVALID
    assert p(FAKE, 1 << 10, 1 << 22, FAKE, 1 << 10, FAKE, 2, FAKE, 16, 64,
             None) == INVALID                                                     # EP*T_K
    assert p(None, 2, 0, None, 8, None, 2, None, 16, 64, None) == OK              # T_K == 0


@host_only
def test_shuffling_rejects(lib):
    c, sp = lib.moe_combine_shuffling, lib.moe_split_shuffling
    ws = 1 << 22
    args = [FAKE, 64, FAKE, 64, 64, FAKE, 4, 8, 0, 8, -1, FAKE, FAKE, ws, None]

    def call(f, **kw):
        a = list(args)
        names = ["in_", "in_rows", "out", "out_rows", "D", "counts", "EP", "C", "lo", "hi",
                 "stride", "oc", "ws", "wsb", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    assert call(c, EP=0) == UNSUPPORTED
    assert call(c, EP=65) == UNSUPPORTED
    assert call(c, lo=5, hi=4) == INVALID
    assert call(c, hi=9) == INVALID
    assert call(c, C=4096, hi=4096, EP=2) == UNSUPPORTED      # 8192 segments > 4096
    assert call(c, D=60) == INVALID
    assert call(c, counts=None) == INVALID
    assert call(c, oc=None) == INVALID                        # required for combine
    assert call(c, wsb=8) == WORKSPACE
    assert call(c, in_=FAKE + 8) == INVALID
    assert call(c, stride=1 << 30) == INVALID                 # EP * stride >= 2^31
    assert call(sp, in_rows=1 << 31) == INVALID
    assert lib.moe_shuffling_workspace_bytes(4, 8, 64) == 2 * 256 + 256


@host_only
def test_finalize_rejects(lib):
    f = lib.moe_finalize_rmsnorm
    args = dict(y=FAKE, rows=64, w=FAKE, rop=FAKE, sh=FAKE, g=FAKE, eps=1e-6, T=8, K=8,
                D=256, flags=0, out=FAKE, mc=None, ms=None)

    def call(**kw):
        a = {**args, **kw}
        return f(a["y"], a["rows"], a["w"], a["rop"], a["sh"], a["g"], a["eps"], a["T"],
                 a["K"], a["D"], a["flags"], a["out"], a["mc"], a["ms"], None)

    assert call(mc=FAKE) == INVALID                       # codes without scales
    assert call(mc=FAKE, ms=FAKE, D=264) == INVALID       # D % 32 for MXFP8
    assert call(flags=8) == INVALID                       # unknown bit
    assert call(flags=4) == INVALID                       # swizzled scales without MXFP8
    assert call(flags=4, mc=FAKE, ms=FAKE, D=288) == INVALID  # swizzled needs D % 128
    assert call(flags=2, w=FAKE + 2, T=0) == OK           # bf16 weights: 2-byte alignment
    assert lib.moe_mxfp8_scale_bytes(130, 512, 0) == 130 * 16
    assert lib.moe_mxfp8_scale_bytes(130, 512, 4) == 256 * 16
    assert lib.moe_mxfp8_scale_bytes(1, 128, 4) == 128 * 4
    assert call(K=0) == INVALID
    assert call(K=65) == UNSUPPORTED
    assert call(D=1 << 17) == UNSUPPORTED
    assert call(g=None) == INVALID
    assert call(sh=FAKE + 8) == INVALID
    assert call(T=0) == OK


@host_only
def test_finalize_mhc_rejects(lib):
    f = lib.moe_finalize_mhc
    args = dict(y=FAKE, rows=64, w=FAKE, rop=FAKE, sh=FAKE, res=FAKE, post=FAKE, comb=FAKE,
                pre=FAKE, g=FAKE, eps=1e-6, T=8, K=8, D=256, hc=4, flags=0, ro=FAKE,
                out=FAKE, mc=None, ms=None)

    def call(**kw):
        a = {**args, **kw}
        return f(a["y"], a["rows"], a["w"], a["rop"], a["sh"], a["res"], a["post"], a["comb"],
                 a["pre"], a["g"], a["eps"], a["T"], a["K"], a["D"], a["hc"], a["flags"],
                 a["ro"], a["out"], a["mc"], a["ms"], None)

    assert call(hc=0) == INVALID
    assert call(hc=5) == UNSUPPORTED
    assert call(pre=None) == INVALID                      # residual only: out must be NULL
    assert call(pre=None, out=None, mc=FAKE, ms=FAKE) == INVALID  # and no MXFP8
    assert call(pre=None, out=None, g=None, T=0) == OK
    assert call(mc=FAKE) == INVALID                       # codes without scales
    assert call(flags=8) == INVALID
    assert call(flags=4) == INVALID                       # swizzled scales without MXFP8
    assert call(D=260) == INVALID                         # D % 8
    assert call(D=1 << 16) == UNSUPPORTED
    assert call(K=65) == UNSUPPORTED
    assert call(res=None) == INVALID
    assert call(comb=None) == INVALID
    assert call(ro=None) == INVALID
    assert call(g=None) == INVALID                        # gamma needed with pre
    assert call(ro=FAKE + 8) == INVALID                   # 16-byte rows
    assert call(post=FAKE + 2) == INVALID
    assert call(T=0) == OK


@host_only
def test_convert_rejects(lib):
    assert lib.moe_convert_check(None, 4, None, None, None) == INVALID
    assert lib.moe_convert_check(None, 0, None, None, None) == OK


def test_ops_raise_without_gpu_tensors():
    import torch

    from combine_moe_shuffle_amd import ops
    with pytest.raises(ValueError):
        ops.moe_gather_scale(torch.zeros(4, 16, dtype=torch.bfloat16),
                             torch.zeros(8, dtype=torch.int32),
                             torch.zeros(8, dtype=torch.int32), torch.zeros(4, 2))


def test_fast_call_module_covers_every_launching_entry_point(lib):
    """The compiled fast-call extension wraps every status-returning entry
    point of the signature table, with the same arity."""
    fast = _lib.fast()
    assert fast is not None, "the fast-call extension is built with the library"
    for name, (res, args) in _lib.SIGNATURES.items():
        if res is not ctypes.c_int or not args:
            continue
        f = getattr(fast, name)
        with pytest.raises(TypeError):
            f(*([0] * (len(args) - 1)))  # one argument short


@host_only
def test_fast_call_rejects_like_ctypes(lib):
    """Host-side rejections give the same status and message through the
    extension as through ctypes."""
    fast = _lib.fast()
    calls = [
        ("moe_finalize_rmsnorm",
         (FAKE, 64, FAKE, FAKE, 0, FAKE, 1e-6, 8, 65, 256, 0, FAKE, 0, 0, 0)),
        ("moe_shuffle", (FAKE, 8, 1, 4, 8, 9, 0, FAKE, FAKE, FAKE, 0, FAKE, 1 << 20, 0)),
        ("moe_scatter_add", (FAKE, 8, FAKE, FAKE, 16, 64, 0, FAKE, 16, 0)),
    ]
    for name, args in calls:
        s_fast = getattr(fast, name)(*args)
        m_fast = fast.last_error()
        s_ct = getattr(lib, name)(*args)
        m_ct = lib.moe_last_error().decode()
        assert s_fast == s_ct != OK and m_fast == m_ct, name


def test_prepare_records_and_replays_library_calls(monkeypatch):
    """ops.prepare: the op runs once with its checks; each replay repeats the
    recorded library calls with the same arguments and the then-current
    stream, keeps alive every tensor whose address a call takes (workspaces
    the op allocated itself included) and returns the op's result."""
    import gc
    import weakref

    import torch

    from combine_moe_shuffle_amd import ops

    seen = []

    def entry(*args):
        seen.append(args)
        return 0

    monkeypatch.setattr(_lib, "fn", lambda name: entry)
    streams = iter([11, 22, 33])
    monkeypatch.setattr(ops, "_stream", lambda device: next(streams))
    refs = []

    def op(t):
        scratch = torch.empty(16, dtype=torch.uint8)   # the op's own workspace
        refs.append(weakref.ref(scratch))
        ops._call("moe_a", ops._ptr(t), 7, ops._ptr(scratch), ops._stream(t.device))
        ops._call("moe_b", ops._ptr(t), 2.5, ops._stream(t.device))
        return t

    x = torch.zeros(4)
    p = ops.prepare(op, x)
    gc.collect()
    assert refs[0]() is not None, "the op's workspace must outlive the op"
    assert len(seen) == 2                                # the set-up run
    assert p() is x
    assert seen[2][:-1] == seen[0][:-1] and seen[3][:-1] == seen[1][:-1]
    assert seen[2][-1] == seen[3][-1] == 33              # the replay's stream
    assert seen[0][2] == refs[0]().data_ptr()
    del p
    gc.collect()
    assert refs[0]() is None

    with pytest.raises(ValueError, match="no library call"):
        ops.prepare(lambda: None)

    def nested():
        ops.prepare(op, x)
    with pytest.raises(RuntimeError, match="does not nest"):
        ops.prepare(nested)
    assert getattr(ops._rec, "calls", None) is None

    # a call made by another thread while prepare() runs is not recorded
    import threading
    other = threading.Thread(target=lambda: ops._call("moe_c", 1, 0))

    def op_with_thread(t):
        other.start()
        other.join()
        ops._call("moe_a", ops._ptr(t), ops._stream(t.device))
        return t
    monkeypatch.setattr(ops, "_stream", lambda device: 44)
    n0 = len(seen)
    p = ops.prepare(op_with_thread, x)
    assert len(seen) == n0 + 2                     # both calls ran once
    p()
    assert seen[-1] == seen[-2] and seen[-1][0] == x.data_ptr()   # only moe_a replayed
