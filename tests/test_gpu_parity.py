"""GPU parity: every stage through the C ABI against the CPU oracle, on the
same seeded inputs.

Bar: integer outputs (shuffle) and the bf16 gather are bit-exact; the combine
is designed bit-exact (same fp32 addition order as the oracle); the finalize
output must be within |gpu - ref| <= 2e-2 + 1e-2 * |ref| and is designed
bit-exact too (both sides take the row's sum of squares in fp64 and round it
once to fp32, so the kernel's tree and the oracle's sequence agree); FP8 and
MXFP8 codes may differ by at most one code on at most 0.1 % of elements
(expected exact). MXFP8 is checked twice: end to end against the oracle's
own codes and scales, and split (the oracle quantising the GPU's own bf16
output), which separates quantiser parity from RMSNorm rounding.

Sizes: small shapes spanning several slices and a ragged tail, the edge cases
(empty, single token, K = E, valid count 0 / T / beyond T, ties, strided
scores, tokens with more than 64 rows), and the full workload sizes in the
launch configuration the benchmark times.
"""
import os

import numpy as np
import pytest
import torch

import oracle as orc
from combine_moe_shuffle_amd import ops
from combine_moe_shuffle_amd import workloads as W

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5A5


def say(*a):
    print("[gpu-case]", *a, flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    from combine_moe_shuffle_amd import _lib
    _lib.load()
    return torch.device("cuda:0")


def bf_dev(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def bits_host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def i32_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def scalar_dev(v, dev):
    return None if v is None else torch.tensor([v], dtype=torch.int32, device=dev)


def ordinal(codes):
    """E4M3 sign-magnitude code -> monotone integer."""
    c = codes.astype(np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def assert_fp8_close(got, want, what):
    d = np.abs(ordinal(got) - ordinal(want))
    bad = d > 0
    assert d.max(initial=0) <= 1, f"{what}: code distance {d.max()}"
    assert bad.mean() <= 1e-3, f"{what}: {bad.mean():.2e} of codes differ"


# ---------------------------------------------------------------- conversions
def test_device_conversions_match_oracle_encoders(dev):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    allbf = orc.bf16_to_f32(h)
    allbf = allbf[np.isfinite(allbf)]
    g = np.random.default_rng(5)
    rnd = g.integers(0, 2**32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    rnd[:100_000] = (rnd[:100_000] & 0xFFFF0000) | 0x8000          # bf16 ties
    rnd = rnd.view(np.float32)
    rnd = rnd[np.isfinite(rnd)]
    vals = np.concatenate([allbf * np.float32(s) for s in (1.0, 0.125, 3.7, 1e-3, 97.0,
                                                             2.0 ** -12)] + [rnd])
    vals = vals.astype(np.float32)
    say("convert_check", vals.size)
    bf, e4 = ops.moe_convert_check(torch.from_numpy(vals).to(dev))
    bf = bf.cpu().numpy().view(np.uint16)
    e4 = e4.cpu().numpy()
    fin = np.isfinite(vals)
    assert np.array_equal(bf[fin], orc.f32_to_bf16(vals)[fin])
    clipped = np.clip(vals, -448.0, 448.0).astype(np.float32)
    assert np.array_equal(e4[fin], orc.f32_to_e4m3(clipped)[fin])


def test_launch_floor_kernels(dev):
    """The latency-floor kernels of the finalize's launch shape run, and the
    two-load kernel computes dst[i] = sum of the words of src[src[i].x % n]."""
    from combine_moe_shuffle_amd import _lib
    lib = _lib.load()
    for T, D in ((1, 7168), (128, 7168), (5, 1024)):
        threads = lib.moe_launch_floor_threads(T, D)
        assert threads % 64 == 0 and 64 <= threads <= 1024
        n = T * threads
        g = np.random.default_rng(T)
        src = g.integers(0, 1 << 20, size=(n, 4)).astype(np.int32)
        say("launch floor", T, D, threads)
        dst = ops.moe_launch_floor(1, T, D, src=torch.from_numpy(src).to(dev))
        ops.moe_launch_floor(0, T, D, device=dev)
        torch.cuda.synchronize()
        pick = src[src[:, 0].astype(np.uint32) % n]
        want = pick.astype(np.uint32).sum(axis=1, dtype=np.uint32).view(np.int32)
        assert np.array_equal(dst.cpu().numpy(), want)


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("R,W,units", [(1, 1, 1), (9, 1, 1001), (1, 8, 999), (32, 32, 6),
                                       (10, 3, 257)])
def test_stream_probe(dev, R, W, units, layout):
    """The contiguous-stream aid writes the wave's w-th destination KiB as
    the wrapping uint32 sum (word by word) of its R source KiB, xor w, with
    the KiB of wave u at u*R + r / u*W + w (blocked) or r*units + u /
    w*units + u (interleaved), and nothing past units * W KiB."""
    g = np.random.default_rng(R * 100 + W)
    src = g.integers(0, 1 << 32, size=units * R * 256, dtype=np.uint32)
    extra = 4096
    dst = torch.full((units * W * 1024 + extra,), 0xA5, dtype=torch.uint8, device=dev)
    say("stream probe", layout, R, W, units)
    ops.moe_stream_probe(R, W, units, src=torch.from_numpy(src.view(np.uint8)).to(dev),
                         dst=dst, layout=layout)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    body = got[:units * W * 1024].view(np.uint32)
    if layout == 0:
        acc = np.add.reduce(src.reshape(units, R, 256), axis=1, dtype=np.uint32)
        body = body.reshape(units, W, 256).transpose(1, 0, 2)
    else:
        acc = np.add.reduce(src.reshape(R, units, 256), axis=0, dtype=np.uint32)
        body = body.reshape(W, units, 256)
    want = acc[None, :, :] ^ np.arange(W, dtype=np.uint32)[:, None, None]
    assert np.array_equal(body, want)
    assert np.all(got[units * W * 1024:] == 0xA5)


# ---------------------------------------------------------------- shuffle
SHUFFLE_CASES = [
    # (name, T, E, K, vtc, score kind)
    ("tiny-workload", None, None, None, None, "tiny"),
    ("quant-workload", None, None, None, None, "quant"),
    ("zipf-workload", None, None, None, 6000, "zipf"),
    ("single", 1, 1, 1, None, "normal"),
    ("K=E", 63, 8, 8, None, "normal"),
    ("ragged", 200, 257, 3, 137, "normal"),
    ("wide", 130, 1024, 64, None, "normal"),
    ("ties", 300, 40, 6, 250, "ties"),
    ("strided", 150, 48, 5, None, "strided"),
    ("vtc0", 100, 16, 2, 0, "normal"),
    ("vtc-beyond", 100, 16, 2, 99999, "normal"),
    ("vtc-negative", 100, 16, 2, -5, "normal"),
    ("T0", 0, 16, 2, None, "normal"),
    ("large-T", 70000, 64, 4, 65000, "normal"),
    # histogram sizes E * ceil(T/32) around the one-launch scan-and-place limit
    ("hist-8192", 1024, 256, 8, 1000, "normal"),
    ("hist-8448", 1056, 256, 8, 1000, "normal"),
    # more than 4096 blocks of 32 tokens; experts of ~10000 rows; E not a
    # multiple of 8
    ("many-blocks", 140000, 8, 2, 139000, "normal"),
    ("big-experts", 20000, 2, 1, None, "normal"),
    ("E12", 3000, 12, 3, 2900, "normal"),
    # the one-launch form (up to 32 tokens; up to 64 when K * ceil(E/64) <= 8
    # and E <= 256) with 1, 2 and 4 tokens per wave, and just past its limits
    ("small-ties", 64, 40, 6, 50, "ties"),
    ("small-T64-E128-K4", 64, 128, 4, 60, "ties"),
    ("small-top64", 32, 256, 64, None, "normal"),
    ("small-strided", 33, 48, 5, None, "strided"),
    ("small-vtc0", 10, 16, 2, 0, "normal"),
    ("small-E384", 32, 384, 8, 30, "normal"),
    ("small-E1024-top64", 16, 1024, 64, None, "ties"),
    ("small-T17", 17, 256, 8, None, "normal"),
    ("T64-E256-K8", 64, 256, 8, 50, "normal"),
    ("T65", 65, 256, 8, None, "normal"),
    ("E257-T64", 64, 257, 3, 60, "normal"),
    ("E300-T33", 33, 300, 4, None, "strided"),
]


def _scores_for(kind, T, E, seed=0):
    g = np.random.default_rng(seed)
    if kind == "ties":
        s = g.integers(0, 4, size=(T, E)).astype(np.float32)
        s[g.random((T, E)) < 0.3] = -0.0
        return s
    if kind == "strided":
        return g.standard_normal((E, T)).astype(np.float32).T   # (T, E) view
    return g.standard_normal((T, E)).astype(np.float32)


@pytest.mark.parametrize("case", SHUFFLE_CASES, ids=[c[0] for c in SHUFFLE_CASES])
def test_shuffle_bit_exact(dev, case):
    name, T, E, K, vtc, kind = case
    if kind in W.WORKLOADS:
        wl = W.WORKLOADS[kind]
        s = W.router_scores(wl)
        T, E, K = wl.T, wl.E, wl.K
    else:
        s = _scores_for(kind, T, E)
    say("shuffle", name, T, E, K, vtc)
    counts, ei, ti, rop = orc.shuffle(s, K, vtc)
    if kind == "strided":
        base = torch.from_numpy(np.ascontiguousarray(s.T)).to(dev)
        sd = base.t()                                  # strides (1, T)
    else:
        sd = torch.from_numpy(np.ascontiguousarray(s)).to(dev)
    gc, gei, gti, grop = ops.moe_shuffle(sd, K, scalar_dev(vtc, dev))
    assert np.array_equal(gc.cpu().numpy(), counts)
    assert np.array_equal(gei.cpu().numpy(), ei)
    assert np.array_equal(gti.cpu().numpy(), ti)
    assert np.array_equal(grop.cpu().numpy(), rop)
    # deterministic: a second run gives the same bits
    gc2, gei2, gti2, grop2 = ops.moe_shuffle(sd, K, scalar_dev(vtc, dev))
    assert torch.equal(gti, gti2) and torch.equal(grop, grop2)


# ---------------------------------------------------------------- gather
GATHER_CASES = [
    # (name, T, D, E, K, vtc)
    ("tiny-workload", 64, 1024, 8, 2, None),
    ("ragged-D", 77, 8 * (64 * 7 + 3), 9, 3, 70),      # partial last slice
    ("short-row", 33, 8, 4, 2, None),                  # one chunk per row
    ("odd", 129, 8 * 1000, 13, 4, 100),
    ("vtc0", 16, 512, 4, 2, 0),
    ("K16", 40, 8 * 70, 32, 16, 30),                   # four groups of rows in flight
    ("K64", 10, 256, 64, 64, None),                    # a full wave of rows per token
]


def _dispatch_case(T, D, E, K, vtc, seed=0):
    wl = W.WORKLOADS["tiny"]
    wl = W.Workload(**{**wl.__dict__, "router": "softmax"})
    inp = W.dispatch_inputs(wl, T=T, D=D, E=E, K=K, vtc=vtc, seed=seed, out0="normal")
    counts, ei, ti, rop = orc.shuffle(inp.scores, K, vtc)
    return inp, counts, ei, ti, rop


@pytest.mark.parametrize("case", GATHER_CASES, ids=[c[0] for c in GATHER_CASES])
@pytest.mark.parametrize("path", ["lists", "rows", "by_token"])
def test_gather_scale_bit_exact(dev, case, path):
    name, T, D, E, K, vtc = case
    inp, counts, ei, ti, rop = _dispatch_case(T, D, E, K, vtc)
    V = int(counts[E])
    say("gather", path, name, T, D, E, K, V)
    want = np.full((T * K, D), SENTINEL, np.uint16)
    orc.gather_scale(inp.x, ti, ei, inp.scores, V, want)
    out = torch.full((T * K, D), SENTINEL - 65536, dtype=torch.int16,
                     device=dev).view(torch.bfloat16)
    x = bf_dev(inp.x, dev)
    s = torch.from_numpy(inp.scores).to(dev)
    vr = scalar_dev(V, dev)
    if path != "by_token":
        ops.moe_gather_scale(x, i32_dev(ti, dev), i32_dev(ei, dev), s, vr, out,
                             row_order=path == "rows")
    else:
        ops.moe_gather_scale_by_token(x, i32_dev(rop, dev), i32_dev(ei, dev), s, vr, out)
    assert np.array_equal(bits_host(out), want)


@pytest.mark.parametrize("ub", [None, 1200.0, 1e-3])
@pytest.mark.parametrize("shape", [(96, 8 * (64 * 5 + 7), 6, 2, 90), (40, 5120, 16, 1, None),
                                   (20, 8, 3, 2, None), (6, 65536, 4, 1, None),
                                   (30, 8 * 637, 16, 2, 25)],
                         ids=["ragged", "D5120", "D8", "Dmax", "one-wave-ragged"])
def test_gather_scale_quant(dev, ub, shape):
    T, D, E, K, vtc = shape
    inp, counts, ei, ti, rop = _dispatch_case(T, D, E, K, vtc, seed=3)
    x = inp.x.copy()
    x[ti[0]] = 0                                   # an all-zero row
    V = int(counts[E])
    say("quant", shape, ub, V)
    wc = np.full((T * K, D), 0x5A, np.uint8)
    ws = np.full(T * K, -7.0, np.float32)
    orc.gather_scale_quant(x, ti, ei, inp.scores, ub, V, wc, ws)
    codes = torch.full((T * K, D), 0x5A, dtype=torch.uint8, device=dev)
    scale = torch.full((T * K,), -7.0, dtype=torch.float32, device=dev)
    ubd = None if ub is None else torch.tensor([ub], dtype=torch.float32, device=dev)
    ops.moe_gather_scale_quant(bf_dev(x, dev), i32_dev(ti, dev), i32_dev(ei, dev),
                               torch.from_numpy(inp.scores).to(dev), ubd, scalar_dev(V, dev),
                               codes, scale)
    gc, gs = codes.cpu().numpy(), scale.cpu().numpy()
    assert np.array_equal(gs.view(np.uint32), ws.view(np.uint32))   # scales exact
    assert np.array_equal(gc[V:], wc[V:])                            # untouched rows
    assert_fp8_close(gc[:V], wc[:V], "rowwise fp8")
    assert np.array_equal(gc, wc)                                    # expected exact


# ---------------------------------------------------------------- scatter
@pytest.mark.parametrize("case", GATHER_CASES, ids=[c[0] for c in GATHER_CASES])
@pytest.mark.parametrize("path", ["general", "by_token"])
def test_scatter_add_bit_exact(dev, case, path):
    name, T, D, E, K, vtc = case
    inp, counts, ei, ti, rop = _dispatch_case(T, D, E, K, vtc, seed=1)
    V = int(counts[E])
    say("scatter", path, name, T, D, K, V)
    want = orc.scatter_add(inp.out0.copy(), inp.y, ti, V)
    out = bf_dev(inp.out0, dev)
    y = bf_dev(inp.y, dev)
    if path == "general":
        ops.moe_scatter_add(out, y, i32_dev(ti, dev), scalar_dev(V, dev))
    else:
        ops.moe_scatter_add_by_token(out, y, i32_dev(rop, dev), scalar_dev(V, dev))
    assert np.array_equal(bits_host(out), want)


def test_scatter_add_general_long_lists(dev):
    """Arbitrary token_indices: a token owning 100 rows (beyond one wave's
    sort), unsorted rows, rows of no token."""
    g = np.random.default_rng(9)
    T, D, a = 12, 8 * 70, 400
    ti = g.integers(0, T, size=a).astype(np.int32)
    ti[g.permutation(a)[:100]] = 5
    y = W.to_bf16_bits(g.standard_normal((a, D)).astype(np.float32))
    out0 = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    V = 350
    say("scatter long lists", T, D, a, V)
    want = orc.scatter_add(out0.copy(), y, ti, V)
    out = bf_dev(out0, dev)
    ops.moe_scatter_add(out, bf_dev(y, dev), i32_dev(ti, dev), scalar_dev(V, dev))
    assert np.array_equal(bits_host(out), want)


@pytest.mark.parametrize("V", [2997, 3000, 3001])
def test_token_lists_unaligned_indices(dev, V):
    """The row lists of the general combine and gather built from a
    token_indices array that is 4- but not 16-byte aligned and from an aligned
    one, with valid counts on and off a multiple of four: same bits as the
    oracle."""
    g = np.random.default_rng(V)
    T, D, E, a = 700, 8 * 24, 16, 3001
    ti = g.integers(0, T, size=a).astype(np.int32)
    ei = g.integers(0, E, size=a).astype(np.int32)
    x = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    sc = g.random((T, E)).astype(np.float32)
    y = W.to_bf16_bits(g.standard_normal((a, D)).astype(np.float32))
    out0 = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    want_out = orc.scatter_add(out0.copy(), y, ti, V)
    want_rows = orc.gather_scale(x, ti, ei, sc, V)
    for offset in (0, 1):
        buf = torch.zeros(a + 4, dtype=torch.int32, device=dev)
        tid = buf[offset:offset + a]
        tid.copy_(torch.from_numpy(ti))
        assert (tid.data_ptr() % 16 == 0) == (offset == 0)
        say("token lists", V, offset)
        out = bf_dev(out0, dev)
        ops.moe_scatter_add(out, bf_dev(y, dev), tid, scalar_dev(V, dev))
        assert np.array_equal(bits_host(out), want_out), offset
        rows = torch.zeros((a, D), dtype=torch.bfloat16, device=dev)
        ops.moe_gather_scale(bf_dev(x, dev), tid, i32_dev(ei, dev), torch.from_numpy(sc).to(dev),
                             scalar_dev(V, dev), rows)
        assert np.array_equal(bits_host(rows)[:V], want_rows[:V]), offset


@pytest.mark.parametrize("row_order", [False, True], ids=["lists", "rows"])
def test_gather_scale_general_long_lists(dev, row_order):
    """Arbitrary token_indices: a token owning 100 rows (more than one pass of
    the token-order gather), unsorted rows, a valid bound below a; and a > 131072
    rows, where the token lists are built in four launches."""
    g = np.random.default_rng(10)
    T, D, E, a, V = 12, 8 * 70, 6, 400, 350
    ti = g.integers(0, T, size=a).astype(np.int32)
    ti[g.permutation(a)[:100]] = 5
    ei = g.integers(0, E, size=a).astype(np.int32)
    x = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    sc = g.random((T, E)).astype(np.float32)
    say("gather long lists", row_order, T, D, E, a, V)
    want = np.full((a, D), SENTINEL, np.uint16)
    orc.gather_scale(x, ti, ei, sc, V, want)
    out = torch.full((a, D), SENTINEL - 65536, dtype=torch.int16, device=dev).view(torch.bfloat16)
    ops.moe_gather_scale(bf_dev(x, dev), i32_dev(ti, dev), i32_dev(ei, dev),
                         torch.from_numpy(sc).to(dev), scalar_dev(V, dev), out,
                         row_order=row_order)
    assert np.array_equal(bits_host(out), want)

    T, D, E, K = 70000, 64, 8, 2
    inp, counts, ei, ti, rop = _dispatch_case(T, D, E, K, None, seed=4)
    V = int(counts[E])
    say("gather multi-launch lists", row_order, T, D, E, K, V)
    want = np.full((T * K, D), SENTINEL, np.uint16)
    orc.gather_scale(inp.x, ti, ei, inp.scores, V, want)
    out = torch.full((T * K, D), SENTINEL - 65536, dtype=torch.int16,
                     device=dev).view(torch.bfloat16)
    ops.moe_gather_scale(bf_dev(inp.x, dev), i32_dev(ti, dev), i32_dev(ei, dev),
                         torch.from_numpy(inp.scores).to(dev), scalar_dev(V, dev), out,
                         row_order=row_order)
    assert np.array_equal(bits_host(out), want)


def test_scatter_add_by_token_any_inverse_map(dev):
    """An inverse map that no shuffle makes: rows dealt to tokens by a random
    permutation, half of them valid, so tokens past V/K still own valid rows
    and tokens before it may own none (the early initial-row load guesses
    wrong both ways). The result equals the oracle's and the general path's."""
    g = np.random.default_rng(31)
    T, K, D = 300, 6, 8 * 90
    a = T * K
    perm = g.permutation(a).astype(np.int32)
    rop = perm.reshape(T, K)
    ti = np.empty(a, np.int32)
    ti[perm] = np.repeat(np.arange(T, dtype=np.int32), K)
    V = a // 2
    y = W.to_bf16_bits(g.standard_normal((a, D)).astype(np.float32))
    out0 = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    say("scatter by token, any inverse map", T, K, D, V)
    want = orc.scatter_add(out0.copy(), y, ti, V)
    out = bf_dev(out0, dev)
    ops.moe_scatter_add_by_token(out, bf_dev(y, dev), i32_dev(rop, dev), scalar_dev(V, dev))
    assert np.array_equal(bits_host(out), want)
    out2 = bf_dev(out0, dev)
    ops.moe_scatter_add(out2, bf_dev(y, dev), i32_dev(ti, dev), scalar_dev(V, dev))
    assert np.array_equal(bits_host(out2), want)


MANY_SMALL_K_CASES = [
    # (name, T, D, E, K, vtc): top-1 and top-2 on grids of more than 4096
    # (token, slice) waves, where a wave takes several consecutive tokens
    ("K1-ragged-D", 4099, 8 * (64 * 4 + 5), 16, 1, 4000),  # partial last slice
    ("K2", 5003, 512, 16, 2, 4990),                        # T not a multiple of the tokens
    ("K1-quant-D", 4110, 5120, 16, 1, None),               # per wave
    ("K2-vtc0", 5000, 1024, 8, 2, 0),                      # no routed token: out unchanged
    ("K1-D8-4097", 4097, 8, 4, 1, None),                   # one chunk per row, 4097 waves
    ("K2-D8-4097", 4097, 8, 4, 2, 3001),                   # the first grid past 4096 waves
]


@pytest.mark.parametrize("case", MANY_SMALL_K_CASES, ids=[c[0] for c in MANY_SMALL_K_CASES])
def test_scatter_add_by_token_many_tokens_small_k(dev, case):
    name, T, D, E, K, vtc = case
    inp, counts, ei, ti, rop = _dispatch_case(T, D, E, K, vtc, seed=4)
    V = int(counts[E])
    say("scatter by token, small K", name, T, D, K, V)
    want = orc.scatter_add(inp.out0.copy(), inp.y, ti, V)
    out = bf_dev(inp.out0, dev)
    ops.moe_scatter_add_by_token(out, bf_dev(inp.y, dev), i32_dev(rop, dev), scalar_dev(V, dev))
    assert np.array_equal(bits_host(out), want)


def test_scatter_add_by_token_small_k_any_inverse_map(dev):
    """Top-2 on a large grid with an inverse map no shuffle makes: rows dealt
    to tokens by a random permutation, 60 % of them valid, so a token may own
    0, 1 or 2 valid rows in either slot order, and tokens past V/K still own
    some. Equal to the oracle and to the general path."""
    g = np.random.default_rng(41)
    T, K, D = 4600, 2, 8 * 100
    a = T * K
    perm = g.permutation(a).astype(np.int32)
    rop = perm.reshape(T, K)
    ti = np.empty(a, np.int32)
    ti[perm] = np.repeat(np.arange(T, dtype=np.int32), K)
    V = a * 3 // 5
    y = W.to_bf16_bits(g.standard_normal((a, D)).astype(np.float32))
    out0 = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    say("scatter by token, small K, any inverse map", T, K, D, V)
    want = orc.scatter_add(out0.copy(), y, ti, V)
    out = bf_dev(out0, dev)
    ops.moe_scatter_add_by_token(out, bf_dev(y, dev), i32_dev(rop, dev), scalar_dev(V, dev))
    assert np.array_equal(bits_host(out), want)
    out2 = bf_dev(out0, dev)
    ops.moe_scatter_add(out2, bf_dev(y, dev), i32_dev(ti, dev), scalar_dev(V, dev))
    assert np.array_equal(bits_host(out2), want)


# ---------------------------------------------------------------- padded combine
PADDED_CASES = [
    # (name, T, D, E, K, EP)
    ("ep1", 40, 256, 8, 2, 1),
    ("ep2-ragged-D", 77, 8 * (64 * 5 + 3), 10, 3, 2),
    ("ep4", 129, 1024, 16, 4, 4),
    ("ep8-wide", 64, 8 * 1000, 64, 8, 8),
    ("E1024-ep64", 50, 64, 1024, 16, 64),   # the most experts and ranks
]


@pytest.mark.parametrize("case", PADDED_CASES, ids=[c[0] for c in PADDED_CASES])
def test_scatter_add_padded_bit_exact(dev, case):
    name, T, D, E, K, EP = case
    inp, counts, ei, ti, rop = _dispatch_case(T, D, E, K, None, seed=2)
    g = np.random.default_rng(5)
    slabs = W.to_bf16_bits(g.standard_normal((EP, T * K, D)).astype(np.float32))
    say("padded", name, T, D, E, K, EP)
    want = orc.scatter_add_padded(inp.out0.copy(), slabs, counts[:E], ti)
    out = bf_dev(inp.out0, dev)
    ops.moe_scatter_add_padded(bf_dev(slabs, dev), i32_dev(counts[:E], dev), i32_dev(ti, dev),
                               out)
    assert np.array_equal(bits_host(out), want)
    out = bf_dev(inp.out0, dev)
    ops.moe_scatter_add_padded_by_token(bf_dev(slabs, dev), i32_dev(counts[:E], dev),
                                        i32_dev(rop, dev), out)
    assert np.array_equal(bits_host(out), want)


def test_scatter_add_padded_by_token_any_inverse_map(dev):
    """The by-token padded combine with an inverse map no shuffle makes: rows
    dealt to tokens by a random permutation and counts whose total (V) is
    60 % of the rows, so a token may own none, some or all of its K slots,
    in any order, and tokens past V/K still own rows. Equal to the oracle,
    which takes the same map's token_indices."""
    g = np.random.default_rng(43)
    T, K, D, E, EP = 700, 6, 8 * 70, 24, 4
    T_K = T * K
    perm = g.permutation(T_K).astype(np.int32)
    rop = perm.reshape(T, K)
    ti = np.empty(T_K, np.int32)
    ti[perm] = np.repeat(np.arange(T, dtype=np.int32), K)
    V = T_K * 3 // 5
    counts = np.bincount(np.sort(g.integers(0, E, size=V)), minlength=E).astype(np.int32)
    slabs = W.to_bf16_bits(g.standard_normal((EP, T_K, D)).astype(np.float32))
    out0 = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    say("padded by token, any inverse map", T, K, D, E, EP, V)
    want = orc.scatter_add_padded(out0.copy(), slabs, counts, ti)
    out = bf_dev(out0, dev)
    ops.moe_scatter_add_padded_by_token(bf_dev(slabs, dev), i32_dev(counts, dev),
                                        i32_dev(rop, dev), out)
    assert np.array_equal(bits_host(out), want)


def test_scatter_add_padded_long_lists(dev):
    """A token owning 100 rows (beyond one wave's sort), empty experts, and a
    count total below T_K."""
    g = np.random.default_rng(12)
    T, D, E, EP, T_K = 10, 8 * 40, 12, 4, 300
    counts = np.array([30, 0, 25, 40, 0, 0, 35, 20, 10, 0, 50, 20], np.int32)  # 230 rows
    ti = g.integers(0, T, size=T_K).astype(np.int32)
    ti[g.permutation(230)[:100]] = 3
    slabs = W.to_bf16_bits(g.standard_normal((EP, T_K, D)).astype(np.float32))
    out0 = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    say("padded long lists", T, D, E, EP, T_K)
    want = orc.scatter_add_padded(out0.copy(), slabs, counts, ti)
    out = bf_dev(out0, dev)
    ops.moe_scatter_add_padded(bf_dev(slabs, dev), i32_dev(counts, dev), i32_dev(ti, dev), out)
    assert np.array_equal(bits_host(out), want)


def test_scatter_add_csr_multi_launch(dev):
    """More rows than the two-launch CSR build takes (131072): the general
    and padded combines build the CSR in four launches."""
    T, D, E, K, EP = 70000, 64, 8, 2, 2
    inp, counts, ei, ti, rop = _dispatch_case(T, D, E, K, None, seed=4)
    V = int(counts[E])
    say("csr multi-launch", T, D, E, K, EP, V)
    y = W.to_bf16_bits(np.random.default_rng(8).standard_normal((T * K, D)).astype(np.float32))
    want = orc.scatter_add(inp.out0.copy(), y, ti, V)
    out = bf_dev(inp.out0, dev)
    ops.moe_scatter_add(out, bf_dev(y, dev), i32_dev(ti, dev), scalar_dev(V, dev))
    assert np.array_equal(bits_host(out), want)
    slabs = W.to_bf16_bits(np.random.default_rng(9).standard_normal(
        (EP, T * K, D)).astype(np.float32))
    want = orc.scatter_add_padded(inp.out0.copy(), slabs, counts[:E], ti)
    out = bf_dev(inp.out0, dev)
    ops.moe_scatter_add_padded(bf_dev(slabs, dev), i32_dev(counts[:E], dev), i32_dev(ti, dev),
                               out)
    assert np.array_equal(bits_host(out), want)


def test_scatter_add_csr_stage_overflow(dev):
    """One 128-token range owning more rows (10000) than the CSR build stages
    in LDS (8192): the build falls back to a second pass over the indices."""
    g = np.random.default_rng(13)
    T, D, a = 100, 64, 10000
    ti = g.integers(0, T, size=a).astype(np.int32)
    y = W.to_bf16_bits(g.standard_normal((a, D)).astype(np.float32))
    out0 = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    say("csr stage overflow", T, D, a)
    want = orc.scatter_add(out0.copy(), y, ti, a)
    out = bf_dev(out0, dev)
    ops.moe_scatter_add(out, bf_dev(y, dev), i32_dev(ti, dev))
    assert np.array_equal(bits_host(out), want)
    # the padded layout: 4 experts over 2 ranks, all rows valid
    counts = np.array([3000, 2500, 2500, 2000], np.int32)
    slabs = W.to_bf16_bits(g.standard_normal((2, a, D)).astype(np.float32))
    want = orc.scatter_add_padded(out0.copy(), slabs, counts, ti)
    out = bf_dev(out0, dev)
    ops.moe_scatter_add_padded(bf_dev(slabs, dev), i32_dev(counts, dev), i32_dev(ti, dev), out)
    assert np.array_equal(bits_host(out), want)


@pytest.mark.parametrize("a", [600, 2000, 6000])
def test_out_of_range_indices_are_skipped(dev, a):
    """Token, expert and slot indices out of range (negative, or past T, E, V
    or rows) are preconditions the kernels check before addressing memory:
    such a row or slot is skipped. Valid rows equal the oracle on the input
    with the bad rows dropped; rows with a bad index are left unwritten.
    a = 600, 2000, 6000 take the per-wave row search, the one-workgroup build
    and the two-launch build of the token_indices paths."""
    g = np.random.default_rng(a)
    T, D, E, K = 50, 64, 8, 4
    V = a - 37
    ti = g.integers(0, T, size=a).astype(np.int32)
    ei = g.integers(0, E, size=a).astype(np.int32)
    bad_t = g.random(a) < 0.1
    ti[bad_t] = np.where(g.random(int(bad_t.sum())) < 0.5, -3, T + 7)
    bad_e = g.random(a) < 0.05
    ei[bad_e] = np.where(g.random(int(bad_e.sum())) < 0.5, -1, E + 2)
    x = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    s = g.standard_normal((T, E)).astype(np.float32)
    y = W.to_bf16_bits(g.standard_normal((a, D)).astype(np.float32))
    out0 = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    say("out-of-range indices", a, int(bad_t.sum()), int(bad_e.sum()))
    ok_rows = (np.arange(a) < V) & ~bad_t & ~bad_e
    # gather: the valid rows as the oracle computes them, the others untouched
    want_rows = orc.gather_scale(x, np.where(ok_rows, ti, 0).astype(np.int32),
                                 np.where(ok_rows, ei, 0).astype(np.int32), s, V,
                                 np.full((a, D), SENTINEL, np.uint16))
    want_rows[~ok_rows] = SENTINEL
    for row_order in (False, True):
        rows = bf_dev(np.full((a, D), SENTINEL, np.uint16), dev)
        ops.moe_gather_scale(bf_dev(x, dev), i32_dev(ti, dev), i32_dev(ei, dev),
                             torch.from_numpy(s).to(dev), scalar_dev(V, dev), out=rows,
                             row_order=row_order)
        assert np.array_equal(bits_host(rows), want_rows), row_order
    q, qs = ops.moe_gather_scale_quant(bf_dev(x, dev), i32_dev(ti, dev), i32_dev(ei, dev),
                                       torch.from_numpy(s).to(dev), None, scalar_dev(V, dev))
    wq, wqs = orc.gather_scale_quant(x, np.where(ok_rows, ti, 0).astype(np.int32),
                                     np.where(ok_rows, ei, 0).astype(np.int32), s, None, V)
    assert np.array_equal(q.cpu().numpy()[ok_rows], wq[ok_rows])
    assert np.array_equal(qs.cpu().numpy()[ok_rows], wqs[ok_rows])
    # general combine: a row with a bad token adds nothing (expert ids unused)
    keep = (np.arange(a) < V) & ~bad_t
    want = orc.scatter_add(out0.copy(), np.ascontiguousarray(y[keep]),
                           np.ascontiguousarray(ti[keep]))
    out = bf_dev(out0, dev)
    ops.moe_scatter_add(out, bf_dev(y, dev), i32_dev(ti, dev), scalar_dev(V, dev))
    assert np.array_equal(bits_host(out), want)
    # by-token paths and the finalize: slots outside [0, V) (and past the rows)
    rop = g.permutation(V)[:T * K].reshape(T, K).astype(np.int32)  # no row twice
    bad = g.random((T, K)) < 0.15
    rop[bad] = g.choice(np.array([-1, -9, V, V + 3, a + 100], np.int32), size=int(bad.sum()))
    okp = (rop >= 0) & (rop < V)
    rows = bf_dev(np.full((a, D), SENTINEL, np.uint16), dev)
    ops.moe_gather_scale_by_token(bf_dev(x, dev), i32_dev(rop, dev), i32_dev(ei, dev),
                                  torch.from_numpy(s).to(dev), scalar_dev(V, dev), rows)
    got = bits_host(rows)
    tt, kk = np.nonzero(okp)
    for t_, r_ in zip(tt, rop[okp]):
        e_ = ei[r_]
        if 0 <= e_ < E:
            w1 = orc.gather_scale(x, np.array([t_], np.int32), np.array([e_], np.int32), s, 1)
            assert np.array_equal(got[r_], w1[0]), (t_, r_)
    touched = np.zeros(a, bool)
    touched[rop[okp]] = True
    assert np.all(got[~touched] == SENTINEL)
    # by-token combine: each token adds its valid slots' rows in ascending order
    want = out0.copy()
    for t_ in range(T):
        rr = np.sort(rop[t_][okp[t_]])
        if rr.size:
            want[t_] = orc.scatter_add(out0[t_:t_ + 1].copy(), np.ascontiguousarray(y[rr]),
                                       np.zeros(rr.size, np.int32))[0]
    out = bf_dev(out0, dev)
    ops.moe_scatter_add_by_token(out, bf_dev(y, dev), i32_dev(rop, dev), scalar_dev(V, dev))
    assert np.array_equal(bits_host(out), want)
    # padded by-token combine: the same slots (counts summing to V), each row
    # read from the slab of the rank that owns its expert
    EPp = 2
    cnt = np.bincount(g.integers(0, E, size=V), minlength=E).astype(np.int32)
    owner = np.searchsorted(np.concatenate([[0], np.cumsum(cnt)]), np.arange(a), "right") - 1
    slabs = W.to_bf16_bits(g.standard_normal((EPp, a, D)).astype(np.float32))
    want = out0.copy()
    for t_ in range(T):
        rr = np.sort(rop[t_][okp[t_]])
        if rr.size:
            src = np.ascontiguousarray(slabs[owner[rr] // (E // EPp), rr])
            want[t_] = orc.scatter_add(out0[t_:t_ + 1].copy(), src,
                                       np.zeros(rr.size, np.int32))[0]
    out = bf_dev(out0, dev)
    ops.moe_scatter_add_padded_by_token(bf_dev(slabs, dev), i32_dev(cnt, dev),
                                        i32_dev(rop, dev), out)
    assert np.array_equal(bits_host(out), want)
    # finalize: a slot past the permuted rows is not held
    rop_f = rop.copy()
    rop_f[rop_f >= a] = a + 5
    w = g.random((T, K)).astype(np.float32)
    gamma = W.to_bf16_bits(g.uniform(0.5, 1.5, D).astype(np.float32))
    want_o = orc.finalize_rmsnorm(y, w, np.where((rop_f >= 0) & (rop_f < a), rop_f, -1)
                                  .astype(np.int32), None, gamma, 1e-6)
    o = ops.moe_finalize_rmsnorm(bf_dev(y, dev), torch.from_numpy(w).to(dev),
                                 i32_dev(rop_f, dev), None, bf_dev(gamma, dev), 1e-6)
    _close(bits_host(o), want_o, "finalize, slots past the rows")


@pytest.mark.parametrize("T,a", [(4096, 4096), (1, 4096), (4097, 300), (300, 4097)])
def test_csr_small_build_limits(dev, T, a):
    """The one-workgroup row-list build (up to 4096 rows and 4096 tokens) at its
    limits and just past them (the two-launch build): the general gather and
    combine, and the padded combine, against the oracle."""
    g = np.random.default_rng(T * 7 + a)
    D, V = 64, a - a // 5
    ti = g.integers(0, T, size=a).astype(np.int32)
    ti[: min(a, 70)] = T - 1  # one token with more than 64 rows
    x = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    s = g.standard_normal((T, 4)).astype(np.float32)
    ei = g.integers(0, 4, size=a).astype(np.int32)
    y = W.to_bf16_bits(g.standard_normal((a, D)).astype(np.float32))
    out0 = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    say("csr small build limits", T, a, V)
    rows0 = np.full((a, D), SENTINEL, np.uint16)
    want_rows = orc.gather_scale(x, ti, ei, s, V, rows0.copy())
    rows = bf_dev(rows0, dev)
    ops.moe_gather_scale(bf_dev(x, dev), i32_dev(ti, dev), i32_dev(ei, dev),
                         torch.from_numpy(s).to(dev), scalar_dev(V, dev), out=rows)
    assert np.array_equal(bits_host(rows), want_rows)
    want = orc.scatter_add(out0.copy(), y, ti, V)
    out = bf_dev(out0, dev)
    ops.moe_scatter_add(out, bf_dev(y, dev), i32_dev(ti, dev), scalar_dev(V, dev))
    assert np.array_equal(bits_host(out), want)
    # padded: 4 experts over 2 ranks covering the first V rows
    counts = np.array([V // 4, V // 4, V // 4, V - 3 * (V // 4)], np.int32)
    slabs = W.to_bf16_bits(g.standard_normal((2, a, D)).astype(np.float32))
    want = orc.scatter_add_padded(out0.copy(), slabs, counts, ti)
    out = bf_dev(out0, dev)
    ops.moe_scatter_add_padded(bf_dev(slabs, dev), i32_dev(counts, dev), i32_dev(ti, dev), out)
    assert np.array_equal(bits_host(out), want)


@pytest.mark.parametrize("T", [2048 * 128, 2048 * 128 + 1])
def test_scatter_add_csr_most_ranges(dev, T):
    """The most token ranges the two-launch CSR build takes (2048 of 128
    tokens), and one token more (four launches), with 131072 rows of which
    the first 120000 are valid."""
    g = np.random.default_rng(T)
    D, a, V = 64, 131072, 120000
    ti = g.integers(0, T, size=a).astype(np.int32)
    ti[:80] = T - 1  # the last token, a list of more than 64 rows
    y = W.to_bf16_bits(g.standard_normal((a, D)).astype(np.float32))
    out0 = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    say("csr most ranges", T, D, a, V)
    want = orc.scatter_add(out0.copy(), y, ti, V)
    out = bf_dev(out0, dev)
    ops.moe_scatter_add(out, bf_dev(y, dev), i32_dev(ti, dev), scalar_dev(V, dev))
    assert np.array_equal(bits_host(out), want)


# ---------------------------------------------------------------- EP re-sort
SHUFFLING_CASES = [
    # (name, EP, C, c_lo, c_hi, packed, max count, D)
    ("dynamic-ep4", 4, 16, 0, 16, True, 9, 256),
    ("dynamic-ep8-ragged-D", 8, 32, 0, 32, True, 7, 8 * (64 * 3 + 5)),
    ("static-ep8-local-range", 8, 64, 16, 24, False, 12, 1024),
    ("static-ep2-empty-range", 2, 8, 3, 3, False, 5, 64),
    ("static-ep64", 64, 32, 0, 32, False, 3, 512),
    ("static-4096-segments", 64, 64, 0, 64, False, 2, 64),  # the most segments
]


@pytest.mark.parametrize("case", SHUFFLING_CASES, ids=[c[0] for c in SHUFFLING_CASES])
def test_combine_split_shuffling_bit_exact(dev, case):
    name, EP, C, lo, hi, packed, mx, D = case
    g = np.random.default_rng(21)
    counts = g.integers(0, mx + 1, size=(EP, C)).astype(np.int32)
    counts[0, :2] = 0                                    # empty segments
    stride = None if packed else int(counts.sum(axis=1).max() + 3)
    rows = int(counts.sum()) if packed else EP * stride
    tok = W.to_bf16_bits(g.standard_normal((rows, D)).astype(np.float32))
    say("shuffling", name, EP, C, lo, hi, rows, D)
    want, woc = orc.combine_shuffling(tok, counts, lo, hi, stride,
                                      out=np.full((rows, D), SENTINEL, np.uint16))
    out0 = torch.full((rows, D), SENTINEL - 65536, dtype=torch.int16,
                      device=dev).view(torch.bfloat16)
    out, oc = ops.moe_combine_shuffling(bf_dev(tok, dev), i32_dev(counts, dev), lo, hi, stride,
                                        out=out0)
    assert np.array_equal(oc.cpu().numpy(), woc)
    assert np.array_equal(bits_host(out), want)
    # split back into a fresh buffer: the moved rows return, others untouched
    wback = orc.split_shuffling(want, counts, lo, hi, stride,
                                out=np.full((rows, D), SENTINEL, np.uint16))
    back0 = torch.full((rows, D), SENTINEL - 65536, dtype=torch.int16,
                       device=dev).view(torch.bfloat16)
    back = ops.moe_split_shuffling(out, i32_dev(counts, dev), lo, hi, stride, out=back0)
    assert np.array_equal(bits_host(back), wback)


# ---------------------------------------------------------------- finalize
def _close(got_bits, want_bits, what):
    """The finalize bar (|gpu - ref| <= 2e-2 + 1e-2 |ref|), then bit-exactness,
    which the fp64 sum of squares on both sides is designed to give."""
    g = orc.bf16_to_f32(got_bits).astype(np.float64)
    r = orc.bf16_to_f32(want_bits).astype(np.float64)
    err = np.abs(g - r)
    tol = 2e-2 + 1e-2 * np.abs(r)
    assert np.all(err <= tol), f"{what}: max abs {err.max():.3e}"
    ndiff = int(np.count_nonzero(got_bits != want_bits))
    if ndiff:
        say(what, f"differs from the oracle in {ndiff} of {got_bits.size} elements, "
                  f"max abs {err.max():.3e}")
    assert ndiff == 0, f"{what}: {ndiff} elements differ from the oracle (within tolerance)"


def assert_mx_end_to_end(codes, scales, want_codes, want_scales, what):
    """MXFP8 codes and UE8M0 scales against the oracle's own end-to-end output:
    codes at most one code apart on at most 0.1 % of elements; reported, then
    required exact (as designed)."""
    d = np.abs(ordinal(codes) - ordinal(want_codes))
    sd = np.abs(scales.astype(np.int32) - want_scales.astype(np.int32))
    say(what, f"end to end: codes differ {np.mean(d > 0):.2e} (max distance "
              f"{d.max(initial=0)}), scale bytes differ {np.mean(sd > 0):.2e}")
    assert_fp8_close(codes, want_codes, what)
    assert np.array_equal(scales, want_scales), f"{what}: scale bytes differ"
    assert np.array_equal(codes, want_codes), f"{what}: codes differ"


FIN_CASES = [
    # (name, T, D, K, hole_frac, shared, flags, mxfp8)
    ("decode-1", 1, 7168, 8, 0.0, True, 0, False),
    ("decode-8", 8, 7168, 8, 0.0, True, 0, False),
    ("decode-32", 32, 7168, 8, 0.0, True, 0, False),
    ("decode-128", 128, 7168, 8, 0.0, True, 0, False),
    ("holes-noshared", 50, 1024, 4, 0.3, False, 0, True),
    ("bf16-squares", 20, 2048, 8, 0.1, True, 1, False),
    ("ragged-D", 33, 32 * 49, 3, 0.0, True, 0, True),   # partial last wave
    ("many-tokens", 2100, 640, 4, 0.05, True, 0, True),  # the many-token shape
    ("K1", 9, 256, 1, 0.0, False, 0, True),
    ("Dmax", 3, 65536, 2, 0.0, True, 0, True),         # the widest row
    ("tiny-ragged", 5, 32 * 49, 8, 0.1, True, 0, True),  # <= 32 tokens, partial last wave
]


@pytest.mark.parametrize("case", FIN_CASES, ids=[c[0] for c in FIN_CASES])
def test_finalize_rmsnorm(dev, case):
    name, T, D, K, holes, with_shared, flags, mx = case
    wl = W.WORKLOADS["decode"] if D == 7168 else W.WORKLOADS["prefill"]
    fi = W.finalize_inputs(wl, T=T, D=D, K=K, hole_frac=holes)
    shared = fi.shared if with_shared else None
    say("finalize", name, T, D, K, flags, mx)
    want = orc.finalize_rmsnorm(fi.y, fi.w, fi.row_of_pair, shared, fi.gamma, fi.eps,
                                flags=flags, mxfp8=mx)
    res = ops.moe_finalize_rmsnorm(bf_dev(fi.y, dev), torch.from_numpy(fi.w).to(dev),
                                   i32_dev(fi.row_of_pair, dev),
                                   None if shared is None else bf_dev(shared, dev),
                                   bf_dev(fi.gamma, dev), fi.eps, flags=flags, mxfp8=mx)
    out = res[0] if mx else res
    got = bits_host(out)
    _close(got, want[0] if mx else want, name)
    if mx:
        codes, scales = res[1].cpu().numpy(), res[2].cpu().numpy()
        assert_mx_end_to_end(codes, scales, want[1], want[2], name)
        oc, os_ = orc.mxfp8_quantize(got)        # the split check
        assert np.array_equal(scales, os_)
        assert_fp8_close(codes, oc, "mxfp8")
        assert np.array_equal(codes, oc)


FIN_VARIANT_CASES = [
    # (name, T, D, K, holes, bf16 weights, swizzled scales)
    ("bf16-weights", 40, 1024, 8, 0.1, True, False),
    ("swizzled-130", 130, 1024, 4, 0.0, False, True),
    ("swizzled-1", 1, 7168, 8, 0.0, True, True),
    ("swizzled-256", 256, 512, 2, 0.2, False, True),
]


@pytest.mark.parametrize("case", FIN_VARIANT_CASES, ids=[c[0] for c in FIN_VARIANT_CASES])
def test_finalize_variants(dev, case):
    name, T, D, K, holes, bfw, swz = case
    fi = W.finalize_inputs(W.WORKLOADS["prefill"], T=T, D=D, K=K, hole_frac=holes)
    flags = (2 if bfw else 0)
    w = W.to_bf16_bits(fi.w) if bfw else fi.w
    say("finalize variant", name, T, D, K, bfw, swz)
    want, wcodes, wscales = orc.finalize_rmsnorm(
        fi.y, w, fi.row_of_pair, fi.shared, fi.gamma, fi.eps,
        flags=flags | (4 if swz else 0), mxfp8=True)
    wd = bf_dev(w, dev) if bfw else torch.from_numpy(w).to(dev)
    out, codes, scales = ops.moe_finalize_rmsnorm(
        bf_dev(fi.y, dev), wd, i32_dev(fi.row_of_pair, dev), bf_dev(fi.shared, dev),
        bf_dev(fi.gamma, dev), fi.eps, mxfp8=True,
        scale_layout="swizzled" if swz else "rowmajor")
    got = bits_host(out)
    _close(got, want, name)
    assert_mx_end_to_end(codes.cpu().numpy(), scales.cpu().numpy(), wcodes, wscales, name)
    oc, rm = orc.mxfp8_quantize(got)            # split check on the GPU's own output
    assert np.array_equal(codes.cpu().numpy(), oc)
    want_scales = orc.mxfp8_swizzle(rm) if swz else rm
    assert np.array_equal(scales.cpu().numpy(), want_scales)


MHC_CASES = [
    # (name, T, D, K, holes, hc, mode, swizzled, flags)
    #   mode: "mx" (layer input + MXFP8), "norm" (layer input), "res" (residual only)
    ("hc4-mx", 40, 1024, 8, 0.1, 4, "mx", False, 0),
    ("hc4-swizzled-130", 130, 5120, 4, 0.0, 4, "mx", True, 0),
    ("hc1", 17, 7168, 8, 0.0, 1, "norm", False, 0),
    ("hc3-ragged", 33, 32 * 49, 3, 0.2, 3, "mx", False, 0),   # partial last wave
    ("hc2-residual-only", 20, 2048, 2, 0.0, 2, "res", False, 0),
    ("hc4-wide", 5, 16384 + 8192, 2, 0.0, 4, "norm", False, 0),  # four chunks per lane
    ("hc4-flags", 64, 2048, 8, 0.1, 4, "mx", True, 1 | 2),     # bf16 squares + weights
    ("hc4-T1", 1, 5120, 4, 0.0, 4, "mx", True, 0),
    ("hc4-Dmax", 2, 32768, 2, 0.0, 4, "mx", True, 0),     # the widest row
]


@pytest.mark.parametrize("case", MHC_CASES, ids=[c[0] for c in MHC_CASES])
def test_finalize_mhc(dev, case):
    name, T, D, K, holes, hc, mode, swz, flags = case
    wl = W.WORKLOADS["mhc"]
    fi = W.finalize_inputs(wl, T=T, D=D, K=K, hole_frac=holes)
    m = W.mhc_inputs(wl, T=T, D=D, hc=hc)
    bfw = bool(flags & 2)
    w = W.to_bf16_bits(fi.w) if bfw else fi.w
    mx = mode == "mx"
    pre = None if mode == "res" else m.pre
    say("finalize mhc", name, T, D, K, hc, mode, swz, flags)
    want = orc.finalize_mhc(fi.y, w, fi.row_of_pair, fi.shared, m.residual, m.post, m.comb,
                            pre, fi.gamma if pre is not None else None, fi.eps,
                            flags=flags | (4 if (mx and swz) else 0), mxfp8=mx)
    wd = bf_dev(w, dev) if bfw else torch.from_numpy(w).to(dev)
    f32 = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
    res = ops.moe_finalize_mhc(
        bf_dev(fi.y, dev), wd, i32_dev(fi.row_of_pair, dev), bf_dev(fi.shared, dev),
        bf_dev(m.residual, dev), f32(m.post), f32(m.comb), None if pre is None else f32(pre),
        bf_dev(fi.gamma, dev), fi.eps, flags=flags & 1, mxfp8=mx,
        scale_layout="swizzled" if swz else "rowmajor")
    got_res = bits_host(res[0])
    _close(got_res, want[0], name + " residual_out")
    if pre is None:
        assert res[1] is None
        return
    got = bits_host(res[1])
    _close(got, want[1], name)
    if mx:
        assert_mx_end_to_end(res[2].cpu().numpy(), res[3].cpu().numpy(), want[2], want[3], name)
        oc, rm = orc.mxfp8_quantize(got)        # split check on the GPU's own output
        assert np.array_equal(res[2].cpu().numpy(), oc)
        assert np.array_equal(res[3].cpu().numpy(), orc.mxfp8_swizzle(rm) if swz else rm)


# ---------------------------------------------------------------- empty inputs
def test_empty_inputs_leave_outputs_alone(dev):
    """Zero tokens, zero rows or zero counts: every entry point returns
    without touching its outputs."""
    say("empty inputs")
    D, K, E = 64, 2, 4
    bf = lambda *sh: torch.randn(sh, device=dev).to(torch.bfloat16)  # noqa: E731
    i32 = lambda *sh: torch.zeros(sh, dtype=torch.int32, device=dev)  # noqa: E731
    f32 = lambda *sh: torch.rand(sh, device=dev)  # noqa: E731
    # zero tokens
    ops.moe_gather_scale(bf(0, D), i32(0), i32(0), f32(0, E), out=bf(0, D))
    ops.moe_gather_scale_by_token(bf(0, D), i32(0, K), i32(0), f32(0, E), out=bf(0, D))
    ops.moe_gather_scale_quant(bf(0, D), i32(0), i32(0), f32(0, E))
    out = bf(0, D)
    ops.moe_scatter_add_by_token(out, bf(0, D), i32(0, K))
    fin = ops.moe_finalize_rmsnorm(bf(0, D), f32(0, K), i32(0, K), None, bf(D), 1e-6,
                                   mxfp8=True)
    assert fin[0].shape == (0, D)
    r = ops.moe_finalize_mhc(bf(0, D), f32(0, K), i32(0, K), None, bf(0, 4, D), f32(0, 4),
                             f32(0, 4, 4), f32(0, 4), bf(D), 1e-6)
    assert r[0].shape == (0, 4, D)
    # rows present, none valid: outputs keep their bits
    T = 5
    out = bf(T, D)
    keep = out.clone()
    ops.moe_scatter_add(out, bf(T * K, D), i32(T * K), scalar_dev(0, dev))
    ops.moe_scatter_add_by_token(out, bf(T * K, D), i32(T, K) - 1)
    ops.moe_scatter_add_padded(bf(2, T * K, D), i32(E), i32(T * K), out)
    assert torch.equal(out, keep)
    rows = bf(T * K, D)
    keep = rows.clone()
    ops.moe_gather_scale(bf(T, D), i32(T * K), i32(T * K), f32(T, E), scalar_dev(0, dev), rows)
    assert torch.equal(rows, keep)
    # all counts zero: nothing moves, the column counts are zero
    tok = bf(8, D)
    em = bf(8, D)
    keep = em.clone()
    em2, oc = ops.moe_combine_shuffling(tok, i32(2, 4), 0, 4, None, out=em)
    assert torch.equal(em2, keep) and int(oc.abs().sum()) == 0
    back = bf(8, D)
    keep = back.clone()
    ops.moe_split_shuffling(em, i32(2, 4), 0, 4, 4, out=back)
    assert torch.equal(back, keep)


# ---------------------------------------------------------------- HIP graphs
def test_graph_replay_matches_eager(dev):
    """shuffle -> gather (by token) -> scatter (by token) -> padded scatter (by
    token, two ranks' slabs) -> finalize + MXFP8 (128x4-tiled scales) -> mHC
    finalize, captured in one HIP graph. Every replay, with eager work
    (buffers overwritten) and synchronisations between replays, equals the
    eager run bit for bit."""
    wl = W.WORKLOADS["zipf"]
    T, D, E, K, vtc, hc = 200, 1024, 16, 4, 150, 4
    inp = W.dispatch_inputs(wl, T=T, D=D, E=E, K=K, vtc=vtc, out0="normal")
    fi = W.finalize_inputs(W.WORKLOADS["mhc"], T=T, D=D, K=K, hole_frac=0.1)
    m = W.mhc_inputs(W.WORKLOADS["mhc"], T=T, D=D, hc=hc)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    s, x, y, out0 = f32(inp.scores), bf_dev(inp.x, dev), bf_dev(inp.y, dev), bf_dev(inp.out0, dev)
    vtc_d = scalar_dev(vtc, dev)
    yf, wf, ropf = bf_dev(fi.y, dev), f32(fi.w), i32_dev(fi.row_of_pair, dev)
    shf, gf = bf_dev(fi.shared, dev), bf_dev(fi.gamma, dev)
    res, post, comb, pre = bf_dev(m.residual, dev), f32(m.post), f32(m.comb), f32(m.pre)
    slabs = bf_dev(W.to_bf16_bits(np.random.default_rng(9).standard_normal(
        (2, T * K, D)).astype(np.float32)), dev)

    def buffers():
        i32 = lambda *sh: torch.empty(sh, dtype=torch.int32, device=dev)  # noqa: E731
        u8 = lambda *sh: torch.empty(sh, dtype=torch.uint8, device=dev)  # noqa: E731
        nsc = 256 * (D // 32)  # 128x4-tiled scales of T=200 rows, padded to 256
        return dict(
            ws=u8(ops._lib.load().moe_shuffle_workspace_bytes(T, E, K)),
            shuf=(i32(E + 1), i32(T * K), i32(T * K), i32(T, K)),
            rows=torch.empty((T * K, D), dtype=torch.bfloat16, device=dev),
            out=out0.clone(), pout=out0.clone(),
            fin=torch.empty((T, D), dtype=torch.bfloat16, device=dev),
            codes=u8(T, D), scales=u8(nsc), res_out=torch.empty_like(res),
            mout=torch.empty((T, D), dtype=torch.bfloat16, device=dev), mcodes=u8(T, D),
            mscales=u8(nsc))

    def path(b):
        counts, ei, ti, rop = ops.moe_shuffle(s, K, vtc_d, workspace=b["ws"], out=b["shuf"])
        ops.moe_gather_scale_by_token(x, rop, ei, s, counts[E:], b["rows"])
        ops.moe_scatter_add_by_token(b["out"], y, rop, counts[E:])
        ops.moe_scatter_add_padded_by_token(slabs, counts[:E], rop, b["pout"])
        ops.moe_finalize_rmsnorm(yf, wf, ropf, shf, gf, fi.eps, out=b["fin"], mxfp8=True,
                                 scale_layout="swizzled", mx_codes=b["codes"],
                                 mx_scales=b["scales"])
        ops.moe_finalize_mhc(yf, wf, ropf, shf, res, post, comb, pre, gf, fi.eps,
                             residual_out=b["res_out"], out=b["mout"], mxfp8=True,
                             scale_layout="swizzled", mx_codes=b["mcodes"],
                             mx_scales=b["mscales"])

    def snapshot(b):
        V = int(b["shuf"][0][E].item())
        snap = {k: b[k].cpu().clone() for k in ("out", "pout", "fin", "codes", "scales",
                                                 "res_out", "mout", "mcodes", "mscales")}
        snap["rows"] = b["rows"][:V].cpu().clone()
        for i, t in enumerate(b["shuf"]):
            snap[f"shuf{i}"] = t.cpu().clone()
        return snap

    say("graph replay", T, D, E, K, vtc, hc)
    eager = buffers()
    path(eager)
    torch.cuda.synchronize()
    want = snapshot(eager)

    b = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one eager pass on the capture stream first
        path(b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path(b)
    for rep in range(3):
        # eager work between replays: reset the accumulated output, spoil the rest
        b["out"].copy_(out0)
        b["pout"].copy_(out0)
        for k in ("fin", "res_out", "mout", "rows"):
            b[k].view(torch.int16).fill_(0x7E00 + rep)
        for k in ("codes", "scales", "mcodes", "mscales"):
            b[k].fill_(0xA5)
        for t in b["shuf"]:
            t.fill_(-3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot(b)
        for k, v in want.items():
            assert torch.equal(got[k], v), (rep, k)


@pytest.mark.parametrize("K", [1, 2])
def test_graph_replay_small_k_combine(dev, K):
    """The top-1/top-2 combine on a grid of more than 4096 waves (several
    tokens per wave), captured in a HIP graph: every replay, with the output
    reset eagerly between replays, equals the eager run and the oracle."""
    T, D, E, vtc = 4200, 1024, 8, 4100
    inp, counts, ei, ti, rop = _dispatch_case(T, D, E, K, vtc, seed=6)
    V = int(counts[E])
    want = orc.scatter_add(inp.out0.copy(), inp.y, ti, V)
    out0, y = bf_dev(inp.out0, dev), bf_dev(inp.y, dev)
    rop_d, v_d = i32_dev(rop, dev), scalar_dev(V, dev)
    say("graph replay, small-K combine", T, D, K, V)
    out = out0.clone()
    ops.moe_scatter_add_by_token(out, y, rop_d, v_d)
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(out), want)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out.copy_(out0)
        ops.moe_scatter_add_by_token(out, y, rop_d, v_d)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.moe_scatter_add_by_token(out, y, rop_d, v_d)
    for rep in range(3):
        out.copy_(out0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_host(out), want), rep


@pytest.mark.parametrize("T", [300, 100])
def test_graph_replay_general_paths(dev, T):
    """The entry points the first graph test leaves out, captured in one HIP
    graph with caller workspaces: the shuffle that allocates nothing, the
    general gather (token order), the FP8 rowwise gather, the
    general and padded combines, and the EP re-sort both ways. Every replay,
    with the outputs spoiled by eager work in between, equals the eager run
    bit for bit. T = 300 (1200 rows) builds row lists in one workgroup;
    T = 100 (400 rows) takes the per-wave row search and the shuffle's
    16-token blocks."""
    wl = W.WORKLOADS["zipf"]
    D, E, K, vtc, EP = 512, 16, 4, T - 50, 4
    inp = W.dispatch_inputs(wl, T=T, D=D, E=E, K=K, vtc=vtc, out0="normal")
    a = T * K
    g = np.random.default_rng(31)
    s = torch.from_numpy(np.ascontiguousarray(inp.scores)).to(dev)
    x, y, out0 = bf_dev(inp.x, dev), bf_dev(inp.y, dev), bf_dev(inp.out0, dev)
    slabs = bf_dev(W.to_bf16_bits(g.standard_normal((EP, a, D)).astype(np.float32)), dev)
    C, lo, hi = 16, 4, 12
    rcounts = g.integers(0, 6, size=(EP, C)).astype(np.int32)
    nrows = int(rcounts.sum())
    tok = bf_dev(W.to_bf16_bits(g.standard_normal((nrows, D)).astype(np.float32)), dev)
    rc = i32_dev(rcounts, dev)
    vtc_d = scalar_dev(vtc, dev)
    lib = ops._lib.load()

    def buffers():
        i32 = lambda *sh: torch.empty(sh, dtype=torch.int32, device=dev)  # noqa: E731
        u8 = lambda n: torch.empty(max(n, 1), dtype=torch.uint8, device=dev)  # noqa: E731
        bf = lambda *sh: torch.empty(sh, dtype=torch.bfloat16, device=dev)  # noqa: E731
        return dict(
            shuf=(i32(E + 1), i32(a), i32(a), i32(T, K)), rows=bf(a, D),
            gws=u8(lib.moe_gather_scale_workspace_bytes(T, a)),
            codes=torch.empty((a, D), dtype=torch.uint8, device=dev),
            qs=torch.empty(a, dtype=torch.float32, device=dev),
            out=out0.clone(), sws=u8(lib.moe_scatter_add_workspace_bytes(T, a)),
            pout=out0.clone(), pws=u8(lib.moe_scatter_add_padded_workspace_bytes(T, a, E)),
            cs=bf(nrows, D), cws=u8(lib.moe_shuffling_workspace_bytes(EP, hi - lo, nrows)),
            ss=bf(nrows, D), sws2=u8(lib.moe_shuffling_workspace_bytes(EP, hi - lo, nrows)))

    def path(b):
        counts, ei, ti, rop = ops.moe_shuffle_noalloc(s, K, vtc_d, out=b["shuf"])
        vr = counts[E:]
        ops.moe_gather_scale(x, ti, ei, s, vr, out=b["rows"], workspace=b["gws"])
        ops.moe_gather_scale_quant(x, ti, ei, s, None, vr, out=b["codes"], out_scale=b["qs"])
        ops.moe_scatter_add(b["out"], y, ti, vr, workspace=b["sws"])
        ops.moe_scatter_add_padded(slabs, counts[:E], ti, b["pout"], workspace=b["pws"])
        _, oc = ops.moe_combine_shuffling(tok, rc, lo, hi, None, out=b["cs"],
                                          workspace=b["cws"])
        ops.moe_split_shuffling(b["cs"], rc, lo, hi, None, out=b["ss"], workspace=b["sws2"])
        b["oc"] = oc

    def snapshot(b):
        V = int(b["shuf"][0][E].item())
        n = int(b["oc"][-1].item())
        snap = {k: b[k].cpu().clone() for k in ("out", "pout", "oc")}
        snap.update(rows=b["rows"][:V].cpu().clone(), codes=b["codes"][:V].cpu().clone(),
                    qs=b["qs"][:V].cpu().clone(), cs=b["cs"][:n].cpu().clone())
        for i, t in enumerate(b["shuf"]):
            snap[f"shuf{i}"] = t.cpu().clone()
        # the split writes back the rows of the local columns only
        snap["ss"] = b["ss"].cpu().clone()
        return snap

    say("graph replay, general paths", T, D, E, K, vtc, EP, nrows)
    eager = buffers()
    eager["ss"].view(torch.int16).fill_(0x7E00)
    path(eager)
    torch.cuda.synchronize()
    want = snapshot(eager)

    b = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one eager pass on the capture stream first
        path(b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        path(b)
    for rep in range(3):
        b["out"].copy_(out0)
        b["pout"].copy_(out0)
        for k in ("rows", "cs"):
            b[k].view(torch.int16).fill_(0x7E01 + rep)
        b["ss"].view(torch.int16).fill_(0x7E00)
        b["codes"].fill_(0xA5)
        b["qs"].fill_(-1.0)
        b["oc"].fill_(-7)
        for t in b["shuf"]:
            t.fill_(-3)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        got = snapshot(b)
        for k, v in want.items():
            assert torch.equal(got[k], v), (rep, k)


# ---------------------------------------------------------------- full sizes
@pytest.fixture(scope="module")
def zipf_inputs():
    wl = W.WORKLOADS["zipf"]
    inp = W.dispatch_inputs(wl)
    counts, ei, ti, rop = orc.shuffle(inp.scores, wl.K, wl.vtc)
    return wl, inp, counts, ei, ti, rop


def test_zipf_pipeline_full_size(dev, zipf_inputs):
    """shuffle -> gather (by token) -> scatter (by token) at T=8192, D=7168,
    E=256, K=8, valid_token_count=6000, as the benchmark launches it (row
    bound read from counts[E] on the device); every element checked."""
    wl, inp, counts, ei, ti, rop = zipf_inputs
    V = int(counts[wl.E])
    say("zipf pipeline", wl.T, wl.D, wl.E, wl.K, wl.vtc, V)
    s = torch.from_numpy(inp.scores).to(dev)
    gc, gei, gti, grop = ops.moe_shuffle(s, wl.K, scalar_dev(wl.vtc, dev))
    assert np.array_equal(gc.cpu().numpy(), counts)
    assert np.array_equal(grop.cpu().numpy(), rop)
    vr = gc[wl.E:]
    x = bf_dev(inp.x, dev)
    rows = torch.empty((wl.T * wl.K, wl.D), dtype=torch.bfloat16, device=dev)
    ops.moe_gather_scale_by_token(x, grop, gei, s, vr, rows)
    want_rows = np.zeros((wl.T * wl.K, wl.D), np.uint16)
    orc.gather_scale(inp.x, ti, ei, inp.scores, V, want_rows)
    assert np.array_equal(bits_host(rows[:V]), want_rows[:V])
    del want_rows
    out = torch.zeros((wl.T, wl.D), dtype=torch.bfloat16, device=dev)
    y = bf_dev(inp.y, dev)
    ops.moe_scatter_add_by_token(out, y, grop, vr)
    want = orc.scatter_add(inp.out0.copy(), inp.y, ti, V)
    assert np.array_equal(bits_host(out), want)
    # the general combine and both visit orders of the general gather agree
    # with the same oracle
    out2 = torch.zeros_like(out)
    ops.moe_scatter_add(out2, y, gti, vr)
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    for row_order in (False, True):
        rows2 = torch.empty_like(rows)
        ops.moe_gather_scale(x, gti, gei, s, vr, rows2, row_order=row_order)
        assert torch.equal(rows2[:V].view(torch.int16), rows[:V].view(torch.int16))


def test_quant_workload_full_size(dev):
    wl = W.WORKLOADS["quant"]
    inp = W.dispatch_inputs(wl)
    counts, ei, ti, rop = orc.shuffle(inp.scores, wl.K, None)
    V = int(counts[wl.E])
    say("quant workload", wl.T, wl.D, wl.E, wl.K)
    s = torch.from_numpy(inp.scores).to(dev)
    gc, gei, gti, grop = ops.moe_shuffle(s, wl.K)
    ub = torch.tensor([wl.scale_ub], dtype=torch.float32, device=dev)
    codes, scale = ops.moe_gather_scale_quant(bf_dev(inp.x, dev), gti, gei, s, ub, gc[wl.E:])
    wc, ws = orc.gather_scale_quant(inp.x, ti, ei, inp.scores, wl.scale_ub, V)
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), ws.view(np.uint32))
    assert_fp8_close(codes.cpu().numpy(), wc, "quant workload")
    out = torch.zeros((wl.T, wl.D), dtype=torch.bfloat16, device=dev)
    ops.moe_scatter_add_by_token(out, bf_dev(inp.y, dev), grop, gc[wl.E:])
    assert np.array_equal(bits_host(out), orc.scatter_add(inp.out0.copy(), inp.y, ti, V))


def test_prefill_finalize_full_size(dev):
    wl = W.WORKLOADS["prefill"]
    fi = W.finalize_inputs(wl)
    say("prefill finalize", wl.T, wl.D, wl.K)
    out, codes, scales = ops.moe_finalize_rmsnorm(
        bf_dev(fi.y, dev), torch.from_numpy(fi.w).to(dev), i32_dev(fi.row_of_pair, dev),
        bf_dev(fi.shared, dev), bf_dev(fi.gamma, dev), fi.eps, mxfp8=True)
    got = bits_host(out)
    want, wcodes, wscales = orc.finalize_rmsnorm(fi.y, fi.w, fi.row_of_pair, fi.shared,
                                                 fi.gamma, fi.eps, mxfp8=True)
    _close(got, want, "prefill")
    # MXFP8 end to end: the GPU's codes and scales against the oracle's own
    assert_mx_end_to_end(codes.cpu().numpy(), scales.cpu().numpy(), wcodes, wscales,
                         "prefill mxfp8")
    oc, os_ = orc.mxfp8_quantize(got)
    assert np.array_equal(scales.cpu().numpy(), os_)
    assert_fp8_close(codes.cpu().numpy(), oc, "prefill mxfp8")


def test_prefill_swizzled_finalize_full_size(dev):
    """The prefill finalize with bf16 routing weights and 128x4-tiled MXFP8
    scales at T=16384, D=5120, K=4, as the benchmark launches it."""
    wl = W.WORKLOADS["prefill"]
    fi = W.finalize_inputs(wl)
    wb = W.to_bf16_bits(fi.w)
    say("prefill-swizzled finalize", wl.T, wl.D, wl.K)
    out, codes, scales = ops.moe_finalize_rmsnorm(
        bf_dev(fi.y, dev), bf_dev(wb, dev), i32_dev(fi.row_of_pair, dev),
        bf_dev(fi.shared, dev), bf_dev(fi.gamma, dev), fi.eps, mxfp8=True,
        scale_layout="swizzled")
    got = bits_host(out)
    want, wcodes, wscales = orc.finalize_rmsnorm(fi.y, wb, fi.row_of_pair, fi.shared, fi.gamma,
                                                 fi.eps, flags=2 | 4, mxfp8=True)
    _close(got, want, "prefill-swizzled")
    assert_mx_end_to_end(codes.cpu().numpy(), scales.cpu().numpy(), wcodes, wscales,
                         "prefill-swizzled mxfp8")
    oc, os_ = orc.mxfp8_quantize(got)
    assert np.array_equal(scales.cpu().numpy(), orc.mxfp8_swizzle(os_))
    assert_fp8_close(codes.cpu().numpy(), oc, "prefill-swizzled mxfp8")


def test_mhc_finalize_full_size(dev):
    """The hc = 4 mHC finalize at T=16384, D=5120, K=4 with MXFP8 and swizzled
    scales, as the benchmark launches it."""
    wl = W.WORKLOADS["mhc"]
    fi = W.finalize_inputs(wl)
    m = W.mhc_inputs(wl)
    say("mhc finalize", wl.T, wl.D, wl.K, wl.hc)
    f32 = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
    res_out, out, codes, scales = ops.moe_finalize_mhc(
        bf_dev(fi.y, dev), f32(fi.w), i32_dev(fi.row_of_pair, dev), bf_dev(fi.shared, dev),
        bf_dev(m.residual, dev), f32(m.post), f32(m.comb), f32(m.pre), bf_dev(fi.gamma, dev),
        fi.eps, mxfp8=True, scale_layout="swizzled")
    want = orc.finalize_mhc(fi.y, fi.w, fi.row_of_pair, fi.shared, m.residual, m.post, m.comb,
                            m.pre, fi.gamma, fi.eps, flags=4, mxfp8=True)
    _close(bits_host(res_out), want[0], "mhc residual_out")
    got = bits_host(out)
    _close(got, want[1], "mhc out")
    assert_mx_end_to_end(codes.cpu().numpy(), scales.cpu().numpy(), want[2], want[3],
                         "mhc mxfp8")
    oc, rm = orc.mxfp8_quantize(got)
    assert np.array_equal(scales.cpu().numpy(), orc.mxfp8_swizzle(rm))
    assert_fp8_close(codes.cpu().numpy(), oc, "mhc mxfp8")


def test_padded_combine_full_routing(dev):
    """The padded workload's routing at full size (zipf scores, T=8192, E=256,
    K=8, valid_token_count=6000, EP=8 static buffer), shuffled on the device
    as the benchmark does; rows of D=256 keep the host copy of the eight
    slabs small. Every element checked, through token_indices and through
    row_of_pair."""
    wl = W.WORKLOADS["padded"]
    D = 256
    inp = W.dispatch_inputs(wl, D=D, with_y=False)
    counts, ei, ti, rop = orc.shuffle(inp.scores, wl.K, wl.vtc)
    say("padded full routing", wl.T, D, wl.E, wl.K, wl.ep, int(counts[wl.E]))
    s = torch.from_numpy(inp.scores).to(dev)
    gc, gei, gti, grop = ops.moe_shuffle(s, wl.K, scalar_dev(wl.vtc, dev))
    assert np.array_equal(gti.cpu().numpy(), ti)
    slabs = W.to_bf16_bits(np.random.default_rng(6).standard_normal(
        (wl.ep, wl.T * wl.K, D), dtype=np.float32))
    want = orc.scatter_add_padded(np.zeros((wl.T, D), np.uint16), slabs, counts[:wl.E], ti)
    out = torch.zeros((wl.T, D), dtype=torch.bfloat16, device=dev)
    ops.moe_scatter_add_padded(bf_dev(slabs, dev), gc[:wl.E].contiguous(), gti, out)
    assert np.array_equal(bits_host(out), want)
    out = torch.zeros((wl.T, D), dtype=torch.bfloat16, device=dev)
    ops.moe_scatter_add_padded_by_token(bf_dev(slabs, dev), gc[:wl.E].contiguous(), grop, out)
    assert np.array_equal(bits_host(out), want)


def test_padded_combine_full_size(dev):
    """The padded workload exactly as the benchmark launches it: T=8192,
    D=7168, E=256, K=8, valid_token_count=6000, eight (T*K, D) slabs drawn
    on the device. Every 7th 16-byte chunk of each output row -- every slice
    of the launch, lanes at every offset -- is checked against the oracle run
    on those columns (the combine is independent per column); the by-token
    form (row_of_pair) equals it bit for bit on every element."""
    wl = W.WORKLOADS["padded"]
    T, D, E, K, EP = wl.T, wl.D, wl.E, wl.K, wl.ep
    inp = W.dispatch_inputs(wl, with_y=False)
    counts, ei, ti, rop = orc.shuffle(inp.scores, K, wl.vtc)
    say("padded full size", T, D, E, K, EP, int(counts[E]))
    gc, gei, gti, grop = ops.moe_shuffle(torch.from_numpy(inp.scores).to(dev), K,
                                         scalar_dev(wl.vtc, dev))
    assert np.array_equal(gti.cpu().numpy(), ti)
    gen = torch.Generator(device=dev)
    gen.manual_seed(6006)
    slabs = torch.empty((EP, T * K, D), dtype=torch.bfloat16, device=dev)
    for r in range(EP):
        slabs[r] = torch.randn((T * K, D), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.zeros((T, D), dtype=torch.bfloat16, device=dev)
    ops.moe_scatter_add_padded(slabs, gc[:E].contiguous(), gti, out)
    out_t = torch.zeros((T, D), dtype=torch.bfloat16, device=dev)
    ops.moe_scatter_add_padded_by_token(slabs, gc[:E].contiguous(), grop, out_t)
    assert torch.equal(out_t.view(torch.int16), out.view(torch.int16))
    del out_t
    chunks = torch.arange(0, D // 8, 7, device=dev)
    cols = (chunks[:, None] * 8 + torch.arange(8, device=dev)).reshape(-1)
    sub = bits_host(slabs.index_select(2, cols))
    del slabs
    want = orc.scatter_add_padded(np.zeros((T, cols.numel()), np.uint16), sub, counts[:E], ti)
    assert np.array_equal(bits_host(out.index_select(1, cols)), want)


def test_shuffling_workload_full_size(dev):
    """The EP re-sort as the benchmark runs it: eight source ranks of 8192
    tokens routed over E=256 with K=8, rank 0's 32 local experts, packed
    layout, D=7168; combine and split, every element checked."""
    wl = W.WORKLOADS["shuffling"]
    EG = wl.E // wl.ep
    per_src = []
    for r in range(wl.ep):
        c, _, _, _ = orc.shuffle(W.router_scores(wl, seed=r), wl.K)
        per_src.append(c[:EG])
    cnt = np.stack(per_src).astype(np.int32)
    rows = int(cnt.sum())
    say("shuffling full size", wl.ep, EG, rows, wl.D)
    tok = W.to_bf16_bits(np.random.default_rng(7).standard_normal((rows, wl.D),
                                                                  dtype=np.float32))
    want, woc = orc.combine_shuffling(tok, cnt, 0, EG, None)
    cd = i32_dev(cnt, dev)
    em, oc = ops.moe_combine_shuffling(bf_dev(tok, dev), cd, 0, EG)
    assert np.array_equal(oc.cpu().numpy(), woc)
    assert np.array_equal(bits_host(em), want)
    back = ops.moe_split_shuffling(em, cd, 0, EG)
    assert np.array_equal(bits_host(back), tok)


def test_c_abi_consumer(dev, tmp_path):
    """A plain C program (tests/c_abi_consumer.c: gcc, the header and the HIP
    runtime only) runs moe_shuffle, moe_gather_scale (token_indices) and its
    by-token form, moe_gather_scale_quant, moe_scatter_add (token_indices) and
    its by-token form, and moe_finalize_rmsnorm with MXFP8 on the tiny
    workload, as a child process; every output equals the oracle's."""
    import subprocess
    exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_consumer")
    assert os.path.exists(exe), "build the library first: it also builds the C consumer"
    wl = W.WORKLOADS["tiny"]
    T, D, E, K = wl.T, wl.D, wl.E, wl.K
    a = T * K
    inp = W.dispatch_inputs(wl, out0="normal")
    fi = W.finalize_inputs(W.WORKLOADS["decode"], T=T, D=D, K=K)
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(fin, "wb") as f:
        f.write(np.array([T, E, K, D], np.int32).tobytes())
        for arr in (inp.scores, inp.x, inp.y, inp.out0, fi.w, fi.shared, fi.gamma,
                    np.array([fi.eps], np.float32)):
            f.write(np.ascontiguousarray(arr).tobytes())
    say("c consumer", T, D, E, K)
    r = subprocess.run([exe, str(fin), str(fout)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    buf = np.fromfile(fout, dtype=np.uint8)
    sizes = [(E + 1) * 4, a * 4, a * 4, a * 4, a * D * 2, a * D * 2, a * D, a * 4,
             T * D * 2, T * D * 2, T * D * 2, T * D, T * D // 32]
    assert buf.size == sum(sizes)
    parts = np.split(buf, np.cumsum(sizes)[:-1])
    gc, gei, gti, grop = (p.view(np.int32) for p in parts[:4])
    rows, rows_g = (p.view(np.uint16).reshape(a, D) for p in parts[4:6])
    codes, qscale = parts[6].reshape(a, D), parts[7].view(np.float32)
    out, out_g, fo = (p.view(np.uint16).reshape(T, D) for p in parts[8:11])
    mc, ms = parts[11].reshape(T, D), parts[12].reshape(T, D // 32)
    counts, ei, ti, rop = orc.shuffle(inp.scores, K)
    V = int(counts[E])
    assert np.array_equal(gc, counts) and np.array_equal(gei, ei) and np.array_equal(gti, ti)
    assert np.array_equal(grop, rop.ravel())
    want_rows = orc.gather_scale(inp.x, ti, ei, inp.scores, V)
    assert np.array_equal(rows[:V], want_rows[:V])
    assert np.array_equal(rows_g[:V], want_rows[:V])
    wq, ws = orc.gather_scale_quant(inp.x, ti, ei, inp.scores, None, V)
    assert np.array_equal(codes[:V], wq[:V])
    assert np.array_equal(qscale[:V].view(np.uint32), ws[:V].view(np.uint32))
    want_out = orc.scatter_add(inp.out0.copy(), inp.y, ti, V)
    assert np.array_equal(out, want_out) and np.array_equal(out_g, want_out)
    wo, wc, wsc = orc.finalize_rmsnorm(inp.y, fi.w, rop.reshape(T, K), fi.shared, fi.gamma,
                                       fi.eps, mxfp8=True)
    _close(fo, wo, "c consumer finalize")
    assert_mx_end_to_end(mc, ms, wc, wsc, "c consumer mxfp8")


def _large_seed(seed):
    """Seeds 24-31, and every fifth seed from 32 on, draw the large shapes."""
    return 24 <= seed < 32 or (seed >= 32 and seed % 5 == 0)


def test_randomized_shapes_against_oracle(dev, random_seed):
    """Seeded random shapes through every entry point: T, D, E, K, the valid
    count, score strides and EP drawn per seed; every output checked. The
    large seeds draw thousands of tokens and up to 1024 experts (narrow rows),
    so the shuffle takes its three-launch form there. `--random-shape-seeds N`
    runs seeds F .. F+N-1 (`--random-shape-first F`, default 0; N default 32)."""
    seed = random_seed
    g = np.random.default_rng(1000 + seed)
    if not _large_seed(seed):
        T = int(g.integers(1, 300))
        E = int(g.integers(1, 300))
        K = int(g.integers(1, min(E, 16) + 1))
        D = 8 * int(g.integers(1, 260))
    else:
        T = int(g.integers(2000, 6000))
        E = int(g.integers(300, 1025))
        K = int(g.integers(1, 17))
        D = 8 * int(g.integers(1, 33))
    vtc = None if g.random() < 0.3 else int(g.integers(0, T + 1))
    say("random", seed, T, D, E, K, vtc)
    s = g.standard_normal((T, E)).astype(np.float32)
    if g.random() < 0.3:
        s = np.round(s * 2) / 2                        # ties
    x = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    y = W.to_bf16_bits(g.standard_normal((T * K, D)).astype(np.float32))
    out0 = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    counts, ei, ti, rop = orc.shuffle(s, K, vtc)
    V = int(counts[E])
    if g.random() < 0.5:
        sd = torch.from_numpy(np.ascontiguousarray(s.T)).to(dev).t()
    else:
        sd = torch.from_numpy(s).to(dev)
    gc, gei, gti, grop = ops.moe_shuffle(sd, K, scalar_dev(vtc, dev))
    assert np.array_equal(gc.cpu().numpy(), counts)
    assert np.array_equal(gti.cpu().numpy(), ti) and np.array_equal(gei.cpu().numpy(), ei)
    assert np.array_equal(grop.cpu().numpy(), rop)
    vr = gc[E:]
    want_rows = orc.gather_scale(x, ti, ei, s, V)
    for path in ("lists", "rows", "by_token"):
        rows = torch.zeros((T * K, D), dtype=torch.bfloat16, device=dev)
        if path != "by_token":
            ops.moe_gather_scale(bf_dev(x, dev), gti, gei, sd, vr, rows,
                                 row_order=path == "rows")
        else:
            ops.moe_gather_scale_by_token(bf_dev(x, dev), grop, gei, sd, vr, rows)
        assert np.array_equal(bits_host(rows)[:V], want_rows[:V]), path
    wq, wsc = orc.gather_scale_quant(x, ti, ei, s, None, V)
    q, qs = ops.moe_gather_scale_quant(bf_dev(x, dev), gti, gei, sd, None, vr)
    assert np.array_equal(q.cpu().numpy()[:V], wq[:V])
    assert np.array_equal(qs.cpu().numpy()[:V].view(np.uint32), wsc[:V].view(np.uint32))
    want = orc.scatter_add(out0.copy(), y, ti, V)
    for path in ("general", "by_token"):
        out = bf_dev(out0, dev)
        if path == "general":
            ops.moe_scatter_add(out, bf_dev(y, dev), gti, vr)
        else:
            ops.moe_scatter_add_by_token(out, bf_dev(y, dev), grop, vr)
        assert np.array_equal(bits_host(out), want), path
    # padded combine over a divisor of E
    EP = int(g.choice([d for d in range(1, min(E, 8) + 1) if E % d == 0]))
    slabs = W.to_bf16_bits(g.standard_normal((EP, T * K, D)).astype(np.float32))
    want = orc.scatter_add_padded(out0.copy(), slabs, counts[:E], ti)
    out = bf_dev(out0, dev)
    ops.moe_scatter_add_padded(bf_dev(slabs, dev), gc[:E].contiguous(), gti, out)
    assert np.array_equal(bits_host(out), want)
    out = bf_dev(out0, dev)
    ops.moe_scatter_add_padded_by_token(bf_dev(slabs, dev), gc[:E].contiguous(), grop, out)
    assert np.array_equal(bits_host(out), want)
    # finalize and mHC on the shuffle's rows (D a multiple of 32 for MXFP8);
    # the finalize's flags drawn per seed: bf16 squares, bf16 weights, and the
    # 128x4-tiled scales where D allows them
    Df = 32 * max(1, D // 32)
    yf = W.to_bf16_bits(g.standard_normal((T * K, Df)).astype(np.float32))
    w = g.random((T, K)).astype(np.float32)
    shared = W.to_bf16_bits(g.standard_normal((T, Df)).astype(np.float32))
    gamma = W.to_bf16_bits(g.uniform(0.5, 1.5, Df).astype(np.float32))
    fl = int(g.integers(0, 8)) & (7 if Df % 128 == 0 else 3)
    wk = W.to_bf16_bits(w) if fl & 2 else w
    say("random finalize flags", fl)
    want_o, want_c, want_s = orc.finalize_rmsnorm(yf, wk, rop, shared, gamma, 1e-6, flags=fl,
                                                  mxfp8=True)
    wdev = bf_dev(wk, dev) if fl & 2 else torch.from_numpy(w).to(dev)
    o, mc, ms = ops.moe_finalize_rmsnorm(bf_dev(yf, dev), wdev, grop, bf_dev(shared, dev),
                                         bf_dev(gamma, dev), 1e-6, flags=fl & 1, mxfp8=True,
                                         scale_layout="swizzled" if fl & 4 else "rowmajor")
    _close(bits_host(o), want_o, "finalize")
    assert_mx_end_to_end(mc.cpu().numpy(), ms.cpu().numpy().reshape(-1), want_c,
                         np.asarray(want_s).reshape(-1), "finalize MXFP8")
    hc = int(g.integers(1, 5))
    res = W.to_bf16_bits(g.standard_normal((T, hc, Df)).astype(np.float32))
    post = g.uniform(0, 2, (T, hc)).astype(np.float32)
    comb = g.random((T, hc, hc)).astype(np.float32)
    pre = g.random((T, hc)).astype(np.float32)
    wres, wout, wmc, wms = orc.finalize_mhc(yf, wk, rop, shared, res, post, comb, pre, gamma,
                                            1e-6, flags=fl, mxfp8=True)
    f32 = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
    r_out, m_out, mmc, mms = ops.moe_finalize_mhc(
        bf_dev(yf, dev), wdev, grop, bf_dev(shared, dev), bf_dev(res, dev), f32(post),
        f32(comb), f32(pre), bf_dev(gamma, dev), 1e-6, flags=fl & 1, mxfp8=True,
        scale_layout="swizzled" if fl & 4 else "rowmajor")
    _close(bits_host(r_out), wres, "mhc residual")
    _close(bits_host(m_out), wout, "mhc out")
    assert_mx_end_to_end(mmc.cpu().numpy(), mms.cpu().numpy().reshape(-1), wmc,
                         np.asarray(wms).reshape(-1), "mhc MXFP8")
    # the EP re-sort both ways: ranks, columns, local range and layout drawn
    EP, C = int(g.integers(1, 9)), int(g.integers(1, 65))
    lo = int(g.integers(0, C + 1))
    hi = int(g.integers(lo, C + 1))
    rc = g.integers(0, 7, size=(EP, C)).astype(np.int32)
    packed = bool(g.random() < 0.5)
    stride = None if packed else int(rc.sum(axis=1).max() + g.integers(0, 4))
    nrows = max(1, int(rc.sum()) if packed else EP * stride)
    Dr = 8 * int(g.integers(1, 100))
    say("random re-sort", EP, C, lo, hi, packed, nrows, Dr)
    tok = W.to_bf16_bits(g.standard_normal((nrows, Dr)).astype(np.float32))
    want_c, want_oc = orc.combine_shuffling(tok, rc, lo, hi, stride,
                                            out=np.full((nrows, Dr), SENTINEL, np.uint16))
    out_c = torch.full((nrows, Dr), SENTINEL - 65536, dtype=torch.int16,
                       device=dev).view(torch.bfloat16)
    out_c, oc = ops.moe_combine_shuffling(bf_dev(tok, dev), i32_dev(rc, dev), lo, hi, stride,
                                          out=out_c)
    assert np.array_equal(oc.cpu().numpy(), want_oc)
    assert np.array_equal(bits_host(out_c), want_c)
    want_s = orc.split_shuffling(want_c, rc, lo, hi, stride,
                                 out=np.full((nrows, Dr), SENTINEL, np.uint16))
    out_s = torch.full((nrows, Dr), SENTINEL - 65536, dtype=torch.int16,
                       device=dev).view(torch.bfloat16)
    ops.moe_split_shuffling(out_c, i32_dev(rc, dev), lo, hi, stride, out=out_s)
    assert np.array_equal(bits_host(out_s), want_s)


def test_every_op_is_deterministic(dev):
    """Each entry point run three times on the same inputs gives the same
    bits, including the combines whose row lists are built with atomics
    (here with up to 40 rows on one token)."""
    g = np.random.default_rng(77)
    T, D, E, K = 300, 640, 32, 8
    s = torch.from_numpy(g.standard_normal((T, E)).astype(np.float32)).to(dev)
    x = bf_dev(W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32)), dev)
    y = bf_dev(W.to_bf16_bits(g.standard_normal((T * K, D)).astype(np.float32)), dev)
    out0 = bf_dev(W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32)), dev)
    ti_hot = np.where(g.random(T * K) < 0.02, 7, g.integers(0, T, T * K)).astype(np.int32)
    ti_hot = i32_dev(ti_hot, dev)
    say("determinism", T, D, E, K)

    def run_once():
        counts, ei, ti, rop = ops.moe_shuffle(s, K, scalar_dev(250, dev))
        vr = counts[E:]
        rows = ops.moe_gather_scale_by_token(x, rop, ei, s, vr,
                                             torch.zeros((T * K, D), dtype=torch.bfloat16,
                                                         device=dev))
        q, qs = ops.moe_gather_scale_quant(x, ti, ei, s, None, vr)
        a = out0.clone()
        ops.moe_scatter_add(a, y, ti_hot)
        b = out0.clone()
        ops.moe_scatter_add_padded(y.view(2, T * K // 2, D).repeat(1, 2, 1).contiguous(),
                                   torch.full((E,), T * K // E, dtype=torch.int32, device=dev),
                                   ti_hot, b)
        c = out0.clone()
        ops.moe_scatter_add_by_token(c, y, rop, vr)
        w = torch.rand((T, K), device=dev)
        o, mc, ms = ops.moe_finalize_rmsnorm(y, w, rop, out0, x[0].contiguous(), 1e-6,
                                             mxfp8=True)
        torch.cuda.synchronize()
        V = int(counts[E].item())  # rows past V of the FP8 outputs are not written
        return [t.cpu() for t in (counts, ei, ti, rop, rows, q[:V], qs[:V], a, b, c,
                                  o, mc, ms)], w

    first, w0 = run_once()
    for _ in range(2):
        again, w = run_once()
        for i, (u, v) in enumerate(zip(first[:10], again[:10])):
            assert torch.equal(u, v), i
    # the finalize with the same weights both times
    counts, ei, ti, rop = ops.moe_shuffle(s, K, scalar_dev(250, dev))
    outs = [ops.moe_finalize_rmsnorm(y, w0, rop, out0, x[0].contiguous(), 1e-6,
                                     mxfp8=True) for _ in range(3)]
    for o, mc, ms in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(mc, outs[0][1])
        assert torch.equal(ms, outs[0][2])


def test_prepared_calls_match_checked_calls(dev):
    """ops.prepare: each replay gives the bits of the checked op on the
    current inputs (changed in place between replays), and the workspace the
    shuffle allocated for itself survives allocator churn between replays."""
    T, D, E, K, vtc = 300, 1024, 16, 4, 250
    inp, _, _, _, _ = _dispatch_case(T, D, E, K, vtc)
    s = torch.from_numpy(inp.scores).to(dev)
    x = bf_dev(inp.x, dev)
    vtc_d = scalar_dev(vtc, dev)
    say("prepared", T, D, E, K, vtc)
    shuffle = ops.prepare(ops.moe_shuffle, s, K, vtc_d)
    counts, ei, ti, rop = shuffle()
    rows = torch.zeros((T * K, D), dtype=torch.bfloat16, device=dev)
    gather = ops.prepare(ops.moe_gather_scale_by_token, x, rop, ei, s, counts[E:], rows)
    g = np.random.default_rng(5)
    for rep in range(3):
        junk = [torch.full((1 << 20,), rep, dtype=torch.int32, device=dev) for _ in range(4)]
        del junk                                   # the caching allocator reuses these
        new_s = g.standard_normal((T, E)).astype(np.float32)
        s.copy_(torch.from_numpy(new_s))
        got = shuffle()
        assert got[0] is counts and got[3] is rop
        gather()
        wc, wei, wti, wrop = orc.shuffle(new_s, K, vtc)
        assert np.array_equal(counts.cpu().numpy(), wc), rep
        assert np.array_equal(ti.cpu().numpy(), wti), rep
        assert np.array_equal(rop.cpu().numpy(), wrop), rep
        V = int(wc[E])
        want = orc.gather_scale(inp.x, wti, wei, new_s, V)
        assert np.array_equal(bits_host(rows)[:V], want[:V]), rep

    fi = W.finalize_inputs(W.WORKLOADS["decode"], T=32, D=7168, K=8)
    y = bf_dev(fi.y, dev)
    args = (y, torch.from_numpy(fi.w).to(dev), i32_dev(fi.row_of_pair, dev),
            bf_dev(fi.shared, dev), bf_dev(fi.gamma, dev), fi.eps)
    fin = ops.prepare(ops.moe_finalize_rmsnorm, *args, mxfp8=True)
    for rep in range(2):
        y.copy_(bf_dev(W.to_bf16_bits(g.standard_normal(fi.y.shape).astype(np.float32)), dev))
        o, mc, ms = fin()
        ro, rmc, rms = ops.moe_finalize_rmsnorm(*args, mxfp8=True)
        assert torch.equal(o, ro) and torch.equal(mc, rmc) and torch.equal(ms, rms), rep


def test_prepared_calls_cover_every_op(dev):
    """Every other op prepared once and replayed twice gives the bits of two
    checked calls on twin buffers; the in-place combines accumulate twice
    either way."""
    g = np.random.default_rng(9)
    T, D, E, K = 200, 640, 16, 4
    rnd = lambda *sh: W.to_bf16_bits(g.standard_normal(sh).astype(np.float32))  # noqa: E731
    s = torch.from_numpy(g.standard_normal((T, E)).astype(np.float32)).to(dev)
    x, y, out0 = bf_dev(rnd(T, D), dev), bf_dev(rnd(T * K, D), dev), rnd(T, D)
    counts, ei, ti, rop = ops.moe_shuffle(s, K, scalar_dev(180, dev))
    vr = counts[E:]
    fi = W.finalize_inputs(W.WORKLOADS["mhc"], T=8, D=1024, K=4)
    m = W.mhc_inputs(W.WORKLOADS["mhc"], T=8, D=1024, hc=4)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    cnt = g.integers(0, 6, size=(4, 8)).astype(np.int32)
    tok = bf_dev(rnd(int(cnt.sum()), 256), dev)
    slabs = bf_dev(rnd(2, T * K, D), dev)

    def zeros_like_rows():
        return torch.zeros((T * K, D), dtype=torch.bfloat16, device=dev)

    cases = {
        "gather lists": lambda o: ops.moe_gather_scale(x, ti, ei, s, vr, o),
        "gather rows": lambda o: ops.moe_gather_scale(x, ti, ei, s, vr, o, row_order=True),
        "quant": lambda o: ops.moe_gather_scale_quant(x, ti, ei, s, None, vr, o[0], o[1]),
        "scatter": lambda o: ops.moe_scatter_add(o, y, ti, vr),
        "scatter by token": lambda o: ops.moe_scatter_add_by_token(o, y, rop, vr),
        "padded": lambda o: ops.moe_scatter_add_padded(slabs, counts[:E].contiguous(), ti, o),
        "padded by token": lambda o: ops.moe_scatter_add_padded_by_token(
            slabs, counts[:E].contiguous(), rop, o),
        "combine_shuffling": lambda o: ops.moe_combine_shuffling(tok, i32_dev(cnt, dev), 2, 6,
                                                                 out=o),
        "mhc": lambda o: ops.moe_finalize_mhc(
            bf_dev(fi.y, dev), f32(fi.w), i32_dev(fi.row_of_pair, dev), bf_dev(fi.shared, dev),
            bf_dev(m.residual, dev), f32(m.post), f32(m.comb), f32(m.pre),
            bf_dev(fi.gamma, dev), fi.eps, residual_out=o[0], out=o[1], mxfp8=True,
            mx_codes=o[2], mx_scales=o[3]),
    }

    def buffers(name):
        if name.startswith("gather"):
            return zeros_like_rows()
        if name == "quant":
            return (torch.zeros((T * K, D), dtype=torch.uint8, device=dev),
                    torch.zeros(T * K, dtype=torch.float32, device=dev))
        if name.startswith("scatter") or name.startswith("padded"):
            return bf_dev(out0, dev)
        if name == "combine_shuffling":
            return torch.zeros_like(tok)
        return (torch.zeros((8, 4, 1024), dtype=torch.bfloat16, device=dev),
                torch.zeros((8, 1024), dtype=torch.bfloat16, device=dev),
                torch.zeros((8, 1024), dtype=torch.uint8, device=dev),
                torch.zeros(ops._lib.load().moe_mxfp8_scale_bytes(8, 1024, 0), dtype=torch.uint8,
                            device=dev))

    def flat(r):
        return [t for t in (r if isinstance(r, tuple) else (r,)) if isinstance(t, torch.Tensor)]

    for name, run in cases.items():
        say("prepared", name)
        a, b = buffers(name), buffers(name)
        run(a)
        ra = run(a)
        p = ops.prepare(run, b)
        rb = p()
        torch.cuda.synchronize()
        for u, v in zip(flat(a) + flat(ra), flat(b) + flat(rb)):
            assert torch.equal(u, v), name


def test_binding_checks_caller_workspaces(dev):
    """A workspace the caller passes must be a contiguous tensor on the same
    GPU (else ValueError before any launch); any dtype works, its size counted
    in bytes."""
    say("binding workspaces")
    T, E, K, D = 40, 8, 2, 64
    s = torch.rand((T, E), device=dev)
    counts, ei, ti, rop = ops.moe_shuffle(s, K)
    x = torch.randn((T, D), device=dev).to(torch.bfloat16)
    y = torch.randn((T * K, D), device=dev).to(torch.bfloat16)
    lib = ops._lib.load()
    calls = {
        "shuffle": (lib.moe_shuffle_workspace_bytes(T, E, K),
                    lambda ws: ops.moe_shuffle(s, K, workspace=ws)),
        "gather": (lib.moe_gather_scale_workspace_bytes(T, T * K),
                   lambda ws: ops.moe_gather_scale(x, ti, ei, s, counts[E:], workspace=ws)),
        "scatter": (lib.moe_scatter_add_workspace_bytes(T, T * K),
                    lambda ws: ops.moe_scatter_add(x.clone(), y, ti, counts[E:], workspace=ws)),
        "padded": (lib.moe_scatter_add_padded_workspace_bytes(T, T * K, E),
                   lambda ws: ops.moe_scatter_add_padded(y.view(1, T * K, D), counts[:E].clone(),
                                                         ti, x.clone(), workspace=ws)),
        "combine_shuffling": (lib.moe_shuffling_workspace_bytes(2, 4, T * K),
                              lambda ws: ops.moe_combine_shuffling(
                                  y, counts[:E].view(2, 4).contiguous(), workspace=ws)),
    }
    for name, (need, call) in calls.items():
        with pytest.raises(ValueError):
            call(torch.empty(need + 256, dtype=torch.uint8))                  # host memory
        with pytest.raises(ValueError):
            call(torch.empty((need + 256) * 2, dtype=torch.uint8, device=dev)[::2])  # strided
        call(torch.empty((need + 3) // 4 + 64, dtype=torch.float32, device=dev))   # bytes
    torch.cuda.synchronize()


def test_binding_checks_caller_outputs(dev):
    """Outputs the caller passes must have the exact shape (or, for the EP
    re-sort, D columns), dtype and device; a wrong one raises ValueError
    before any launch."""
    say("binding outputs")
    T, E, K, D = 16, 4, 2, 64
    s = torch.rand((T, E), device=dev)
    counts, ei, ti, rop = ops.moe_shuffle(s, K)
    x = torch.randn((T, D), device=dev).to(torch.bfloat16)
    y = torch.randn((T * K, D), device=dev).to(torch.bfloat16)
    w = torch.rand((T, K), device=dev)
    g = torch.ones(D, dtype=torch.bfloat16, device=dev)
    res = torch.randn((T, 2, D), device=dev).to(torch.bfloat16)
    post, comb, pre = torch.rand((T, 2), device=dev), torch.rand((T, 2, 2), device=dev), \
        torch.rand((T, 2), device=dev)
    bf, u8, f32 = torch.bfloat16, torch.uint8, torch.float32
    bad = [
        lambda: ops.moe_gather_scale(x, ti, ei, s, out=torch.empty((T * K - 1, D), dtype=bf,
                                                                   device=dev)),
        lambda: ops.moe_gather_scale_quant(x, ti, ei, s, out=torch.empty((T * K, D - 16),
                                                                         dtype=u8, device=dev)),
        lambda: ops.moe_gather_scale_quant(x, ti, ei, s, out_scale=torch.empty(
            T * K - 1, dtype=f32, device=dev)),
        lambda: ops.moe_finalize_rmsnorm(y, w, rop, None, g, 1e-6, out=torch.empty(
            (T, D // 2), dtype=bf, device=dev)),
        lambda: ops.moe_finalize_rmsnorm(y, w, rop, None, g, 1e-6, out=torch.empty(
            (T, D), dtype=bf)),
        lambda: ops.moe_finalize_mhc(y, w, rop, None, res, post, comb, pre, g, 1e-6,
                                     residual_out=torch.empty((T, 1, D), dtype=bf, device=dev)),
        lambda: ops.moe_finalize_mhc(y, w, rop, None, res, post, comb, pre, g, 1e-6,
                                     out=torch.empty((T - 1, D), dtype=bf, device=dev)),
        lambda: ops.moe_combine_shuffling(y, counts[:E].view(2, 2).contiguous(),
                                          out=torch.empty((T * K, D // 2), dtype=bf, device=dev)),
    ]
    for i, call in enumerate(bad):
        with pytest.raises(ValueError):
            call()
    torch.cuda.synchronize()


def test_zero_width_rows_are_no_ops(dev):
    """D = 0: every row entry point returns without touching anything."""
    say("zero-width rows")
    T, E, K = 6, 4, 2
    z = torch.empty((T, 0), dtype=torch.bfloat16, device=dev)
    zi = torch.zeros(T * K, dtype=torch.int32, device=dev)
    s = torch.rand((T, E), device=dev)
    ops.moe_gather_scale(z, zi, zi, s, out=torch.empty((T * K, 0), dtype=torch.bfloat16,
                                                      device=dev))
    ops.moe_gather_scale_quant(z, zi, zi, s)
    ops.moe_scatter_add(z.clone(), torch.empty((T * K, 0), dtype=torch.bfloat16, device=dev), zi)
    ops.moe_scatter_add_by_token(z.clone(), torch.empty((T * K, 0), dtype=torch.bfloat16,
                                                        device=dev), zi.view(T, K))
    torch.cuda.synchronize()
