"""Pins for the oracle's combine stages: scatter_add, the MoE finalize with
RMSNorm, and its MXFP8 output (CPU only).

scatter_add: gather-then-scatter with unit scores reproduces K*x exactly; a
pure-Python fp32 brute force on tiny inputs; torch.index_add_ in fp64 within
bf16 rounding; untouched tokens keep their bits.
finalize: special cases that reduce to torch.nn.functional.rms_norm; an fp64
evaluation of the weighted sum; the constant-row closed form; exact invariance
under power-of-two scaling (eps = 0); the bf16-square mode against torch's
bf16 multiply; the RMSNorm bit for bit against exact rational arithmetic (the
sum of squares rounded once to fp32 from its exact value, the correctly
rounded inverse square root), on rows where a plain fp32 running sum rounds
differently.
MXFP8: the scale byte is the round-up power of two of each block's max; codes
are torch's E4M3 cast of the scaled block; re-quantising the dequantised block
is the identity.
"""
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

from combine_moe_shuffle_amd import workloads as W


def _bf(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- scatter_add
@pytest.mark.parametrize("K", [1, 2, 4, 8])
def test_gather_scatter_roundtrip_unit_scores(orc, K):
    g = np.random.default_rng(K)
    T, D, E = 37, 96, 9
    x = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    s = g.standard_normal((T, E)).astype(np.float32)
    counts, ei, ti, rop = orc.shuffle(s, K)
    ones = np.ones((T, E), np.float32)
    rows = orc.gather_scale(x, ti, ei, ones)
    out = np.zeros((T, D), np.uint16)
    orc.scatter_add(out, rows, ti, counts[E])
    want = _bits((_bf(x).float() * K).to(torch.bfloat16))
    assert np.array_equal(out, want)            # K * x, exact for K = 2^j


def test_scatter_add_brute_force_tiny(orc):
    g = np.random.default_rng(11)
    for trial in range(6):
        T, D, a = int(g.integers(1, 9)), int(g.integers(1, 20)), int(g.integers(0, 30))
        out0 = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
        inp = W.to_bf16_bits((g.standard_normal((a, D)) * 10).astype(np.float32))
        ti = g.integers(0, T, size=a).astype(np.int32)
        V = int(g.integers(0, a + 1))
        got = orc.scatter_add(out0.copy(), inp, ti, V)
        want = out0.copy()
        for t in range(T):
            rs = [r for r in range(V) if ti[r] == t]
            if not rs:
                continue
            for d in range(D):
                acc = np.float32(orc.bf16_to_f32(out0[t:t + 1, d])[0])
                for r in rs:
                    acc = np.float32(acc + orc.bf16_to_f32(inp[r:r + 1, d])[0])
                want[t, d] = W.to_bf16_bits(np.array([acc], np.float32))[0]
        assert np.array_equal(got, want)


def test_scatter_add_vs_index_add_fp64(orc):
    wl = W.WORKLOADS["zipf"]
    inp = W.dispatch_inputs(wl, T=300, D=128, E=32, K=8, vtc=250, out0="normal")
    counts, ei, ti, rop = orc.shuffle(inp.scores, 8, 250)
    V = int(counts[-1])
    got = orc.scatter_add(inp.out0.copy(), inp.y, ti, V)
    ref = _bf(inp.out0).double()
    ref.index_add_(0, torch.from_numpy(ti[:V].astype(np.int64)), _bf(inp.y[:V]).double())
    g = _bf(got).double()
    assert torch.allclose(g, ref, rtol=2.0 ** -8, atol=1e-6)
    assert np.array_equal(got[250:], inp.out0[250:])      # no rows: untouched


def test_scatter_add_untouched_rows_keep_bits(orc):
    T, D = 6, 16
    out0 = np.full((T, D), 0x7FC1, np.uint16)            # a NaN payload
    inp = np.zeros((3, D), np.uint16)
    ti = np.array([1, 1, 4], np.int32)
    got = orc.scatter_add(out0.copy(), inp, ti, 2)
    assert np.array_equal(got[[0, 2, 3, 4, 5]], out0[[0, 2, 3, 4, 5]])


# ---------------------------------------------------------------- finalize
def _fin(orc, fi, **kw):
    return orc.finalize_rmsnorm(fi.y, fi.w, fi.row_of_pair, fi.shared, fi.gamma,
                                fi.eps, **kw)


def test_finalize_k1_reduces_to_rms_norm(orc):
    g = np.random.default_rng(5)
    T, D = 7, 512
    y = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    gamma = W.to_bf16_bits(g.uniform(0.5, 1.5, D).astype(np.float32))
    rop = np.arange(T, dtype=np.int32).reshape(T, 1)
    w = np.ones((T, 1), np.float32)
    got = orc.finalize_rmsnorm(y, w, rop, None, gamma, 1e-6)
    ref = torch.nn.functional.rms_norm(_bf(y).float(), (D,), _bf(gamma).float(), 1e-6)
    diff = (_bf(got).float() - ref.to(torch.bfloat16).float()).abs()
    assert torch.all(diff <= 2.0 ** -7 * ref.abs() + 1e-6)


def test_finalize_all_slots_missing_is_rms_norm_of_shared(orc):
    fi = W.finalize_inputs(W.WORKLOADS["decode"], T=5, D=256, K=4)
    fi.row_of_pair[:] = -1
    got = _fin(orc, fi)
    ref = torch.nn.functional.rms_norm(_bf(fi.shared).float(), (256,),
                                       _bf(fi.gamma).float(), fi.eps)
    diff = (_bf(got).float() - ref).abs()
    assert torch.all(diff <= 2.0 ** -8 * ref.abs() * 1.01 + 1e-6)


def test_finalize_matches_fp64_evaluation(orc):
    fi = W.finalize_inputs(W.WORKLOADS["prefill"], T=33, D=320, K=4, hole_frac=0.2)
    got = _bf(_fin(orc, fi)).double()
    y = _bf(fi.y).double()
    w = torch.from_numpy(fi.w).double()
    rop = torch.from_numpy(fi.row_of_pair.astype(np.int64))
    h = _bf(fi.shared).double().clone()
    for k in range(4):
        r = rop[:, k]
        ok = (r >= 0).double()[:, None]
        h += ok * w[:, k:k + 1] * y[r.clamp(min=0)]
    ref = h * torch.rsqrt((h * h).mean(dim=1, keepdim=True) + fi.eps) * _bf(fi.gamma).double()
    # h is rounded to bf16 before the norm, the output once more
    assert torch.allclose(got, ref, rtol=2.0 ** -7, atol=1e-3)


def test_finalize_constant_row(orc):
    T, D = 3, 128
    c = np.array([0.75, -2.0, 3.0], np.float32)
    shared = W.to_bf16_bits(np.repeat(c[:, None], D, axis=1))
    gamma = W.to_bf16_bits(np.linspace(0.5, 1.5, D).astype(np.float32))
    rop = np.full((T, 2), -1, np.int32)
    w = np.zeros((T, 2), np.float32)
    eps = 1e-6
    got = orc.finalize_rmsnorm(np.zeros((1, D), np.uint16), w, rop, shared, gamma, eps)
    gf = orc.bf16_to_f32(gamma).astype(np.float64)
    want = gf[None, :] * (c[:, None] / np.sqrt(c[:, None] ** 2 + eps))
    assert np.allclose(orc.bf16_to_f32(got), want, rtol=2.0 ** -8, atol=0)


def test_finalize_power_of_two_scaling_invariance(orc):
    fi = W.finalize_inputs(W.WORKLOADS["decode"], T=6, D=384, K=8)
    base = orc.finalize_rmsnorm(fi.y, fi.w, fi.row_of_pair, fi.shared, fi.gamma, 0.0)
    for j in (-3, 2, 5):
        f = np.float32(2.0 ** j)
        y2 = W.to_bf16_bits(orc.bf16_to_f32(fi.y) * f)
        s2 = W.to_bf16_bits(orc.bf16_to_f32(fi.shared) * f)
        got = orc.finalize_rmsnorm(y2, fi.w, fi.row_of_pair, s2, fi.gamma, 0.0)
        assert np.array_equal(got, base)


def test_finalize_bf16_square_mode(orc):
    fi = W.finalize_inputs(W.WORKLOADS["decode"], T=4, D=512, K=2)
    got = _bf(_fin(orc, fi, flags=1)).float()
    # h from the default mode's pipeline is the same; recompute the norm with
    # torch's bf16 multiply for the squares
    w = torch.from_numpy(fi.w)
    y = _bf(fi.y).float()
    rop = torch.from_numpy(fi.row_of_pair.astype(np.int64))
    acc = torch.zeros(4, 512)
    for k in range(2):
        acc = torch.addcmul(acc, w[:, k:k + 1], y[rop[:, k]])
    h = (acc + _bf(fi.shared).float()).to(torch.bfloat16)
    sq = (h * h).float()
    inv = torch.rsqrt(sq.sum(1, keepdim=True) / 512 + fi.eps)
    ref = ((h.float() * inv) * _bf(fi.gamma).float()).to(torch.bfloat16).float()
    assert torch.allclose(got, ref, rtol=2.0 ** -7, atol=1e-6)


def _f32_nearest(q):
    """The binary32 value nearest the positive rational q, ties to even (q in
    the normal range)."""
    q = Fraction(q)
    assert q > 0
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    scaled = q / Fraction(2) ** (e - 23)          # in [2^23, 2^24)
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return np.float32(m * 2.0 ** (e - 23))        # m <= 2^24: exact


def _rmsnorm_exact(h_bits, gamma_bits, eps, bf16_squares=False):
    """RMSNorm of bf16 rows from exact arithmetic: squares in fp32 (exact for
    bf16 values; rounded to bf16 in the bf16-square mode), their exact
    rational sum rounded once to fp32, mean and mean + eps in fp32, inverse
    square root rounded once from a 60-digit decimal value, then
    bf16((h * inv) * gamma) in fp32 with torch's bf16 cast."""
    h = _bf(h_bits).float().numpy()
    g = _bf(gamma_bits).float().numpy()
    T, D = h.shape
    out = np.empty_like(h)
    for t in range(T):
        sq = (h[t] * h[t]).astype(np.float32)
        if bf16_squares:
            sq = _bf(W.to_bf16_bits(sq)).float().numpy()
        ss = _f32_nearest(sum(Fraction(float(v)) for v in sq))
        arg = np.float32(np.float32(ss / np.float32(D)) + np.float32(eps))
        with localcontext() as ctx:
            ctx.prec = 60
            inv = _f32_nearest(Fraction(Decimal(1) / Decimal(float(arg)).sqrt()))
        out[t] = (h[t] * inv).astype(np.float32) * g
    return W.to_bf16_bits(out.astype(np.float32))


def _rmsnorm_fp32_running_sum(h_bits, gamma_bits, eps):
    """The same with the squares added one by one in fp32 (the reading the
    exact-sum pin must tell apart)."""
    h = _bf(h_bits).float().numpy()
    g = _bf(gamma_bits).float().numpy()
    D = h.shape[1]
    ss = np.add.accumulate((h * h).astype(np.float32), axis=1, dtype=np.float32)[:, -1]
    arg = (ss / np.float32(D) + np.float32(eps)).astype(np.float32)
    inv = (1.0 / np.sqrt(arg.astype(np.float64))).astype(np.float32)
    return W.to_bf16_bits(((h * inv[:, None]).astype(np.float32) * g).astype(np.float32))


@pytest.mark.parametrize("flags", [0, 1])
def test_finalize_rmsnorm_exact_sum_of_squares(orc, flags):
    g = np.random.default_rng(11)
    T, D = 6, 4096
    y = g.standard_normal((T, D)).astype(np.float32)
    y[:3, 0] = 4096.0          # a large first square: a running fp32 sum drops the rest
    y[3, :] *= np.float32(1e-3)
    y = W.to_bf16_bits(y)
    gamma = W.to_bf16_bits(g.uniform(0.5, 1.5, D).astype(np.float32))
    rop = np.arange(T, dtype=np.int32).reshape(T, 1)
    w = np.ones((T, 1), np.float32)     # h = y exactly (fma(1, y, 0), one bf16 rounding)
    got = orc.finalize_rmsnorm(y, w, rop, None, gamma, 1e-6, flags=flags)
    want = _rmsnorm_exact(y, gamma, 1e-6, bf16_squares=bool(flags))
    assert np.array_equal(got, want)
    if not flags:
        # the crafted rows tell the two readings apart
        running = _rmsnorm_fp32_running_sum(y, gamma, 1e-6)
        assert not np.array_equal(running[:3], want[:3])


# ---------------------------------------------------------------- MXFP8
def _mx_check(orc, o_bits, codes, scales):
    T, D = o_bits.shape
    o = orc.bf16_to_f32(o_bits).reshape(T, D // 32, 32)
    amax = np.abs(o).max(axis=2)
    # scale byte: least n with 2^n >= amax * fp32(1/448) (fp32 product), +127
    p = (amax.astype(np.float32) * (np.float32(1) / np.float32(448))).astype(np.float64)
    b = scales.astype(np.int64)
    nz = p > 0
    assert np.all(np.exp2(b[nz] - 127.0) >= p[nz])
    lo = nz & (b > 0)                       # byte 0 may be a clamp
    assert np.all(np.exp2(b[lo] - 128.0) < p[lo])
    assert np.all(b[~nz] == 0)
    # codes: torch's E4M3 cast of the block scaled by 2^(127 - byte)
    mult = np.exp2(127.0 - b).astype(np.float32)[:, :, None]
    scaled = (o * mult).astype(np.float32)
    want = torch.from_numpy(scaled.reshape(T, D)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, want)
    dq = orc.e4m3_to_f32(codes).reshape(T, D // 32, 32)
    assert np.all(np.abs(dq) <= 448.0)
    return dq


def test_mxfp8_of_finalize_output(orc):
    fi = W.finalize_inputs(W.WORKLOADS["prefill"], T=20, D=640, K=4)
    out, codes, scales = _fin(orc, fi, mxfp8=True)
    assert np.array_equal(out, _fin(orc, fi))           # quantising adds no change
    dq = _mx_check(orc, out, codes, scales)
    # block max lands in [224, 448]
    assert np.all(np.abs(dq).max(axis=2)[scales > 0] >= 224.0)
    # re-quantising the dequantised block is the identity
    back = (dq * np.exp2(scales.astype(np.float64) - 127.0)[:, :, None]).astype(np.float32)
    out2 = W.to_bf16_bits(back.reshape(20, 640))
    assert np.array_equal(orc.f32_to_e4m3(
        (orc.bf16_to_f32(out2).reshape(20, 20, 32) *
         np.exp2(127.0 - scales.astype(np.float64))[:, :, None]).astype(np.float32)
    ).reshape(20, 640), codes)


def test_mxfp8_crafted_blocks(orc):
    """A row with h = 1 everywhere has rms 1, so with eps = 0 the finalize
    output is gamma itself; gamma then carries crafted 32-element blocks."""
    cases = [  # (block max, expected UE8M0 byte)
        (448.0, 127),                    # 448 * 2^0
        (896.0, 128),                    # 448 * 2^1
        (448.0 * (1 + 2.0 ** -7), 128),  # just above a power: rounds up
        (448.0 * (1 - 2.0 ** -7), 127),  # just below: same power
        (1.0, 119),                      # ceil(log2(1/448)) = -8
        (3.0, 120),                      # ceil(log2(3/448)) = -7
        (0.0, 0),                        # zero block
        (2.0 ** -130, 0),                # below 2^-127 * 448: clamped to 0
    ]
    D = 32 * len(cases)
    gam = np.zeros(D, np.float32)
    for j, (amax, _) in enumerate(cases):
        blk = np.zeros(32, np.float32)
        blk[::5] = amax
        blk[1::5] = -amax / 3
        blk[2] = -amax
        gam[32 * j:32 * j + 32] = blk
    gamma = W.to_bf16_bits(gam)
    shared = W.to_bf16_bits(np.ones((1, D), np.float32))
    out, codes, scales = orc.finalize_rmsnorm(
        np.zeros((1, D), np.uint16), np.zeros((1, 1), np.float32),
        np.full((1, 1), -1, np.int32), shared, gamma, 0.0, mxfp8=True)
    assert np.array_equal(out[0], gamma)
    assert scales[0].tolist() == [b for _, b in cases]
    _mx_check(orc, out, codes, scales)
    # exact powers land on the largest code
    assert codes[0, 0] == 0x7E and codes[0, 2] == 0xFE
    assert codes[0, 32] == 0x7E
    assert np.all(codes[0, 6 * 32:7 * 32] & 0x7F == 0)     # +-0 (sign kept)
