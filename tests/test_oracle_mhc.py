"""Pins for the oracle's mHC finalize (post-mix of the hc residual streams,
pre-mix collapse, RMSNorm, MXFP8), CPU only:

* hc streams with post = e_0, comb = 0, pre = e_0 reduce it to the plain
  finalize (stream 0 carries h, the collapse is h);
* small dyadic inputs for which every fp32 step is exact: the residual
  output is checked bit for bit against exact rational arithmetic, the
  prenorm against torch's bf16 rounding of the exact collapse;
* a permutation comb moves stream s to stream pi(s) unchanged (catches a
  transposed [source, target] index);
* residual-only mode writes the same streams;
* realistic inputs against an fp64 evaluation.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from combine_moe_shuffle_amd import workloads as W

WL = W.WORKLOADS["mhc"]


def _f(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).double().numpy()


def _bf(x):
    return W.to_bf16_bits(np.asarray(x, dtype=np.float32))


def _fin(T, D, K, seed, holes=0.0):
    return W.finalize_inputs(WL, T=T, D=D, K=K, seed=seed, hole_frac=holes)


@pytest.mark.parametrize("hc", [1, 3])
def test_mhc_identity_mix_is_plain_finalize(orc, hc):
    T, D, K = 37, 256, 4
    f = _fin(T, D, K, 1, holes=0.2)
    m = W.mhc_inputs(WL, T=T, D=D, hc=hc, seed=1)
    post = np.zeros((T, hc), np.float32)
    post[:, 0] = 1.0
    pre = post.copy()
    comb = np.zeros((T, hc, hc), np.float32)
    res, out, codes, scales = orc.finalize_mhc(f.y, f.w, f.row_of_pair, f.shared, m.residual,
                                               post, comb, pre, f.gamma, f.eps, mxfp8=True)
    want, wc, ws = orc.finalize_rmsnorm(f.y, f.w, f.row_of_pair, f.shared, f.gamma, f.eps,
                                        mxfp8=True)
    assert np.array_equal(out, want)
    assert np.array_equal(codes, wc) and np.array_equal(scales, ws)
    # streams past 0 are h * 0 + r * 0: a zero of either sign
    assert np.all(_f(res[:, 1:, :]) == 0)
    # stream 0 is h: within one bf16 rounding of the fp64 sum
    h = np.zeros((T, D))
    for t in range(T):
        for k in range(K):
            r = f.row_of_pair[t, k]
            if r >= 0:
                h[t] += float(f.w[t, k]) * _f(f.y[r])
    h += _f(f.shared)
    got = _f(res[:, 0, :])
    assert np.all(np.abs(got - h) <= 2.0 ** -8 * np.abs(h) + 1e-5)


def test_mhc_exact_dyadic(orc):
    """Integers and halves: every fp32 product and sum is exact, so the
    residual output equals the exact value, which is representable in bf16."""
    T, D, K, hc = 9, 64, 2, 4
    g = np.random.default_rng(5)
    y = _bf(g.integers(-4, 5, size=(T * K, D)))
    rop = g.permutation(T * K).astype(np.int32).reshape(T, K)
    w = np.full((T, K), 0.5, np.float32)
    shared = _bf(g.integers(-4, 5, size=(T, D)))
    residual = _bf(g.integers(-4, 5, size=(T, hc, D)))
    post = g.choice([0.5, 1.0], size=(T, hc)).astype(np.float32)
    pre = g.choice([0.5, 1.0], size=(T, hc)).astype(np.float32)
    comb = g.choice([0.0, 0.5, 1.0], size=(T, hc, hc)).astype(np.float32)
    gamma = _bf(np.ones(D))
    res, out, _, _ = orc.finalize_mhc(y, w, rop, shared, residual, post, comb, pre, gamma, 0.0)
    q = lambda v: Fraction(float(v))  # noqa: E731
    yf, sf, rf = _f(y), _f(shared), _f(residual)
    prenorm = np.zeros((T, D))
    for t in range(T):
        for d in range(D):
            h = sum(q(w[t, k]) * q(yf[rop[t, k], d]) for k in range(K)) + q(sf[t, d])
            col = Fraction(0)
            for j in range(hc):
                mixed = h * q(post[t, j]) + sum(q(rf[t, s, d]) * q(comb[t, s, j])
                                                for s in range(hc))
                assert _f(res[t, j, d:d + 1])[0] == float(mixed), (t, j, d)
                col += mixed * q(pre[t, j])
            prenorm[t, d] = float(col)  # exact: at most 10 significant bits
    pn = _f(_bf(prenorm))  # torch's round-to-nearest-even of the exact collapse
    # gamma = 1, eps = 0: out = bf16(pn / rms(pn)); rms in fp64
    rms = np.sqrt((pn ** 2).mean(axis=1, keepdims=True))
    want = pn / rms
    assert np.all(np.abs(_f(out) - want) <= 2.0 ** -8 * np.abs(want) + 1e-6)


def test_mhc_permutation_moves_streams(orc):
    T, D, K, hc = 11, 128, 3, 4
    f = _fin(T, D, K, 2)
    m = W.mhc_inputs(WL, T=T, D=D, hc=hc, seed=2)
    pi = [1, 2, 3, 0]  # stream s goes to target pi[s]; not an involution
    comb = np.zeros((T, hc, hc), np.float32)
    for s in range(hc):
        comb[:, s, pi[s]] = 1.0
    post = np.zeros((T, hc), np.float32)
    res, _, _, _ = orc.finalize_mhc(f.y, f.w, f.row_of_pair, f.shared, m.residual, post, comb,
                                    None, None, f.eps)
    for s in range(hc):
        assert np.array_equal(res[:, pi[s], :], m.residual[:, s, :])


def test_mhc_residual_only_matches_full(orc):
    T, D, K, hc = 20, 256, 8, 4
    f = _fin(T, D, K, 3, holes=0.1)
    m = W.mhc_inputs(WL, T=T, D=D, hc=hc, seed=3)
    full = orc.finalize_mhc(f.y, f.w, f.row_of_pair, f.shared, m.residual, m.post, m.comb, m.pre,
                            f.gamma, f.eps)
    ro = orc.finalize_mhc(f.y, f.w, f.row_of_pair, f.shared, m.residual, m.post, m.comb, None,
                          None, f.eps)
    assert np.array_equal(full[0], ro[0]) and ro[1] is None


def test_mhc_vs_fp64(orc):
    T, D, K, hc = 24, 512, 4, 4
    f = _fin(T, D, K, 4, holes=0.1)
    m = W.mhc_inputs(WL, T=T, D=D, hc=hc, seed=4)
    res, out, codes, scales = orc.finalize_mhc(f.y, f.w, f.row_of_pair, f.shared, m.residual,
                                               m.post, m.comb, m.pre, f.gamma, f.eps)
    h = _f(f.shared).copy()
    for t in range(T):
        for k in range(K):
            r = f.row_of_pair[t, k]
            if r >= 0:
                h[t] += float(f.w[t, k]) * _f(f.y[r])
    rf = _f(m.residual)
    mixed = h[:, None, :] * m.post[:, :, None].astype(np.float64) + np.einsum(
        "tsd,tsj->tjd", rf, m.comb.astype(np.float64))
    got = _f(res)
    # h is bf16-rounded before the mix: allow that rounding times post, plus
    # the output rounding
    slack = 2.0 ** -8 * np.abs(h)[:, None, :] * m.post[:, :, None]
    assert np.all(np.abs(got - mixed) <= 2.0 ** -8 * np.abs(mixed) + slack + 1e-5)
    col = (got * m.pre[:, :, None]).sum(axis=1)
    g = _f(f.gamma)
    want = col / np.sqrt((col ** 2).mean(axis=1, keepdims=True) + f.eps) * g
    assert np.all(np.abs(_f(out) - want) <= 2e-2 + 1e-2 * np.abs(want))


def test_mhc_swizzled_scales_and_padding(orc):
    T, D, K, hc = 130, 256, 2, 2
    f = _fin(T, D, K, 6)
    m = W.mhc_inputs(WL, T=T, D=D, hc=hc, seed=6)
    res, out, codes, scales = orc.finalize_mhc(f.y, f.w, f.row_of_pair, f.shared, m.residual,
                                               m.post, m.comb, m.pre, f.gamma, f.eps, flags=4,
                                               mxfp8=True)
    oc, rm = orc.mxfp8_quantize(out)
    assert np.array_equal(codes, oc)
    assert scales.size == 256 * (D // 32)
    assert np.array_equal(scales, orc.mxfp8_swizzle(rm))
    # the padding rows' scales are zero
    for mrow in range(T, 256):
        for kcol in range(D // 32):
            assert scales[orc.mxfp8_swizzle_offset(mrow, kcol, D // 32)] == 0


def test_mhc_rejects_bad_arguments(orc):
    T, D, K, hc = 4, 64, 2, 2
    f = _fin(T, D, K, 7)
    m = W.mhc_inputs(WL, T=T, D=D, hc=hc, seed=7)
    with pytest.raises(ValueError):  # swizzled scales without MXFP8
        orc.finalize_mhc(f.y, f.w, f.row_of_pair, f.shared, m.residual, m.post, m.comb, m.pre,
                         f.gamma, f.eps, flags=4)
    with pytest.raises(ValueError):  # MXFP8 in residual-only mode
        orc.finalize_mhc(f.y, f.w, f.row_of_pair, f.shared, m.residual, m.post, m.comb, None,
                         None, f.eps, mxfp8=True)
