"""Pins for the oracle's finalize variants, CPU only.

bf16 routing weights: with weights that are bf16 values, the bf16-weight path
equals the (pinned) fp32-weight path fed the widened weights, and an fp64
evaluation agrees. The swizzled 128x4 MXFP8 scale layout (a reading: the
pages call an absent helper) is checked against an independent numpy
reshape/transpose of the same tiling, for bijectivity over the padded
buffer, zero padding rows, and hand-derived offsets."""
import numpy as np
import pytest
import torch

from combine_moe_shuffle_amd import workloads as W


def _fi(T=24, D=512, K=4, holes=0.1):
    return W.finalize_inputs(W.WORKLOADS["prefill"], T=T, D=D, K=K, hole_frac=holes)


def test_bf16_weights_equal_widened_fp32_weights(orc):
    fi = _fi()
    wb = W.to_bf16_bits(fi.w)
    wf = orc.bf16_to_f32(wb).reshape(fi.w.shape)
    a = orc.finalize_rmsnorm(fi.y, wb, fi.row_of_pair, fi.shared, fi.gamma, fi.eps, flags=2)
    b = orc.finalize_rmsnorm(fi.y, np.ascontiguousarray(wf), fi.row_of_pair, fi.shared,
                             fi.gamma, fi.eps, flags=0)
    assert np.array_equal(a, b)


def test_bf16_weights_fp64_evaluation(orc):
    fi = _fi(T=16, D=256, K=3)
    wb = W.to_bf16_bits(fi.w)
    got = orc.bf16_to_f32(orc.finalize_rmsnorm(fi.y, wb, fi.row_of_pair, fi.shared, fi.gamma,
                                               fi.eps, flags=2)).astype(np.float64)
    w = orc.bf16_to_f32(wb).reshape(fi.w.shape).astype(np.float64)
    y = orc.bf16_to_f32(fi.y).astype(np.float64)
    h = orc.bf16_to_f32(fi.shared).astype(np.float64)
    for k in range(3):
        r = fi.row_of_pair[:, k]
        h = h + np.where(r[:, None] >= 0, w[:, k:k + 1] * y[np.maximum(r, 0)], 0.0)
    ref = h / np.sqrt((h * h).mean(axis=1, keepdims=True) + fi.eps)
    ref = ref * orc.bf16_to_f32(fi.gamma).astype(np.float64)
    assert np.allclose(got, ref, rtol=2.0 ** -7, atol=1e-3)


def _swizzle_numpy(rowmajor):
    """The same 128x4 tiling written as a reshape/transpose: row m = 128*mt +
    32*g + i and column k = 4*kt + kk go to tile (mt, kt), then i, g, kk."""
    M, cols = rowmajor.shape
    Mp = -(-M // 128) * 128
    kp = -(-cols // 4) * 4
    pad = np.zeros((Mp, kp), np.uint8)
    pad[:M, :cols] = rowmajor
    t = pad.reshape(Mp // 128, 4, 32, kp // 4, 4)       # (mt, g, i, kt, kk)
    return t.transpose(0, 3, 2, 1, 4).reshape(-1)       # (mt, kt, i, g, kk)


@pytest.mark.parametrize("M,cols", [(1, 4), (127, 8), (128, 4), (200, 160), (300, 6)])
def test_swizzle_matches_reshape_formulation(orc, M, cols):
    g = np.random.default_rng(M + cols)
    rm = g.integers(1, 255, size=(M, cols)).astype(np.uint8)
    got = orc.mxfp8_swizzle(rm)
    assert got.size == orc.mxfp8_scale_bytes(M, 32 * cols, True)
    assert np.array_equal(got, _swizzle_numpy(rm))


def test_swizzle_is_a_bijection_with_zero_padding(orc):
    M, cols = 130, 8
    Mp, kp = 256, 8
    offs = [orc.mxfp8_swizzle_offset(m, k, cols) for m in range(Mp) for k in range(kp)]
    assert sorted(offs) == list(range(Mp * kp))
    rm = np.full((M, cols), 7, np.uint8)
    sw = orc.mxfp8_swizzle(rm)
    live = {orc.mxfp8_swizzle_offset(m, k, cols) for m in range(M) for k in range(cols)}
    dead = np.array([i not in live for i in range(sw.size)])
    assert np.all(sw[dead] == 0) and np.all(sw[~dead] == 7)


@pytest.mark.parametrize("M,cols", [(1, 4), (130, 8), (200, 160), (129, 12)])
def test_swizzle_padding_words_as_the_page_stores_them(orc, M, cols):
    """The "all_reduce_mhc" page (_LamportMHCDeviceKernel, the zeroing of the
    padding rows' scales) zeroes the padding with one 32-bit store per padding
    row and 4-column group, at the offset of (row, 4j). For those stores to
    clear exactly the padding, the layout must keep the 4 scales of a row and
    column group in 4 contiguous bytes from a 4-aligned offset, and those words
    must cover the padding entries and no live one. The page fixes this much of
    the tile order; the order of rows inside a tile stays a reading."""
    Mp = -(-M // 128) * 128
    words = set()
    for row in range(M, Mp):
        for j in range(cols // 4):
            base = orc.mxfp8_swizzle_offset(row, 4 * j, cols)
            assert base % 4 == 0
            for kk in range(4):
                assert orc.mxfp8_swizzle_offset(row, 4 * j + kk, cols) == base + kk
            words.update(range(base, base + 4))
    pad = {orc.mxfp8_swizzle_offset(m, k, cols) for m in range(M, Mp) for k in range(cols)}
    live = {orc.mxfp8_swizzle_offset(m, k, cols) for m in range(M) for k in range(cols)}
    assert words == pad and not (words & live)
    assert len(pad) + len(live) == orc.mxfp8_scale_bytes(M, 32 * cols, True)


def test_swizzle_hand_offsets(orc):
    # cols = 8: two 4-column tiles per 128-row band, 512 bytes each
    cases = {(0, 0): 0, (1, 0): 16, (32, 0): 4, (96, 3): 12 + 3, (0, 1): 1,
             (0, 4): 512, (128, 0): 1024, (33, 5): 512 + 16 + 4 + 1, (159, 7): 1536 + 31 * 16 + 0 * 4 + 3}  # 159 % 128 = 31: group 0
    for (m, k), want in cases.items():
        assert orc.mxfp8_swizzle_offset(m, k, 8) == want, (m, k)


def test_finalize_swizzled_scales_are_the_swizzled_rowmajor(orc):
    fi = _fi(T=150, D=256, K=4)
    out, codes, rm = orc.finalize_rmsnorm(fi.y, fi.w, fi.row_of_pair, fi.shared, fi.gamma,
                                          fi.eps, mxfp8=True)
    out2, codes2, sw = orc.finalize_rmsnorm(fi.y, fi.w, fi.row_of_pair, fi.shared, fi.gamma,
                                            fi.eps, flags=4, mxfp8=True)
    assert np.array_equal(out, out2) and np.array_equal(codes, codes2)
    assert np.array_equal(sw, _swizzle_numpy(rm))
