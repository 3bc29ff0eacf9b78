"""Pins for the oracle's expert-parallel re-sort (combine_shuffling) and its
inverse (split_shuffling), CPU only: a sort-based brute force (label every
row with its (rank, column) by walking the layout, then a stable sort by
column then rank), the identity special case, the round trip, and counts."""
import numpy as np
import pytest


def _labels(counts, rank_stride, rows):
    """(rank, column, position-in-segment) of every input row that belongs
    to a segment, by walking the layout; None for padding rows."""
    EP, C = counts.shape
    lab = [None] * rows
    chunk = 0
    for r in range(EP):
        base = r * rank_stride if rank_stride is not None else chunk
        off = 0
        for c in range(C):
            for j in range(int(counts[r, c])):
                lab[base + off + j] = (r, c, j)
            off += int(counts[r, c])
        chunk = base + off
    return lab


def _case(seed, packed):
    g = np.random.default_rng(seed)
    EP = int(g.integers(1, 5))
    C = int(g.integers(1, 7))
    counts = g.integers(0, 4, size=(EP, C)).astype(np.int32)
    stride = None if packed else int(counts.sum(axis=1).max() + g.integers(0, 3))
    rows = int(counts.sum()) if packed else EP * stride
    rows = max(rows, 1)
    D = 8
    tok = g.integers(0, 2**16, size=(rows, D)).astype(np.uint16)
    c_lo = int(g.integers(0, C))
    c_hi = int(g.integers(c_lo, C + 1))
    return tok, counts, stride, c_lo, c_hi


@pytest.mark.parametrize("seed", range(10))
@pytest.mark.parametrize("packed", [True, False])
def test_combine_matches_sort_brute_force(orc, seed, packed):
    tok, counts, stride, c_lo, c_hi = _case(seed, packed)
    out, oc = orc.combine_shuffling(tok, counts, c_lo, c_hi, stride)
    lab = _labels(counts, stride, tok.shape[0])
    keep = [(c, r, j, i) for i, L in enumerate(lab) if L is not None
            for (r, c, j) in [L] if c_lo <= c < c_hi]
    order = [i for (_, _, _, i) in sorted(keep)]
    assert np.array_equal(out[:len(order)], tok[order])
    assert oc[:-1].tolist() == [int(counts[:, c].sum()) for c in range(c_lo, c_hi)]
    assert oc[-1] == len(order)


@pytest.mark.parametrize("seed", range(10))
@pytest.mark.parametrize("packed", [True, False])
def test_split_inverts_combine(orc, seed, packed):
    tok, counts, stride, c_lo, c_hi = _case(seed, packed)
    mid, oc = orc.combine_shuffling(tok, counts, c_lo, c_hi, stride)
    back = orc.split_shuffling(mid, counts, c_lo, c_hi, stride,
                               out=np.full_like(tok, 0xBEEF))
    lab = _labels(counts, stride, tok.shape[0])
    moved = np.array([L is not None and c_lo <= L[1] < c_hi for L in lab])
    assert np.array_equal(back[moved], tok[moved])
    assert np.all(back[~moved] == 0xBEEF)


def test_single_rank_full_range_is_identity(orc):
    g = np.random.default_rng(3)
    counts = g.integers(0, 9, size=(1, 12)).astype(np.int32)
    n = int(counts.sum())
    tok = g.integers(0, 2**16, size=(n, 16)).astype(np.uint16)
    out, oc = orc.combine_shuffling(tok, counts)
    assert np.array_equal(out, tok)
    assert oc.tolist() == counts[0].tolist() + [n]
