"""Pins for the oracle's padded (static-shape expert-parallel) combine, CPU
only: pure-Python brute force on tiny inputs, the EP = 1 case against the
dense scatter_add, rank selection with per-slab constants (closed form), and
torch.index_add_ in fp64."""
import numpy as np
import torch

from combine_moe_shuffle_amd import workloads as W


def _bf(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def _setup(orc, T, D, E, K, EP, seed, out0="normal"):
    wl = W.Workload(**{**W.WORKLOADS["zipf"].__dict__, "router": "softmax"})
    inp = W.dispatch_inputs(wl, T=T, D=D, E=E, K=K, vtc=None, seed=seed, out0=out0,
                            with_y=False)
    counts, ei, ti, rop = orc.shuffle(inp.scores, K)
    g = np.random.default_rng(seed + 100)
    slabs = W.to_bf16_bits(g.standard_normal((EP, T * K, D)).astype(np.float32))
    return inp, counts[:E].copy(), ei, ti, slabs


def test_padded_brute_force_tiny(orc):
    for seed in range(5):
        g = np.random.default_rng(seed)
        EP = int(g.choice([1, 2, 4]))
        E = EP * int(g.integers(1, 4))
        K = int(g.integers(1, E + 1))
        T, D = int(g.integers(1, 12)), 8 * int(g.integers(1, 3))
        inp, counts, ei, ti, slabs = _setup(orc, T, D, E, K, EP, seed)
        got = orc.scatter_add_padded(inp.out0.copy(), slabs, counts, ti)
        want = inp.out0.copy()
        off = np.concatenate([[0], np.cumsum(counts)])
        for t in range(T):
            rows = [r for r in range(int(off[-1])) if ti[r] == t]
            if not rows:
                continue
            for d in range(D):
                acc = np.float32(orc.bf16_to_f32(inp.out0[t:t + 1, d])[0])
                for r in rows:
                    e = int(np.searchsorted(off, r, side="right") - 1)
                    rank = e // (E // EP)
                    acc = np.float32(acc + orc.bf16_to_f32(slabs[rank, r:r + 1, d])[0])
                want[t, d] = W.to_bf16_bits(np.array([acc], np.float32))[0]
        assert np.array_equal(got, want), seed


def test_padded_ep1_is_dense_scatter_add(orc):
    inp, counts, ei, ti, slabs = _setup(orc, 70, 64, 12, 3, 1, 7)
    got = orc.scatter_add_padded(inp.out0.copy(), slabs, counts, ti)
    want = orc.scatter_add(inp.out0.copy(), np.ascontiguousarray(slabs[0]), ti, int(counts.sum()))
    assert np.array_equal(got, want)


def test_padded_selects_the_owning_rank(orc):
    """Slab r is filled with the constant r+1: each token's output is the
    exact sum of (rank+1) over its routes, with out0 = 0."""
    T, D, E, K, EP = 50, 16, 8, 3, 4
    inp, counts, ei, ti, _ = _setup(orc, T, D, E, K, EP, 3, out0="zeros")
    slabs = np.stack([W.to_bf16_bits(np.full((T * K, D), r + 1.0, np.float32))
                      for r in range(EP)])
    got = orc.bf16_to_f32(orc.scatter_add_padded(inp.out0.copy(), slabs, counts, ti))
    V = int(counts.sum())
    want = np.zeros(T)
    for r in range(V):
        want[ti[r]] += ei[r] // (E // EP) + 1
    assert np.array_equal(got, np.repeat(want[:, None], D, axis=1).astype(np.float32))


def test_padded_vs_index_add_fp64(orc):
    T, D, E, K, EP = 200, 96, 16, 4, 4
    inp, counts, ei, ti, slabs = _setup(orc, T, D, E, K, EP, 11)
    got = orc.scatter_add_padded(inp.out0.copy(), slabs, counts, ti)
    V = int(counts.sum())
    ref = _bf(inp.out0).double()
    src = torch.stack([_bf(slabs[ei[r] // (E // EP), r]).double() for r in range(V)])
    ref.index_add_(0, torch.from_numpy(ti[:V].astype(np.int64)), src)
    assert torch.allclose(_bf(got).double(), ref, rtol=2.0 ** -8, atol=1e-6)
