"""Pins for the oracle's dispatch stages: top-k, shuffle, gather_scale and the
FP8 rowwise gather (CPU only).

Top-k and shuffle are checked against pure-Python brute force on tiny inputs
(including crafted ties), against torch.topk on tie-free inputs, and by the
invariants of a stable counting sort at the full zipf size. gather_scale is
checked against torch's CPU bf16 arithmetic and closed forms; the FP8 rowwise
gather against its defining properties (the row max lands on 448, the
dequantisation error bound, saturation under a tiny scale_ub).
"""
import numpy as np
import pytest
import torch

from combine_moe_shuffle_amd import workloads as W


def _brute_topk(s, K):
    T, E = s.shape
    return [sorted(range(E), key=lambda e: (-float(s[t, e]), e))[:K] for t in range(T)]


def _brute_shuffle(s, K, vtc):
    T, E = s.shape
    sel = _brute_topk(s[:vtc], K) if vtc > 0 else []
    pairs = sorted([(e, t, k) for t in range(vtc) for k, e in enumerate(sel[t])])
    counts = [0] * (E + 1)
    for e, _, _ in pairs:
        counts[e] += 1
    counts[E] = len(pairs)
    ti, ei = [], []
    rop = [[-1] * K for _ in range(T)]
    for r, (e, t, k) in enumerate(pairs):
        ti.append(t)
        ei.append(e)
        rop[t][k] = r
    for t in range(vtc, T):
        for k in range(K):
            ti.append(t)
            ei.append(-1)
    return counts, ei, ti, rop


@pytest.mark.parametrize("seed", range(12))
def test_shuffle_brute_force_tiny(orc, seed):
    g = np.random.default_rng(seed)
    T = int(g.integers(1, 17))
    E = int(g.integers(1, 9))
    K = int(g.integers(1, E + 1))
    if seed % 3 == 0:   # heavy ties: few distinct values, signed zeros
        s = g.integers(-2, 3, size=(T, E)).astype(np.float32) * np.float32(0.5)
        s[g.random((T, E)) < 0.2] = -0.0
    else:
        s = g.standard_normal((T, E)).astype(np.float32)
    vtc = int(g.integers(0, T + 1)) if seed % 2 else T
    counts, ei, ti, rop = orc.shuffle(s, K, vtc)
    bc, bei, bti, brop = _brute_shuffle(s, K, vtc)
    assert counts.tolist() == bc
    assert ei.tolist() == bei
    assert ti.tolist() == bti
    assert rop.tolist() == brop


def test_topk_ties_go_to_lower_expert(orc):
    s = np.array([[1.0, 2.0, 2.0, 1.0, 2.0],
                  [0.0, -0.0, 0.0, -0.0, 0.0],
                  [-0.0, 0.0, 0.0, 0.0, 0.0]], np.float32)
    sel = orc.topk(s, 3)
    assert sel.tolist() == [[1, 2, 4], [0, 1, 2], [0, 1, 2]]


def test_topk_matches_torch_tie_free(orc):
    g = np.random.default_rng(7)
    s = g.standard_normal((500, 64)).astype(np.float32)
    for K in (1, 2, 5, 8):
        sel = orc.topk(s, K)
        v, i = torch.topk(torch.from_numpy(s), K, dim=1, largest=True, sorted=True)
        assert np.array_equal(sel, i.numpy().astype(np.int32))


def test_shuffle_strided_scores(orc):
    g = np.random.default_rng(8)
    base = g.standard_normal((16, 40)).astype(np.float32)
    view = base.T            # (40, 16) with strides (1, 40) elements
    cont = np.ascontiguousarray(view)
    a = orc.shuffle(view, 3, 31)
    b = orc.shuffle(cont, 3, 31)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def _check_shuffle_invariants(scores, K, vtc, counts, ei, ti, rop):
    T, E = scores.shape
    V = vtc * K
    assert counts[:E].sum() == counts[E] == V
    # token_indices is the multiset {t repeated K times}
    assert np.array_equal(np.sort(ti), np.repeat(np.arange(T), K))
    # expert-major, stable in token order
    assert np.all(np.diff(ei[:V]) >= 0)
    starts = np.concatenate([[0], np.cumsum(counts[:E])])
    for e in range(E):
        seg = ti[starts[e]:starts[e + 1]]
        assert np.all(ei[starts[e]:starts[e + 1]] == e)
        assert np.all(np.diff(seg) > 0)
    # tail: invalid tokens in (t, k) order, expert -1
    assert np.array_equal(ti[V:], np.repeat(np.arange(vtc, T), K))
    assert np.all(ei[V:] == -1)
    # row_of_pair is the inverse map
    r = rop[:vtc].reshape(-1)
    assert np.array_equal(np.sort(r), np.arange(V))
    tt = np.repeat(np.arange(vtc), K)
    assert np.array_equal(ti[r], tt)
    assert np.all(rop[vtc:] == -1)
    # selected experts are the top K of each valid token: every unselected
    # score is <= the smallest selected one, ties resolved to lower ids
    sel = ei[rop[:vtc]]
    s = scores[:vtc]
    chosen = np.take_along_axis(s, sel, axis=1)
    assert np.all(np.diff(chosen, axis=1) <= 0)
    mask = np.ones_like(s, dtype=bool)
    np.put_along_axis(mask, sel, False, axis=1)
    worst = chosen[:, -1:]
    assert np.all(np.where(mask, s, -np.inf) <= worst)
    for t in range(min(vtc, 4096)):
        assert len(set(sel[t].tolist())) == K


def test_shuffle_invariants_zipf_full_size(orc):
    wl = W.WORKLOADS["zipf"]
    s = W.router_scores(wl)
    counts, ei, ti, rop = orc.shuffle(s, wl.K, wl.vtc)
    _check_shuffle_invariants(s, wl.K, wl.vtc, counts, ei, ti, rop)
    # Zipf skew: the most popular expert is far above the mean
    assert counts[:wl.E].max() > 4 * counts[:wl.E].mean()


@pytest.mark.parametrize("name", ["tiny", "quant"])
def test_shuffle_invariants_other_workloads(orc, name):
    wl = W.WORKLOADS[name]
    s = W.router_scores(wl)
    counts, ei, ti, rop = orc.shuffle(s, wl.K, None)
    _check_shuffle_invariants(s, wl.K, wl.T, counts, ei, ti, rop)


def test_tiny_workload_masked_scores_select_the_kept_pair(orc):
    wl = W.WORKLOADS["tiny"]
    s = W.router_scores(wl)
    counts, ei, ti, rop = orc.shuffle(s, wl.K, None)
    sel = ei[rop]
    assert np.all(np.take_along_axis(s, sel, axis=1) > 0)
    assert np.all((s > 0).sum(axis=1) == wl.K)


# ---------------------------------------------------------------- gather
def _torch_gather(x_bits, ti, ei, scores, V):
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16)
    s = torch.from_numpy(scores)
    rows = []
    for i in range(V):
        rows.append((x[ti[i]].float() * s[ti[i], ei[i]]).to(torch.bfloat16))
    return torch.stack(rows).view(torch.int16).numpy().view(np.uint16)


def test_gather_scale_matches_torch(orc):
    wl = W.WORKLOADS["tiny"]
    inp = W.dispatch_inputs(wl, T=40, D=136, E=6, K=3, vtc=33)
    counts, ei, ti, rop = orc.shuffle(inp.scores, 3, 33)
    out = np.full((40 * 3, 136), 0xA5A5, np.uint16)
    orc.gather_scale(inp.x, ti, ei, inp.scores, counts[6], out)
    V = int(counts[6])
    assert np.array_equal(out[:V], _torch_gather(inp.x, ti, ei, inp.scores, V))
    assert np.all(out[V:] == 0xA5A5)


def test_gather_scale_closed_forms(orc):
    g = np.random.default_rng(4)
    T, D, E = 9, 64, 4
    x = W.to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    ti = np.repeat(np.arange(T, dtype=np.int32), 2)
    ei = np.tile(np.array([1, 3], np.int32), T)
    xf = orc.bf16_to_f32(x)
    ones = np.ones((T, E), np.float32)
    out = orc.gather_scale(x, ti, ei, ones)
    assert np.array_equal(out, x[ti])           # score 1 copies the row
    for j in (1, 3, 7):
        pw = np.full((T, E), 2.0 ** -j, np.float32)
        out = orc.gather_scale(x, ti, ei, pw)
        assert np.array_equal(orc.bf16_to_f32(out) * np.float32(2.0 ** j), xf[ti])


# ---------------------------------------------------------------- FP8 rowwise
def _quant_setup(orc, T=48, D=256, E=5, K=2, vtc=40, seed=0):
    wl = W.WORKLOADS["quant"]
    inp = W.dispatch_inputs(wl, T=T, D=D, E=E, K=K, vtc=vtc, seed=seed, with_y=False)
    counts, ei, ti, rop = orc.shuffle(inp.scores, K, vtc)
    return inp, counts, ei, ti


@pytest.mark.parametrize("ub", [None, 1200.0])
def test_quant_row_max_hits_448_and_error_bound(orc, ub):
    inp, counts, ei, ti = _quant_setup(orc)
    V = int(counts[-1])
    codes, scale = orc.gather_scale_quant(inp.x, ti, ei, inp.scores, ub, V)
    xf = orc.bf16_to_f32(inp.x)
    sc = inp.scores[ti[:V], ei[:V]]
    v = xf[ti[:V]] * sc[:, None]                      # fp32 products
    deq = orc.e4m3_to_f32(codes[:V]).astype(np.float64) * scale[:V, None]
    m = np.abs(v).max(axis=1)
    # the stored scale is m/448 up to two fp32 roundings
    assert np.allclose(scale[:V], m / 448.0, rtol=2.5e-7, atol=0)
    # each row's max element encodes to +-448
    arg = np.abs(v).argmax(axis=1)
    top = codes[np.arange(V), arg]
    assert np.all((top == 0x7E) | (top == 0xFE))
    # dequantisation error: half a step of E4M3 (relative 2^-4 in the normal
    # range, absolute 2^-10 * scale in the subnormal range), plus fp32 slack
    err = np.abs(deq - v)
    bound = np.maximum(2.0 ** -4 * np.abs(v), 2.0 ** -10 * scale[:V, None])
    assert np.all(err <= bound * (1 + 1e-5) + 1e-30)
    # rows >= V untouched
    assert np.all(codes[V:] == 0) and np.all(scale[V:] == 0)


def test_quant_tiny_scale_ub_saturates(orc):
    inp, counts, ei, ti = _quant_setup(orc, seed=1)
    V = int(counts[-1])
    codes, scale = orc.gather_scale_quant(inp.x, ti, ei, inp.scores, 1e-3, V)
    assert np.allclose(scale[:V], 1e-3 / 448.0, rtol=2.5e-7)
    xf = orc.bf16_to_f32(inp.x)
    v = xf[ti[:V]] * inp.scores[ti[:V], ei[:V]][:, None]
    big = np.abs(v) >= 1e-3
    assert np.all(np.where(big & (v > 0), codes[:V] == 0x7E, True))
    assert np.all(np.where(big & (v < 0), codes[:V] == 0xFE, True))


def test_quant_zero_row_gives_zero_codes(orc):
    T, D, E = 4, 64, 2
    x = np.zeros((T, D), np.uint16)
    ti = np.arange(T, dtype=np.int32)
    ei = np.zeros(T, np.int32)
    s = np.ones((T, E), np.float32)
    codes, scale = orc.gather_scale_quant(x, ti, ei, s)
    assert np.all(codes == 0)
    assert np.all(scale > 0) and np.all(scale < 1e-10)   # EPS-floored (value unpinned)
