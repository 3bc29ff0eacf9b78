"""The shuffle entry point that allocates nothing (moe_shuffle_noalloc),
through the C ABI, against moe_shuffle (the same kernels with a caller's
workspace) and the oracle, bit for bit.

Two calls in a row share the library's static scratch: the routing workload
at full size (T=8192, E=256, K=8, 6000 valid tokens), then a smaller one
(fewer tokens, experts and slots), whose outputs must not depend on what the
first call left there. Outputs are preallocated, so no call in the sequence
allocates device memory.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from combine_moe_shuffle_amd import _lib, ops
from combine_moe_shuffle_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-case]", *a, flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    _lib.load()
    return torch.device("cuda:0")


def _outputs(T, E, K, dev, fill):
    return (torch.full((E + 1,), fill, dtype=torch.int32, device=dev),
            torch.full((T * K,), fill, dtype=torch.int32, device=dev),
            torch.full((T * K,), fill, dtype=torch.int32, device=dev),
            torch.full((T, K), fill, dtype=torch.int32, device=dev))


def _case(wl, T, E, K, vtc, transposed=False):
    scores = W.router_scores(W.Workload(**{**wl.__dict__, "K": K}), T, E)
    return scores, vtc, transposed


def test_noalloc_shuffle_matches_workspace_shuffle(dev):
    zipf = W.WORKLOADS["zipf"]
    cases = [
        ("zipf-full", _case(zipf, zipf.T, zipf.E, zipf.K, zipf.vtc)),
        ("smaller-transposed", _case(W.WORKLOADS["quant"], 700, 48, 4, 650, transposed=True)),
    ]
    for name, (scores, vtc, transposed) in cases:
        T, E = scores.shape
        K = {"zipf-full": zipf.K}.get(name, 4)
        say("noalloc shuffle", name, T, E, K, vtc)
        if transposed:
            s = torch.from_numpy(np.ascontiguousarray(scores.T)).to(dev).t()
        else:
            s = torch.from_numpy(scores).to(dev)
        v = torch.tensor([vtc], dtype=torch.int32, device=dev)
        got = _outputs(T, E, K, dev, -7)
        ops.moe_shuffle_noalloc(s, K, v, out=got)
        want = ops.moe_shuffle(s, K, v, out=_outputs(T, E, K, dev, -9))
        torch.cuda.synchronize()
        for g, w_, what in zip(got, want, ("counts", "expert_indices", "token_indices",
                                            "row_of_pair")):
            assert torch.equal(g, w_), (name, what)
        counts, ei, ti, rop = orc.shuffle(scores, K, vtc)
        assert np.array_equal(got[0].cpu().numpy(), counts), name
        assert np.array_equal(got[1].cpu().numpy(), ei), name
        assert np.array_equal(got[2].cpu().numpy(), ti), name
        assert np.array_equal(got[3].cpu().numpy().reshape(-1), rop.reshape(-1)), name


def test_noalloc_shuffle_on_a_side_stream(dev):
    """On a stream of its own (the scratch address is checked against the
    stream's device), then on the default stream with fewer tokens: both equal
    moe_shuffle."""
    wl = W.WORKLOADS["zipf"]
    for T, stream in ((3000, torch.cuda.Stream()), (100, None)):
        scores = torch.from_numpy(W.router_scores(wl, T=T)).to(dev)
        say("noalloc shuffle, stream", T, stream is not None)
        got = _outputs(T, wl.E, wl.K, dev, -5)
        if stream is not None:
            stream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(stream):
                ops.moe_shuffle_noalloc(scores, wl.K, out=got)
            torch.cuda.current_stream().wait_stream(stream)
        else:
            ops.moe_shuffle_noalloc(scores, wl.K, out=got)
        want = ops.moe_shuffle(scores, wl.K)
        torch.cuda.synchronize()
        for g, w_ in zip(got, want):
            assert torch.equal(g.view(-1), w_.view(-1))


def test_noalloc_shuffle_rejects_beyond_scratch(dev):
    # T = 2^20 tokens at E = 256, K = 8 needs 32 MiB + 32 MiB of workspace
    T, E, K = 1 << 20, 256, 8
    need = _lib.load().moe_shuffle_workspace_bytes(T, E, K)
    assert need > 8 << 20
    s = torch.empty((T, E), dtype=torch.float32, device=dev)
    with pytest.raises(_lib.MoeError) as ei:
        ops.moe_shuffle_noalloc(s, K)
    assert ei.value.status == 3 and "scratch" in str(ei.value)
