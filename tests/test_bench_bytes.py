"""The algorithmic bytes bench.py divides by a kernel's time (the roofline's
numerator), checked against budgets derived here term by term from each
workload's shapes. No GPU needed."""
import bench

MB = 1e6


def _close(got, want_mb, rel=1e-3):
    assert abs(got / MB - want_mb) <= rel * want_mb, (got / MB, want_mb)


def test_zipf_dispatch_bytes():
    # T=8192, D=7168, E=256, K=8, 6000 routed tokens -> 48000 routed rows
    b = bench.dispatch_bytes(8192, 7168, 256, 8, 6000, quant=False)
    # scores 8192*256*4 = 8.39 MB; three index outputs 3*65536*4 = 0.79 MB
    _close(b["shuffle"], 8.389 + 0.786)
    # x once per routed token 6000*14336 = 86.0 MB; rows out 48000*14336 = 688.1 MB;
    # row_of_pair, expert ids and scores of the routed rows 0.65 MB
    _close(b["gather"], 86.016 + 688.128 + 0.646)
    # rows in 688.1 MB; the 6000 token rows read and written 2*86.0 MB; row_of_pair
    _close(b["scatter"], 688.128 + 2 * 86.016 + 0.262)
    _close(sum(b.values()), 1644.4)


def test_zipf_general_dispatch_bytes():
    # the entry points that take token_indices read the 48000 valid rows' token
    # indices (0.19 MB) where the by-token ones read row_of_pair (8192*8 words)
    b = bench.dispatch_bytes(8192, 7168, 256, 8, 6000, quant=False, general=True)
    byt = bench.dispatch_bytes(8192, 7168, 256, 8, 6000, quant=False)
    assert b["shuffle"] == byt["shuffle"]
    assert b["gather"] == byt["gather"] - 8192 * 8 * 4 + 48000 * 4
    assert b["scatter"] == byt["scatter"] - 8192 * 8 * 4 + 48000 * 4
    _close(b["scatter"], 688.128 + 2 * 86.016 + 0.192)


def test_tiny_dispatch_bytes():
    # T=64, D=1024, E=8, K=2, every token valid: 128 rows of 2048 bytes
    b = bench.dispatch_bytes(64, 1024, 8, 2, 64, quant=False)
    assert b["shuffle"] == 64 * 8 * 4 + 3 * 128 * 4 + 9 * 4
    assert b["gather"] == 64 * 2048 + 128 * 2048 + 128 * 4 + 2 * 128 * 4
    assert b["scatter"] == 128 * 2048 + 2 * 64 * 2048 + 128 * 4
    _close(sum(b.values()), 0.9232)


def test_quant_dispatch_bytes():
    # T=4096, D=5120, E=16, K=1: one row per token, FP8 codes 1 byte per element
    b = bench.dispatch_bytes(4096, 5120, 16, 1, 4096, quant=True)
    _close(b["shuffle"], 0.3114)   # scores 0.262 + indices 0.049
    _close(b["gather"], 41.943 + 20.972 + 0.066)   # x rows, codes, scale + indices + score
    _close(b["scatter"], 3 * 41.943 + 0.016)


def test_finalize_bytes():
    # decode, K=8 rows of 14336 bytes, shared and out rows, gamma, slots and weights
    for T, want in ((1, 0.1578), (8, 1.162), (32, 4.604), (128, 18.37)):
        _close(bench.finalize_bytes(T, 7168, 8), want)
    # prefill, T=16384, D=5120, K=4, MXFP8 with row-major scales (T * D/32 bytes)
    T, D, K = 16384, 5120, 4
    want = (671.089 + 2 * 167.772 + 0.010 + 0.524   # rows, shared + out, gamma, slots
            + 83.886 + 2.621)                        # codes, scales
    _close(bench.finalize_bytes(T, D, K, scale_bytes=T * D // 32), want)
    # bf16 weights: 2 bytes per weight instead of 4
    assert (bench.finalize_bytes(T, D, K, bf16_weights=True)
            == bench.finalize_bytes(T, D, K) - 2 * T * K)


def test_mhc_padded_shuffling_bytes():
    T, D, K, hc = 16384, 5120, 4, 4
    sb = 123456
    plain = bench.finalize_bytes(T, D, K, scale_bytes=sb)
    # the hc streams in and out, post and pre (hc each) and comb (hc*hc), fp32
    assert bench.mhc_bytes(T, D, K, hc, sb) == plain + 2 * T * hc * D * 2 + T * hc * 8 + \
        T * hc * hc * 4
    # the padded combine reads the same rows as the dense one, plus the expert counts
    # and the rows' token indices instead of row_of_pair
    dense = bench.dispatch_bytes(8192, 7168, 256, 8, 6000, False)["scatter"]
    assert bench.padded_bytes(7168, 256, 8, 6000) == dense - 8192 * 8 * 4 + 48000 * 4 + 256 * 4
    # the by-token form reads the inverse map (T*K words) as the dense by-token combine does
    assert bench.padded_bytes(7168, 256, 8, 6000, T=8192) == dense + 256 * 4
    # a re-sort moves every row once each way
    assert bench.shuffling_bytes(1000, 256, 8, 32) == 2 * 1000 * 512 + 8 * 32 * 4 + 33 * 4


def test_stream_mix():
    """The contiguous-stream probe's R:W and wave count carry the roofline
    kernel's row bytes: the zipf scatter reads 9 rows' KiB for each KiB it
    writes, the zipf gather writes 8 for each it reads, the MXFP8 prefill
    finalize reads 5 bf16 rows per token and writes 1.5 (bf16 row and codes)."""
    tok_kib = 6000 * 7168 * 2 // 1024
    assert bench.stream_mix(9 * tok_kib, tok_kib) == (9, 1, 84000)
    assert bench.stream_mix(tok_kib, 8 * tok_kib) == (1, 8, 84000)
    row_kib = 16384 * 5120 * 2 // 1024
    assert bench.stream_mix(5 * row_kib, 1.5 * row_kib) == (10, 3, 81920)
    # mhc: K + 1 + hc = 9 rows in, hc + 1.5 = 5.5 out
    assert bench.stream_mix(9 * row_kib, 5.5 * row_kib) == (18, 11, 81920)
    for R, Wm, u in ((9, 1, 84000), (10, 3, 81920), (18, 11, 81920)):
        assert 1 <= R <= 32 and 1 <= Wm <= 32 and u > 0
    # not whole KiB, or no ratio within 32:32
    assert bench.stream_mix(1.5, 1) is None
    assert bench.stream_mix(33, 1) is None
    assert bench.stream_mix(0, 4) is None


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU: --gpus above 1 exits with status 2 and a
    message, before touching any device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
