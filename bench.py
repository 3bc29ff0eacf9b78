"""Benchmark of the MoE dispatch/combine hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload zipf]

A step is one pass of the path over one batch of synthetic input, already
resident in HBM:
  zipf      (default; T=8192, D=7168, E=256, K=8, valid_token_count=6000)
            moe_shuffle -> moe_gather_scale_by_token -> moe_scatter_add_by_token
  zipf-general  the same step through the entry points that take
            token_indices (the pages' gather/scatter arguments): moe_shuffle ->
            moe_gather_scale (with a workspace) -> moe_scatter_add
  quant     (T=4096, D=5120, E=16, K=1)
            moe_shuffle -> moe_gather_scale_quant -> moe_scatter_add_by_token
  tiny      (T=64, D=1024, E=8, K=2) the zipf step's calls, launch-bound; the
            line's "sweep" times the zipf step's calls, by token and through
            token_indices, at decode batch sizes, T = 1, 8, 32, 64 and 128 at
            D=7168, E=256, K=8
  prefill   (T=16384, D=5120, K=4) moe_finalize_rmsnorm with MXFP8
  decode    (T=128, D=7168, K=8)   moe_finalize_rmsnorm; the line's "sweep"
            also times T = 1, 8, 32 and 128 (per call and per kernel)
  prefill-swizzled  prefill with bf16 routing weights and 128x4-tiled scales
  mhc       (T=16384, D=5120, K=4, hc=4) moe_finalize_mhc with MXFP8
            (128x4-tiled scales)
  padded    the zipf routing combined from a static (EP=8, T*K, D) buffer:
            moe_scatter_add_padded_by_token (the shuffle's inverse map)
  padded-general  the same through token_indices (the pages' arguments):
            moe_scatter_add_padded
  shuffling rows from EP=8 source ranks for one rank's 32 local experts:
            moe_combine_shuffling -> moe_split_shuffling
A step launches its kernels from Python through calls prepared once
(ops.prepare: the op's checks run at set-up, each step repeats its library
calls; --checked runs the checked op every step). --graph replays a HIP graph
of the step instead; a graph launch costs more than a few kernel launches here.

1. W untimed steps, then exactly K timed steps between two device
   synchronisations (wall clock, and a HIP event pair around the region): the
   warm steps, reported under "warm" (the previous step's data still in L2
   and the 256 MB Infinity Cache). Then K steps one at a time, each between
   an event pair with the host waiting for it: p10 / p50 / p90 of an isolated
   step's latency, launch included ("step_us_isolated").
2. K cold steps, each after a flush of L2 and the Infinity Cache -- a 1 GiB
   read (clean eviction) or a 1 GiB write (whose dirty lines the step then
   writes back) -- in 5 blocks of K/5, each block between two device
   synchronisations and followed by a block of the flushes alone timed the
   same way: the median over the blocks of the per-step difference; each
   stage alone after a read flush too. The steps after a read flush are the
   headline: `value`, `ms_per_step` and `hbm_frac` (--no-cold skips the cold
   steps, for profiling runs; the headline is then the warm steps).
3. Each stage alone: K launches captured back to back in one HIP graph,
   replayed once between one HIP event pair on the stream the kernels run on:
   each stage's average duration per launch, the kernels' own time.

An event between two kernels costs the stream ~10 us, so no region records
one inside. The longest stage is the roofline kernel: its algorithmic bytes
per launch (unique inputs read once, outputs written once, valid rows only)
over that duration, against the 8 TB/s HBM peak.
4. "stream_ceiling": for each streaming stage (the roofline kernel among
   them), its row bytes in the same read:write mix moved by a plain contiguous
   stream (moe_stream_probe: R KiB read and W KiB written per wave, blocked
   per wave or interleaved over R + W streams, consecutive waves on
   consecutive memory either way), timed as in 3 and after a read flush as in
   2; the faster layout is the reference: the rate a plain stream of the
   same bytes reaches on this GPU, and the stage's rate as a fraction of it
   (--no-ceiling skips it). It is a reference, not a bound: an order that
   spreads writes over many rows can beat it.

One JSON line on stdout. value = valid tokens (routed rows for padded and
shuffling) per second of the whole step. cpu_baseline = the CPU oracle
(single-threaded C) timed on a bounded sample of the same step, pinned to one
core; "host" names the CPU model and core counts, "stage_s" the dispatch
workloads' per-stage times.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
COLD_BLOCKS = 5  # blocks of steps after a flush, alternated with the flush alone
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
WORKLOAD_CHOICES = ["zipf", "zipf-general", "quant", "tiny", "prefill", "decode",
                    "prefill-swizzled", "mhc", "padded", "padded-general", "shuffling"]
DISPATCH_METRIC = "dispatch+combine tokens/s and achieved HBM GB/s (% of peak), 1xMI355X"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed steps (default 50; 1000 for decode and tiny, whose steps "
                        "take a few us)")
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed steps first (default 5; 50 for decode and tiny)")
    p.add_argument("--workload", default="zipf", choices=WORKLOAD_CHOICES)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-cold", action="store_true",
                   help="skip the cold-cache steps (profiling runs: every launch then warm)")
    p.add_argument("--checked", action="store_true",
                   help="launch every stage through the checked op call (dtype, shape and "
                        "device checks each call) instead of a call prepared once")
    p.add_argument("--no-sweep", action="store_true",
                   help="skip the decode and tiny lines' token-count sweeps (profiling runs: every "
                        "launch at the workload's size)")
    p.add_argument("--graph", action="store_true",
                   help="replay a HIP graph of the step instead of launching its kernels from "
                        "Python (a graph launch costs more than a few kernel launches here)")
    p.add_argument("--no-ceiling", action="store_true",
                   help="skip the contiguous-stream probe timed beside the roofline kernel")
    p.add_argument("--copy-bytes", type=int, default=0,
                   help="after the timed region, run one plain device copy of this many "
                        "bytes (the calibration kernel of the HBM counter runs)")
    return p.parse_args()


# headers every kernel source includes: part of each kernel's identity
KERNEL_HEADERS = ["device.hpp", "launch.hpp"]


def source_hash(names):
    """Hash of the kernel sources `names` and the headers they include."""
    h = hashlib.sha256()
    for n in list(names) + KERNEL_HEADERS:
        with open(os.path.join(ROOT, "combine_moe_shuffle_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def capture(torch, fn):
    """A HIP graph of fn(): one eager pass on a side stream, then the
    capture (torch's capture stream is the current stream inside it, and the
    bindings launch on the current stream)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def stage_ms(torch, fn, reps):
    """Average duration of one launch of a stage: `reps` launches captured back
    to back in one HIP graph, replayed once between a pair of HIP events on
    the stream the kernels run on. Without Python between launches and
    without an event between kernels this is the kernels' own time (what the
    rocprofv3 kernel trace shows), not the launch overhead."""
    def many():
        for _ in range(reps):
            fn()
    g = capture(torch, many)
    g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


# ------------------------------------------------------------------ algorithmic bytes
# Per launch: unique inputs read once, outputs written once, valid rows only
# (rows past the valid count are neither read nor written). bf16 rows are 2*D
# bytes; indices, counts, scores and fp32 weights 4 bytes.
def dispatch_bytes(T, D, E, K, vtc, quant, general=False):
    """shuffle: scores + token/expert indices and row_of_pair + counts;
    gather: x once per routed token (bf16) or per row (FP8 rowwise, codes and
    scales out) + the routed rows + the indices and scores it reads;
    scatter: the routed rows + each routed token's row read and written +
    row_of_pair. The general entry points read the valid rows' token indices
    instead of row_of_pair (V instead of T*K index words)."""
    a, V, row_b = T * K, vtc * K, D * 2
    shuffle = T * E * 4 + 3 * a * 4 + (E + 1) * 4
    idx = V * 4 if general else T * K * 4
    if quant:
        gather = V * row_b + V * D + V * 4 + 2 * V * 4 + V * 4
    else:
        gather = vtc * row_b + V * row_b + idx + V * 4 + V * 4
    scatter = V * row_b + 2 * vtc * row_b + idx
    return {"shuffle": shuffle, "gather": gather, "scatter": scatter}


def finalize_bytes(T, D, K, scale_bytes=None, bf16_weights=False):
    """K expert rows, shared row and output per token, gamma once, the slot
    rows and weights; with MXFP8 (scale_bytes given) the codes and scales."""
    row_b = D * 2
    b = T * K * row_b + 2 * T * row_b + row_b + T * K * (6 if bf16_weights else 8)
    if scale_bytes is not None:
        b += T * D + scale_bytes
    return b


def mhc_bytes(T, D, K, hc, scale_bytes):
    """The finalize's bytes plus the hc residual streams read and written and
    the per-token mixing coefficients (post, pre: hc each; comb: hc*hc)."""
    row_b = D * 2
    return (T * K * row_b + T * row_b + 2 * T * hc * row_b + T * row_b + row_b + T * K * 8 +
            T * hc * 8 + T * hc * hc * 4 + T * D + scale_bytes)


def padded_bytes(D, E, K, vtc, T=None):
    """The routed rows from the slabs, each routed token's row read and
    written, the expert counts, and the rows' token indices (V words) or,
    given T, the inverse map the by-token form reads (T*K words)."""
    V, row_b = vtc * K, D * 2
    idx = V * 4 if T is None else T * K * 4
    return V * row_b + 2 * vtc * row_b + idx + E * 4


def shuffling_bytes(rows, D, EP, EG):
    """Every moved row read and written once, the count matrix and the
    output counts."""
    return 2 * rows * D * 2 + EP * EG * 4 + (EG + 1) * 4


def stream_mix(read_kib, write_kib):
    """(R, W, units) of the contiguous-stream probe that moves read_kib KiB in
    and write_kib KiB out: the smallest R:W (each <= 32) equal to the
    kernel's read:write ratio, units = write_kib / W; None when the byte
    counts are not whole KiB or no such R, W exist."""
    from math import gcd
    if read_kib <= 0 or write_kib <= 0 or read_kib != int(read_kib) or \
            write_kib != int(write_kib):
        return None
    read_kib, write_kib = int(read_kib), int(write_kib)
    g = gcd(read_kib, write_kib)
    R, Wm = read_kib // g, write_kib // g
    if R > 32 or Wm > 32:
        return None
    return (R, Wm, write_kib // Wm)


# ------------------------------------------------------------------ workloads
def setup_dispatch(ctx, wl, with_cpu, general=False):
    """general: gather and scatter through the entry points that take
    token_indices (moe_gather_scale with a workspace, moe_scatter_add)
    instead of the shuffle's inverse map."""
    torch, ops, W, dev = ctx.torch, ctx.ops, ctx.W, ctx.dev
    inp = W.dispatch_inputs(wl)
    T, D, E, K = wl.T, wl.D, wl.E, wl.K
    vtc = wl.vtc if wl.vtc is not None else T
    a = T * K
    V = vtc * K
    scores = torch.from_numpy(inp.scores).to(dev)
    x = ctx.bf(inp.x)
    y = ctx.bf(inp.y)
    out = torch.zeros((T, D), dtype=torch.bfloat16, device=dev)
    vtc_d = torch.tensor([vtc], dtype=torch.int32, device=dev) if wl.vtc else None
    quant = wl.quant
    if quant:
        rows = torch.empty((a, D), dtype=torch.uint8, device=dev)
        rscale = torch.empty(a, dtype=torch.float32, device=dev)
        ub = torch.tensor([wl.scale_ub], dtype=torch.float32, device=dev)
    else:
        rows = torch.empty((a, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, ctx.lib.moe_shuffle_workspace_bytes(T, E, K)), dtype=torch.uint8,
                     device=dev)
    shuf_out = (torch.empty(E + 1, dtype=torch.int32, device=dev),
                torch.empty(a, dtype=torch.int32, device=dev),
                torch.empty(a, dtype=torch.int32, device=dev),
                torch.empty((T, K), dtype=torch.int32, device=dev))

    counts, ei, ti, rop = shuf_out
    vr = counts[E:]
    if general:
        ws_g = torch.empty(max(1, ctx.lib.moe_gather_scale_workspace_bytes(T, a)),
                           dtype=torch.uint8, device=dev)
        ws_s = torch.empty(max(1, ctx.lib.moe_scatter_add_workspace_bytes(T, a)),
                           dtype=torch.uint8, device=dev)

    def shuffle():
        ops.moe_shuffle(scores, K, vtc_d, workspace=ws, out=shuf_out)

    def gather():
        if quant:
            ops.moe_gather_scale_quant(x, ti, ei, scores, ub, vr, rows, rscale)
        elif general:
            ops.moe_gather_scale(x, ti, ei, scores, vr, rows, workspace=ws_g)
        else:
            ops.moe_gather_scale_by_token(x, rop, ei, scores, vr, rows)

    def scatter():
        if general:
            ops.moe_scatter_add(out, y, ti, vr, workspace=ws_s)
        else:
            ops.moe_scatter_add_by_token(out, y, rop, vr)

    name = wl.name + ("-general" if general else "")
    # the row bytes of gather and scatter (indices and scores left out)
    tok_kib = vtc * D * 2 / 1024
    ceiling = {"gather": stream_mix(2 * V * D / 1024, V * D / 1024) if quant else
               stream_mix(tok_kib, K * tok_kib),
               "scatter": stream_mix((K + 1) * tok_kib, tok_kib)}
    stage_names = (("gather_scale_quant", "scatter_add_by_token") if quant else
                   ("gather_scale (token_indices, workspace)", "scatter_add (token_indices)")
                   if general else ("gather_scale_by_token", "scatter_add_by_token"))
    return SimpleNamespace(
        stages={"shuffle": shuffle, "gather": gather, "scatter": scatter},
        stage_bytes=dispatch_bytes(T, D, E, K, vtc, quant, general),
        units_per_step=vtc, unit="tokens/s", metric=DISPATCH_METRIC,
        config={"workload": f"{name}: T={T} D={D} E={E} K={K} valid_token_count={vtc}",
                "tokens": T, "hidden": D, "experts": E, "top_k": K,
                "valid_token_count": vtc, "routed_rows": V,
                "stages": "shuffle -> " + " -> ".join(stage_names)},
        traffic_key=name, ceiling=ceiling,
        dtype="bf16" if not quant else "bf16->fp8e4m3",
        kernel_src={"shuffle": ["shuffle.hip"],
                    # the general gather builds its row lists with combine.hip's kernel
                    "gather": ["gather.hip", "combine.hip"] if general else ["gather.hip"],
                    "scatter": ["combine.hip"]},
        cpu=cpu_baseline_dispatch(ctx.orc, inp, wl, vtc) if with_cpu else None)


def setup_finalize(ctx, wl, with_cpu, variant=False, T=None):
    """variant: bf16 routing weights and the 128x4-tiled scale layout. T: the
    token count, if not the workload's (the decode sweep)."""
    torch, ops, W, dev = ctx.torch, ctx.ops, ctx.W, ctx.dev
    T = wl.T if T is None else T
    fi = W.finalize_inputs(wl, T=T)
    D, K = wl.D, wl.K
    w = W.to_bf16_bits(fi.w) if variant else fi.w
    yd = ctx.bf(fi.y)
    wd = ctx.bf(w) if variant else torch.from_numpy(w).to(dev)
    ropd = torch.from_numpy(fi.row_of_pair).to(dev)
    shd = ctx.bf(fi.shared)
    gd = ctx.bf(fi.gamma)
    outd = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    mx = wl.mxfp8
    layout = "swizzled" if variant else "rowmajor"
    sbytes = ctx.lib.moe_mxfp8_scale_bytes(T, D, 4 if variant else 0) if mx else 0
    codes = torch.empty((T, D), dtype=torch.uint8, device=dev) if mx else None
    scales = torch.empty(sbytes, dtype=torch.uint8, device=dev) if mx else None

    def finalize():
        ops.moe_finalize_rmsnorm(yd, wd, ropd, shd, gd, wl.eps, out=outd, mxfp8=mx,
                                 scale_layout=layout, mx_codes=codes, mx_scales=scales)

    fin_bytes = finalize_bytes(T, D, K, sbytes if mx else None, bf16_weights=variant)
    name = wl.name + ("-swizzled" if variant else "")
    row_kib = T * D * 2 / 1024  # expert and shared rows in, bf16 rows (and codes) out
    ceiling = {"finalize": stream_mix((K + 1) * row_kib, row_kib * (1.5 if mx else 1))}
    return SimpleNamespace(
        stages={"finalize": finalize}, stage_bytes={"finalize": fin_bytes},
        units_per_step=T, unit="tokens/s",
        metric="finalize+RMSNorm tokens/s and achieved HBM GB/s (% of peak), 1xMI355X",
        config={"workload": f"{name}: T={T} D={D} K={K}" + (" MXFP8" if mx else "") +
                (" bf16 weights, 128x4-tiled scales" if variant else ""),
                "tokens": T, "hidden": D, "top_k": K,
                "stages": "finalize_rmsnorm" + (" + mxfp8" if mx else "")},
        dtype="bf16" if not mx else "bf16->mxfp8", kernel_src={"finalize": ["finalize.hip"]},
        traffic_key=name, ceiling=ceiling,
        cpu=cpu_baseline_finalize(ctx.orc, fi, wl, w, 2 if variant else 0, name)
        if with_cpu else None)


def setup_mhc(ctx, wl, with_cpu):
    torch, ops, W, dev = ctx.torch, ctx.ops, ctx.W, ctx.dev
    fi = W.finalize_inputs(wl)
    m = W.mhc_inputs(wl)
    T, D, K, hc = wl.T, wl.D, wl.K, wl.hc
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    yd, wd, ropd = ctx.bf(fi.y), f32(fi.w), torch.from_numpy(fi.row_of_pair).to(dev)
    shd, gd = ctx.bf(fi.shared), ctx.bf(fi.gamma)
    resd, postd, combd, pred = ctx.bf(m.residual), f32(m.post), f32(m.comb), f32(m.pre)
    res_out = torch.empty_like(resd)
    outd = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    sbytes = ctx.lib.moe_mxfp8_scale_bytes(T, D, 4)
    codes = torch.empty((T, D), dtype=torch.uint8, device=dev)
    scales = torch.empty(sbytes, dtype=torch.uint8, device=dev)

    def finalize_mhc():
        ops.moe_finalize_mhc(yd, wd, ropd, shd, resd, postd, combd, pred, gd, wl.eps,
                             residual_out=res_out, out=outd, mxfp8=True,
                             scale_layout="swizzled", mx_codes=codes, mx_scales=scales)

    row_kib = T * D * 2 / 1024  # rows in: K experts, shared, hc streams; out: hc, bf16, codes
    ceiling = {"finalize_mhc": stream_mix((K + 1 + hc) * row_kib, (hc + 1.5) * row_kib)}
    return SimpleNamespace(
        stages={"finalize_mhc": finalize_mhc}, ceiling=ceiling,
        stage_bytes={"finalize_mhc": mhc_bytes(T, D, K, hc, sbytes)},
        units_per_step=T, unit="tokens/s",
        metric="mHC finalize+RMSNorm tokens/s and achieved HBM GB/s (% of peak), 1xMI355X",
        config={"workload": f"{wl.name}: T={T} D={D} K={K} hc={hc} MXFP8 128x4-tiled scales",
                "tokens": T, "hidden": D, "top_k": K, "hc": hc,
                "stages": "finalize_mhc + mxfp8"},
        dtype="bf16->mxfp8", kernel_src={"finalize_mhc": ["finalize.hip"]},
        cpu=cpu_baseline_mhc(ctx.orc, fi, m, wl) if with_cpu else None)


def _device_normal_bf16(torch, shape, seed, dev):
    """Seeded N(0,1) bf16 tensor made on the device, one leading slice at a
    time (a host draw of several GB would dominate the set-up)."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    for i in range(shape[0]):
        out[i].copy_(torch.randn(shape[1:], generator=g, device=dev))
    return out


def setup_padded(ctx, wl, with_cpu, general=False):
    """general: through token_indices (moe_scatter_add_padded, which builds
    per-token row lists in its workspace) instead of the shuffle's inverse map
    (moe_scatter_add_padded_by_token)."""
    torch, ops, W, dev = ctx.torch, ctx.ops, ctx.W, ctx.dev
    T, D, E, K, EP = wl.T, wl.D, wl.E, wl.K, wl.ep
    inp = W.dispatch_inputs(wl, with_y=False)
    vtc = wl.vtc
    scores = torch.from_numpy(inp.scores).to(dev)
    counts, ei, ti, rop = ops.moe_shuffle(scores, K, torch.tensor([vtc], dtype=torch.int32,
                                                                  device=dev))
    counts_e = counts[:E].contiguous()
    V = int(counts[E].item())
    T_K = T * K
    slabs = _device_normal_bf16(torch, (EP, T_K, D), 6000 + wl.cfg_id, dev)
    out = torch.zeros((T, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, ctx.lib.moe_scatter_add_padded_workspace_bytes(T, T_K, E)),
                     dtype=torch.uint8, device=dev)

    def padded_scatter():
        if general:
            ops.moe_scatter_add_padded(slabs, counts_e, ti, out, workspace=ws)
        else:
            ops.moe_scatter_add_padded_by_token(slabs, counts_e, rop, out)

    tok_kib = vtc * D * 2 / 1024
    name = wl.name + ("-general" if general else "")
    return SimpleNamespace(
        stages={"padded_scatter": padded_scatter},
        ceiling={"padded_scatter": stream_mix((K + 1) * tok_kib, tok_kib)},
        stage_bytes={"padded_scatter": padded_bytes(D, E, K, vtc, None if general else T)},
        units_per_step=vtc, unit="tokens/s", metric=DISPATCH_METRIC,
        config={"workload": f"{name}: T={T} D={D} E={E} K={K} EP={EP} "
                            f"valid_token_count={vtc} static (EP, T*K, D) buffer",
                "tokens": T, "hidden": D, "experts": E, "top_k": K, "ep": EP,
                "valid_token_count": vtc, "routed_rows": V,
                "stages": "scatter_add_padded (token_indices)" if general else
                          "scatter_add_padded_by_token (row_of_pair)"},
        traffic_key=name,
        dtype="bf16", kernel_src={"padded_scatter": ["combine.hip"]},
        cpu=cpu_baseline_padded(ctx.orc, ctx.W, wl) if with_cpu else None)


def setup_shuffling(ctx, wl, with_cpu):
    torch, ops, W, dev = ctx.torch, ctx.ops, ctx.W, ctx.dev
    T, D, E, K, EP = wl.T, wl.D, wl.E, wl.K, wl.ep
    EG = E // EP  # rank 0's local experts: columns [0, EG)
    per_src = []
    for r in range(EP):  # source rank r routes its own T tokens
        sc = torch.from_numpy(W.router_scores(wl, seed=r)).to(dev)
        c, _, _, _ = ops.moe_shuffle(sc, K, None, row_of_pair=False)
        per_src.append(c[:EG])
    counts = torch.stack(per_src).contiguous()  # (EP, EG): rows rank r sends per expert
    rows = int(counts.sum().item())
    tokens = _device_normal_bf16(torch, (1, rows, D), 7000 + wl.cfg_id, dev)[0]
    em = torch.empty_like(tokens)
    back = torch.empty_like(tokens)
    ws_bytes = max(1, ctx.lib.moe_shuffling_workspace_bytes(EP, EG, rows))
    ws_c = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_s = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def combine_shuffling():
        ops.moe_combine_shuffling(tokens, counts, 0, EG, None, out=em, workspace=ws_c)

    def split_shuffling():
        ops.moe_split_shuffling(em, counts, 0, EG, None, out=back, workspace=ws_s)

    nb = shuffling_bytes(rows, D, EP, EG)
    mix = stream_mix(rows * D * 2 / 1024, rows * D * 2 / 1024)
    return SimpleNamespace(
        ceiling={"combine_shuffling": mix, "split_shuffling": mix},
        stages={"combine_shuffling": combine_shuffling, "split_shuffling": split_shuffling},
        stage_bytes={"combine_shuffling": nb, "split_shuffling": nb},
        units_per_step=rows, unit="rows/s",
        metric="EP re-sort (combine_shuffling + split_shuffling) routed rows/s and achieved "
               "HBM GB/s (% of peak), 1xMI355X",
        config={"workload": f"{wl.name}: EP={EP} source ranks x T={T} tokens, E={E}, K={K}, "
                            f"softmax routing; rank 0's {EG} local experts, {rows} rows, "
                            f"D={D}, packed layout",
                "ep": EP, "tokens_per_rank": T, "experts": E, "top_k": K,
                "local_experts": EG, "rows": rows, "hidden": D,
                "stages": "combine_shuffling -> split_shuffling"},
        dtype="bf16", kernel_src={"combine_shuffling": ["reorder.hip"],
                                  "split_shuffling": ["reorder.hip"]},
        cpu=cpu_baseline_shuffling(ctx.orc, counts.cpu().numpy(), D, wl)
        if with_cpu else None)


# ------------------------------------------------------------------ main
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the path runs on a single MI355X and "
              f"has no multi-GPU mode (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import oracle as orc
    from combine_moe_shuffle_amd import _lib, ops
    from combine_moe_shuffle_amd import workloads as W

    dev = torch.device("cuda:0")

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(
            torch.bfloat16)

    ctx = SimpleNamespace(torch=torch, ops=ops, W=W, orc=orc, dev=dev, bf=bf, lib=_lib.load())
    with_cpu = not args.no_cpu_baseline
    name = args.workload
    if name in ("zipf", "quant", "tiny"):
        s = setup_dispatch(ctx, W.WORKLOADS[name], with_cpu)
    elif name == "zipf-general":
        s = setup_dispatch(ctx, W.WORKLOADS["zipf"], with_cpu, general=True)
    elif name in ("prefill", "decode"):
        s = setup_finalize(ctx, W.WORKLOADS[name], with_cpu)
    elif name == "prefill-swizzled":
        s = setup_finalize(ctx, W.WORKLOADS["prefill"], with_cpu, variant=True)
    elif name == "mhc":
        s = setup_mhc(ctx, W.WORKLOADS["mhc"], with_cpu)
    elif name in ("padded", "padded-general"):
        s = setup_padded(ctx, W.WORKLOADS["padded"], with_cpu, general=name == "padded-general")
    else:
        s = setup_shuffling(ctx, W.WORKLOADS["shuffling"], with_cpu)
    if s.cpu:
        s.cpu["host"] = _host()
    # a few us per step: more steps amortise the region's ends
    short = name in ("decode", "tiny")
    steps = args.steps if args.steps is not None else (1000 if short else 50)
    warm = args.warmup if args.warmup is not None else (50 if short else 5)
    # each stage's library calls, checked and converted once (ops.prepare: the
    # first call runs the op with every check); --checked goes through the
    # checked op call every time
    stages = [(n, fn if args.checked else ctx.ops.prepare(fn)) for n, fn in s.stages.items()]
    graph = args.graph

    def step():
        for _, fn in stages:
            fn()

    run_step = capture(torch, step).replay if graph else step
    # ---- warmup, then exactly `steps` timed steps (no event inside a step:
    # each event record between kernels costs the stream ~10 us)
    for _ in range(warm):
        run_step()
    torch.cuda.synchronize()
    region = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    t0 = time.perf_counter()
    region[0].record()
    for _ in range(steps):
        run_step()
    region[1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    region_ms = region[0].elapsed_time(region[1])
    # ---- the spread over steps: each step alone between an event pair, the
    # host waiting for it before the next (the latency of one isolated step,
    # launch included)
    isolated = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run_step()
        e1.record()
        torch.cuda.synchronize()
        isolated.append(e0.elapsed_time(e1) * 1e3)
    p10, p50, p90 = (float(v) for v in np.percentile(isolated, [10, 50, 90]))
    # ---- cold steps: before each step a 1 GiB buffer is read (a sum), which
    # evicts the step's data from L2 and the 256 MB Infinity Cache without
    # leaving dirty lines behind; the same with a 1 GiB write, whose dirty
    # lines the next step then writes back. Each flush alone is timed the same
    # way and subtracted, so no event sits between a flush and its step.
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    flush_sum = torch.empty((), dtype=torch.float32, device=dev)

    def flush_read():
        torch.sum(flush_buf, dim=0, out=flush_sum)

    def flush_write():
        flush_buf.fill_(1.0)

    def time_region(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def after_flush(fl, fn):
        """Device time per call of fn after flush fl: COLD_BLOCKS blocks of
        flush + fn and of the flush alone, alternated; the median over the
        blocks of the per-call difference (a flush takes ~150 us, so a drift
        of a few per cent in its own time would swamp a step of a few us)."""
        def both():
            fl()
            fn()
        both()
        n = max(1, steps // COLD_BLOCKS)
        diffs = [(time_region(both, n) - time_region(fl, n)) / n for _ in range(COLD_BLOCKS)]
        return float(np.median(diffs))

    cold = {}
    cold_stage = {}
    kinds = () if args.no_cold else (("read", flush_read), ("write", flush_write))
    for kind, fl in kinds:
        cold[kind] = after_flush(fl, run_step)
    # each stage alone after a read flush
    for n, fn in ([] if args.no_cold else stages):
        cold_stage[n] = after_flush(flush_read, fn)
    # ---- each stage alone, `steps` launches back to back: its average
    # duration per launch, the denominator of the roofline
    names = [n for n, _ in stages]
    st_ms = {n: stage_ms(torch, fn, steps) for n, fn in stages}
    dom = max(names, key=lambda n: st_ms[n])
    # ---- each streaming stage's read and write bytes moved by a plain stream
    # (consecutive waves on consecutive memory, two layouts): the rate that mix
    # reaches on this GPU, timed the same two ways as the stage
    ceiling = None
    mixes = {n: m for n, m in getattr(s, "ceiling", {}).items() if m}
    if mixes and not args.no_ceiling:
        ceiling = {"roofline_kernel": dom, "probe": "moe_stream_probe", "stages": {}}
        for n, (R, Wm, units) in mixes.items():
            p_src = torch.zeros(units * R * 1024, dtype=torch.uint8, device=dev)
            p_dst = torch.empty(units * Wm * 1024, dtype=torch.uint8, device=dev)
            p_bytes = units * (R + Wm) * 1024
            rec = {"R_kib": R, "W_kib": Wm, "waves": units, "bytes": p_bytes}
            for layout, lname in ((0, "blocked"), (1, "interleaved")):
                probe = ctx.ops.prepare(ctx.ops.moe_stream_probe, R, Wm, units, src=p_src,
                                        dst=p_dst, layout=layout)
                lrec = {"us": round(stage_ms(torch, probe, steps) * 1e3, 2)}
                if not args.no_cold:
                    lrec["us_after_read"] = round(after_flush(flush_read, probe) * 1e3, 2)
                rec[lname] = lrec
                del probe
            # the faster layout is the reference, each way of timing on its own
            best = min(rec["blocked"]["us"], rec["interleaved"]["us"])
            p_gbps = p_bytes / (best * 1e-6) / 1e9
            k_gbps = s.stage_bytes[n] / (st_ms[n] * 1e-3) / 1e9
            rec.update({"gbps": round(p_gbps, 1), "frac_of_peak": p_gbps / HBM_PEAK_GBPS,
                        "kernel_vs_probe": k_gbps / p_gbps})
            if not args.no_cold:
                bc = min(rec["blocked"]["us_after_read"], rec["interleaved"]["us_after_read"])
                pc_gbps = p_bytes / (bc * 1e-6) / 1e9
                kc_gbps = s.stage_bytes[n] / (cold_stage[n] * 1e-3) / 1e9
                rec.update({"gbps_after_read": round(pc_gbps, 1),
                            "kernel_vs_probe_after_read": kc_gbps / pc_gbps})
            ceiling["stages"][n] = rec
            del p_src, p_dst
    del flush_buf
    if args.copy_bytes > 0:
        n = args.copy_bytes // 2
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    warm_ms = elapsed * 1e3 / steps
    # the headline: the steps after a read flush (inputs in HBM, not in the
    # caches); the warm steps when the cold ones were skipped
    ms_step = cold["read"] if "read" in cold else warm_ms
    total_bytes = sum(s.stage_bytes.values())
    achieved = s.stage_bytes[dom] / (st_ms[dom] * 1e-3) / 1e9
    traffic = load_traffic(dom, s.kernel_src[dom], getattr(s, "traffic_key", name))

    def rates(ms):
        return {"ms_per_step": ms, "value": s.units_per_step / (ms * 1e-3),
                "hbm_gbps": total_bytes / (ms * 1e-3) / 1e9,
                "hbm_frac": total_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}

    line = {
        "metric": s.metric,
        "value": s.units_per_step / (ms_step * 1e-3),
        "unit": s.unit,
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": ms_step,
        "headline": ("cold: K steps, each after a 1 GiB read that evicts L2 and the "
                     "Infinity Cache, device time with the reads' own time subtracted "
                     "(median over 5 blocks of K/5 steps, each against a block of reads "
                     "alone)"
                     if "read" in cold else
                     "warm: K steps back to back (cold steps skipped)"),
        "warm": {**rates(warm_ms), "ms_per_step_device": region_ms / steps,
                 "step_us_isolated": {"p10": round(p10, 2), "p50": round(p50, 2),
                                      "p90": round(p90, 2)}},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {**s.config, "launch": ("one HIP graph per step" if graph else
                   "eager (kernels launched from Python)") +
                   (", checked op calls" if args.checked else
                    ", prepared calls (arguments checked once)")},
        "cold": None if args.no_cold else {
            **{kind: rates(ms) for kind, ms in cold.items()},
            "stage_us_after_read": {n: round(cold_stage[n] * 1e3, 2) for n in names},
            "roofline_frac_after_read":
                s.stage_bytes[dom] / (cold_stage[dom] * 1e-3) / 1e9 / HBM_PEAK_GBPS},
        "routed_rows_per_s": (s.config["routed_rows"] / (ms_step * 1e-3)
                              if "routed_rows" in s.config else None),
        "hbm_gbps": total_bytes / (ms_step * 1e-3) / 1e9,
        "hbm_frac": total_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "stage_us": {n: round(st_ms[n] * 1e3, 2) for n in names},
        "stage_gbps": {n: round(s.stage_bytes[n] / (st_ms[n] * 1e-3) / 1e9, 1)
                       for n in names},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "bytes_per_launch": s.stage_bytes[dom], "traffic": traffic,
                     "duration": "the kernel's average launch duration, launches back to "
                                 "back (what the rocprofv3 kernel trace shows); after a "
                                 "read flush: cold.roofline_frac_after_read"},
        "stream_ceiling": ceiling,
        "cpu_baseline": s.cpu,
    }
    if name == "decode" and not args.no_sweep:
        line["sweep"] = decode_sweep(ctx, W.WORKLOADS[name], steps, warm, args.checked)
    if name == "tiny" and not args.no_sweep:
        line["sweep"] = dispatch_sweep(ctx, W.WORKLOADS["zipf"], steps, warm, args.checked)
    print(json.dumps(line), flush=True)


DISPATCH_SWEEP_T = (1, 8, 32, 64, 128)


def dispatch_sweep(ctx, wl, steps, warm, checked):
    """The zipf step's calls at decode batch sizes, every token valid: by token
    (shuffle, gather and scatter through the inverse map) and through the
    entry points that take token_indices ("general"). Each is launched from
    Python `steps` times back to back (wall clock per step, launches included)
    and each stage's kernels are timed alone per launch (graph replay)."""
    torch = ctx.torch
    out = []
    for T in DISPATCH_SWEEP_T:
        rec = {"tokens": T}
        for key, general in (("", False), ("general_", True)):
            sub = setup_dispatch(ctx, ctx.W.Workload(**{**wl.__dict__, "T": T, "vtc": None}),
                                 False, general=general)
            fns = [(n, f if checked else ctx.ops.prepare(f)) for n, f in sub.stages.items()]

            def step():
                for _, f in fns:
                    f()

            for _ in range(warm):
                step()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                step()
            torch.cuda.synchronize()
            step_us = (time.perf_counter() - t0) * 1e6 / steps
            rec[key + "step_us"] = round(step_us, 2)
            rec[key + "stage_kernel_us"] = {n: round(stage_ms(torch, f, steps) * 1e3, 2)
                                            for n, f in fns}
        rec["tokens_per_s"] = T / (rec["step_us"] * 1e-6)
        out.append(rec)
    return out


def decode_sweep(ctx, wl, steps, warm, checked):
    """The decode finalize at every token count of the sweep: the step launched
    from Python `steps` times back to back (wall clock per call, launch
    included) and the kernel's own duration per launch (graph replay)."""
    torch = ctx.torch
    out = []
    for T in wl.sweep_T:
        sub = setup_finalize(ctx, wl, False, T=T)
        fn = sub.stages["finalize"]
        fn = fn if checked else ctx.ops.prepare(fn)
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        step_us = (time.perf_counter() - t0) * 1e6 / steps
        k_ms = stage_ms(torch, fn, steps)
        b = sub.stage_bytes["finalize"]
        rec = {"tokens": T, "step_us": round(step_us, 2), "kernel_us": round(k_ms * 1e3, 2),
               "tokens_per_s": T / (step_us * 1e-6), "bytes": b,
               "kernel_gbps": round(b / (k_ms * 1e-3) / 1e9, 1)}
        # floors on the same launch path and shape: an empty kernel, and two
        # dependent 16-byte loads + a store per thread
        for kind, key in ((0, "floor_empty"), (1, "floor_2loads")):
            ff = ctx.ops.prepare(ctx.ops.moe_launch_floor, kind, T, wl.D, device=ctx.dev)
            for _ in range(warm):
                ff()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                ff()
            torch.cuda.synchronize()
            rec[key + "_step_us"] = round((time.perf_counter() - t0) * 1e6 / steps, 2)
            rec[key + "_kernel_us"] = round(stage_ms(torch, ff, steps) * 1e3, 2)
        out.append(rec)
    return out


def load_traffic(kernel, srcs, workload):
    """HBM bytes per launch from the committed counter runs, if they were
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get(f"{workload}/{kernel}")
    if not rec or rec.get("source_hash") != source_hash(srcs):
        return None
    return rec.get("bytes_per_launch")


# ------------------------------------------------------------------ CPU oracle
CPU_SAMPLE_S = 10.0  # about this much single-core oracle time per baseline


def _median_time(fn):
    """Median wall time of runs of fn, the process pinned to one core meanwhile
    (the oracle is single-threaded): at least 3 runs, more while they add up
    to under CPU_SAMPLE_S seconds (at most 25). Returns (median, runs)."""
    old = os.sched_getaffinity(0)
    os.sched_setaffinity(0, {min(old)})
    try:
        ts = []
        while len(ts) < 3 or (sum(ts) < CPU_SAMPLE_S and len(ts) < 25):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
    finally:
        os.sched_setaffinity(0, old)
    return float(np.median(ts)), len(ts)


def _host():
    """The host the CPU baseline ran on: its CPU model, the logical CPUs the
    system has and those this process may use."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu": model, "nproc": os.cpu_count(), "usable": len(os.sched_getaffinity(0))}


def cpu_baseline_dispatch(orc, inp, wl, vtc):
    """The oracle on the same step (shuffle, gather, scatter-add), single
    thread; the median over about CPU_SAMPLE_S seconds of runs."""
    K = wl.K
    stage_t = {"shuffle": [], "gather": [], "scatter": []}
    rows = np.empty((wl.T * K, wl.D), np.uint16)

    def run():
        t0 = time.perf_counter()
        counts, ei, ti, rop = orc.shuffle(inp.scores, K, wl.vtc)
        V = int(counts[wl.E])
        t1 = time.perf_counter()
        if wl.quant:
            orc.gather_scale_quant(inp.x, ti, ei, inp.scores, wl.scale_ub, V)
        else:
            orc.gather_scale(inp.x, ti, ei, inp.scores, V, rows)
        t2 = time.perf_counter()
        orc.scatter_add(inp.out0.copy(), inp.y, ti, V)
        t3 = time.perf_counter()
        for k, d in zip(stage_t, (t1 - t0, t2 - t1, t3 - t2)):
            stage_t[k].append(d)

    t, runs = _median_time(run)
    return {"value": vtc / t, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole step (shuffle, gather, scatter-add) of the {wl.name} "
                      f"workload, {vtc} valid tokens; median of {runs} runs, "
                      f"{t:.2f} s each",
            "stage_s": {k: round(float(np.median(v)), 4) for k, v in stage_t.items()}}


def cpu_baseline_finalize(orc, fi, wl, w, flags, name):
    T = wl.T
    n = min(T, 4096)
    sub = slice(0, n)

    def run():
        orc.finalize_rmsnorm(fi.y, np.ascontiguousarray(w[sub]),
                             np.ascontiguousarray(fi.row_of_pair[sub]),
                             np.ascontiguousarray(fi.shared[sub]), fi.gamma, fi.eps,
                             flags=flags | (4 if flags & 2 else 0), mxfp8=wl.mxfp8)

    t, runs = _median_time(run)
    return {"value": n / t, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} of {T} tokens of the {name} finalize; median of {runs} "
                      f"runs, {t:.2f} s each"}


def cpu_baseline_mhc(orc, fi, m, wl):
    n = min(wl.T, 2048)
    sub = slice(0, n)
    c = np.ascontiguousarray

    def run():
        orc.finalize_mhc(fi.y, c(fi.w[sub]), c(fi.row_of_pair[sub]), c(fi.shared[sub]),
                         c(m.residual[sub]), c(m.post[sub]), c(m.comb[sub]), c(m.pre[sub]),
                         fi.gamma, fi.eps, flags=4, mxfp8=True)

    t, runs = _median_time(run)
    return {"value": n / t, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} of {wl.T} tokens of the mhc finalize; median of {runs} runs, "
                      f"{t:.2f} s each"}


def cpu_baseline_padded(orc, W, wl):
    """The oracle's padded combine on a T=1024 draw of the same routing
    (valid_token_count scaled to 750); every rank's slab holds the same
    N(0,1) rows (the oracle reads one row per routed pair either way)."""
    T = 1024
    vtc = wl.vtc * T // wl.T
    inp = W.dispatch_inputs(wl, T=T, vtc=vtc, with_y=False)
    counts, ei, ti, rop = orc.shuffle(inp.scores, wl.K, vtc)
    g = np.random.default_rng(6000)
    slab = W.to_bf16_bits(g.standard_normal((T * wl.K, wl.D), dtype=np.float32))
    slabs = np.ascontiguousarray(np.broadcast_to(slab, (wl.ep,) + slab.shape))
    out0 = np.zeros((T, wl.D), np.uint16)

    def run():
        orc.scatter_add_padded(out0.copy(), slabs, counts[:wl.E], ti)

    t, runs = _median_time(run)
    return {"value": vtc / t, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"T={T} tokens of the same routing ({vtc} valid), EP={wl.ep}; median "
                      f"of {runs} runs, {t:.2f} s each"}


def cpu_baseline_shuffling(orc, counts, D, wl):
    """The oracle's combine + split on the same counts; the rows are zeros
    (a row copy does not depend on its values)."""
    rows = int(counts.sum())
    EG = counts.shape[1]
    tok = np.zeros((rows, D), np.uint16)

    def run():
        em, _ = orc.combine_shuffling(tok, counts, 0, EG, None, out=np.empty_like(tok))
        orc.split_shuffling(em, counts, 0, EG, None, out=np.empty_like(tok))

    t, runs = _median_time(run)
    return {"value": rows / t, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole step ({rows} rows, combine + split); median of {runs} runs, "
                      f"{t:.2f} s each"}


if __name__ == "__main__":
    main()
