"""Benchmark of the MoE dispatch/combine hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload zipf]

A step is one pass of the path over one batch of synthetic input, already
resident in HBM:
  zipf     (default; T=8192, D=7168, E=256, K=8, valid_token_count=6000)
           moe_shuffle -> moe_gather_scale_by_token -> moe_scatter_add_by_token
  quant    (T=4096, D=5120, E=16, K=1)
           moe_shuffle -> moe_gather_scale_quant -> moe_scatter_add_by_token
  prefill  (T=16384, D=5120, K=4) moe_finalize_rmsnorm with MXFP8
  decode   (T=128, D=7168, K=8)   moe_finalize_rmsnorm
W untimed steps, then exactly K timed steps between two device
synchronisations (wall clock, and a HIP event pair around the region). Then
the same K steps once more with HIP events around every stage on the stream
the kernels run on (an event between two kernels costs the stream ~10 us, so
the headline region carries none): each stage's average duration. The
longest stage is the roofline kernel: its algorithmic bytes per launch
(unique inputs read once, outputs written once, valid rows only) over that
duration, against the 8 TB/s HBM peak.

One JSON line on stdout. value = valid tokens per second of the whole step.
cpu_baseline = the CPU oracle (single-threaded C) timed on the same step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="zipf",
                   choices=["zipf", "quant", "prefill", "decode"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-bytes", type=int, default=0,
                   help="after the timed region, run one plain device copy of this many "
                        "bytes (the calibration kernel of the HBM counter runs)")
    return p.parse_args()


def source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "combine_moe_shuffle_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Timer:
    """HIP events around named stages on the current stream."""

    def __init__(self, torch, names, steps):
        self.torch = torch
        self.ev = {n: [(torch.cuda.Event(enable_timing=True),
                        torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
                   for n in names}

    def mean_ms(self, name):
        pairs = self.ev[name]
        return sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build's path runs on a single MI355X and "
              f"has no multi-GPU mode (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import oracle as orc
    from combine_moe_shuffle_amd import ops
    from combine_moe_shuffle_amd import workloads as W

    dev = torch.device("cuda:0")
    wl = W.WORKLOADS[args.workload]

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(
            torch.bfloat16)

    steps, warm = args.steps, args.warmup
    cpu = None

    if args.workload in ("zipf", "quant"):
        inp = W.dispatch_inputs(wl)
        T, D, E, K = wl.T, wl.D, wl.E, wl.K
        vtc = wl.vtc if wl.vtc is not None else T
        a = T * K
        V = vtc * K
        scores = torch.from_numpy(inp.scores).to(dev)
        x = bf(inp.x)
        y = bf(inp.y)
        out = torch.zeros((T, D), dtype=torch.bfloat16, device=dev)
        vtc_d = torch.tensor([vtc], dtype=torch.int32, device=dev) if wl.vtc else None
        quant = wl.quant
        if quant:
            rows = torch.empty((a, D), dtype=torch.uint8, device=dev)
            rscale = torch.empty(a, dtype=torch.float32, device=dev)
            ub = torch.tensor([wl.scale_ub], dtype=torch.float32, device=dev)
        else:
            rows = torch.empty((a, D), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(1, _lib_ws(T, E, K)), dtype=torch.uint8, device=dev)
        shuf_out = (torch.empty(E + 1, dtype=torch.int32, device=dev),
                    torch.empty(a, dtype=torch.int32, device=dev),
                    torch.empty(a, dtype=torch.int32, device=dev),
                    torch.empty((T, K), dtype=torch.int32, device=dev))
        names = ["shuffle", "gather", "scatter"]

        def step(tm=None, i=0):
            def mark(n, k):
                if tm is not None:
                    tm.ev[n][i][k].record()
            mark("shuffle", 0)
            counts, ei, ti, rop = ops.moe_shuffle(scores, K, vtc_d, workspace=ws, out=shuf_out)
            mark("shuffle", 1)
            vr = counts[E:]
            mark("gather", 0)
            if quant:
                ops.moe_gather_scale_quant(x, ti, ei, scores, ub, vr, rows, rscale)
            else:
                ops.moe_gather_scale_by_token(x, rop, ei, scores, vr, rows)
            mark("gather", 1)
            mark("scatter", 0)
            ops.moe_scatter_add_by_token(out, y, rop, vr)
            mark("scatter", 1)

        # algorithmic bytes per launch (unique data read once, written once)
        row_b = D * 2
        shuffle_bytes = T * E * 4 + 3 * a * 4 + (E + 1) * 4
        if quant:
            gather_bytes = V * row_b + V * D + V * 4 + 2 * V * 4 + V * 4
        else:
            gather_bytes = vtc * row_b + V * row_b + T * K * 4 + V * 4 + V * 4
        scatter_bytes = V * row_b + 2 * vtc * row_b + T * K * 4
        stage_bytes = {"shuffle": shuffle_bytes, "gather": gather_bytes,
                       "scatter": scatter_bytes}
        tokens_per_step = vtc
        workload_cfg = {"workload": f"{wl.name}: T={T} D={D} E={E} K={K} "
                        f"valid_token_count={vtc}", "tokens": T, "hidden": D,
                        "experts": E, "top_k": K, "valid_token_count": vtc,
                        "routed_rows": V,
                        "stages": "shuffle -> " + ("gather_scale_quant" if quant else
                                                   "gather_scale_by_token") +
                        " -> scatter_add_by_token"}
        dtype = "bf16" if not quant else "bf16->fp8e4m3"
        kernel_src = {"shuffle": ["shuffle.hip"], "gather": ["gather.hip"],
                      "scatter": ["combine.hip"]}

        if not args.no_cpu_baseline:
            cpu = cpu_baseline_dispatch(orc, inp, wl, vtc)
    else:
        T_ = wl.T
        fi = W.finalize_inputs(wl)
        T, D, K = T_, wl.D, wl.K
        yd = bf(fi.y)
        wd = torch.from_numpy(fi.w).to(dev)
        ropd = torch.from_numpy(fi.row_of_pair).to(dev)
        shd = bf(fi.shared)
        gd = bf(fi.gamma)
        outd = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
        names = ["finalize"]
        mx = wl.mxfp8

        def step(tm=None, i=0):
            if tm is not None:
                tm.ev["finalize"][i][0].record()
            ops.moe_finalize_rmsnorm(yd, wd, ropd, shd, gd, wl.eps, out=outd, mxfp8=mx)
            if tm is not None:
                tm.ev["finalize"][i][1].record()

        row_b = D * 2
        fin_bytes = T * K * row_b + 2 * T * row_b + row_b + T * K * 8
        if mx:
            fin_bytes += T * D + T * (D // 32)
        stage_bytes = {"finalize": fin_bytes}
        tokens_per_step = T
        workload_cfg = {"workload": f"{wl.name}: T={T} D={D} K={K}" +
                        (" MXFP8" if mx else ""), "tokens": T, "hidden": D, "top_k": K,
                        "stages": "finalize_rmsnorm" + (" + mxfp8" if mx else "")}
        dtype = "bf16" if not mx else "bf16->mxfp8"
        kernel_src = {"finalize": ["finalize.hip"]}
        if not args.no_cpu_baseline:
            cpu = cpu_baseline_finalize(orc, fi, wl)

    # ---- warmup, then exactly `steps` timed steps (no event inside a step:
    # each event record between kernels costs the stream ~10 us)
    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    region = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    t0 = time.perf_counter()
    region[0].record()
    for i in range(steps):
        step()
    region[1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    region_ms = region[0].elapsed_time(region[1])
    # ---- the same steps again with HIP events around every stage: the
    # per-kernel durations behind the roofline
    tm = Timer(torch, names, steps)
    for i in range(steps):
        step(tm, i)
    torch.cuda.synchronize()
    if args.copy_bytes > 0:
        n = args.copy_bytes // 2
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    ms_step = elapsed * 1e3 / steps
    stage_ms = {n: tm.mean_ms(n) for n in names}
    total_bytes = sum(stage_bytes.values())
    dom = max(names, key=lambda n: stage_ms[n])
    achieved = stage_bytes[dom] / (stage_ms[dom] * 1e-3) / 1e9
    traffic = load_traffic(dom, kernel_src[dom], wl.name)

    line = {
        "metric": "dispatch+combine tokens/s and achieved HBM GB/s (% of peak), 1xMI355X"
        if args.workload in ("zipf", "quant") else
        "finalize+RMSNorm tokens/s and achieved HBM GB/s (% of peak), 1xMI355X",
        "value": tokens_per_step / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": ms_step,
        "ms_per_step_device": region_ms / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": workload_cfg,
        "hbm_gbps": total_bytes / (ms_step * 1e-3) / 1e9,
        "hbm_frac": total_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "stage_us": {n: round(stage_ms[n] * 1e3, 2) for n in names},
        "stage_gbps": {n: round(stage_bytes[n] / (stage_ms[n] * 1e-3) / 1e9, 1)
                       for n in names},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "bytes_per_launch": stage_bytes[dom], "traffic": traffic},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def _lib_ws(T, E, K):
    from combine_moe_shuffle_amd import _lib
    return _lib.load().moe_shuffle_workspace_bytes(T, E, K)


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


def _median_time(fn, reps):
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def cpu_baseline_dispatch(orc, inp, wl, vtc):
    """The oracle on the same step (shuffle, gather, scatter-add), single
    thread; median of 3 runs."""
    K = wl.K

    def run():
        counts, ei, ti, rop = orc.shuffle(inp.scores, K, wl.vtc)
        V = int(counts[wl.E])
        rows = np.empty((wl.T * K, wl.D), np.uint16)
        if wl.quant:
            orc.gather_scale_quant(inp.x, ti, ei, inp.scores, wl.scale_ub, V)
        else:
            orc.gather_scale(inp.x, ti, ei, inp.scores, V, rows)
        orc.scatter_add(inp.out0.copy(), inp.y, ti, V)

    t = _median_time(run, 3)
    return {"value": vtc / t, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole step (shuffle, gather, scatter-add) of the {wl.name} "
                      f"workload, {vtc} valid tokens; median of 3 runs, "
                      f"{t:.2f} s each"}


def cpu_baseline_finalize(orc, fi, wl):
    T = wl.T
    n = min(T, 4096)
    sub = slice(0, n)

    def run():
        orc.finalize_rmsnorm(fi.y, np.ascontiguousarray(fi.w[sub]),
                             np.ascontiguousarray(fi.row_of_pair[sub]),
                             np.ascontiguousarray(fi.shared[sub]), fi.gamma, fi.eps,
                             mxfp8=wl.mxfp8)

    t = _median_time(run, 3)
    return {"value": n / t, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} of {T} tokens of the {wl.name} finalize; median of 3 "
                      f"runs, {t:.2f} s each"}


if __name__ == "__main__":
    main()
