"""Seeded synthetic inputs for the MoE dispatch/combine workloads.

This module only draws random inputs of the right shapes and distributions; it
holds none of the dispatch/combine arithmetic, so the CPU oracle and the GPU
path can both be fed from it. Every tensor has its own generator,
``PCG64(SeedSequence([seed, cfg_id, tensor_id]))``, so any one tensor can be
regenerated alone. bf16 values are returned as ``np.uint16`` bit patterns made
by torch's round-to-nearest-even cast of fp32 draws.

Workloads (the problem sizes are those of the MoE layers the pages describe:
hidden 7168 for the Kimi/DeepSeek-style 256-expert top-8 router, hidden 5120
for the DeepSeek-V4.1 finalize presets):

  tiny     T=64,    D=1024, E=8,   K=2  softmax router, top-2 kept, rest zeroed
  quant    T=4096,  D=5120, E=16,  K=1  softmax router, FP8 rowwise dispatch,
                                        scale_ub = 1200
  zipf     T=8192,  D=7168, E=256, K=8  sigmoid router, Zipf(1.2) expert
                                        popularity, valid_token_count = 6000
  decode   T in {1,8,32,128}, D=7168, K=8   finalize + RMSNorm
  prefill  T=16384, D=5120, E=128, K=4      finalize + RMSNorm + MXFP8
  mhc      T=16384, D=5120, E=128, K=4, hc=4 finalize + mHC post-mix and
                                        collapse + RMSNorm + MXFP8 (swizzled)
  padded   the zipf routing, combined from a static (EP=8, T*K, D) buffer
  shuffling EP=8 source ranks of T=8192 tokens, softmax routing over E=256,
           K=8; the rows for one rank's 32 local experts re-sorted and back
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

# tensor ids: one generator per tensor
(_X, _LOGITS, _Y, _OUT0, _PERM, _W, _SHARED, _GAMMA, _ZIPF, _GUMBEL, _HOLES,
 _RESID, _POST, _COMB, _PRE) = range(15)


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    T: int
    D: int
    E: int
    K: int
    router: str = "softmax"          # softmax | softmax_topk | zipf_sigmoid
    vtc: int | None = None           # valid_token_count (None: all tokens)
    quant: bool = False              # FP8 rowwise dispatch
    scale_ub: float | None = None
    zipf_s: float = 1.2
    eps: float = 1e-6                # finalize RMSNorm epsilon
    mxfp8: bool = False
    sweep_T: tuple = field(default_factory=tuple)
    hc: int = 0                      # mHC residual streams (0: plain finalize)
    ep: int = 1                      # expert-parallel ranks (padded combine, EP re-sort)


WORKLOADS = {
    "tiny": Workload("tiny", 0, T=64, D=1024, E=8, K=2, router="softmax_topk"),
    "quant": Workload("quant", 1, T=4096, D=5120, E=16, K=1, quant=True,
                      scale_ub=1200.0),
    "zipf": Workload("zipf", 2, T=8192, D=7168, E=256, K=8,
                     router="zipf_sigmoid", vtc=6000),
    "decode": Workload("decode", 3, T=128, D=7168, E=256, K=8,
                       sweep_T=(1, 8, 32, 128)),
    "prefill": Workload("prefill", 4, T=16384, D=5120, E=128, K=4, mxfp8=True),
    "mhc": Workload("mhc", 5, T=16384, D=5120, E=128, K=4, mxfp8=True, hc=4),
    "padded": Workload("padded", 6, T=8192, D=7168, E=256, K=8, router="zipf_sigmoid",
                       vtc=6000, ep=8),
    "shuffling": Workload("shuffling", 7, T=8192, D=7168, E=256, K=8, ep=8),
}


def rng(cfg_id: int, tensor_id: int, seed: int = 0) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([seed, cfg_id, tensor_id])))


def to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns via torch's round-to-nearest-even cast."""
    t = torch.from_numpy(np.ascontiguousarray(f, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(g: np.random.Generator, shape) -> np.ndarray:
    return to_bf16_bits(g.standard_normal(size=shape, dtype=np.float32))


def _softmax64(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float64)
    z = z - z.max(axis=-1, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=-1, keepdims=True)


def router_scores(wl: Workload, T: int | None = None, E: int | None = None,
                  seed: int = 0) -> np.ndarray:
    """Router output (T, E) fp32 for the workload's router model.

    softmax       softmax of N(0,1) logits (fp64, cast to fp32).
    softmax_topk  the same, keeping each token's K largest probabilities and
                  zeroing the rest (input construction with numpy's sort; the
                  dispatch path selects its own top-k from these scores).
    zipf_sigmoid  expert e has popularity p_pi(e) with p_r proportional to
                  r^-s (r = 1..E) under a seeded permutation pi; logits are
                  ln p_pi(e) + Gumbel(0,1) noise, so a token's top-K experts
                  are a draw of K experts without replacement weighted by p;
                  scores = sigmoid(logits).
    """
    T = wl.T if T is None else T
    E = wl.E if E is None else E
    if wl.router in ("softmax", "softmax_topk"):
        logits = rng(wl.cfg_id, _LOGITS, seed).standard_normal(size=(T, E))
        probs = _softmax64(logits)
        if wl.router == "softmax_topk":
            order = np.argsort(-probs, axis=1, kind="stable")
            keep = np.zeros_like(probs, dtype=bool)
            np.put_along_axis(keep, order[:, :wl.K], True, axis=1)
            probs = np.where(keep, probs, 0.0)
        return probs.astype(np.float32)
    if wl.router == "zipf_sigmoid":
        ranks = np.arange(1, E + 1, dtype=np.float64)
        p = ranks ** (-wl.zipf_s)
        p /= p.sum()
        perm = rng(wl.cfg_id, _ZIPF, seed).permutation(E)
        logp = np.log(p[perm])
        gumbel = rng(wl.cfg_id, _GUMBEL, seed).gumbel(size=(T, E))
        logits = logp[None, :] + gumbel
        return (1.0 / (1.0 + np.exp(-logits))).astype(np.float32)
    raise ValueError(f"unknown router {wl.router}")


@dataclass
class DispatchInputs:
    x: np.ndarray          # (T, D) bf16 bits
    scores: np.ndarray     # (T, E) fp32
    y: np.ndarray          # (T*K, D) bf16 bits: stand-in expert outputs
    out0: np.ndarray       # (T, D) bf16 bits: initial combine output
    vtc: int | None


def dispatch_inputs(wl: Workload, seed: int = 0, T: int | None = None,
                    D: int | None = None, E: int | None = None,
                    K: int | None = None, vtc: int | None = -1,
                    out0: str = "zeros", with_y: bool = True) -> DispatchInputs:
    """Inputs of shuffle -> gather_scale[_quant] -> scatter_add.

    Sizes default to the workload's; ``vtc=-1`` keeps the workload's valid
    token count. ``out0`` is "zeros" (the workloads) or "normal" (N(0,1)
    bf16, the shared-expert-output case)."""
    T = wl.T if T is None else T
    D = wl.D if D is None else D
    E = wl.E if E is None else E
    K = wl.K if K is None else K
    if vtc == -1:
        vtc = wl.vtc
    wl_k = Workload(**{**wl.__dict__, "K": K})
    x = normal_bf16(rng(wl.cfg_id, _X, seed), (T, D))
    scores = router_scores(wl_k, T, E, seed)
    y = normal_bf16(rng(wl.cfg_id, _Y, seed), (T * K, D)) if with_y else None
    if out0 == "zeros":
        o = np.zeros((T, D), dtype=np.uint16)
    else:
        o = normal_bf16(rng(wl.cfg_id, _OUT0, seed), (T, D))
    return DispatchInputs(x=x, scores=scores, y=y, out0=o, vtc=vtc)


@dataclass
class FinalizeInputs:
    y: np.ndarray            # (rows, D) bf16 bits: unweighted expert outputs
    w: np.ndarray            # (T, K) fp32 routing weights
    row_of_pair: np.ndarray  # (T, K) int32, -1 = slot not held
    shared: np.ndarray       # (T, D) bf16 bits
    gamma: np.ndarray        # (D,) bf16 bits
    eps: float


def finalize_inputs(wl: Workload, T: int | None = None, D: int | None = None,
                    K: int | None = None, seed: int = 0,
                    hole_frac: float = 0.0) -> FinalizeInputs:
    """Inputs of the MoE finalize.

    The expert rows are T*K N(0,1) bf16 rows. Each (token, slot) pair owns one
    of them through a seeded random bijection (the permuted order a dispatch
    produces); ``hole_frac`` of the pairs are marked -1 (expert not held).
    Weights are a softmax over K N(0,1) draws per token (fp64, cast to fp32).
    Shared output N(0,1) bf16; gamma = bf16(U(0.5, 1.5))."""
    T = wl.T if T is None else T
    D = wl.D if D is None else D
    K = wl.K if K is None else K
    rows = T * K
    y = normal_bf16(rng(wl.cfg_id, _Y, seed), (rows, D))
    w = _softmax64(rng(wl.cfg_id, _W, seed).standard_normal(size=(T, K)))
    w = w.astype(np.float32)
    rop = rng(wl.cfg_id, _PERM, seed).permutation(rows).astype(np.int32)
    rop = rop.reshape(T, K)
    if hole_frac > 0.0:
        holes = rng(wl.cfg_id, _HOLES, seed).random(size=(T, K)) < hole_frac
        rop = np.where(holes, np.int32(-1), rop).astype(np.int32)
    shared = normal_bf16(rng(wl.cfg_id, _SHARED, seed), (T, D))
    g = rng(wl.cfg_id, _GAMMA, seed).uniform(0.5, 1.5, size=D).astype(np.float32)
    return FinalizeInputs(y=y, w=np.ascontiguousarray(w), row_of_pair=rop,
                          shared=shared, gamma=to_bf16_bits(g), eps=wl.eps)


@dataclass
class MhcInputs:
    residual: np.ndarray     # (T, hc, D) bf16 bits: the hc residual streams
    post: np.ndarray         # (T, hc) fp32 post-mix
    comb: np.ndarray         # (T, hc, hc) fp32 residual mix [source, target]
    pre: np.ndarray          # (T, hc) fp32 pre-mix of the collapse


def mhc_inputs(wl: Workload, T: int | None = None, D: int | None = None,
               hc: int | None = None, seed: int = 0) -> MhcInputs:
    """Inputs of the mHC stage, shaped like those of a trained hyper-connection
    layer: residual streams N(0,1) bf16; post = 2*sigmoid(N(0,1)) in (0, 2);
    pre = sigmoid(N(0,1)) in (0, 1); comb a doubly stochastic matrix per token
    (20 alternating row/column normalisations of exp(N(0,1)), in fp64)."""
    T = wl.T if T is None else T
    D = wl.D if D is None else D
    hc = (wl.hc or 4) if hc is None else hc
    residual = normal_bf16(rng(wl.cfg_id, _RESID, seed), (T, hc, D))
    post = 2.0 / (1.0 + np.exp(-rng(wl.cfg_id, _POST, seed).standard_normal((T, hc))))
    pre = 1.0 / (1.0 + np.exp(-rng(wl.cfg_id, _PRE, seed).standard_normal((T, hc))))
    c = np.exp(rng(wl.cfg_id, _COMB, seed).standard_normal((T, hc, hc)))
    for _ in range(20):
        c = c / c.sum(axis=2, keepdims=True)
        c = c / c.sum(axis=1, keepdims=True)
    return MhcInputs(residual=residual, post=post.astype(np.float32),
                     comb=np.ascontiguousarray(c.astype(np.float32)),
                     pre=pre.astype(np.float32))
