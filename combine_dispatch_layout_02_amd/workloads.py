"""Seeded synthetic inputs for the dispatch / combine workloads.

This module only draws inputs: token rows, routing, top-k weights and the
per-expert factors of the scaled expert stage.  It holds none of the
method's arithmetic (no deduplication, no slot assignment, no quantization,
no reduction), so both the HIP path and the CPU oracle can be fed from it.

Workloads (shapes and value distributions follow the pages' test setup:
bf16 N(0,1) token rows, 256 experts, top-8, hidden 7168, 4096 tokens per
rank, two nodes of eight ranks for the RDMA accounting):

  tiny        T=64,   H=256,  E=16,  R=4,  N=1, k=2, uniform, identity expert
  decode      T=128,  H=7168, E=256, R=8,  N=1, k=8, uniform, expert scales
              each expert's rows by a seeded fp32 factor in [0.5, 1.5)
  prefill2n   T=4096, H=7168, E=256, R=16, N=2, k=8, uniform, identity
  skewed      T=8192, H=7168, E=256, R=8,  N=1, k=8, Zipf(1.2) popularity
              over a seeded expert permutation, without replacement
  quant       T=4096, H=7168, E=256, R=8,  N=1, k=8, uniform; rows travel
              as fp8 e4m3 + fp32 scale per 128, the expert returns mxfp8
  nvfp4       as quant, but bf16 rows out and an nvfp4 payload back (16
              e2m1 + one bf16 scale per 16 elements)

Draw order from one numpy PCG64 stream per workload (seed 0 unless given):
x, routing, weight logits, expert factors.  bf16 rows are the round-to-
nearest-even cast of float32 N(0,1) draws (torch's cast).  Weights are the
float32 softmax of N(0,1) logits over the k slots.
"""
from __future__ import annotations

import numpy as np

WORKLOADS = {
    "tiny": dict(T=64, H=256, E=16, R=4, N=1, k=2, routing="uniform", expert="identity",
                 x_fmt="bf16"),
    "decode": dict(T=128, H=7168, E=256, R=8, N=1, k=8, routing="uniform", expert="scale",
                   x_fmt="bf16"),
    "prefill2n": dict(T=4096, H=7168, E=256, R=16, N=2, k=8, routing="uniform",
                      expert="identity", x_fmt="bf16"),
    "skewed": dict(T=8192, H=7168, E=256, R=8, N=1, k=8, routing="zipf", zipf_s=1.2,
                   expert="identity", x_fmt="bf16"),
    "quant": dict(T=4096, H=7168, E=256, R=8, N=1, k=8, routing="uniform", expert="identity",
                  x_fmt="fp8"),
    "nvfp4": dict(T=4096, H=7168, E=256, R=8, N=1, k=8, routing="uniform", expert="identity",
                  x_fmt="bf16", y_fmt="nvfp4"),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16 bit patterns (torch's cast)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _route_uniform(rng, T, E, k):
    # a uniformly random ordering of all experts per token; its first k are k
    # distinct experts drawn uniformly, in draw order
    return np.argsort(rng.random((T, E)), axis=1, kind="stable")[:, :k].astype(np.int64)


def _route_with_replacement(rng, T, E, k):
    return rng.integers(0, E, size=(T, k)).astype(np.int64)


def _route_zipf(rng, T, E, k, s):
    # popularity rank i has weight (i + 1)^-s; expert id = perm[i].  Sorting
    # Gumbel-perturbed log-weights yields a draw without replacement in the
    # order a sequential sampler would produce it.
    perm = rng.permutation(E)
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    gumbel = -np.log(-np.log(rng.random((T, E))))
    order = np.argsort(-(logp[None, :] + gumbel), axis=1, kind="stable")[:, :k]
    return perm[order].astype(np.int64)


def make_inputs(name: str = "tiny", seed: int = 0, **overrides) -> dict:
    """Draw one workload.  Keyword overrides change any shape or routing
    field; edge-case knobs:

      mask_frac    fraction of (t, j) slots set to -1 (masked)
      mask_tokens  fraction of tokens whose every slot is masked
      routing      "uniform" | "zipf" | "replace" (duplicates allowed)
    """
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    T, H, E, R, N, k = (int(cfg[n]) for n in ("T", "H", "E", "R", "N", "k"))
    rng = np.random.default_rng(seed)

    x = f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))

    routing = cfg.get("routing", "uniform")
    if routing == "uniform":
        idx = _route_uniform(rng, T, E, k)
    elif routing == "zipf":
        idx = _route_zipf(rng, T, E, k, float(cfg.get("zipf_s", 1.2)))
    elif routing == "replace":
        idx = _route_with_replacement(rng, T, E, k)
    else:
        raise ValueError(f"unknown routing {routing!r}")

    logits = rng.standard_normal((T, k), dtype=np.float32)
    m = logits.max(axis=1, keepdims=True) if k > 0 else logits
    ex = np.exp(logits - m, dtype=np.float32)
    w = (ex / ex.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)

    factor = rng.uniform(0.5, 1.5, size=E).astype(np.float32)

    mask_frac = float(cfg.get("mask_frac", 0.0))
    if mask_frac > 0:
        idx = idx.copy()
        idx[rng.random((T, k)) < mask_frac] = -1
    mask_tokens = float(cfg.get("mask_tokens", 0.0))
    if mask_tokens > 0:
        idx = idx.copy()
        idx[rng.random(T) < mask_tokens, :] = -1

    out = dict(cfg)
    out.update(name=name, seed=seed, T=T, H=H, E=E, R=R, N=N, k=k,
               x=x, topk_idx=np.ascontiguousarray(idx), topk_w=np.ascontiguousarray(w),
               expert_factor=factor if cfg.get("expert") == "scale" else None)
    return out
