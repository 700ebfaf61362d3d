"""The routing draw of the pages' worked example, written from its description.

MORI-EP Benchmark page, "Reference: print_bw_values.py": for logical rank r
the script seeds torch's CPU generator with r, draws (and discards) a bf16
N(0,1) token matrix [T, H], draws fp32 scores |N(0,1)| + 1 of shape [T, E],
keeps per token the min(nodes, 4) node groups with the largest per-group
maximum score (the other groups' scores become 0) and routes each token to
the k experts with the largest remaining scores.  Only the set of experts per
token matters for the layout counts, so the order of the k ids is whatever
torch's top-k returns.

This is input generation for the oracle's worked-example pin, not part of
either implementation.
"""
from __future__ import annotations

import numpy as np


def pages_routing(rank: int, T: int = 4096, H: int = 7168, E: int = 256, N: int = 2,
                  k: int = 8) -> np.ndarray:
    import torch

    gen = torch.Generator().manual_seed(rank)
    torch.randn((T, H), dtype=torch.bfloat16, generator=gen)  # advances the stream
    scores = torch.randn((T, E), dtype=torch.float32, generator=gen).abs() + 1
    groups = min(N, 4)
    per_node = scores.view(T, N, E // N)
    best_groups = per_node.amax(dim=-1).topk(groups, dim=-1, sorted=False).indices
    keep = torch.zeros((T, N), dtype=torch.bool)
    keep[torch.arange(T).unsqueeze(1), best_groups] = True
    masked = (per_node * keep.unsqueeze(-1)).view(T, E)
    idx = masked.topk(k, dim=-1, largest=True, sorted=False).indices
    return idx.to(torch.int64).numpy()
