"""The routing of the pages' worked example, as input for the oracle's pin.

MORI-EP Benchmark page, "Reference: print_bw_values.py": each logical rank
seeds torch's CPU generator with its rank, spends the stream on a bf16
N(0,1) token matrix [T, H], then draws fp32 scores |N(0,1)| + 1 of shape
[T, E].  A token may use at most min(nodes, 4) nodes -- those holding its
highest scores -- and is routed to its k highest-scoring experts there.

Only the seeded draw has to match the page (the 8166 pin depends on the exact
random stream), so the draw uses torch's generator in the page's order.  The
selection is this module's own: per token, rank the nodes by their best
score, keep the allowed ones, and take the k largest scores among their
experts with numpy's argpartition.  Only the set of experts per token matters
for the layout counts, so their order within a row is arbitrary.

This is input generation for a test, not part of either implementation.
"""
from __future__ import annotations

import numpy as np


def _scores(rank: int, T: int, H: int, E: int) -> np.ndarray:
    """The page's draw at seed `rank`: [T, E] fp32 scores."""
    import torch

    gen = torch.Generator().manual_seed(rank)
    torch.randn((T, H), dtype=torch.bfloat16, generator=gen)   # consumed first in the page's stream
    return (torch.randn((T, E), dtype=torch.float32, generator=gen).abs() + 1).numpy()


def pages_routing(rank: int, T: int = 4096, H: int = 7168, E: int = 256, N: int = 2,
                  k: int = 8) -> np.ndarray:
    scores = _scores(rank, T, H, E)
    per_node = E // N
    allowed_nodes = min(N, 4)
    node_best = scores.reshape(T, N, per_node).max(axis=2)                 # [T, N]
    # nodes by descending best score; the first allowed_nodes of each row stay
    order = np.argsort(-node_best, axis=1, kind="stable")[:, :allowed_nodes]
    node_ok = np.zeros((T, N), dtype=bool)
    np.put_along_axis(node_ok, order, True, axis=1)
    expert_ok = np.repeat(node_ok, per_node, axis=1)                       # [T, E]
    candidates = np.where(expert_ok, scores, -np.inf)
    return np.argpartition(-candidates, k - 1, axis=1)[:, :k].astype(np.int64)
