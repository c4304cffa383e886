"""Stage plan: which contiguous layer range each pipeline stage owns.

Follows the memra ``pp`` module docs (header: stage map; functions pp_cuts and
stage_of) and the ninfer "Multi-GPU: layer pipeline stages" page (How it works:
StagePlan with per-stage layer counts).  Test infrastructure only.
"""
from __future__ import annotations


def stage_plan(n_layers: int, n_stages: int, cuts=None) -> list[int]:
    """Fence [0, c1, .., cN-1, n_layers]; stage s runs [fence[s], fence[s+1]).

    Without explicit cuts the split is even: cut s = s * n_layers / N with
    integer (floor) division.  Explicit cuts must be strictly increasing and
    each lie in (0, n_layers); anything else is refused (ValueError) rather
    than silently falling back to one stage."""
    if n_layers < 1:
        raise ValueError("n_layers must be >= 1")
    if n_stages < 1 or n_stages > n_layers:
        raise ValueError("n_stages must be in [1, n_layers]")
    if cuts is None:
        cuts = [s * n_layers // n_stages for s in range(1, n_stages)]
    cuts = list(cuts)
    if len(cuts) != n_stages - 1:
        raise ValueError("need exactly n_stages - 1 cuts")
    prev = 0
    for c in cuts:
        if not (0 < c < n_layers) or c <= prev:
            raise ValueError("cuts must be strictly increasing inside (0, n_layers)")
        prev = c
    return [0, *cuts, n_layers]


def stage_plan_counts(n_layers: int, counts) -> list[int]:
    """Per-stage layer counts (each >= 1, summing to n_layers) -> fence."""
    counts = list(counts)
    if not counts or any(c < 1 for c in counts) or sum(counts) != n_layers:
        raise ValueError("counts must be >= 1 and sum to n_layers")
    fence = [0]
    for c in counts:
        fence.append(fence[-1] + c)
    return stage_plan(n_layers, len(counts), fence[1:-1])


def stage_of(fence, layer: int) -> int:
    """The stage whose range [fence[s], fence[s+1]) holds ``layer``."""
    if not (0 <= layer < fence[-1]):
        raise ValueError("layer outside the model")
    for s in range(len(fence) - 1):
        if fence[s] <= layer < fence[s + 1]:
            return s
    raise AssertionError("unreachable")
