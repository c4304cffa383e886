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


def _stage_groups(free, overhead, fixed, kv, a, b, s, max_groups):
    """Page groups stage s can hold for layers [a, b): floor((free - overhead -
    fixed bytes) / KV bytes per group), capped at max_groups; -1 when the stage
    cannot even hold its layers' fixed bytes; max_groups when it holds no KV."""
    need = overhead[s] + sum(fixed[a:b])
    if need > free[s]:
        return -1
    per = sum(kv[a:b])
    if per == 0:
        return max_groups
    return min(max_groups, (free[s] - need) // per)


def solve_stage_plan(free, overhead, fixed, kv, n_stages: int, max_groups: int):
    """Memory-balancing split, by enumeration of every fence (the brute-force
    partition oracle of ninfer "Multi-GPU: layer pipeline stages", How it works
    and Verification).

    Inputs are bytes: free[s] and overhead[s] per stage (device), fixed[l] (the
    layer's weights and per-slot state) and kv[l] (its KV bytes per page group)
    per layer.  Reading of "maximum page groups every stage can hold, then
    least-full stage": every stage must hold the same number P of page groups of
    its own layers' KV; the split maximises P; among the splits reaching it, the
    one whose fullest stage, (overhead + fixed + P * kv) / free, is least full;
    remaining ties go to the lexicographically smallest fence.  Returns
    (fence, P); ValueError when no split holds even P = 0."""
    from fractions import Fraction
    from itertools import combinations
    L = len(fixed)
    if len(kv) != L or len(free) != n_stages or len(overhead) != n_stages:
        raise ValueError("array lengths")
    if not (1 <= n_stages <= L) or max_groups < 0:
        raise ValueError("n_stages must lie in [1, n_layers]; max_groups >= 0")
    if any(f <= 0 for f in free) or any(x < 0 for x in (*overhead, *fixed, *kv)):
        raise ValueError("free > 0 and sizes >= 0")
    best = None
    for cuts in combinations(range(1, L), n_stages - 1):
        fence = (0, *cuts, L)
        groups = [_stage_groups(free, overhead, fixed, kv, fence[s], fence[s + 1], s, max_groups)
                  for s in range(n_stages)]
        P = min(groups)
        if P < 0:
            continue
        fill = max(Fraction(overhead[s] + sum(fixed[fence[s]:fence[s + 1]])
                            + P * sum(kv[fence[s]:fence[s + 1]]), free[s]) for s in range(n_stages))
        key = (-P, fill, fence)
        if best is None or key < best[0]:
            best = (key, list(fence), P)
    if best is None:
        raise ValueError("no split holds the layers")
    return best[1], best[2]
