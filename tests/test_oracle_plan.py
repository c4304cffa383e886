"""Pins of oracle.plan: the pages' printed fences, the closed form, brute force."""
import itertools
import os

import pytest

from oracle.plan import stage_plan, stage_plan_counts, stage_of

GOLD = os.path.join(os.path.dirname(__file__), "golden", "stage_plan.txt")


def _golden():
    for line in open(GOLD):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        head, arg, fence = (p.strip() for p in line.split("|"))
        kind, L, N = head.split()
        yield kind, int(L), int(N), [int(a) for a in arg.split()] if arg != "-" else None, \
            [int(f) for f in fence.split()]


@pytest.mark.parametrize("row", list(_golden()))
def test_golden_fences(row):
    kind, L, N, arg, fence = row
    if kind == "even":
        assert stage_plan(L, N) == fence
    elif kind == "counts":
        assert stage_plan_counts(L, arg) == fence
    else:
        assert stage_plan(L, N, arg) == fence


@pytest.mark.parametrize("L", range(1, 11))
def test_every_cut_set_brute_force(L):
    """All 2^(L-1) cut sets: the fence covers every layer exactly once, stages
    are contiguous and non-empty, and stage_of agrees with counting the cuts at
    or below the layer."""
    for r in range(0, L):
        for cuts in itertools.combinations(range(1, L), r):
            fence = stage_plan(L, r + 1, list(cuts))
            assert fence[0] == 0 and fence[-1] == L and len(fence) == r + 2
            owners = []
            for s in range(r + 1):
                assert fence[s + 1] > fence[s]
                owners += [s] * (fence[s + 1] - fence[s])
            assert owners == [sum(1 for c in cuts if c <= l) for l in range(L)]
            assert [stage_of(fence, l) for l in range(L)] == owners


@pytest.mark.parametrize("L,N", [(L, N) for L in range(1, 13) for N in range(1, L + 1)])
def test_even_split_closed_form(L, N):
    f = stage_plan(L, N)
    assert f == [s * L // N for s in range(N)] + [L]
    sizes = [f[s + 1] - f[s] for s in range(N)]
    assert max(sizes) - min(sizes) <= 1


@pytest.mark.parametrize("L,N,cuts", [
    (4, 0, None), (4, 5, None), (0, 1, None),
    (4, 2, [0]), (4, 2, [4]), (4, 3, [2, 2]), (4, 3, [3, 1]), (4, 3, [1]), (4, 2, [1, 2]),
    (4, 2, [-1]),
])
def test_invalid_plans_refused(L, N, cuts):
    with pytest.raises(ValueError):
        stage_plan(L, N, cuts)


def test_invalid_counts_and_layers():
    for counts in ([], [0, 4], [2, 3], [5, -1]):
        with pytest.raises(ValueError):
            stage_plan_counts(4, counts)
    with pytest.raises(ValueError):
        stage_of([0, 2, 4], 4)
    with pytest.raises(ValueError):
        stage_of([0, 2, 4], -1)
