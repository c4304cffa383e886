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


# ---- memory-balancing split (ninfer "Multi-GPU: layer pipeline stages", How it works
# and Verification; the plan loading test: the head stage gets fewer layers, a device
# with twice the memory more) ----------------------------------------------------

from oracle.plan import solve_stage_plan


def test_solver_identical_stages_split_evenly_closed_form():
    # 8 layers of 10 fixed bytes and 3 KV bytes per group over 4 stages of 1000 free:
    # two layers per stage hold (1000 - 20) // 6 = 163 groups; any uneven split puts
    # 3 layers somewhere: (1000 - 30) // 9 = 107
    fence, P = solve_stage_plan([1000] * 4, [0] * 4, [10] * 8, [3] * 8, 4, 10**9)
    assert fence == [0, 2, 4, 6, 8] and P == 163


def test_solver_twice_the_memory_gets_more_layers():
    fence, P = solve_stage_plan([2000, 1000], [0, 0], [10] * 9, [2] * 9, 2, 10**9)
    counts = [fence[1] - fence[0], fence[2] - fence[1]]
    assert counts[0] > counts[1]
    # hand check: 6 / 3 -> min((2000-60)//12, (1000-30)//6) = min(161, 161) = 161
    assert fence == [0, 6, 9] and P == 161


def test_solver_head_stage_gets_fewer_layers():
    # the last stage also holds the head (overhead); equal devices
    fence, P = solve_stage_plan([1000, 1000], [0, 400], [10] * 8, [2] * 8, 2, 10**9)
    assert fence[1] - fence[0] > fence[2] - fence[1]
    # 5 / 3: min((1000-50)//10, (1000-400-30)//6) = min(95, 95) = 95
    assert fence == [0, 5, 8] and P == 95


def test_solver_tie_goes_to_least_full_then_smallest_fence():
    # layers 0..3 fixed 0, kv [1, 1, 1, 1]: [0,2,4] gives P = 50 on both stages;
    # [0,1,4] / [0,3,4] give min(100, 33) = 33
    fence, P = solve_stage_plan([100, 100], [0, 0], [0, 0, 0, 0], [1, 1, 1, 1], 2, 10**9)
    assert fence == [0, 2, 4] and P == 50
    # no KV at all: every split holds max_groups; fill = fixed / free decides:
    # fixed [30, 10, 10, 30] -> [0,2,4] (40 / 40) beats [0,1,4] (30 / 50) and [0,3,4]
    fence, P = solve_stage_plan([100, 100], [0, 0], [30, 10, 10, 30], [0, 0, 0, 0], 2, 7)
    assert fence == [0, 2, 4] and P == 7
    # symmetric fills: [0,1,3] and [0,2,3] both fill 20/100 at worst -> smallest fence
    fence, _ = solve_stage_plan([100, 100], [0, 0], [10, 10, 10], [0, 0, 0], 2, 5)
    assert fence == [0, 1, 3]


def test_solver_single_stage_and_infeasible():
    fence, P = solve_stage_plan([100], [10], [20, 30], [5, 5], 1, 10**9)
    assert fence == [0, 2] and P == (100 - 10 - 50) // 10
    with pytest.raises(ValueError):
        solve_stage_plan([50, 50], [0, 0], [40, 40, 40], [1, 1, 1], 2, 10)   # 80 > 50 somewhere
    with pytest.raises(ValueError):
        solve_stage_plan([50], [0, 0], [1], [1], 1, 10)                       # lengths
