"""Pins of oracle.moe: top-k by exhaustive search, routing special cases, the
FP16 pieces and aliased-combine invariants of strata PR #3648, closed forms."""
import itertools
from dataclasses import replace

import numpy as np
import pytest

import synth
from oracle.moe import (softmax, top_k, piece_bounds, f16_pieces_to_f32, combine, moe_layer,
                        MoEStack, expert)
from oracle.numerics import to_f32

SMALL = synth.MoEConfig("moe-small", n_layers=2, d=64, n_experts=8, top_k=3, ff=32,
                        remote_from=4, prefill_T=37, steps=3)


@pytest.mark.parametrize("k", [1, 2, 3])
def test_top_k_brute_force(k):
    rng = np.random.default_rng(k)
    r = rng.standard_normal((50, 8))
    pi = softmax(r)
    idx, w = top_k(pi, k)
    for t in range(50):
        best = max(itertools.combinations(range(8), k), key=lambda S: sum(pi[t, list(S)]))
        assert set(idx[t]) == set(best)
        assert list(idx[t]) == sorted(best, key=lambda e: -pi[t, e])
        assert abs(w[t].sum() - 1) < 1e-15
        assert np.allclose(w[t], pi[t, idx[t]] / pi[t, idx[t]].sum())


def test_softmax_and_ties():
    r = np.array([[0.0, 1.0, 1.0, 0.5, 1.0, -2.0]])
    pi = softmax(r)
    assert abs(pi.sum() - 1) < 1e-15
    assert np.allclose(softmax(r + 123.0), pi, rtol=1e-14)
    idx, w = top_k(pi, 2)
    assert list(idx[0]) == [1, 2]                   # equal logits: the lower ids first
    idx, w = top_k(softmax(np.zeros((1, 8))), 3)    # zero router -> experts 0,1,2, 1/3 each
    assert list(idx[0]) == [0, 1, 2] and np.allclose(w, 1 / 3)


@pytest.mark.parametrize("T", [0, 1, 7, 8, 9, 37, 16384])
def test_piece_bounds_cover_rows(T):
    b = piece_bounds(T, 8)
    assert b[0][0] == 0 and b[-1][1] == T
    assert all(b[i][1] == b[i + 1][0] for i in range(7))
    if T == 1:
        assert [hi - lo for lo, hi in b] == [0] * 7 + [1]


def test_pieces_equal_one_piece_bit_for_bit():
    rng = np.random.default_rng(9)
    rem = (rng.standard_normal((37, 64)) * np.exp(rng.uniform(-8, 8, (37, 1)))).astype(np.float32)
    one = f16_pieces_to_f32(rem, 1)
    for P in (2, 3, 8, 37):
        buf = np.full_like(rem, np.nan)               # poisoned, as a reused buffer would be
        assert np.array_equal(f16_pieces_to_f32(rem, P, out=buf), one)
    # f16 -> f32 is exact: widening and narrowing again is the identity
    assert np.array_equal(one.astype(np.float16).astype(np.float32), one)


def test_aliased_combine_equals_separate():
    rng = np.random.default_rng(10)
    x, sh, lo, r = (rng.standard_normal((5, 16)).astype(np.float32) for _ in range(4))
    ref = combine(x, sh, lo, r)
    lo2 = lo.copy()
    assert np.array_equal(combine(x, sh, lo2, r, out=lo2), ref)
    r2 = r.copy()
    assert np.array_equal(combine(x, sh, lo, r2, out=r2), ref)


def test_identical_experts_reduce_to_one_expert():
    """With every routed expert equal, the normalised weights sum to 1 so the
    routed part is one expert's output: y = shared(h) + e(h) (no FP16 half)."""
    cfg = replace(SMALL, remote_from=SMALL.n_experts)
    m = synth.make_moe(cfg)
    L = m["layers"][0]
    L["w_gu_e"][:] = L["w_gu_e"][0]
    L["w_d_e"][:] = L["w_d_e"][0]
    x = m["x_prefill"][:5]
    out = moe_layer(x, L, cfg)
    xx = x.astype(np.float64)
    h = xx / np.sqrt(np.mean(xx ** 2, axis=1, keepdims=True) + cfg.eps)
    y = to_f32(expert(h, L["w_gu_s"], L["w_d_s"], cfg.ff)).astype(np.float64) + \
        to_f32(expert(h, L["w_gu_e"][0], L["w_d_e"][0], cfg.ff)).astype(np.float64)
    ref = to_f32(xx + y)
    assert np.max(np.abs(out - ref)) <= 4 * np.spacing(np.abs(ref).max())


def test_remote_half_goes_through_f16():
    """Moving the split point changes only the rounding of the moved terms, and
    never by more than f16 precision of the remote sum."""
    m = synth.make_moe(SMALL)
    L = m["layers"][0]
    x = m["x_prefill"][:9]
    a, b = {}, {}
    out_half = moe_layer(x, L, SMALL, trace=a)
    out_none = moe_layer(x, L, replace(SMALL, remote_from=SMALL.n_experts), trace=b)
    assert np.array_equal(a["idx"], b["idx"])
    tol = np.abs(a["remote"]).max() * 2 ** -10 + 4 * np.spacing(np.abs(out_none).max())
    assert np.max(np.abs(out_half - out_none)) <= tol
    assert np.array_equal(a["r32"], a["remote"].astype(np.float32).astype(np.float16).astype(np.float32))


def test_moe_pieces_and_rows_independent():
    m = synth.make_moe(SMALL)
    st = MoEStack(m)
    X = m["x_prefill"]
    one = st.forward(X, prefill=True, n_pieces=1)
    eight = st.forward(X, prefill=True, n_pieces=8)
    assert np.array_equal(one, eight)
    rows = [0, 5, 36]
    assert np.array_equal(st.forward(X[rows], prefill=True, n_pieces=8), one[rows])
    # decode of one row equals its single-row forward
    assert np.array_equal(st.forward(X[3]), st.forward(X[3:4])[0])


def test_forced_routing_is_used():
    m = synth.make_moe(SMALL)
    L = m["layers"][0]
    x = m["x_prefill"][:4]
    tr = {}
    moe_layer(x, L, SMALL, trace=tr)
    forced = tr["idx"][:, ::-1].copy()                    # same set, other order
    tr2 = {}
    out2 = moe_layer(x, L, SMALL, forced_idx=forced, trace=tr2)
    assert np.array_equal(tr2["idx"], forced)
    assert np.allclose(out2, moe_layer(x, L, SMALL), rtol=0, atol=1e-6)
