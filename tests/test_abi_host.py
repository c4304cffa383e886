"""The C-ABI library loads on a machine without a GPU, exports every symbol
include/lps.h declares, and its host-only logic (stage plan, validation that
runs before anything is enqueued) behaves as specified."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from oracle.plan import stage_plan as oracle_plan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from layer_pipeline_stage_amd import lps
    lps.load()
    return lps


def declared_functions():
    src = open(os.path.join(ROOT, "include", "lps.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(lps_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 35
    lib = C.CDLL(L.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding wraps exactly the declared set
    assert set(L.SIGS) == set(names)


def test_stage_plan_matches_oracle_everywhere(L):
    import itertools
    for nl in range(1, 9):
        for n in range(1, nl + 1):
            assert L.stage_plan(nl, n) == oracle_plan(nl, n)
        for r in range(nl):
            for cuts in itertools.combinations(range(1, nl), r):
                f = L.stage_plan(nl, r + 1, list(cuts))
                assert f == oracle_plan(nl, r + 1, list(cuts))
                assert [L.stage_of(f, l) for l in range(nl)] == \
                    [sum(c <= l for c in cuts) for l in range(nl)]


@pytest.mark.parametrize("nl,n,cuts", [
    (4, 0, None), (4, 5, None), (0, 1, None), (4, 2, [0]), (4, 2, [4]), (4, 3, [2, 2]),
    (4, 3, [3, 1]), (4, 3, [1]), (4, 2, [1, 2]), (4, 2, [-1]),
])
def test_invalid_plans_refused_with_text(L, nl, n, cuts):
    with pytest.raises(L.LpsError) as e:
        L.stage_plan(nl, n, cuts)
    assert e.value.code == L.LPS_EINVAL
    assert "lps_stage_plan" in str(e.value)


def test_counts_and_stage_of_errors(L):
    assert L.stage_plan_counts(64, [30, 34]) == [0, 30, 64]
    for counts in ([0, 4], [2, 3], [5, -1]):
        with pytest.raises(L.LpsError):
            L.stage_plan_counts(4, counts)
    with pytest.raises(L.LpsError) as e:
        L.stage_of([0, 2, 4], 4)
    assert e.value.code == L.LPS_ERANGE
    with pytest.raises(L.LpsError):
        L.stage_of([0, 2, 2], 1)


def test_validation_before_enqueue(L):
    """Bad descriptors and arguments are refused before any HIP call, so the
    refusals are observable without a GPU."""
    d = L.LayerDesc()
    d.d, d.nq, d.nkv, d.hd, d.ff = 256, 4, 3, 64, 704          # nq % nkv != 0
    d.wdtype, d.kvdtype, d.ctx_max = 0, 0, 16
    with pytest.raises(L.LpsError) as e:
        L.lps_layer_forward(C.byref(d), 16, 0, 16, 1 << 20, None)
    assert e.value.code == L.LPS_EUNSUP and "lps_layer_forward" in str(e.value)
    d.nkv, d.hd = 2, 96                                         # head dim not built
    with pytest.raises(L.LpsError) as e:
        L.lps_layer_forward(C.byref(d), 16, 0, 16, 1 << 20, None)
    assert e.value.code == L.LPS_EUNSUP
    d.hd = 64
    with pytest.raises(L.LpsError) as e:                        # null weights
        L.lps_layer_forward(C.byref(d), 16, 0, 16, 1 << 20, None)
    assert e.value.code == L.LPS_EINVAL
    assert L.lps_layer_scratch_bytes(C.byref(d)) == 0           # invalid desc -> 0
    with pytest.raises(L.LpsError):
        L.lps_gemv(2, 16, 16, 8, 100, 16, None, 0.0, 16, 0, None)   # K % 32 for MXFP4
    with pytest.raises(L.LpsError):
        L.lps_gemv(1, 16, None, 7, 64, 16, None, 0.0, 16, 2, None)  # SwiGLU needs even N
    with pytest.raises(L.LpsError):
        L.lps_attention_decode(4, 2, 64, 0, 16, 16, 8, 9, 16, 16, 16, 1 << 20, None)  # n_rows > ctx
    with pytest.raises(L.LpsError):
        L.lps_moe_combine(16, 16, 16, 16, 16, 16, 4, 64, 0, None, None)    # 0 pieces
    with pytest.raises(L.LpsError) as e:
        L.lps_hbm_stream_read(16, 24, 16, None)                 # bytes not a multiple of 16
    assert e.value.code == L.LPS_EINVAL
    with pytest.raises(L.LpsError):
        L.lps_hbm_stream_read(8, 32, 16, None)                  # unaligned source
    assert L.lps_attention_scratch_bytes(32, 8, 128, 4224) > 0

    assert L.lps_attention_scratch_bytes(3, 2, 128, 10) == 0


def test_error_text_is_thread_local_and_cleared(L):
    with pytest.raises(L.LpsError):
        L.stage_plan(4, 9)
    assert "n_stages" in L.last_error()
    L.stage_plan(4, 2)
    assert L.last_error() == ""


def test_stage_solver_matches_the_brute_force_oracle(L):
    """lps_stage_solve (exact DP) against the oracle's enumeration of every fence,
    on seeded random instances that include zero-KV layers, head overheads, tight
    memory and max_groups caps; infeasible instances must be refused by both."""
    from oracle.plan import solve_stage_plan
    rng = np.random.default_rng(20261202)
    checked = 0
    for _ in range(400):
        nl = int(rng.integers(1, 10))
        ns = int(rng.integers(1, min(nl, 4) + 1))
        fixed = [int(v) for v in rng.integers(0, 50, nl)]
        kv = [int(v) * int(rng.random() < 0.8) for v in rng.integers(0, 8, nl)]
        free = [int(v) for v in rng.integers(20, 400, ns)]
        over = [int(v) for v in rng.integers(0, 60, ns)]
        mg = int(rng.choice([0, 3, 50, 10**6]))
        try:
            want = solve_stage_plan(free, over, fixed, kv, ns, mg)
        except ValueError:
            with pytest.raises(L.LpsError) as e:
                L.stage_solve(free, over, fixed, kv, ns, mg)
            assert e.value.code == L.LPS_EUNSUP
            continue
        assert L.stage_solve(free, over, fixed, kv, ns, mg) == (want[0], want[1]), (
            free, over, fixed, kv, ns, mg)
        checked += 1
    assert checked > 150


def test_stage_solver_refuses_bad_arguments(L):
    with pytest.raises(L.LpsError) as e:
        L.stage_solve([100], [0], [1, 1], [1, 1], 3, 10)          # more stages than layers
    assert e.value.code == L.LPS_EINVAL
    with pytest.raises(L.LpsError):
        L.stage_solve([0, 100], [0, 0], [1, 1], [1, 1], 2, 10)    # a stage with no free bytes
    with pytest.raises(L.LpsError):
        L.stage_solve([100, 100], [0, 0], [1, -1], [1, 1], 2, 10)  # negative size


def test_memory_balanced_fence_for_the_dense_slice():
    """The dense 8B-class slice (8 layers, bf16) over four equal 288 GB devices:
    the embedding sits on stage 0 and the head on stage 3 (equal sizes), so the
    split is even; giving stage 0 half the memory moves layers off it."""
    from layer_pipeline_stage_amd.runtime import memory_balanced_fence
    geo = dict(n_layers=8, d=4096, nq=32, nkv=8, hd=128, ff=14336, vocab=32000, wdtype="bf16",
               kvdtype="bf16")
    fence, groups = memory_balanced_fence(n_stages=4, free_bytes=[288 << 30] * 4, **geo)
    assert fence == [0, 2, 4, 6, 8] and groups > 0
    fence2, groups2 = memory_balanced_fence(n_stages=4, free_bytes=[144 << 30] + [288 << 30] * 3, **geo)
    assert fence2[1] - fence2[0] < 2 and groups2 < groups


def test_rope_table_matches_the_oracle_rotation(L):
    """lps_rope_table (the device-position walk's cos / sin table) against the
    oracle's rotation applied to unit vectors: rotating e_i at position p
    yields cos(p theta_i) at i and sin(p theta_i) at i + hd/2.  The table is
    the f64 values rounded once to f32, so it is within one f32 ulp."""
    from oracle.decoder import rope
    for hd, base, n_pos in ((64, 10000.0, 300), (128, 500000.0, 4200)):
        half = hd // 2
        tab = L.rope_table(hd, base, n_pos)
        assert tab.shape == (n_pos, half, 2) and tab.dtype == np.float32
        eye = np.eye(half, hd)
        for p in list(range(0, n_pos, 97)) + [n_pos - 1]:
            r = rope(eye, p, base)
            want = np.stack([r[np.arange(half), np.arange(half)],
                             r[np.arange(half), half + np.arange(half)]], axis=-1)
            ulp = np.spacing(np.abs(want).astype(np.float32))
            assert np.all(np.abs(tab[p].astype(np.float64) - want) <= ulp), (hd, p)
        assert np.array_equal(tab[0, :, 0], np.ones(half, np.float32))
        assert np.array_equal(tab[0, :, 1], np.zeros(half, np.float32))


def test_graph_and_device_state_entry_points_refuse_bad_arguments(L):
    """The whole-pass graph entry points validate on the host first."""
    for args in ((0, 1e4, 4), (63, 1e4, 4), (64, 1e4, 0), (64, 0.0, 4)):
        with pytest.raises(L.LpsError) as e:
            L.lps_rope_table(*args, 16)
        assert e.value.code == L.LPS_EINVAL
    with pytest.raises(L.LpsError):
        L.lps_rope_table(64, 1e4, 4, None)
    bad_adv = [
        (None, 8, 16, 16, None, 0, None, 0, None, 0, None, None),   # null state
        (16, 0, 16, 16, None, 0, None, 0, None, 0, None, None),     # pos_limit < 1
        (16, 8, 16, 16, None, 3, None, 0, None, 0, None, None),     # feed ids without feed
        (16, 8, 16, 16, None, 0, None, 4, None, 0, None, None),     # history without tok_hist
        (16, 8, 16, 16, None, 0, 16, 4, None, 0, 16, None),         # logits history, no logits
    ]
    for a in bad_adv:
        with pytest.raises(L.LpsError) as e:
            L.lps_step_advance(*a)
        assert e.value.code == L.LPS_EINVAL, a
    # lps_step_finish: (h, x, logits, state, pos_limit, feed, n_feed, tok_hist,
    # logits_hist, hist_cap, embed, embed_dtype, x_next, tok_cur, ring, scratch,
    # bytes, stream)
    hd = L.HeadDesc()
    hd.d, hd.vocab, hd.wdtype, hd.eps, hd.g_out, hd.w_lm = 256, 100, L.LPS_F32, 1e-6, 16, 16
    ok = [C.byref(hd), 16, 16, 16, 8, None, 0, None, None, 0, 16, L.LPS_F32, 16, None, None, 16,
          1 << 20, None]
    ring0, ring_empty = L.HostRing(), L.HostRing()
    ring0.logits, ring0.tok, ring0.slots = 16, 16, 0
    ring_empty.logits, ring_empty.tok, ring_empty.slots = None, None, 4
    bad_fin = [
        (0, None),              # null head
        (3, None),              # null state
        (4, 0),                 # pos_limit < 1
        (6, 3),                 # feed ids without feed
        (9, 4),                 # history without tok_hist
        (10, None),             # null embedding table
        (11, L.LPS_MXFP4),      # embedding dtype
        (12, None),             # null x_next
        (14, C.byref(ring0)),   # a host ring of no slots
        (14, C.byref(ring_empty)),  # a host ring with neither row
        (16, 16),               # scratch below the head's
    ]
    for i, v in bad_fin:
        a = list(ok)
        a[i] = v
        with pytest.raises(L.LpsError) as e:
            L.lps_step_finish(*a)
        assert e.value.code == L.LPS_EINVAL, (i, v)
    with pytest.raises(L.LpsError) as e:
        L.lps_graph_begin(None)                      # the null stream is not captured
    assert e.value.code == L.LPS_EINVAL
    with pytest.raises(L.LpsError) as e:
        L.lps_graph_end(None, None, 0, None)         # null out
    assert e.value.code == L.LPS_EINVAL
    with pytest.raises(L.LpsError):
        L.lps_graph_launch(None, None)
    assert L.lps_graph_destroy(None) == 0
    fence = L.i32_array([0, 1])
    with pytest.raises(L.LpsError) as e:
        L.lps_stage_forward_dpos(None, fence, 1, 0, 16, 16, 16, 1 << 20, None)
    assert e.value.code == L.LPS_EINVAL
    with pytest.raises(L.LpsError) as e:
        L.lps_stage_forward_dpos_hop(None, fence, 1, 0, 16, 16, 16, 1 << 20, 16, 16, 0, None)
    assert e.value.code == L.LPS_EINVAL
    with pytest.raises(L.LpsError) as e:
        L.lps_stage_prefill(None, fence, 1, 0, 16, 4, 0, 16, 1 << 20, None)
    assert e.value.code == L.LPS_EINVAL
    assert L.lps_prefill_scratch_bytes(None, 4) == 0
    for args in ((16, 1, 10, 8, 16, 0, 16), (16, 2, 10, 8, 16, 4, 16), (None, 1, 10, 8, 16, 4, 16)):
        with pytest.raises(L.LpsError) as e:
            L.lps_embed_rows(*args, None)           # T 0, wdtype MXFP4, null table
        assert e.value.code == L.LPS_EINVAL


def test_prefill_refuses_unsupported_layers_before_enqueue(L):
    """A model handle over valid decode layers that the prefill cannot run
    (f32 weights, a ragged ff) is refused by lps_stage_prefill with the layer
    named, before any HIP call."""
    import ctypes
    d = L.LayerDesc()
    d.d, d.nq, d.nkv, d.hd, d.ff = 256, 4, 2, 64, 704
    d.wdtype, d.kvdtype, d.ctx_max = L.LPS_BF16, L.LPS_BF16, 64
    d.eps, d.rope_base = 1e-6, 1e4
    for k in ("g_attn", "g_ffn", "w_qkv", "w_o", "w_gu", "w_d", "k_cache", "v_cache", "rope_cs"):
        setattr(d, k, 256)
    h = ctypes.c_void_p()
    L.lps_model_create(ctypes.byref(d), 1, ctypes.byref(h))
    try:
        assert L.lps_prefill_scratch_bytes(h, 8) > 0
        fence = L.i32_array([0, 1])
        with pytest.raises(L.LpsError) as e:        # ff 704 is not a multiple of 128
            L.lps_stage_prefill(h, fence, 1, 0, 256, 8, 0, 256, 1 << 30, None)
        assert e.value.code == L.LPS_EUNSUP and "layer 0" in str(e.value)
        with pytest.raises(L.LpsError) as e:        # rows past the cache
            L.lps_stage_prefill(h, fence, 1, 0, 256, 60, 8, 256, 1 << 30, None)
        assert e.value.code in (L.LPS_EUNSUP, L.LPS_ERANGE)
        # the walk with a folded hop: no boundary, no receiver, a misaligned receiver
        for b, xo in ((None, 256), (256, None), (256, 260)):
            with pytest.raises(L.LpsError) as e:
                L.lps_stage_forward_dpos_hop(h, fence, 1, 0, 256, 256, 256, 1 << 30, b, xo, 0, None)
            assert e.value.code == L.LPS_EINVAL, (b, xo)
    finally:
        L.lps_model_destroy(h)


def test_cache_tile_layouts_match_the_documented_offsets():
    """bf16 caches: K element (head j, row r, dim e) sits at
    ((j * rows/16 + r/16) * hd/8 + e/8) * 128 + (r % 16) * 8 + e % 8, V at
    ((j * rows/16 + r/16) * hd + e) * 16 + r % 16; the helpers round-trip
    for numpy arrays and torch tensors."""
    import torch
    from layer_pipeline_stage_amd import layout
    nkv, rows, hd = 3, 48, 16
    x = np.arange(nkv * rows * hd).reshape(nkv, rows, hd)
    kt, vt = layout.k_to_tiles(x), layout.v_to_tiles(x)
    kf, vf = kt.reshape(-1), vt.reshape(-1)
    for j, r, e in ((0, 0, 0), (1, 17, 3), (2, 47, 15), (2, 31, 8), (0, 5, 9)):
        tile = j * (rows // 16) + r // 16
        assert kf[(tile * (hd // 8) + e // 8) * 128 + (r % 16) * 8 + e % 8] == x[j, r, e]
        assert vf[(tile * hd + e) * 16 + r % 16] == x[j, r, e]
    assert np.array_equal(layout.k_from_tiles(kt), x)
    assert np.array_equal(layout.v_from_tiles(vt), x)
    xt = torch.from_numpy(x)
    assert np.array_equal(layout.k_to_tiles(xt).numpy(), kt)
    assert np.array_equal(layout.v_to_tiles(xt).numpy(), vt)
    assert np.array_equal(layout.k_from_tiles(layout.k_to_tiles(xt)).numpy(), x)
    assert np.array_equal(layout.v_from_tiles(layout.v_to_tiles(xt)).numpy(), x)


def test_chunks_past_32_bit_offsets_are_refused_before_enqueue(L):
    """The prefill kernels address every operand with 32-bit byte offsets: a chunk
    whose largest operand reaches 2 GiB is refused (LPS_EUNSUP) with the size in
    the text, before any HIP call.  Dense: T = 140,000 rows of f32 QKV at the 8B
    slice's width; MoE: T = 40,000 at d 2048, top 8 (the [T, 8, d] f32 expert
    outputs)."""
    import ctypes
    d = L.LayerDesc()
    d.d, d.nq, d.nkv, d.hd, d.ff = 4096, 32, 8, 128, 14336
    d.wdtype, d.kvdtype, d.ctx_max = L.LPS_BF16, L.LPS_BF16, 1 << 18
    d.eps, d.rope_base = 1e-6, 1e4
    for k in ("g_attn", "g_ffn", "w_qkv", "w_o", "w_gu", "w_d", "k_cache", "v_cache", "rope_cs"):
        setattr(d, k, 256)
    h = ctypes.c_void_p()
    L.lps_model_create(ctypes.byref(d), 1, ctypes.byref(h))
    try:
        fence = L.i32_array([0, 1])
        with pytest.raises(L.LpsError) as e:
            L.lps_stage_prefill(h, fence, 1, 0, 256, 140000, 0, 256, 1 << 62, None)
        assert e.value.code == L.LPS_EUNSUP and "2 GiB" in str(e.value)
    finally:
        L.lps_model_destroy(h)
    m = L.MoEDesc()
    m.d, m.n_experts, m.top_k, m.ff, m.remote_from, m.eps = 2048, 64, 8, 1024, 32, 1e-6
    for k in ("g_ffn", "w_r", "w_gu_e", "w_d_e", "w_gu_s", "w_d_s"):
        setattr(m, k, 256)
    with pytest.raises(L.LpsError) as e:
        L.lps_moe_prefill(ctypes.byref(m), 256, 40000, 8, 256, 1 << 62, None, None)
    assert e.value.code == L.LPS_EUNSUP and "2 GiB" in str(e.value)
    # the workload's own chunk (16,384 rows) stays below the limit: it fails later,
    # on the scratch size, not on the offsets
    with pytest.raises(L.LpsError) as e:
        L.lps_moe_prefill(ctypes.byref(m), 256, 16384, 8, 256, 16, None, None)
    assert e.value.code == L.LPS_EINVAL and "scratch" in str(e.value)


def test_pending_tokens_refuse_a_second_use(L):
    """A pending readback handle is a token that one wait or drop consumes; a
    token the library never issued (or one already consumed) is refused with
    LPS_ESTATE, before any HIP call."""
    for fn in (L.lps_pending_wait, L.lps_pending_drop):
        with pytest.raises(L.LpsError) as e:
            fn((7 << 32) | 3)
        assert e.value.code == L.LPS_ESTATE and "already waited or dropped" in str(e.value)
    with pytest.raises(L.LpsError) as e:
        L.lps_pending_order((1 << 32) | 1, None)
    assert e.value.code == L.LPS_ESTATE


@pytest.mark.parametrize("ring", [1, 2, 3, 4, 8])
def test_replay_mark_schedule_drains_every_step_after_its_mark(ring):
    """The graph replay loop's marking (runtime.mark_schedule), run as the loop runs
    it: every step is drained once, after a mark at or after it that was already
    launched, before its host-ring row is reused; each mark is waited once and no
    mark is stored over one that was never waited."""
    from layer_pipeline_stage_amd.runtime import mark_schedule
    for total in range(1, 30):
        for every in (1, 2, 3, 5, 64):
            marked, cover = mark_schedule(total, ring, every)
            pend, waited, launched, drained = [None] * ring, set(), -1, []

            def drain(i):
                j = cover(i)
                assert marked(j) and i <= j <= launched < i + ring, (total, every, i, j, launched)
                if pend[j % ring] is not None:
                    assert pend[j % ring] == j
                    waited.add(j)
                    pend[j % ring] = None
                assert j in waited
                drained.append(i)

            for i in range(total):
                if i >= ring:
                    drain(i - ring)
                launched = i
                if marked(i):
                    assert pend[i % ring] is None
                    pend[i % ring] = i
            for i in range(max(0, total - ring), total):
                drain(i)
            assert drained == list(range(total)) and all(p is None for p in pend)
            assert waited == {i for i in range(total) if marked(i)}
