"""Staged decode on the GPU: bit identity of staged vs unstaged runs (every N and
cut set of the tiny model), the deferred readback ring, liveness counters,
and teacher-forced logits against the float64 oracle."""
import itertools
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from oracle.decoder import Decoder
from oracle.plan import stage_plan

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    from layer_pipeline_stage_amd import runtime, lps
    lps.load()
    assert torch.cuda.is_available(), "GPU tests need a visible ROCm GPU"
    return runtime


def _cut_sets(L):
    for r in range(L):
        for cuts in itertools.combinations(range(1, L), r):
            yield list(cuts)


def _check_against_oracle(model, res, tol_rel):
    """Teacher forcing: the oracle is fed the GPU's token sequence; logits per
    step within tol_rel * max|oracle logits|; the GPU's argmax must be the
    oracle's, unless the oracle's top two logits are closer than the tolerance
    (a certified near tie, counted)."""
    dec = Decoder(model)
    _, am, lg = dec.greedy([], 0, feed=res.fed)
    near = 0
    for i, (a, b) in enumerate(zip(res.logits, lg)):
        tol = tol_rel * np.abs(b).max()
        assert np.max(np.abs(a - b)) <= tol, (i, np.max(np.abs(a - b)), tol)
        if res.argmax[i] != am[i]:
            top2 = np.sort(b)[-2:]
            assert top2[1] - top2[0] <= 2 * tol and b[res.argmax[i]] >= top2[1] - 2 * tol
            near += 1
    return near


def test_tiny_unstaged_matches_oracle(rt):
    cfg = synth.TINY
    m = synth.make_tiny(cfg)
    dd = rt.DeviceDecoder(m)
    res = dd.run_tokens(m["prompt"], cfg.steps)
    assert len(res.logits) == cfg.prompt + cfg.steps
    assert _check_against_oracle(m, res, 1e-5) == 0
    dd.close()


def test_tiny_staged_equals_unstaged_every_cut_set(rt):
    """memra pp docs (header; PendingLogits) and ninfer Verification: staged
    output bit-identical to one stage, for all 8 cut sets of the 4-layer model,
    with the liveness counters proving the staged walk and the slots ran."""
    from layer_pipeline_stage_amd import lps
    cfg = synth.TINY
    m = synth.make_tiny(cfg)
    dd = rt.DeviceDecoder(m)
    ref = dd.run_tokens(m["prompt"], cfg.steps)
    steps = cfg.prompt + cfg.steps
    for cuts in _cut_sets(cfg.n_layers):
        n = len(cuts) + 1
        dd.set_fence(stage_plan(cfg.n_layers, n, cuts))
        dd.reset()
        lps.lps_counters_reset()
        got = dd.run_tokens(m["prompt"], cfg.steps)
        c = lps.counters()
        assert c["stage_walks"] == n * steps
        assert c["boundary_sends"] == c["boundary_recvs"] == (n - 1) * steps
        assert c["drains"] == steps
        assert got.fed == ref.fed and got.argmax == ref.argmax
        assert all(np.array_equal(a, b) for a, b in zip(got.logits, ref.logits)), cuts
    dd.close()


def test_tiny_n4_deferred_per_step_identity_and_soak(rt):
    """Same model at context 32 -> 96: N = 4 (cuts 1, 2, 3) on one device, the
    deferred readback ring letting the host run ahead, 64 greedy steps;
    per-step bit identity against N = 1, repeated 20 times (memra's one-device
    pipelined arm failed 7 of 20 such soaks from a race; here the stages share
    no mutable state beyond the event-ordered slots)."""
    cfg = synth.TINY_N4
    m = synth.make_tiny(cfg)
    dd = rt.DeviceDecoder(m)
    ref = dd.run_tokens(m["prompt"], cfg.steps)
    assert len(ref.logits) == 96
    assert _check_against_oracle(m, ref, 1e-5) == 0
    dd.set_fence(stage_plan(4, 4, [1, 2, 3]))
    for run in range(20):
        dd.reset()
        got = dd.run_tokens(m["prompt"], cfg.steps)
        assert got.argmax == ref.argmax, run
        for i, (a, b) in enumerate(zip(got.logits, ref.logits)):
            assert np.array_equal(a, b), (run, i)
    dd.close()


def test_single_stream_seam_equals_per_stage_streams(rt):
    """The same-stream seam (every stage on one stream, the boundary as plain
    copies) gives the same bits as one stream per stage."""
    cfg = replace(synth.TINY, prompt=5, steps=6)
    m = synth.make_tiny(cfg)
    a = rt.DeviceDecoder(m, fence=[0, 1, 3, 4])
    b = rt.DeviceDecoder(m, fence=[0, 1, 3, 4], streams="single")
    ra = a.run_tokens(m["prompt"], cfg.steps)
    rb = b.run_tokens(m["prompt"], cfg.steps)
    assert ra.argmax == rb.argmax
    assert all(np.array_equal(x, y) for x, y in zip(ra.logits, rb.logits))
    a.close()
    b.close()


def _same(a, b):
    assert a.fed == b.fed and a.argmax == b.argmax
    assert len(a.logits) == len(b.logits)
    for i, (x, y) in enumerate(zip(a.logits, b.logits)):
        assert np.array_equal(x, y), i


def test_graph_replay_equals_eager_tiny(rt):
    """ninfer pipeline stages, How it works (StageLink) and Verification (graphs
    and eager byte-identical): the whole step captured once and replayed, the
    position and next id advanced on the device, gives the eager walk's bits,
    for one stage and for two and three stages on the same-stream seam."""
    cfg = synth.TINY
    m = synth.make_tiny(cfg)
    for fence in ([0, 4], [0, 2, 4], [0, 1, 3, 4]):
        dd = rt.DeviceDecoder(m, fence=fence, streams="single")
        ref = dd.run_tokens(m["prompt"], cfg.steps)
        dd.reset()
        got = dd.run_tokens_graph(m["prompt"], cfg.steps)
        _same(got, ref)
        dd.close()


def test_graph_replay_marks_every_few_steps(rt):
    """The replay loop marks one replay in mark_every (and the last); every step's
    row is still drained after a mark that covers it: the same ids and logits for
    a mark every replay, every second, every third, and more than the ring holds."""
    cfg = replace(synth.TINY, prompt=3, steps=13)
    m = synth.make_tiny(cfg)
    dd = rt.DeviceDecoder(m, fence=[0, 2, 4], streams="single")
    ref = dd.run_tokens(m["prompt"], cfg.steps)
    for me in (1, 2, 3, 9):
        dd.reset()
        _same(dd.run_tokens_graph(m["prompt"], cfg.steps, mark_every=me), ref)
    dd.close()


def test_graph_replay_per_stage_streams_and_eager_after(rt):
    """N = 4 on four streams: the capture forks the later stage streams in
    through the boundary events and joins them back; replays equal the eager
    walk at context 32 -> 96, twice with a fresh capture, and an eager walk
    after the graphs (boundary slots reused across the capture) still gives
    the same bits; teacher forcing through the graph too."""
    cfg = synth.TINY_N4
    m = synth.make_tiny(cfg)
    dd = rt.DeviceDecoder(m, fence=[0, 1, 2, 3, 4])
    ref = dd.run_tokens(m["prompt"], cfg.steps)
    for _ in range(2):
        dd.reset()
        _same(dd.run_tokens_graph(m["prompt"], cfg.steps), ref)
    dd.reset()
    _same(dd.run_tokens(m["prompt"], cfg.steps), ref)
    dd.reset()
    feed = ref.fed[:40]
    got = dd.run_tokens_graph([], feed=feed)
    assert got.fed == feed and got.argmax == ref.argmax[:40]
    assert all(np.array_equal(x, y) for x, y in zip(got.logits, ref.logits[:40]))
    dd.close()


def test_graph_replay_bf16(rt):
    """The device-position walk on bf16 weights and bf16 caches equals the
    eager walk bit for bit (the RoPE table holds the by-value launch's own
    f32 cos / sin values)."""
    cfg = replace(synth.TINY, wdtype="bf16", kvdtype="bf16", prompt=4, steps=8)
    m = synth.make_tiny(cfg)
    dd = rt.DeviceDecoder(m, fence=[0, 2, 4])
    ref = dd.run_tokens(m["prompt"], cfg.steps)
    dd.reset()
    _same(dd.run_tokens_graph(m["prompt"], cfg.steps), ref)
    dd.close()


def test_invalid_fence_refused(rt):
    from layer_pipeline_stage_amd import lps
    m = synth.make_tiny(replace(synth.TINY, prompt=2, steps=1))
    dd = rt.DeviceDecoder(m)
    for bad in ([0, 2, 2, 4], [0, 5], [1, 2, 4], [0, 3, 2, 4]):
        with pytest.raises(lps.LpsError):
            dd.set_fence(bad)
    dd.close()


def test_moe_decode_small_matches_oracle(rt):
    from oracle.moe import MoEStack
    cfg = synth.MoEConfig("moe-gpu-small", n_layers=2, d=512, n_experts=16, top_k=4, ff=128,
                          remote_from=8, prefill_T=0, steps=6)
    m = synth.make_moe(cfg)
    st = rt.DeviceMoEStack(m)
    got = st.decode(m["x_in"])
    ref_st = MoEStack(m)
    for t in range(cfg.steps):
        traces = []
        ref = ref_st.forward(m["x_in"][t], traces=traces)
        tol = 2e-3 * np.abs(ref).max()
        assert np.max(np.abs(got[t] - ref)) <= tol


def test_moe_prefill_small_matches_oracle_and_pieces(rt):
    """Grouped-GEMM prefill over a ragged chunk (T = 300: tiles of 128 rows plus
    a tail, per-expert groups of uneven size): every row within the bf16
    tolerance of the oracle (which rounds the GEMM inputs to bf16 the same
    way), and the 8-piece FP16 transfer bit-identical to the 1-piece one."""
    from oracle.moe import MoEStack
    cfg = synth.MoEConfig("moe-gpu-pf", n_layers=2, d=512, n_experts=16, top_k=4, ff=128,
                          remote_from=8, prefill_T=300, steps=0)
    from layer_pipeline_stage_amd import lps
    m = synth.make_moe(cfg)
    st = rt.DeviceMoEStack(m)
    X = m["x_prefill"]
    lps.lps_counters_reset()
    got8 = st.prefill(X, n_pieces=8)
    c = lps.counters()
    # both halves of the transfer ran in 8 pieces per layer (activations, then sums)
    assert c["act_pieces"] == 8 * cfg.n_layers and c["pieces"] == 8 * cfg.n_layers, c
    got1 = st.prefill(X, n_pieces=1)
    assert np.array_equal(got8, got1)
    # one stream for both halves, and more pieces than rows in a tiny chunk
    got_one_stream = st.prefill(X, n_pieces=8, remote_stream=st.stream)
    assert np.array_equal(got8, got_one_stream)
    lps.lps_counters_reset()
    tiny = st.prefill(X[:5], n_pieces=8)
    assert lps.counters()["act_pieces"] == 5 * cfg.n_layers
    assert np.array_equal(tiny, st.prefill(X[:5], n_pieces=1))
    ref = MoEStack(m).forward(X, prefill=True, n_pieces=8)
    tol = 2e-3 * np.abs(ref).max()
    err = np.abs(got8 - ref).max(axis=1)
    assert np.all(err <= tol), (int(np.argmax(err)), float(err.max()), tol)
    # a single row through the chunk path equals its decode (one-token) path within tolerance
    dec = st.decode(X[:3])
    ref_dec = MoEStack(m).forward(X[:3])
    assert np.max(np.abs(dec - ref_dec)) <= 2e-3 * np.abs(ref_dec).max()


def test_moe_prefill_wide_rows_tile_router(rt):
    """Rows too wide for the matrix-core router's LDS tile (d = 2560: 16 f32 rows
    exceed it) take the 8-token tile router; the chunk still matches the oracle
    row by row, with a ragged last tile (T = 45)."""
    from oracle.moe import MoEStack
    cfg = synth.MoEConfig("moe-gpu-wide", n_layers=1, d=2560, n_experts=16, top_k=4, ff=128,
                          remote_from=8, prefill_T=45, steps=0)
    m = synth.make_moe(cfg)
    st = rt.DeviceMoEStack(m)
    X = m["x_prefill"]
    got = st.prefill(X, n_pieces=3)
    ref = MoEStack(m).forward(X, prefill=True, n_pieces=3)
    tol = 2e-3 * np.abs(ref).max()
    err = np.abs(got - ref).max(axis=1)
    assert np.all(err <= tol), (int(np.argmax(err)), float(err.max()), tol)


def test_moe_prefill_top12_matches_oracle(rt):
    """More selections per token than one pair of 16-byte index words holds (k = 12
    of 16 experts): the grouping takes four words per token; rows match the oracle
    and 8 pieces equal one."""
    from oracle.moe import MoEStack
    cfg = synth.MoEConfig("moe-gpu-k12", n_layers=1, d=512, n_experts=16, top_k=12, ff=128,
                          remote_from=8, prefill_T=700, steps=0)
    m = synth.make_moe(cfg)
    st = rt.DeviceMoEStack(m)
    X = m["x_prefill"]
    got8 = st.prefill(X, n_pieces=8)
    assert np.array_equal(got8, st.prefill(X, n_pieces=1))
    ref = MoEStack(m).forward(X, prefill=True, n_pieces=8)
    tol = 2e-3 * np.abs(ref).max()
    err = np.abs(got8 - ref).max(axis=1)
    assert np.all(err <= tol), (int(np.argmax(err)), float(err.max()), tol)


@pytest.mark.parametrize("remote_from", [0, 16])
def test_moe_prefill_all_remote_or_all_local(rt, remote_from):
    """Every routed expert on the remote half (the local tile list holds only the
    shared expert) or none of them (the remote list is empty and its launches find
    no tile): rows still match the oracle and 8 pieces equal one."""
    from oracle.moe import MoEStack
    cfg = synth.MoEConfig("moe-gpu-edge", n_layers=1, d=512, n_experts=16, top_k=4, ff=128,
                          remote_from=remote_from, prefill_T=260, steps=0)
    m = synth.make_moe(cfg)
    st = rt.DeviceMoEStack(m)
    X = m["x_prefill"]
    got8 = st.prefill(X, n_pieces=8)
    assert np.array_equal(got8, st.prefill(X, n_pieces=1))
    ref = MoEStack(m).forward(X, prefill=True, n_pieces=8)
    tol = 2e-3 * np.abs(ref).max()
    err = np.abs(got8 - ref).max(axis=1)
    assert np.all(err <= tol), (int(np.argmax(err)), float(err.max()), tol)


def test_moe_stack_stages_equal_one_stage_decode_and_prefill(rt):
    """Every cut set of a 4-layer MoE stack, on per-stage streams: decode rows and a
    ragged prefill chunk equal the one-stage run bit for bit, with the walks and
    boundary crossings counted (the staged walk is not vacuous)."""
    from layer_pipeline_stage_amd import lps
    cfg = synth.MoEConfig("moe-stages", n_layers=4, d=512, n_experts=16, top_k=4, ff=128,
                          remote_from=8, prefill_T=200, steps=5)
    m = synth.make_moe(cfg)
    st = rt.DeviceMoEStack(m)
    ref = st.decode(m["x_in"])
    ref_pf = st.prefill(m["x_prefill"], n_pieces=8)
    for cuts in ([1], [2], [3], [1, 2], [1, 3], [2, 3], [1, 2, 3]):
        fence = [0, *cuts, 4]
        n = len(fence) - 1
        st.set_fence(fence)
        lps.lps_counters_reset()
        got = st.decode(m["x_in"])
        c = lps.counters()
        assert c["stage_walks"] == n * cfg.steps and c["boundary_sends"] == (n - 1) * cfg.steps
        assert np.array_equal(got, ref), fence
        got_pf = st.prefill(m["x_prefill"], n_pieces=8)
        assert np.array_equal(got_pf, ref_pf), fence
    st.close()


@pytest.mark.parametrize("wdtype", ["f32", "bf16"])
def test_stage_walk_with_folded_hop_equals_walk_then_hop(rt, wdtype):
    """lps_stage_forward_dpos_hop (the hop's copy folded into the stage's last
    launch) leaves the same bits as lps_stage_forward_dpos followed by
    lps_boundary_hop: the stage's x, the slot of the step (the other slot left
    alone) and the receiver's x, with one send and one receive counted; a step out
    of order and a boundary of another width are refused before anything runs."""
    import ctypes as C
    from layer_pipeline_stage_amd import lps
    from layer_pipeline_stage_amd.runtime import ptr
    cfg = replace(synth.TINY, wdtype=wdtype, kvdtype=wdtype, prompt=2, steps=2)
    m = synth.make_tiny(cfg)
    dd = rt.DeviceDecoder(m, fence=[0, 2, 4], streams="single")
    dd.g_state.copy_(torch.tensor([5, 0, 0, 0], dtype=torch.int32))
    x0 = torch.from_numpy(np.random.default_rng(3).standard_normal(cfg.d).astype(np.float32))
    st = torch.cuda.current_stream().cuda_stream
    fence = lps.i32_array([0, 2, 4])

    def boundary(n):
        s0 = torch.full((n,), float("nan"), device="cuda")
        s1 = torch.full((n,), float("nan"), device="cuda")
        b = C.c_void_p()
        lps.lps_boundary_create(n, ptr(s0), ptr(s1), C.byref(b))
        return b, s0, s1

    xa, xb = x0.cuda(), x0.cuda()
    ya = torch.full((cfg.d,), float("nan"), device="cuda")
    yb = ya.clone()
    ba, sa0, sa1 = boundary(cfg.d)
    bb, sb0, sb1 = boundary(cfg.d)
    lps.lps_stage_forward_dpos(dd.model, fence, 2, 0, ptr(xa), ptr(dd.g_state), ptr(dd.scratch[0]),
                               dd.scratch_bytes, st)
    lps.lps_boundary_hop(ba, ptr(xa), ptr(ya), 0, st)
    torch.cuda.synchronize()
    c0 = lps.counters()
    lps.lps_stage_forward_dpos_hop(dd.model, fence, 2, 0, ptr(xb), ptr(dd.g_state),
                                   ptr(dd.scratch[0]), dd.scratch_bytes, bb, ptr(yb), 0, st)
    torch.cuda.synchronize()
    c1 = lps.counters()
    assert torch.equal(xa, xb) and torch.equal(ya, yb) and torch.equal(sa0, sb0)
    assert torch.equal(sb0, xb) and torch.equal(yb, xb) and not torch.equal(xb, x0.cuda())
    assert torch.isnan(sb1).all()
    assert c1["boundary_sends"] - c0["boundary_sends"] == 1
    assert c1["boundary_recvs"] - c0["boundary_recvs"] == 1
    assert c1["stage_walks"] - c0["stage_walks"] == 1
    before = xb.clone()
    with pytest.raises(lps.LpsError) as e:           # step 0 again
        lps.lps_stage_forward_dpos_hop(dd.model, fence, 2, 0, ptr(xb), ptr(dd.g_state),
                                       ptr(dd.scratch[0]), dd.scratch_bytes, bb, ptr(yb), 0, st)
    assert e.value.code == lps.LPS_ESTATE
    bw, _, _ = boundary(cfg.d + 8)
    with pytest.raises(lps.LpsError) as e:           # rows of another width
        lps.lps_stage_forward_dpos_hop(dd.model, fence, 2, 0, ptr(xb), ptr(dd.g_state),
                                       ptr(dd.scratch[0]), dd.scratch_bytes, bw, ptr(yb), 0, st)
    assert e.value.code == lps.LPS_EINVAL
    torch.cuda.synchronize()
    assert torch.equal(xb, before)
    for b in (ba, bb, bw):
        lps.lps_boundary_destroy(b)
    dd.close()


def test_moe_stage_walk_with_folded_hop_equals_walk_then_hop(rt):
    """The folded hop on an MoE stage (its last launch is the down projections and
    the ordered combine): the same bits as lps_stage_forward + lps_boundary_hop in
    x, the step's slot and the receiver's x."""
    import ctypes as C
    from layer_pipeline_stage_amd import lps
    from layer_pipeline_stage_amd.runtime import ptr
    cfg = synth.MoEConfig("moe-hop", n_layers=2, d=512, n_experts=16, top_k=4, ff=128, remote_from=8,
                          prefill_T=0, steps=1)
    m = synth.make_moe(cfg)
    stk = rt.DeviceMoEStack(m, fence=[0, 1, 2], streams="single")
    st = torch.cuda.current_stream().cuda_stream
    fence = lps.i32_array([0, 1, 2])
    pos = torch.zeros(4, dtype=torch.int32, device="cuda")
    outs = []
    for folded in (False, True):
        s0 = torch.full((cfg.d,), float("nan"), device="cuda")
        s1 = torch.full((cfg.d,), float("nan"), device="cuda")
        b = C.c_void_p()
        lps.lps_boundary_create(cfg.d, ptr(s0), ptr(s1), C.byref(b))
        x = torch.from_numpy(m["x_in"][0].copy()).cuda()
        y = torch.full((cfg.d,), float("nan"), device="cuda")
        if folded:
            lps.lps_stage_forward_dpos_hop(stk.model, fence, 2, 0, ptr(x), ptr(pos), ptr(stk.scratch[0]),
                                           stk.scratch_bytes, b, ptr(y), 0, st)
        else:
            lps.lps_stage_forward(stk.model, fence, 2, 0, ptr(x), 0, ptr(stk.scratch[0]),
                                  stk.scratch_bytes, st)
            lps.lps_boundary_hop(b, ptr(x), ptr(y), 0, st)
        torch.cuda.synchronize()
        outs.append((x.cpu(), y.cpu(), s0.cpu(), s1.cpu()))
        lps.lps_boundary_destroy(b)
    (xa, ya, sa, _), (xb, yb, sb, sb1) = outs
    assert torch.equal(xa, xb) and torch.equal(ya, yb) and torch.equal(sa, sb)
    assert torch.equal(sb, xb) and torch.isnan(sb1).all()
    stk.close()
