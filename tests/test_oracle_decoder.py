"""Pins of oracle.decoder: special cases, brute force on tiny shapes, and the
invariants the pages fix (staged == unstaged, padded == unpadded)."""
import itertools
import math
from dataclasses import replace

import numpy as np
import pytest
from scipy.special import expit

import synth
from oracle.decoder import Decoder, rmsnorm, rope, attend, silu, matvec_grouped
from oracle.numerics import widen_weight
from oracle.plan import stage_plan

SMALL8 = synth.DecoderConfig("small8", n_layers=8, d=64, nq=4, nkv=2, hd=16, ff=96, vocab=64,
                             wdtype="f32", kvdtype="f32", prompt=3, steps=2)
SMALL_PAD = synth.DecoderConfig("small-pad", n_layers=2, d=128, nq=6, nkv=3, hd=32, ff=192,
                                vocab=0, wdtype="mxfp4", kvdtype="bf16", prefix=16, steps=3,
                                nq_real=4, nkv_real=2, ff_real=160)


# ---- RMSNorm ------------------------------------------------------------------
def test_rmsnorm_special_cases():
    g = np.linspace(0.5, 2, 16)
    assert np.array_equal(rmsnorm(np.zeros(16), g, 1e-6), np.zeros(16))
    c = -3.0
    y = rmsnorm(np.full(16, c), g, 1e-6)
    assert np.allclose(y, np.sign(c) * abs(c) / math.sqrt(c * c + 1e-6) * g, rtol=1e-15)
    x = np.random.default_rng(0).standard_normal(16)
    assert np.allclose(rmsnorm(7.5 * x, g, 0.0), rmsnorm(x, g, 0.0), rtol=1e-14)
    # unit gain, eps 0: the output has RMS exactly 1
    assert abs(np.sqrt(np.mean(rmsnorm(x, np.ones(16), 0.0) ** 2)) - 1) < 1e-15


# ---- RoPE -------------------------------------------------------------------
def test_rope_against_complex_rotation():
    """Each pair (i, i + hd/2) is the complex number u_i + j u_{i+hd/2} multiplied
    by e^{j p theta_i}, theta_i = base^(-2i/hd)."""
    rng = np.random.default_rng(1)
    u = rng.standard_normal((3, 8))
    p, base = 37, 10000.0
    z = u[:, :4] + 1j * u[:, 4:]
    th = np.array([base ** (-2 * i / 8) for i in range(4)])
    w = z * np.exp(1j * p * th)
    r = rope(u, p, base)
    assert np.allclose(r[:, :4], w.real, atol=1e-13) and np.allclose(r[:, 4:], w.imag, atol=1e-13)


def test_rope_invariants():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((2, 64)), rng.standard_normal((2, 64))
    assert np.array_equal(rope(q, 0, 1e4), q)
    assert np.array_equal(rope(np.zeros((2, 64)), 123, 1e4), np.zeros((2, 64)))
    assert np.allclose(np.linalg.norm(rope(q, 999, 1e4), axis=1), np.linalg.norm(q, axis=1))
    d1 = np.sum(rope(q, 10, 1e4) * rope(k, 3, 1e4), axis=1)
    d2 = np.sum(rope(q, 107, 1e4) * rope(k, 100, 1e4), axis=1)
    assert np.allclose(d1, d2, rtol=1e-12)


# ---- attention -----------------------------------------------------------------
def _attend_brute(q, K, V):
    nq, hd = len(q), len(q[0])
    nkv, n = len(K), len(K[0])
    G = nq // nkv
    out = []
    for h in range(nq):
        g = h // G
        s = [math.fsum(q[h][i] * K[g][j][i] for i in range(hd)) / math.sqrt(hd) for j in range(n)]
        m = max(s)
        e = [math.exp(v - m) for v in s]
        z = math.fsum(e)
        out.append([math.fsum(e[j] / z * V[g][j][i] for j in range(n)) for i in range(hd)])
    return np.array(out)


@pytest.mark.parametrize("n", [1, 2, 3, 6])
@pytest.mark.parametrize("nq,nkv", [(2, 1), (4, 2), (6, 3)])
def test_attention_brute_force(n, nq, nkv):
    rng = np.random.default_rng(n * 10 + nq)
    q = rng.standard_normal((nq, 4))
    K, V = rng.standard_normal((nkv, n, 4)), rng.standard_normal((nkv, n, 4))
    assert np.allclose(attend(q, K, V), _attend_brute(q.tolist(), K.tolist(), V.tolist()),
                       rtol=1e-13, atol=1e-14)


def test_attention_special_cases():
    rng = np.random.default_rng(4)
    K, V = rng.standard_normal((2, 5, 8)), rng.standard_normal((2, 5, 8))
    q = rng.standard_normal((4, 8))
    # one visible row: the output is that row of V (per kv group h // 2)
    o1 = attend(q, K[:, :1], V[:, :1])
    assert np.allclose(o1, V[[0, 0, 1, 1], 0], rtol=1e-15)
    # zero query: uniform weights -> mean of V
    o0 = attend(np.zeros((4, 8)), K, V)
    assert np.allclose(o0, V.mean(axis=1)[[0, 0, 1, 1]], rtol=1e-14)
    # V = 0 -> 0 (the dummy-head trace of the TP3 padding plan)
    assert np.array_equal(attend(q, K, np.zeros_like(V)), np.zeros((4, 8)))
    # GQA: changing kv head 1 changes only q heads 2, 3
    K2 = K.copy()
    K2[1] += rng.standard_normal(K2[1].shape)
    a, b = attend(q, K, V), attend(q, K2, V)
    assert np.array_equal(a[:2], b[:2]) and not np.allclose(a[2:], b[2:])


def test_silu_and_matvec():
    z = np.linspace(-30, 30, 1001)
    assert np.allclose(silu(z), z * expit(z), rtol=1e-14, atol=1e-300)
    assert silu(np.array([0.0]))[0] == 0.0
    rng = np.random.default_rng(5)
    W, h = rng.standard_normal((7, 96)), rng.standard_normal(96)
    brute = np.array([math.fsum(W[i, j] * h[j] for j in range(96)) for i in range(7)])
    assert np.allclose(W @ h, brute, rtol=1e-14)
    assert np.allclose(matvec_grouped(W, h), brute, rtol=1e-14)
    # zero groups appended at the end of K change nothing, bit for bit
    W2 = np.concatenate([W, np.zeros((7, 64))], axis=1)
    h2 = np.concatenate([h, rng.standard_normal(64)])
    assert np.array_equal(matvec_grouped(W2, h2), matvec_grouped(W, h))


# ---- a whole layer -------------------------------------------------------------
def test_first_token_layer_closed_form():
    """At p = 0 with an empty cache the attention sees one row, so every q head
    returns its kv group's v and RoPE plays no part:
    x1 = f32(x + Wo [v_{h//G}]_h), out = f32(x1 + Wd (silu(Wg h2) * Wu h2))."""
    cfg = synth.TINY
    m = synth.make_tiny(cfg)
    dec = Decoder(m)
    x = dec.embed(int(m["prompt"][0]))
    out = dec.layer(0, x, 0)
    L = m["layers"][0]
    W = lambda n: widen_weight(L[n], "f32")
    xx = x.astype(np.float64)
    h = xx / np.sqrt(np.mean(xx ** 2) + cfg.eps)
    qkv = W("w_qkv") @ h
    off = (cfg.nq + cfg.nkv) * cfg.hd
    v = qkv[off:].reshape(cfg.nkv, cfg.hd)
    G = cfg.nq // cfg.nkv
    o = np.concatenate([v[hh // G] for hh in range(cfg.nq)])
    x1 = (xx + W("w_o") @ o).astype(np.float32).astype(np.float64)
    h2 = x1 / np.sqrt(np.mean(x1 ** 2) + cfg.eps)
    g, u = W("w_gu")[:cfg.ff] @ h2, W("w_gu")[cfg.ff:] @ h2
    ref = (x1 + W("w_d") @ (g * expit(g) * u)).astype(np.float32)
    # both round the residual to f32 twice; a different f64 summation order may
    # move a rounding by one f32 step at the scale of the vector
    assert np.max(np.abs(out - ref)) <= 4 * np.spacing(np.abs(ref).max())


def test_zero_projections_make_identity_layer():
    m = synth.make_tiny()
    for L in m["layers"]:
        L["w_o"] = np.zeros_like(L["w_o"])
        L["w_d"] = np.zeros_like(L["w_d"])
    dec = Decoder(m)
    x = dec.embed(5)
    assert np.array_equal(dec.walk(x, 0), x)


def test_causal_rows_beyond_position_ignored():
    m = synth.make_tiny()
    a, b = Decoder(m), Decoder(m)
    for K in b.K:
        K[:, 3:] = 1e3                         # garbage in rows the step must not read
    for p, t in enumerate(m["prompt"][:3]):
        la, _ = a.step(int(t), p)
        lb, _ = b.step(int(t), p)
        assert np.array_equal(la, lb)


# ---- pages' invariants -----------------------------------------------------------
def _all_cut_sets(L):
    for r in range(L):
        for cuts in itertools.combinations(range(1, L), r):
            yield list(cuts)


def test_staged_equals_unstaged_tiny_every_cut_set():
    """memra pp module docs (header, M2 increment 3) and ninfer Verification:
    staged output is bit-identical to unstaged, for every cut set."""
    cfg = replace(synth.TINY, prompt=4, steps=3)
    m = synth.make_tiny(cfg)
    ref = Decoder(m)
    fed, am, lg = ref.greedy(m["prompt"], cfg.steps)
    for cuts in _all_cut_sets(cfg.n_layers):
        fence = stage_plan(cfg.n_layers, len(cuts) + 1, cuts)
        d = Decoder(m)
        f2, a2, l2 = d.greedy(m["prompt"], cfg.steps, fence=fence)
        assert f2 == fed and a2 == am
        assert all(np.array_equal(x, y) for x, y in zip(lg, l2))
        n = len(cuts) + 1
        assert d.counters["stage_walks"] == n * len(fed)
        assert d.counters["boundary_crossings"] == (n - 1) * len(fed)


def test_staged_equals_unstaged_eight_layers_all_128_cut_sets():
    m = synth.make_tiny(SMALL8)
    ref = Decoder(m)
    _, am, lg = ref.greedy(m["prompt"], SMALL8.steps)
    count = 0
    for cuts in _all_cut_sets(8):
        d = Decoder(m)
        _, a2, l2 = d.greedy(m["prompt"], SMALL8.steps, fence=stage_plan(8, len(cuts) + 1, cuts))
        assert a2 == am and all(np.array_equal(x, y) for x, y in zip(lg, l2))
        count += 1
    assert count == 128


def test_bf16_slot_would_break_identity():
    """Planted mistake, on the CPU: a boundary that rounds the hidden to bf16
    instead of copying f32 must be caught by the staged == unstaged check."""
    from oracle import decoder as dmod
    cfg = replace(synth.TINY, prompt=3, steps=1)
    m = synth.make_tiny(cfg)
    _, _, ref = Decoder(m).greedy(m["prompt"], 1)

    class Lossy(dmod.Decoder):
        def walk(self, x32, p, fence=None):
            x = np.asarray(x32, np.float32)
            for s in range(len(fence) - 1):
                for l in range(fence[s], fence[s + 1]):
                    x = self.layer(l, x, p)
                if s < len(fence) - 2:
                    u = x.view(np.uint32) & np.uint32(0xFFFF0000)
                    x = u.view(np.float32)
            return x
    _, _, got = Lossy(m).greedy(m["prompt"], 1, fence=[0, 2, 4])
    assert not all(np.array_equal(a, b) for a, b in zip(ref, got))


def test_padded_equals_unpadded_bit_for_bit():
    """TP3 zero-padded dummy heads plan: zero dummy heads and FFN rows/columns at
    the end of every padded axis leave the model's output unchanged."""
    pm = synth.make_pad(SMALL_PAD, padded=True)
    um = synth.make_pad(SMALL_PAD, padded=False)
    assert pm["layers"][0]["w_qkv"][0].shape[0] == SMALL_PAD.qkv_rows
    assert um["layers"][0]["w_qkv"][0].shape[0] == SMALL_PAD.real().qkv_rows
    dp, du = Decoder(pm), Decoder(um)
    p0 = SMALL_PAD.prefix
    for t in range(SMALL_PAD.steps):
        a = dp.step(pm["x_in"][t], p0 + t)
        b = du.step(um["x_in"][t], p0 + t)
        assert np.array_equal(a, b)
    # the dummy kv heads' cache rows hold zeros (RoPE may give a signed zero)
    from oracle.numerics import bf16_to_f64
    for K in dp.K:
        assert np.all(bf16_to_f64(K[SMALL_PAD.nkv_real:]) == 0)


def test_pad_generator_geometry_matches_page():
    """Shape self-test of the padded MXFP4 layout against the TP3 plan's tables."""
    import os
    rows = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "pad_geometry.txt")):
        line = line.split("#")[0].strip()
        if line:
            k, a, b = line.split()
            rows[k] = (int(a), int(b))
    P, U = synth.PAD, synth.PAD.real()
    assert rows["num_attention_heads"] == (U.nq, P.nq)
    assert rows["num_key_value_heads"] == (U.nkv, P.nkv)
    assert rows["intermediate_size"] == (U.ff, P.ff)
    assert rows["kv_proj_rows"] == (U.nkv * U.hd, P.nkv * P.hd)
    assert rows["o_proj_packed_cols"] == (U.nq * U.hd // 2, P.nq * P.hd // 2)
    assert rows["o_proj_scale_cols"] == (U.nq * U.hd // 32, P.nq * P.hd // 32)
    assert rows["down_proj_packed_cols"] == (U.ff // 2, P.ff // 2)
    assert rows["down_proj_scale_cols"] == (U.ff // 32, P.ff // 32)
    assert P.ff % 128 == 64            # the K tail the decode GEMM must handle
    # a reduced-size build of the real generator keeps the fill bytes of the plan
    pm = synth.make_pad(SMALL_PAD, padded=True)
    wo_c, wo_s = pm["layers"][0]["w_o"]
    k_real = SMALL_PAD.nq_real * SMALL_PAD.hd
    assert not np.any(wo_c[:, k_real // 2:]) and np.all(wo_s[:, k_real // 32:] == 0x7F)
    wd_c, wd_s = pm["layers"][0]["w_d"]
    assert not np.any(wd_c[:, SMALL_PAD.ff_real // 2:]) and np.all(wd_s[:, SMALL_PAD.ff_real // 32:] == 0x7F)
    assert not np.any(wd_s == 0xFF)


def test_pad_pair_matches_separate_builds():
    pm, um = synth.make_pad_pair(SMALL_PAD)
    pm2 = synth.make_pad(SMALL_PAD, padded=True)
    um2 = synth.make_pad(SMALL_PAD, padded=False)
    for a, b in ((pm, pm2), (um, um2)):
        assert a["cfg"] == b["cfg"]
        for La, Lb in zip(a["layers"], b["layers"]):
            for k in La:
                va, vb = La[k], Lb[k]
                if isinstance(va, tuple):
                    assert all(np.array_equal(x, y) for x, y in zip(va, vb))
                else:
                    assert np.array_equal(va, vb)


def test_mxfp4_row_blocks_equal_whole_matrix():
    pm = synth.make_pad(SMALL_PAD, padded=True)
    a, b = Decoder(pm, weight_cache=True), Decoder(pm, weight_cache=False)
    x = pm["x_in"][0]
    h = rmsnorm(x.astype(np.float64), pm["layers"][0]["g_attn"], SMALL_PAD.eps)
    assert np.array_equal(a.mv(0, "w_gu", h), b._mv_mxfp4_rows(0, "w_gu", h, rows=7))


# ---- chunked prefill (matrix form) -------------------------------------------------
PF_BF16 = synth.DecoderConfig("pf-bf16", n_layers=3, d=64, nq=4, nkv=2, hd=16, ff=96, vocab=64,
                              wdtype="bf16", kvdtype="bf16", prefix=5, prompt=8, steps=0)


@pytest.mark.parametrize("cfg", [replace(SMALL8, prefix=4, prompt=7, steps=0), PF_BF16])
def test_prefill_matrix_form_equals_decode_steps(cfg):
    """With exact operands (act=None) the whole-chunk matrix form — all K/V rows
    of the chunk stored first, then a causal mask — reproduces the decode steps
    fed one id at a time: same last logits, same cache rows."""
    m = synth.make_tiny(cfg) if cfg.vocab == 1024 else synth.make_dense(cfg)
    a, b = Decoder(m), Decoder(m)
    lg, am, X = a.prefill(m["prompt"], act=None)
    _, dam, dlg = b.greedy(m["prompt"], 0)
    assert am == dam[-1]
    assert np.max(np.abs(lg - dlg[-1])) <= 1e-12 * np.abs(dlg[-1]).max()
    for l in range(cfg.n_layers):
        assert np.array_equal(a.K[l], b.K[l]) and np.array_equal(a.V[l], b.V[l])


def test_prefill_chunks_equal_one_chunk_and_stages_equal_one_stage():
    """Splitting the prompt into chunks (each from its own position) or the
    layers into stages changes nothing: rows interact only through the cache,
    causally."""
    m = synth.make_dense(PF_BF16)
    ids = m["prompt"]
    ref = Decoder(m)
    lg, am, X = ref.prefill(ids)
    for chunks in ([3, 5], [1, 1, 6], [7, 1]):
        d = Decoder(m)
        p = PF_BF16.prefix
        for n in chunks:
            lgc, amc, Xc = d.prefill(ids[:n], p0=p)
            ids, p = ids[n:], p + n
        assert amc == am and np.max(np.abs(lgc - lg)) <= 1e-12 * np.abs(lg).max(), chunks
        ids = m["prompt"]
    for fence in ([0, 1, 3], [0, 1, 2, 3]):
        d = Decoder(m)
        lgs, ams, Xs = d.prefill(ids, fence=fence)
        assert np.array_equal(lgs, lg) and np.array_equal(Xs, X)


def test_prefill_pin_catches_an_off_by_one_mask(monkeypatch):
    """The decode comparison is not vacuous: a prefill whose row t also sees
    row p0+t+1 (a planted off-by-one in the oracle) misses it by far."""
    import oracle.decoder as od
    m = synth.make_dense(PF_BF16)
    _, _, dlg = Decoder(m).greedy(m["prompt"], 0)
    real = od.causal_attend

    def leaky(Q, K, V, p0):
        T = Q.shape[0]
        n = K.shape[1]
        out = np.empty_like(Q)
        for t in range(T):
            vis = min(n, p0 + t + 2)
            out[t] = real(Q[t:t + 1], K[:, :vis], V[:, :vis], vis - 1)[0]
        return out

    monkeypatch.setattr(od, "causal_attend", leaky)
    lg, _, _ = Decoder(m).prefill(m["prompt"], act=None)
    assert np.max(np.abs(lg - dlg[-1])) > 1e-3 * np.abs(dlg[-1]).max()


def test_bf16_activation_rounding():
    """bf16_act rounds to nearest even through f32, as the f32 -> bf16 convert
    of the matrix-core operands does (torch's conversion as the reference)."""
    import torch
    from oracle.decoder import bf16_act
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(4096) * 10.0 ** rng.integers(-6, 6, 4096),
                        [1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 2 ** -130]])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_act(x), want)
    assert bf16_act(np.array([1.0 + 2 ** -8]))[0] == 1.0           # tie -> even
    assert bf16_act(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6


def test_causal_attend_closed_forms():
    """causal_attend against hand-solvable cases: (a) K = 0 makes every weight
    e^0 = 1, so each row's output is the plain mean of the V rows it sees (the
    GQA map h // G picks the kv head); (b) one query against two keys, the
    second one's score -q0: the output is (v0 + e^(-q0) v1) / (1 + e^(-q0))."""
    from oracle.decoder import causal_attend
    rng = np.random.default_rng(11)
    T, nq, nkv, hd, p0 = 5, 4, 2, 8, 3
    Q = rng.standard_normal((T, nq, hd))
    K = np.zeros((nkv, p0 + T, hd))
    V = rng.standard_normal((nkv, p0 + T, hd))
    O = causal_attend(Q, K, V, p0)
    for t in range(T):
        for h in range(nq):
            want = V[h // 2, :p0 + t + 1].mean(axis=0)
            assert np.max(np.abs(O[t, h] - want)) <= 1e-14
    q0 = 1.0 + 3 * 2.0 ** -9
    Q = np.zeros((1, 1, 4))
    Q[0, 0, 0] = q0
    K = np.zeros((1, 2, 4))
    K[0, 1, 0] = -2.0                             # score of key 1: -q0 (sqrt(hd) = 2)
    V = np.zeros((1, 2, 4))
    V[0, 0, 0] = 1.0
    V[0, 1, 1] = 1.0
    O = causal_attend(Q, K, V, 1)[0, 0]
    w1 = math.exp(-q0)
    assert abs(O[0] - 1.0 / (1.0 + w1)) <= 1e-15
    assert abs(O[1] - w1 / (1.0 + w1)) <= 1e-15
    assert O[2] == O[3] == 0.0


def test_poisoned_step_stays_poisoned():
    """An id outside the table embeds as a NaN row; NaN logits have no argmax
    and give the out-of-table id vocab, so the poison carries to the next step."""
    m = synth.make_tiny(replace(synth.TINY, prompt=2, steps=1))
    d = Decoder(m)
    V = m["cfg"].vocab
    assert np.all(np.isnan(d.embed(V))) and np.all(np.isnan(d.embed(-1)))
    logits, a = d.step(V, 0)
    assert np.all(np.isnan(logits)) and a == V
    assert not np.isnan(d.embed(V - 1)).any()
