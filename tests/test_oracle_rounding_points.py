"""Pins of the oracle's rounding points and of the gated MLP's operand order, on
hand-built layers whose every step reduces to scalar arithmetic.

Zero, identity and unit-vector weights (exact in bf16) turn a layer into a few
scalar operations that the test writes out for that special case, with torch's
bf16 conversion and numpy's f16 conversion as the rounding references and
scipy's expit for the sigmoid.  Each rounding point is live on these inputs,
and each test also plants the removal of one rounding point (or a swap of the
gate and up operands) in the oracle and requires the pin to fail, so that a
dropped rounding or a transposed operand anywhere in these functions turns a
test red.

Rounding points (the matrix-core operands of a prefill chunk, Q24's reading
extended to the dense prefill): the normed rows H, the attention output O, the
normed rows H2 and the SwiGLU output M of a dense layer; the normed rows and
the SwiGLU output of every expert of a MoE layer.  The residual is f32, the
cache bf16, the remote MoE sum f16."""
from dataclasses import replace

import numpy as np
import pytest
import torch
from scipy.special import expit

import synth
import oracle.moe as om
from oracle.decoder import Decoder, bf16_act

EPS = 1e-6
ONE, ZERO = 0x3F80, 0x0000          # bf16 bit patterns of 1.0 and 0.0


def bf(v):
    """f64 -> f32 -> bf16 (nearest even) -> f64, by torch."""
    return torch.tensor(np.asarray(v, np.float64), dtype=torch.float32).to(
        torch.bfloat16).to(torch.float64).numpy()


def f32(v):
    return np.asarray(v, np.float64).astype(np.float32).astype(np.float64)


def f16(v):
    return np.asarray(v, np.float64).astype(np.float32).astype(np.float16).astype(np.float64)


def silu(z):
    return z * expit(z)


def rms(x):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + EPS)


# ---- dense layer: d 2, one q / kv head of dim 2, ff 1 ---------------------------------
CF = synth.DecoderConfig("cf", n_layers=1, d=2, nq=1, nkv=1, hd=2, ff=1, vocab=0,
                         wdtype="bf16", kvdtype="bf16", prefix=0, steps=3)
X3 = f32(np.array([[1.0, -0.9], [-0.7, 1.9], [0.45, -1.3]]))


def dense_model():
    """q = k = 0 (every score 0: row t's weights are uniform over rows 0..t),
    v = (H[0] + H[1], H[1]), O projection = identity, gate = H2[0], up = H2[1],
    down = [M, 0]."""
    qkv = np.zeros((6, 2), np.uint16)
    qkv[4, 0] = qkv[4, 1] = qkv[5, 1] = ONE
    wo = np.array([[ONE, ZERO], [ZERO, ONE]], np.uint16)
    wgu = np.array([[ONE, ZERO], [ZERO, ONE]], np.uint16)
    wd = np.array([[ONE], [ZERO]], np.uint16)
    L = {"g_attn": np.ones(2, np.float32), "w_qkv": qkv, "w_o": wo,
         "g_ffn": np.ones(2, np.float32), "w_gu": wgu, "w_d": wd}
    return {"cfg": CF, "layers": [L]}


def dense_closed_form(X, rounded=True, swap=False):
    """The layer above at positions 0..T-1 with an empty cache, by hand."""
    r = bf if rounded else (lambda a: a)
    H = r(rms(X))
    Vc = bf(np.stack([H[:, 0] + H[:, 1], H[:, 1]], axis=1))    # the bf16 cache rows
    O = np.stack([Vc[:t + 1].mean(axis=0) for t in range(len(X))])
    X1 = f32(X + r(O))
    H2 = r(rms(X1))
    g, u = (H2[:, 1], H2[:, 0]) if swap else (H2[:, 0], H2[:, 1])
    M = r(silu(g) * u)
    return f32(X1 + np.stack([M, np.zeros_like(M)], axis=1))


def skip_call(k):
    """bf16_act with its k-th call (0-based) left out: a planted missing rounding."""
    n = [0]

    def act(x):
        i = n[0]
        n[0] += 1
        return np.asarray(x, np.float64) if i == k else bf16_act(x)
    return act


def test_dense_prefill_rounding_points_closed_form():
    m = dense_model()
    got = Decoder(m).layer_prefill(0, X3, 0)
    want = dense_closed_form(X3)
    assert np.max(np.abs(got - want)) <= 1e-15
    # exact operands: the same layer without any bf16 rounding
    got = Decoder(m).layer_prefill(0, X3, 0, act=None)
    assert np.max(np.abs(got - dense_closed_form(X3, rounded=False))) <= 1e-15


@pytest.mark.parametrize("k,name", [(0, "H"), (1, "O"), (2, "H2"), (3, "M")])
def test_dense_prefill_pin_catches_a_missing_rounding(k, name):
    """Each of the four rounding points is live: leaving any one out moves the
    layer's output far past the pin's bar."""
    got = Decoder(dense_model()).layer_prefill(0, X3, 0, act=skip_call(k))
    assert np.max(np.abs(got - dense_closed_form(X3))) > 1e-6, name


def test_dense_gate_up_order_is_pinned():
    """A gate/up swap (silu of the up rows) would miss the closed form by far,
    in prefill and in the decode step."""
    want, swapped = dense_closed_form(X3), dense_closed_form(X3, swap=True)
    assert np.max(np.abs(want - swapped)) > 1e-3
    # decode steps of the same layer (exact operands, bf16 cache) give the
    # exact-operand closed form row by row
    d = Decoder(dense_model())
    rows = np.stack([d.layer(0, X3[t], t) for t in range(3)])
    assert np.max(np.abs(rows - dense_closed_form(X3, rounded=False))) <= 1e-15


# ---- MoE layer: d 2, two experts, top 1, ff 1, expert 1 remote --------------------------
MCF = synth.MoEConfig("mcf", n_layers=1, d=2, n_experts=2, top_k=1, ff=1, remote_from=1,
                      prefill_T=0, steps=0)
XM = f32(np.array([[1.0, 0.3], [-0.7, 1.9], [0.45, -1.3]]))   # rows 0, 2 -> expert 0; row 1 -> expert 1


def moe_layer_weights():
    """Router = identity (logits = the unrounded normed row, top 1 = its larger
    component, weight 1).  Expert 0: gate h[0], up h[1], out [m, 0].  Expert 1:
    gate h[1], up h[0], out [0, m].  Shared: gate = up = h[0], out [m, m]."""
    I2 = np.array([[ONE, ZERO], [ZERO, ONE]], np.uint16)
    return {
        "g_ffn": np.ones(2, np.float32),
        "w_r": I2.copy(),
        "w_gu_e": np.stack([I2, I2[::-1].copy()]),
        "w_d_e": np.array([[[ONE], [ZERO]], [[ZERO], [ONE]]], np.uint16),
        "w_gu_s": np.array([[ONE, ZERO], [ONE, ZERO]], np.uint16),
        "w_d_s": np.array([[ONE], [ONE]], np.uint16),
    }


def moe_closed_form(X, prefill, swap=False):
    r = bf if prefill else (lambda a: a)
    h = rms(X)
    sel = (h[:, 1] > h[:, 0]).astype(int)        # top 1 of the router logits (ties -> 0)
    H = r(h)

    def e(g, u):
        if swap:
            g, u = u, g
        return r(silu(g) * u)

    m0, m1, ms = e(H[:, 0], H[:, 1]), e(H[:, 1], H[:, 0]), e(H[:, 0], H[:, 0])
    z = np.zeros_like(m0)
    shared = np.stack([ms, ms], 1)
    local = np.where(sel[:, None] == 0, np.stack([m0, z], 1), 0.0)
    remote = np.where(sel[:, None] == 1, np.stack([z, m1], 1), 0.0)
    y = (f32(shared) + f32(local)) + f16(remote)
    return f32(X + y), sel


@pytest.mark.parametrize("prefill", [False, True])
def test_moe_layer_closed_form(prefill):
    L = moe_layer_weights()
    tr = {}
    got = om.moe_layer(XM, L, MCF, prefill=prefill, trace=tr)
    want, sel = moe_closed_form(XM, prefill)
    assert list(tr["idx"][:, 0]) == list(sel) == [0, 1, 0]
    assert np.max(np.abs(got - want)) <= 1e-15
    # the gate/up order and (at decode) the f16 rounding of the remote sum are live
    assert np.max(np.abs(want - moe_closed_form(XM, prefill, swap=True)[0])) > 1e-3
    if not prefill:
        h1 = rms(XM)[1]
        m1 = silu(h1[1]) * h1[0]
        assert f16(m1) != f32(m1)


def test_expert_gate_up_order_closed_form():
    """expert() alone: gate rows first, then up rows; silu on the gate."""
    h = np.array([[0.8, -1.7], [2.5, 0.4]])
    wgu = np.array([[ONE, ZERO], [ZERO, ONE]], np.uint16)
    wd = np.array([[ONE], [ZERO]], np.uint16)
    out = om.expert(h, wgu, wd, 1)
    assert np.max(np.abs(out[:, 0] - silu(h[:, 0]) * h[:, 1])) <= 1e-15
    assert np.all(out[:, 1] == 0)
    assert np.min(np.abs(silu(h[:, 0]) * h[:, 1] - silu(h[:, 1]) * h[:, 0])) > 0.1


@pytest.mark.parametrize("k,name", [(0, "normed rows"), (1, "shared SwiGLU"),
                                    (2, "expert 0 SwiGLU"), (3, "expert 1 SwiGLU")])
def test_moe_prefill_pin_catches_a_missing_rounding(monkeypatch, k, name):
    n = [0]

    def planted(x):
        i = n[0]
        n[0] += 1
        return np.asarray(x, np.float64) if i == k else bf16_act(x)

    monkeypatch.setattr(om, "bf16_round", planted)
    got = om.moe_layer(XM, moe_layer_weights(), MCF, prefill=True)
    assert n[0] == 4, "the prefill layer rounds the rows once and each expert's output once"
    assert np.max(np.abs(got - moe_closed_form(XM, True)[0])) > 1e-6, name
