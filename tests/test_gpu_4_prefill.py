"""Chunked dense prefill through the stages (bf16 GEMMs and causal attention on
the matrix cores) against the oracle's prefill; stage splits and chunk splits
bit-identical on the GPU with liveness counters that prove the split walk ran
(memra pp module docs, Statics: split counters keep identity gates from passing
vacuously); decode continuing from the prefilled caches; the 8B slice at its
full size."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from oracle.decoder import Decoder

pytestmark = pytest.mark.gpu

TOL = 2e-3   # bf16 weights: of the output scale, per step

# Prefill rounds the matrix-core operands (normed rows, attention output, SwiGLU
# output) to bf16 at every layer.  Two implementations that round the same values
# at the same points but form them with different accumulation orders (f32 on the
# GPU, f64 in the oracle) take opposite sides of a rounding midpoint now and then,
# and a flipped operand perturbs the next layer's inputs, so their rounding
# errors decorrelate over the layers.  The bar therefore comes from the oracle
# itself: the GPU may sit at most twice as far from the bf16-operand oracle as
# that oracle sits from the exact-operand one (the size of the rounding effect),
# plus the bf16-weight bar.  A real mistake (a mask, a position, a layout) moves
# the result by far more: the split identities below are exact.


def _pf_tol(exact, rounded):
    exact, rounded = np.asarray(exact, np.float64), np.asarray(rounded, np.float64)
    return 2.0 * float(np.abs(exact - rounded).max()) + TOL * float(np.abs(rounded).max())

PF = synth.DecoderConfig("pf-small", n_layers=4, d=256, nq=4, nkv=2, hd=64, ff=768, vocab=1024,
                         wdtype="bf16", kvdtype="bf16", prefix=37, prompt=45, steps=6)


@pytest.fixture(scope="module")
def rt():
    from layer_pipeline_stage_amd import runtime, lps
    lps.load()
    assert torch.cuda.is_available(), "GPU tests need a visible ROCm GPU"
    return runtime


@pytest.fixture(scope="module")
def small():
    return synth.make_dense(PF)


def _argmax_ok(a, logits, tol=TOL):
    """The GPU's argmax is the oracle's, or the oracle's top two are a near tie."""
    if a == int(np.argmax(logits)):
        return True
    top2 = np.sort(logits)[-2:]
    scale = tol * np.abs(logits).max()
    return top2[1] - top2[0] <= 2 * scale and logits[a] >= top2[1] - 2 * scale


def _check_prefill(rt, m):
    dd = rt.DeviceDecoder(m)
    lg, am, X = dd.prefill(m["prompt"])
    olg, oam, OX = Decoder(m).prefill(m["prompt"])
    elg, _, EX = Decoder(m).prefill(m["prompt"], act=None)
    for got, want, exact, what in ((X, OX, EX, "hidden rows"), (lg, olg, elg, "logits")):
        err = float(np.max(np.abs(np.asarray(got, np.float64) - want)))
        assert err <= _pf_tol(exact, want), (what, err, _pf_tol(exact, want))
    assert am == oam or _argmax_ok(am, olg, 2 * _pf_tol(elg, olg) / np.abs(olg).max())
    dd.close()


def test_prefill_matches_oracle(rt, small):
    _check_prefill(rt, small)


# the other built head dims and group sizes of the attention kernel: head dim 256
# with 8 q heads per kv head (two key tiles per step, V operands read when used),
# head dim 128 with one; ragged prompts after ragged prefixes
@pytest.mark.parametrize("hd,nq,nkv,prefix,prompt", [(256, 8, 1, 21, 39), (128, 2, 2, 50, 70)])
def test_prefill_other_head_shapes_match_oracle(rt, hd, nq, nkv, prefix, prompt):
    cfg = replace(PF, name=f"pf-hd{hd}-g{nq // nkv}", n_layers=2, nq=nq, nkv=nkv, hd=hd,
                  prefix=prefix, prompt=prompt)
    _check_prefill(rt, synth.make_dense(cfg))


@pytest.mark.parametrize("streams", ["single", "per-stage"])
def test_prefill_stage_and_chunk_splits_bit_identical(rt, small, streams):
    from layer_pipeline_stage_amd import lps
    P = len(small["prompt"])
    dd = rt.DeviceDecoder(small, streams=streams)
    ref_lg, ref_am, ref_X = dd.prefill(small["prompt"])
    for fence in ([0, 2, 4], [0, 1, 3, 4], [0, 1, 2, 3, 4]):
        n = len(fence) - 1
        dd.set_fence(fence)
        dd.reset()
        lps.lps_counters_reset()
        lg, am, X = dd.prefill(small["prompt"])
        c = lps.counters()
        assert c["prefill_walks"] == n and c["boundary_sends"] == n - 1, (fence, c)
        assert am == ref_am and np.array_equal(lg, ref_lg) and np.array_equal(X, ref_X), fence
    # chunks of 16 rows (3 chunks, the last ragged) through 4 stages
    dd.reset()
    lps.lps_counters_reset()
    lg, am, X = dd.prefill(small["prompt"], chunk=16)
    c = lps.counters()
    assert c["prefill_walks"] == 4 * 3 and c["boundary_sends"] == 3 * 3
    assert am == ref_am and np.array_equal(lg, ref_lg)
    assert np.array_equal(X, ref_X[32:P])
    dd.close()


def test_decode_continues_from_the_prefilled_cache(rt, small):
    cfg = small["cfg"]
    P = len(small["prompt"])
    dd = rt.DeviceDecoder(small, fence=[0, 2, 4])
    lg, am, _ = dd.prefill(small["prompt"])
    res = dd.run_tokens([am], cfg.steps - 1, p0=cfg.prefix + P)
    dec, ex = Decoder(small), Decoder(small)
    olg, oam, _ = dec.prefill(small["prompt"])
    elg, _, _ = ex.prefill(small["prompt"], act=None)
    rel = _pf_tol(elg, olg) / np.abs(olg).max()
    assert am == oam or _argmax_ok(am, olg, rel)
    # the decode steps read the prefilled caches: same bar, from the same two oracles
    _, _, olgs = dec.greedy([], 0, p0=cfg.prefix + P, feed=res.fed)
    _, _, elgs = ex.greedy([], 0, p0=cfg.prefix + P, feed=res.fed)
    for i, (a, b, e) in enumerate(zip(res.logits, olgs, elgs)):
        err = float(np.max(np.abs(a - b)))
        assert err <= _pf_tol(e, b), (i, err, _pf_tol(e, b))
    dd.close()


def test_prefill_dense8b_slice_full_size(rt):
    """The 8B slice (8 layers, n_embd 4096, 32q/8kv x 128, SwiGLU 14336, 4096-row
    prefix) with a 128-token prompt through N = 4 stages: the last row's logits
    against the oracle's prefill, N = 4 == N = 1 bit for bit."""
    cfg = replace(synth.DENSE8B, prompt=128, steps=0)
    m = synth.make_dense(cfg)
    dd = rt.DeviceDecoder(m, fence=[0, 2, 4, 6, 8])
    lg, am, X = dd.prefill(m["prompt"])
    dd.set_fence([0, 8])
    dd.reset()
    lg1, am1, X1 = dd.prefill(m["prompt"])
    assert am1 == am and np.array_equal(lg1, lg) and np.array_equal(X1, X)
    dd.close()
    olg, oam, OX = Decoder(m, weight_cache=False).prefill(m["prompt"])
    elg, _, EX = Decoder(m, weight_cache=False).prefill(m["prompt"], act=None)
    for got, want, exact, what in ((lg, olg, elg, "logits"), (X[-1], OX[-1], EX[-1], "last row")):
        err = float(np.max(np.abs(np.asarray(got, np.float64) - want)))
        assert err <= _pf_tol(exact, want), (what, err, _pf_tol(exact, want))
    assert am == oam or _argmax_ok(am, olg, 2 * _pf_tol(elg, olg) / np.abs(olg).max())
