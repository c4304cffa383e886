"""The stage walk that allocates nothing (its layer scratch in the library's static
device buffer) against the walk with caller scratch: the same hidden rows and
cache rows bit for bit, over two models in a row, the second smaller, so the
static buffer holds the first model's leftovers when the second one runs."""
import ctypes as C
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

MID = synth.DecoderConfig("mid-bf16", n_layers=4, d=1024, nq=8, nkv=2, hd=128, ff=2816, vocab=2048,
                          wdtype="bf16", kvdtype="bf16", prefix=200, prompt=4, steps=0)


@pytest.fixture(scope="module")
def rt():
    from layer_pipeline_stage_amd import runtime, lps
    lps.load()
    assert torch.cuda.is_available(), "GPU tests need a visible ROCm GPU"
    return runtime


def _walk_both(rt, m, fence):
    from layer_pipeline_stage_amd import lps
    cfg = m["cfg"]
    a = rt.DeviceDecoder(m, fence=fence, streams="single")
    b = rt.DeviceDecoder(m, fence=fence, streams="single")
    n = len(fence) - 1
    st = a.streams[0]
    p0 = cfg.prefix
    ids = torch.tensor(m["prompt"], dtype=torch.int32, device=a.device)
    for i in range(len(m["prompt"])):
        for dd in (a, b):
            lps.lps_embed(rt.ptr(dd.embed), lps.DTYPES[cfg.wdtype], cfg.vocab, cfg.d,
                          rt.ptr(ids) + 4 * i, rt.ptr(dd.x[0]), rt.sp(st))
        for s in range(n):
            lps.lps_stage_forward(a.model, a._fence_c, n, s, rt.ptr(a.x[0]), p0 + i,
                                  rt.ptr(a.scratch[0]), a.scratch_bytes, rt.sp(st))
            lps.lps_stage_forward_static(b.model, b._fence_c, n, s, rt.ptr(b.x[0]), p0 + i,
                                         rt.sp(b.streams[0]))
        torch.cuda.synchronize()
        assert torch.equal(a.x[0], b.x[0]), (cfg.name, i)
        assert not torch.isnan(a.x[0]).any()
    for la, lb in zip(a.layers, b.layers):
        assert torch.equal(la["k"], lb["k"]) and torch.equal(la["v"], lb["v"])
    a.close()
    b.close()


def test_static_scratch_walk_equals_caller_scratch_walk(rt):
    _walk_both(rt, synth.make_dense(MID), [0, 2, 4])
    # a smaller model next: the static buffer still holds the larger one's scratch
    _walk_both(rt, synth.make_tiny(replace(synth.TINY, prompt=5, steps=0)), [0, 4])


def test_static_scratch_walk_refuses_a_model_too_large(rt):
    """ctx_max large enough that the attention partials pass the static buffer's
    size: refused with LPS_ERANGE before anything is enqueued."""
    from layer_pipeline_stage_amd import lps
    d = lps.LayerDesc()
    d.d, d.nq, d.nkv, d.hd, d.ff = 5120, 36, 6, 256, 17472
    d.wdtype, d.kvdtype, d.ctx_max = lps.LPS_BF16, lps.LPS_BF16, 1 << 16
    d.eps, d.rope_base = 1e-6, 1e4
    for k in ("g_attn", "g_ffn", "w_qkv", "w_o", "w_gu", "w_d", "k_cache", "v_cache"):
        setattr(d, k, 256)
    h = C.c_void_p()
    lps.lps_model_create(C.byref(d), 1, C.byref(h))
    try:
        assert lps.lps_model_scratch_bytes(h) > 8 << 20
        with pytest.raises(lps.LpsError) as e:
            lps.lps_stage_forward_static(h, lps.i32_array([0, 1]), 1, 0, 256, 0, None)
        assert e.value.code == lps.LPS_ERANGE and "static buffer" in str(e.value)
    finally:
        lps.lps_model_destroy(h)
