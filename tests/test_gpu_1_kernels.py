"""Step-level parity of the HIP kernels against the float64 oracle, through the C ABI.

Tolerances for single kernels are derived from the arithmetic: an f32 dot
product of K terms accumulated by 64 lanes (K/64 sequential FMAs each, then a
6-level butterfly) has a relative error below (K/64 + 8) * 2^-24 of
sum_j |w_j x_j|; RMSNorm in f32 adds a few ulps; the tests allow twice that.
"""
import ctypes as C
import math

import numpy as np
import pytest
import torch

import synth
from layer_pipeline_stage_amd import layout
from oracle import numerics as onum
from oracle.decoder import rmsnorm, rope, attend, silu
from oracle.moe import softmax, top_k, f16_pieces_to_f32

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def L():
    from layer_pipeline_stage_amd import lps
    lps.load()
    assert torch.cuda.is_available(), "GPU tests need a visible ROCm GPU"
    return lps


def dev(a):
    from layer_pipeline_stage_amd.runtime import to_dev
    return to_dev(a, DEV)


def ptr(t):
    return t.data_ptr()


def stream():
    return torch.cuda.current_stream().cuda_stream


def dot_bound(W, x):
    """(K/64 + 8) * 2^-24 * sum_j |W_ij x_j| per row, doubled."""
    K = W.shape[1]
    return 2 * (K / 64 + 16) * 2.0 ** -24 * (np.abs(W) @ np.abs(x))


def _weights(wdtype, N, K, seed):
    rng = np.random.default_rng(seed)
    w32 = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    if wdtype == "f32":
        return w32, w32.astype(np.float64), None
    if wdtype == "bf16":
        b = synth.bf16_bits(w32)
        return b, onum.bf16_to_f64(b), None
    c, s = synth.mxfp4_encode(w32)
    return c, onum.mxfp4_to_f64(c, s), s


GEMV_CASES = [
    ("f32", 37, 260), ("f32", 64, 4096), ("bf16", 37, 1032), ("bf16", 130, 4096),
    ("bf16", 66, 14336), ("mxfp4", 37, 17472), ("mxfp4", 70, 5120), ("mxfp4", 8, 96),
]


@pytest.mark.parametrize("wdtype,N,K", GEMV_CASES)
@pytest.mark.parametrize("mode", ["store", "add", "swiglu"])
@pytest.mark.parametrize("norm", [False, True])
def test_gemv_parity(L, wdtype, N, K, mode, norm):
    if mode == "swiglu" and N % 2:
        N += 1
    w, W64, s = _weights(wdtype, N, K, seed=N * 7 + K)
    rng = np.random.default_rng(K)
    x = rng.standard_normal(K).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    xp = rmsnorm(x.astype(np.float64), g, 1e-6) if norm else x.astype(np.float64)
    r = W64 @ xp
    bound = dot_bound(W64, xp)
    if norm:
        bound += 8 * 2.0 ** -24 * (np.abs(W64) @ np.abs(xp))
    if wdtype == "mxfp4":
        # MXFP4 rows meet x as f16 operands (one dot2 per weight pair): x is rounded
        # to nearest once, relative error <= 2^-11 (absolute <= 2^-25 below f16's
        # normal range)
        bound += 2.0 ** -11 * (np.abs(W64) @ np.abs(xp)) + 2.0 ** -25 * np.abs(W64).sum(axis=1)
    y0 = rng.standard_normal(N).astype(np.float32)
    if mode == "store":
        ref, n_out = r, N
    elif mode == "add":
        ref, n_out = y0.astype(np.float64) + r, N
        bound = bound + np.spacing(np.abs(ref).astype(np.float32))
    else:
        h = N // 2
        ref, n_out = silu(r[:h]) * r[h:], h
        # d(silu(a) b) = silu'(a) b da + silu(a) db, |silu'| <= 1.1
        bound = 1.1 * np.abs(r[h:]) * bound[:h] + np.abs(silu(r[:h])) * bound[h:] + \
            4 * np.spacing(np.abs(ref).astype(np.float32))
    wd, xd = dev(w), dev(x)
    sd = dev(s) if s is not None else None
    gd = dev(g) if norm else None
    yd = dev(y0 if mode == "add" else np.zeros(n_out, np.float32))
    L.lps_gemv(L.DTYPES[wdtype], ptr(wd), ptr(sd) if sd is not None else None, N, K, ptr(xd),
               ptr(gd) if gd is not None else None, 1e-6, ptr(yd),
               {"store": 0, "add": 1, "swiglu": 2}[mode], stream())
    got = yd.cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    assert np.all(err <= bound + 1e-30), (err.max(), bound[np.argmax(err - bound)])


@pytest.mark.parametrize("K", [5120, 17472])
def test_mxfp4_gemv_unnormed_vector_past_f16_range(L, K):
    """An un-normed MXFP4 GEMV input (the attention output, the SwiGLU output)
    whose values pass f16's largest finite value: the staging scales the vector by
    a power of two so no operand rounds to infinity, and the products are scaled
    back: every output finite and within the same f16-operand bound of the oracle
    as an ordinary vector; a vector below 2^15 gives the same bits as before the
    scaling existed (it is staged unchanged: scaling by 2^e is exact, so the
    2^e-scaled vector gives the 2^e-scaled result)."""
    N = 66
    w, W64, s = _weights("mxfp4", N, K, seed=K + 5)
    rng = np.random.default_rng(K + 1)
    x = (rng.standard_normal(K) * 1e5).astype(np.float32)       # |x| up to ~5e5
    x[17] = 3.0e6
    wd, sd, xd = dev(w), dev(s), dev(x)
    yd = dev(np.zeros(N, np.float32))
    L.lps_gemv(L.LPS_MXFP4, ptr(wd), ptr(sd), N, K, ptr(xd), None, 1e-6, ptr(yd), 0, stream())
    got = yd.cpu().numpy().astype(np.float64)
    xp = x.astype(np.float64)
    ref = W64 @ xp
    bound = dot_bound(W64, xp) + 2.0 ** -11 * (np.abs(W64) @ np.abs(xp))
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - ref) <= bound), np.max(np.abs(got - ref) - bound)
    # scaling a small vector by 2^e scales the result by exactly 2^e
    xs = rng.standard_normal(K) * 10
    xs = (np.sign(xs) * np.maximum(np.abs(xs), 1e-3)).astype(np.float32)   # no f16 subnormals
    y1 = dev(np.zeros(N, np.float32))
    L.lps_gemv(L.LPS_MXFP4, ptr(wd), ptr(sd), N, K, ptr(dev(xs)), None, 1e-6, ptr(y1), 0, stream())
    y2 = dev(np.zeros(N, np.float32))
    L.lps_gemv(L.LPS_MXFP4, ptr(wd), ptr(sd), N, K, ptr(dev(xs * np.float32(2.0 ** 20))), None,
               1e-6, ptr(y2), 0, stream())
    assert torch.equal(y2, y1 * 2.0 ** 20)


def test_gemv_k_tail_reads_no_next_row(L):
    """K = 17472 (= 136 * 128 + 64): rows are laid out back to back, so a kernel
    that read whole 128-wide slabs past the end of a row would pull in the next
    row's codes.  Give every row a distinct NaN-free pattern and a NaN-filled
    neighbour region after the matrix: the results must stay finite and exact."""
    N, K = 5, 17472
    w, W64, s = _weights("mxfp4", N, K, seed=1)
    big = np.zeros((N + 1, K // 2), np.uint8)
    big[:N] = w
    sbig = np.full((N + 1, K // 32), 0xFF, np.uint8)   # NaN scales just past the last row
    sbig[:N] = s
    x = np.random.default_rng(2).standard_normal(K).astype(np.float32)
    wd, sd, xd = dev(big), dev(sbig), dev(x)
    yd = torch.zeros(N, dtype=torch.float32, device=DEV)
    L.lps_gemv(L.LPS_MXFP4, ptr(wd), ptr(sd), N, K, ptr(xd), None, 0.0, ptr(yd), 0, stream())
    got = yd.cpu().numpy()
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - W64 @ x) <= dot_bound(W64, x.astype(np.float64)))


def test_gemv_zero_padded_k_bit_identical(L):
    """Zero groups appended at the end of K leave every output bit unchanged
    (each chunk lands on the same lane in the same order whatever K is)."""
    N, K, Kp = 64, 17408, 17472
    w, _, s = _weights("mxfp4", N, K, seed=3)
    wp = np.concatenate([w, np.zeros((N, (Kp - K) // 2), np.uint8)], axis=1)
    spd = np.concatenate([s, np.full((N, (Kp - K) // 32), 0x7F, np.uint8)], axis=1)
    x = np.random.default_rng(4).standard_normal(Kp).astype(np.float32)
    outs = []
    for ww, ss, KK in ((w, s, K), (wp, spd, Kp)):
        yd = torch.zeros(N, dtype=torch.float32, device=DEV)
        wd, sd, xd = dev(ww), dev(ss), dev(x[:KK])
        L.lps_gemv(L.LPS_MXFP4, ptr(wd), ptr(sd), N, KK, ptr(xd), None, 0.0, ptr(yd), 0, stream())
        outs.append(yd.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


def test_mxfp4_builtin_nibble_order(L):
    """The gfx950 scaled FP4 conversion must give element 2b from the low nibble:
    a one-hot code in each position of a row selects exactly that x entry."""
    K = 64
    N = 64
    codes = np.zeros((N, K // 2), np.uint8)
    for r in range(N):
        b, hi = divmod(r, 2)
        codes[r, b] = (2 << 4) if hi else 2          # code 2 = 1.0
    scales = np.full((N, K // 32), 127, np.uint8)
    x = np.arange(1, K + 1, dtype=np.float32)
    yd = torch.zeros(N, dtype=torch.float32, device=DEV)
    cd, sd, xd = dev(codes), dev(scales), dev(x)
    L.lps_gemv(L.LPS_MXFP4, ptr(cd), ptr(sd), N, K, ptr(xd), None, 0.0, ptr(yd), 0, stream())
    assert np.array_equal(yd.cpu().numpy(), x[:N])


def test_mxfp4_gemv_refuses_rows_past_its_staging(L):
    """The MXFP4 GEMV stages x from registers held across the norm's sum, so K is
    bounded (24576); a longer row is refused before anything is enqueued (the
    buffers are sized for it all the same)."""
    N, K = 2, 24576 + 32
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.full((N, K // 32), 127, np.uint8)
    x = np.ones(K, np.float32)
    yd = torch.zeros(N, dtype=torch.float32, device=DEV)
    cd, sd, xd = dev(codes), dev(scales), dev(x)
    with pytest.raises(L.LpsError) as e:
        L.lps_gemv(L.LPS_MXFP4, ptr(cd), ptr(sd), N, K, ptr(xd), None, 0.0, ptr(yd), 0, stream())
    assert e.value.code == L.LPS_EUNSUP
    K = 24576                                            # the longest row runs
    L.lps_gemv(L.LPS_MXFP4, ptr(cd), ptr(sd), N, K, ptr(xd), None, 0.0, ptr(yd), 0, stream())
    torch.cuda.synchronize()
    assert np.array_equal(yd.cpu().numpy(), np.zeros(N, np.float32))


def test_rmsnorm_and_embed(L):
    rng = np.random.default_rng(5)
    d = 4096
    x = rng.standard_normal(d).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    yd = torch.zeros(d, dtype=torch.float32, device=DEV)
    xd, gd = dev(x), dev(g)          # keep the inputs alive until the kernel has run
    L.lps_rmsnorm(ptr(xd), ptr(gd), 1e-6, d, ptr(yd), stream())
    ref = rmsnorm(x.astype(np.float64), g, 1e-6)
    assert np.max(np.abs(yd.cpu().numpy() - ref)) <= 1e-6 * np.abs(ref).max()
    for wd in ("f32", "bf16"):
        E32 = rng.standard_normal((50, 264)).astype(np.float32)
        E = E32 if wd == "f32" else synth.bf16_bits(E32)
        Ed = dev(E)
        for t in (0, 17, 49):
            td = torch.tensor([t], dtype=torch.int32, device=DEV)
            xd = torch.zeros(264, dtype=torch.float32, device=DEV)
            L.lps_embed(ptr(Ed), L.DTYPES[wd], 50, 264, ptr(td), ptr(xd), stream())
            assert np.array_equal(xd.cpu().numpy(), onum.widen_weight(E[t], wd).astype(np.float32))
    # a token outside the table poisons the row with NaN
    td = torch.tensor([50], dtype=torch.int32, device=DEV)
    L.lps_embed(ptr(Ed), L.LPS_BF16, 50, 264, ptr(td), ptr(xd), stream())
    assert np.all(np.isnan(xd.cpu().numpy()))


ATTN_CASES = [
    (4, 2, 64, "f32", [1, 2, 63, 64, 65, 96]),
    (32, 8, 128, "bf16", [1, 64, 65, 257, 4097]),
    (36, 6, 256, "bf16", [1, 130, 8193]),
    (8, 8, 128, "f32", [5, 100]),
]


@pytest.mark.parametrize("nq,nkv,hd,kvd,ns", ATTN_CASES)
def test_attention_parity(L, nq, nkv, hd, kvd, ns):
    """Split-context attention against the oracle's softmax; bf16 caches hold V
    transposed.  The rows past the longest context hold NaN: no row at or past
    n_rows may reach the result."""
    ctx_max = max(ns) + 3
    if kvd == "bf16":
        ctx_max = (ctx_max + 15) // 16 * 16
    rng = np.random.default_rng(nq * hd)
    K32 = rng.standard_normal((nkv, ctx_max, hd)).astype(np.float32)
    V32 = rng.standard_normal((nkv, ctx_max, hd)).astype(np.float32)
    Ks = K32 if kvd == "f32" else synth.bf16_bits(K32)
    Vs = V32 if kvd == "f32" else synth.bf16_bits(V32)
    nan = np.float32(np.nan) if kvd == "f32" else np.uint16(0x7FC0)
    Ks[:, max(ns):] = nan
    Vs[:, max(ns):] = nan
    Kd = dev(Ks if kvd == "f32" else layout.k_to_tiles(Ks))
    Vd = dev(Vs if kvd == "f32" else layout.v_to_tiles(Vs))
    sb = L.lps_attention_scratch_bytes(nq, nkv, hd, ctx_max)
    scratch = torch.zeros(sb, dtype=torch.uint8, device=DEV)
    Kw, Vw = onum.widen_cache(Ks, kvd), onum.widen_cache(Vs, kvd)
    for n in ns:
        q = rng.standard_normal((nq, hd)).astype(np.float32)
        od = torch.zeros(nq * hd, dtype=torch.float32, device=DEV)
        qd = dev(q)
        L.lps_attention_decode(nq, nkv, hd, L.DTYPES[kvd], ptr(Kd), ptr(Vd), ctx_max, n,
                               ptr(qd), ptr(od), ptr(scratch), sb, stream())
        ref = attend(q.astype(np.float64), Kw[:, :n], Vw[:, :n])
        got = od.cpu().numpy().reshape(nq, hd)
        # softmax weights carry ~(hd/16 + 8) ulps from the score dots and exp;
        # the output is a convex combination of V rows
        tol = 2e-5 * np.abs(Vw[:, :n]).max()
        assert np.max(np.abs(got - ref)) <= tol, (n, np.max(np.abs(got - ref)))
    # counters are left at zero: a second identical call gives identical bits
    o1 = od.clone()
    L.lps_attention_decode(nq, nkv, hd, L.DTYPES[kvd], ptr(Kd), ptr(Vd), ctx_max, ns[-1],
                           ptr(qd), ptr(od), ptr(scratch), sb, stream())
    assert torch.equal(o1, od)


def _layer_desc(L, cfg, t):
    d = L.LayerDesc()
    d.d, d.nq, d.nkv, d.hd, d.ff = cfg.d, cfg.nq, cfg.nkv, cfg.hd, cfg.ff
    d.wdtype, d.kvdtype, d.ctx_max = L.DTYPES[cfg.wdtype], L.DTYPES[cfg.kvdtype], cfg.ctx_max
    d.eps, d.rope_base = cfg.eps, cfg.rope_base
    for k in ("g_attn", "g_ffn", "w_qkv", "w_o", "w_gu", "w_d"):
        setattr(d, k, ptr(t[k]))
    for k in ("s_qkv", "s_o", "s_gu", "s_d"):
        setattr(d, k, ptr(t[k]) if t.get(k) is not None else None)
    d.k_cache, d.v_cache = ptr(t["k"]), ptr(t["v"])
    return d


@pytest.mark.parametrize("cfg", [synth.TINY, synth.DecoderConfig(
    "qkv-bf16", n_layers=1, d=512, nq=8, nkv=2, hd=128, ff=256, vocab=0, wdtype="bf16",
    kvdtype="bf16", prefix=28, steps=4)])
def test_qkv_rope_append(L, cfg):
    m = synth.make_dense(cfg) if cfg.vocab or cfg.wdtype != "mxfp4" else None
    Lw = m["layers"][0]
    t = {k: dev(Lw[k]) for k in ("g_attn", "g_ffn", "w_qkv", "w_o", "w_gu", "w_d")}
    kvt = torch.float32 if cfg.kvdtype == "f32" else torch.int16
    if cfg.kvdtype == "bf16":     # 16-row tiles
        kshape = (cfg.nkv, cfg.ctx_max // 16, cfg.hd // 8, 16, 8)
        vshape = (cfg.nkv, cfg.ctx_max // 16, cfg.hd, 16)
    else:
        kshape = vshape = (cfg.nkv, cfg.ctx_max, cfg.hd)
    t["k"] = torch.zeros(kshape, dtype=kvt, device=DEV)
    t["v"] = torch.zeros(vshape, dtype=kvt, device=DEV)
    desc = _layer_desc(L, cfg, t)
    rng = np.random.default_rng(8)
    W = onum.widen_weight(Lw["w_qkv"], cfg.wdtype)
    for pos in (0, 3, cfg.ctx_max - 1):
        x = rng.standard_normal(cfg.d).astype(np.float32)
        qd = torch.zeros(cfg.nq * cfg.hd, dtype=torch.float32, device=DEV)
        xd = dev(x)
        L.lps_qkv_rope_append(C.byref(desc), ptr(xd), pos, ptr(qd), stream())
        h = rmsnorm(x.astype(np.float64), Lw["g_attn"], cfg.eps)
        qkv = W @ h
        nq, nkv, hd = cfg.nq, cfg.nkv, cfg.hd
        q = rope(qkv[:nq * hd].reshape(nq, hd), pos, cfg.rope_base)
        k = rope(qkv[nq * hd:(nq + nkv) * hd].reshape(nkv, hd), pos, cfg.rope_base)
        v = qkv[(nq + nkv) * hd:].reshape(nkv, hd)
        bq = dot_bound(W, h)
        tol = 4 * bq.max() + 1e-6 * np.abs(qkv).max()
        assert np.max(np.abs(qd.cpu().numpy().reshape(nq, hd) - q)) <= tol
        kc = t["k"].cpu().numpy()
        vc = t["v"].cpu().numpy()
        if cfg.kvdtype == "bf16":
            kc, vc = layout.k_from_tiles(kc), layout.v_from_tiles(vc)
        if cfg.kvdtype == "bf16":
            kc, vc = kc.view(np.uint16), vc.view(np.uint16)
        kg = onum.widen_cache(kc[:, pos], cfg.kvdtype)
        vg = onum.widen_cache(vc[:, pos], cfg.kvdtype)
        rel = 2.0 ** -8 if cfg.kvdtype == "bf16" else 0.0      # one bf16 rounding
        assert np.all(np.abs(kg - k) <= tol + rel * np.abs(k))
        assert np.all(np.abs(vg - v) <= tol + rel * np.abs(v))


def test_head_argmax(L):
    rng = np.random.default_rng(11)
    for wd, V, d in (("f32", 1024, 256), ("bf16", 32000, 4096), ("bf16", 1001, 512)):
        W32 = (rng.standard_normal((V, d)) * 0.02).astype(np.float32)
        W = W32 if wd == "f32" else synth.bf16_bits(W32)
        g = np.ones(d, np.float32)
        x = rng.standard_normal(d).astype(np.float32)
        hdsc = L.HeadDesc()
        Wd, gd = dev(W), dev(g)
        hdsc.d, hdsc.vocab, hdsc.wdtype, hdsc.eps = d, V, L.DTYPES[wd], 1e-6
        hdsc.g_out, hdsc.w_lm = ptr(gd), ptr(Wd)
        sb = L.lps_head_scratch_bytes(C.byref(hdsc))
        sc = torch.zeros(sb, dtype=torch.uint8, device=DEV)
        lg = torch.zeros(V, dtype=torch.float32, device=DEV)
        tk = torch.zeros(1, dtype=torch.int32, device=DEV)
        for rep in range(2):
            xd = dev(x)
            L.lps_head_forward(C.byref(hdsc), ptr(xd), ptr(lg), ptr(tk), ptr(sc), sb, stream())
            got = lg.cpu().numpy()
            assert int(tk.item()) == int(np.argmax(got))      # exact on the GPU's own logits
            W64 = onum.widen_weight(W, wd)
            h = rmsnorm(x.astype(np.float64), g, 1e-6)
            ref = W64 @ h
            assert np.max(np.abs(got - ref)) <= 2 * dot_bound(W64, h).max() + 1e-6 * np.abs(ref).max()
    # ties resolve to the lowest index
    V, d = 130, 256
    W = np.zeros((V, d), np.float32)
    W[[7, 40, 129], 0] = 1.0
    x = np.zeros(d, np.float32)
    x[0] = 1.0
    Wd = dev(W)
    hdsc.d, hdsc.vocab, hdsc.wdtype = d, V, L.LPS_F32
    hdsc.w_lm = ptr(Wd)
    gd = dev(np.ones(d, np.float32))
    hdsc.g_out = ptr(gd)
    xd = dev(x)
    L.lps_head_forward(C.byref(hdsc), ptr(xd), ptr(lg), ptr(tk), ptr(sc), sb, stream())
    assert int(tk.item()) == 7
    # a NaN logit (one poisoned weight row), or a NaN input (every logit NaN):
    # the step has no argmax and the id is vocab, outside the table, which the
    # next embedding gather turns into a NaN row
    W[50, 0] = np.nan
    Wd = dev(W)
    hdsc.w_lm = ptr(Wd)
    L.lps_head_forward(C.byref(hdsc), ptr(xd), ptr(lg), ptr(tk), ptr(sc), sb, stream())
    assert np.isnan(lg.cpu().numpy()[50]) and int(tk.item()) == V
    W[50, 0] = 0.0
    Wd = dev(W)
    hdsc.w_lm = ptr(Wd)
    x[3] = np.nan
    xd = dev(x)
    L.lps_head_forward(C.byref(hdsc), ptr(xd), ptr(lg), ptr(tk), ptr(sc), sb, stream())
    assert np.all(np.isnan(lg.cpu().numpy()[:V])) and int(tk.item()) == V
    emb = dev(np.ones((V, d), np.float32))
    out = torch.zeros(d, dtype=torch.float32, device=DEV)
    L.lps_embed(ptr(emb), L.LPS_F32, V, d, ptr(tk), ptr(out), stream())
    assert torch.all(torch.isnan(out))


def test_step_finish_equals_head_advance_embed(L):
    """lps_step_finish (head, history copy, one launch for argmax + token chain +
    next embedding row + advance) leaves exactly what lps_head_forward,
    lps_step_advance and lps_embed leave: logits, history rows, token history, next
    id, state and the next input row, for a fed step, a greedy step, the position
    limit, and a step with no finite logit (a NaN row follows)."""
    rng = np.random.default_rng(5)
    V, d = 1003, 512
    W = synth.bf16_bits((rng.standard_normal((V, d)) * 0.05).astype(np.float32))
    E = synth.bf16_bits(rng.standard_normal((V, d)).astype(np.float32))
    hd = L.HeadDesc()
    Wd, gd, Ed = dev(W), dev(np.ones(d, np.float32)), dev(E)
    hd.d, hd.vocab, hd.wdtype, hd.eps, hd.g_out, hd.w_lm = d, V, L.LPS_BF16, 1e-6, ptr(gd), ptr(Wd)
    sb = L.lps_head_scratch_bytes(C.byref(hd))
    feed = dev(np.array([5, 17, 400], np.int32))
    cap = 4

    def run(fused, x, state0, pos_limit, n_feed):
        sc = torch.zeros(sb, dtype=torch.uint8, device=DEV)
        lg = torch.zeros(V, dtype=torch.float32, device=DEV)
        st = dev(np.array(state0, np.int32))
        th = torch.full((cap,), -7, dtype=torch.int32, device=DEV)
        lh = torch.full((cap, V), -7.0, dtype=torch.float32, device=DEV)
        tok = torch.full((1,), -7, dtype=torch.int32, device=DEV)
        xn = torch.full((d,), -7.0, dtype=torch.float32, device=DEV)
        xd = dev(x)
        if fused:
            L.lps_step_finish(C.byref(hd), ptr(xd), ptr(lg), ptr(st), pos_limit, ptr(feed), n_feed,
                              ptr(th), ptr(lh), cap, ptr(Ed), L.LPS_BF16, ptr(xn), ptr(tok),
                              None, ptr(sc), sb, stream())
        else:
            am = torch.zeros(1, dtype=torch.int32, device=DEV)
            L.lps_head_forward(C.byref(hd), ptr(xd), ptr(lg), ptr(am), ptr(sc), sb, stream())
            L.lps_step_advance(ptr(st), pos_limit, ptr(am), ptr(tok), ptr(feed), n_feed, ptr(th),
                               cap, ptr(lg), V, ptr(lh), stream())
            L.lps_embed(ptr(Ed), L.LPS_BF16, V, d, ptr(tok), ptr(xn), stream())
        torch.cuda.synchronize()
        return [t.cpu().numpy() for t in (lg, st, th, lh, tok, xn)]

    x = rng.standard_normal(d).astype(np.float32)
    xnan = x.copy()
    xnan[3] = np.nan
    cases = [(x, [40, 0, 0, 0], 100, 3),      # fed: the next id is feed[1]
             (x, [41, 2, 0, 0], 100, 3),      # past the feed: the argmax
             (x, [99, 1, 0, 0], 100, 0),      # at the position limit: flag set, position kept
             (xnan, [50, 3, 0, 0], 100, 0)]   # no finite logit: id V, a NaN row next
    for xi, s0, lim, nf in cases:
        a, b = run(True, xi, s0, lim, nf), run(False, xi, s0, lim, nf)
        for u, v in zip(a, b):
            assert np.array_equal(u, v, equal_nan=True), (s0, nf)
    assert int(a[4][0]) == V and np.all(np.isnan(a[5]))

    # the host ring: step s's logits and argmax land in pinned row s % slots, read
    # after a pending marked behind the step; the other rows are left alone
    R = 3
    ring_l = torch.full((R, V), -7.0, dtype=torch.float32).pin_memory()
    ring_t = torch.full((R,), -7, dtype=torch.int32).pin_memory()
    ring = L.HostRing()
    ring.logits, ring.tok, ring.slots = ptr(ring_l), ptr(ring_t), R
    for xi, s0, lim, nf in cases + [(x, [60, 7, 0, 0], 100, 0)]:
        ring_l.fill_(-7.0)
        ring_t.fill_(-7)
        sc = torch.zeros(sb, dtype=torch.uint8, device=DEV)
        lg = torch.zeros(V, dtype=torch.float32, device=DEV)
        st = dev(np.array(s0, np.int32))
        tok = torch.full((1,), -7, dtype=torch.int32, device=DEV)
        xn = torch.full((d,), -7.0, dtype=torch.float32, device=DEV)
        L.lps_step_finish(C.byref(hd), ptr(dev(xi)), ptr(lg), ptr(st), lim, ptr(feed), nf, None,
                          None, 0, ptr(Ed), L.LPS_BF16, ptr(xn), ptr(tok), C.byref(ring), ptr(sc),
                          sb, stream())
        h = C.c_void_p()
        L.lps_pending_mark(stream(), C.byref(h))
        L.lps_pending_wait(h)
        ref = run(False, xi, s0, lim, nf)
        k = s0[1] % R
        assert np.array_equal(ring_l[k].numpy(), ref[0], equal_nan=True), s0
        assert int(ring_t[k]) == int(ref[0].argmax()) if np.isfinite(ref[0]).all() else int(ring_t[k]) == V
        for j in range(R):
            if j != k:
                assert np.all(ring_l[j].numpy() == -7.0) and int(ring_t[j]) == -7
        with pytest.raises(L.LpsError) as e:
            L.lps_pending_wait(h)                 # consumed
        assert e.value.code == L.LPS_ESTATE
    dbuf = torch.zeros(V, dtype=torch.float32, device=DEV)
    ring.logits = ptr(dbuf)                       # device memory is not a host ring
    with pytest.raises(L.LpsError) as e:
        L.lps_step_finish(C.byref(hd), ptr(dev(x)), ptr(lg), ptr(st), 100, ptr(feed), 0, None, None,
                          0, ptr(Ed), L.LPS_BF16, ptr(xn), ptr(tok), C.byref(ring), ptr(sc), sb,
                          stream())
    assert e.value.code == L.LPS_EINVAL


@pytest.mark.parametrize("n16", [1, 4097, (1 << 22) + 333])
def test_hbm_stream_read_touches_every_word(L, n16):
    """The read-bandwidth calibration reads every 16-byte chunk exactly once: the
    XOR of its per-block folds equals the XOR of all 32-bit words (exact, any
    order), also for sizes that leave a ragged grid-stride tail."""
    rng = np.random.default_rng(n16)
    words = rng.integers(0, 2**32, size=4 * n16, dtype=np.uint64).astype(np.uint32)
    src = dev(words.view(np.int32))
    sink = torch.zeros(L.STREAM_SINK, dtype=torch.int32, device=DEV)
    L.lps_hbm_stream_read(ptr(src), 16 * n16, ptr(sink), stream())
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(words))


def test_boundary_protocol(L):
    d = 5120
    s0 = torch.full((d,), float("nan"), device=DEV)
    s1 = torch.full((d,), float("nan"), device=DEV)
    b = C.c_void_p()
    L.lps_boundary_create(d, ptr(s0), ptr(s1), C.byref(b))
    prod, cons = torch.cuda.Stream(), torch.cuda.Stream()
    rng = np.random.default_rng(12)
    xs = [dev(rng.standard_normal(d).astype(np.float32)) for _ in range(6)]
    ys = [torch.full((d,), float("nan"), device=DEV) for _ in range(6)]
    with pytest.raises(L.LpsError) as e:
        L.lps_boundary_recv(b, ptr(ys[0]), 0, cons.cuda_stream)
    assert e.value.code == L.LPS_ESTATE
    torch.cuda.synchronize()
    for t in range(6):
        L.lps_boundary_send(b, ptr(xs[t]), t, prod.cuda_stream)
        if t == 0:
            with pytest.raises(L.LpsError):
                L.lps_boundary_send(b, ptr(xs[t]), 5, prod.cuda_stream)   # out of order
        L.lps_boundary_recv(b, ptr(ys[t]), t, cons.cuda_stream)
    torch.cuda.synchronize()
    for t in range(6):
        assert torch.equal(ys[t], xs[t])
    L.lps_boundary_destroy(b)
    # a third send before the first receive would overwrite an unread slot
    b = C.c_void_p()
    L.lps_boundary_create(d, ptr(s0), ptr(s1), C.byref(b))
    L.lps_boundary_send(b, ptr(xs[0]), 0, prod.cuda_stream)
    L.lps_boundary_send(b, ptr(xs[1]), 1, prod.cuda_stream)
    with pytest.raises(L.LpsError) as e:
        L.lps_boundary_send(b, ptr(xs[2]), 2, prod.cuda_stream)
    assert e.value.code == L.LPS_ESTATE
    L.lps_boundary_recv(b, ptr(ys[0]), 0, cons.cuda_stream)
    L.lps_boundary_recv(b, ptr(ys[1]), 1, cons.cuda_stream)
    L.lps_boundary_destroy(b)


def test_pending_readback(L):
    V = 32000
    lg = dev(np.random.default_rng(13).standard_normal(V).astype(np.float32))
    tk = torch.tensor([123], dtype=torch.int32, device=DEV)
    hl = torch.zeros(V, dtype=torch.float32).pin_memory()
    ht = torch.zeros(1, dtype=torch.int32).pin_memory()
    rb = torch.cuda.Stream()
    p = C.c_void_p()
    L.lps_logits_defer(ptr(lg), ptr(tk), V, torch.cuda.current_stream().cuda_stream, rb.cuda_stream,
                       ptr(hl), ptr(ht), C.byref(p))
    L.lps_pending_wait(p)
    assert torch.equal(hl, lg.cpu()) and int(ht[0]) == 123
    p2 = C.c_void_p()
    L.lps_logits_defer(ptr(lg), None, V, torch.cuda.current_stream().cuda_stream, rb.cuda_stream,
                       ptr(hl), None, C.byref(p2))
    L.lps_pending_drop(p2)          # safe without waiting
    torch.cuda.synchronize()
    # a handle is consumed by its wait or drop: a second use is refused
    for fn in (L.lps_pending_wait, L.lps_pending_drop):
        with pytest.raises(L.LpsError) as e:
            fn(p)
        assert e.value.code == L.LPS_ESTATE
    with pytest.raises(L.LpsError) as e:
        L.lps_pending_order(p2, rb.cuda_stream)
    assert e.value.code == L.LPS_ESTATE


def test_boundary_hop_is_send_plus_receive(L):
    """The same-stream hop writes the slot and the receiver's buffer from the sent
    row in one kernel, keeps the protocol's order (a hop out of order is refused,
    as is a hop after a lone send) and counts a send and a receive."""
    d = 4099
    s0 = torch.full((d,), float("nan"), device=DEV)
    s1 = torch.full((d,), float("nan"), device=DEV)
    b = C.c_void_p()
    L.lps_boundary_create(d, ptr(s0), ptr(s1), C.byref(b))
    st = torch.cuda.Stream()
    rng = np.random.default_rng(21)
    xs = [dev(rng.standard_normal(d).astype(np.float32)) for _ in range(4)]
    ys = [torch.full((d,), float("nan"), device=DEV) for _ in range(4)]
    L.lps_counters_reset()
    for t in range(3):
        L.lps_boundary_hop(b, ptr(xs[t]), ptr(ys[t]), t, st.cuda_stream)
    with pytest.raises(L.LpsError) as e:
        L.lps_boundary_hop(b, ptr(xs[3]), ptr(ys[3]), 5, st.cuda_stream)
    assert e.value.code == L.LPS_ESTATE
    L.lps_boundary_send(b, ptr(xs[3]), 3, st.cuda_stream)
    with pytest.raises(L.LpsError):
        L.lps_boundary_hop(b, ptr(xs[3]), ptr(ys[3]), 3, st.cuda_stream)
    L.lps_boundary_recv(b, ptr(ys[3]), 3, st.cuda_stream)
    torch.cuda.synchronize()
    for t in range(4):
        assert torch.equal(ys[t], xs[t]), t
    assert torch.equal(s0, xs[2]) and torch.equal(s1, xs[3])
    c = L.counters()
    assert c["boundary_sends"] == 4 and c["boundary_recvs"] == 4
    L.lps_boundary_destroy(b)


def test_boundary_orders_a_same_stream_receive_before_another_producer(L):
    """Step 0 is sent and received on stream A behind a long read (its receive
    records no event: same stream); step 2 is then sent from stream B into the
    same slot.  B must wait for A's receive copy: the value received for step 0
    is step 0's, not step 2's."""
    d = 1 << 20
    s0 = torch.full((d,), float("nan"), device=DEV)
    s1 = torch.full((d,), float("nan"), device=DEV)
    b = C.c_void_p()
    L.lps_boundary_create(d, ptr(s0), ptr(s1), C.byref(b))
    A, B = torch.cuda.Stream(), torch.cuda.Stream()
    xs = [torch.full((d,), float(t + 1), device=DEV) for t in range(3)]
    ys = [torch.zeros(d, device=DEV) for _ in range(3)]
    busy = torch.empty(1 << 30, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(L.STREAM_SINK, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    L.lps_boundary_send(b, ptr(xs[0]), 0, A.cuda_stream)
    for _ in range(4):     # ~0.6 ms of HBM reads ahead of the receive on A
        L.lps_hbm_stream_read(ptr(busy), busy.numel(), ptr(sink), A.cuda_stream)
    L.lps_boundary_recv(b, ptr(ys[0]), 0, A.cuda_stream)
    L.lps_boundary_send(b, ptr(xs[1]), 1, B.cuda_stream)
    L.lps_boundary_recv(b, ptr(ys[1]), 1, B.cuda_stream)
    L.lps_boundary_send(b, ptr(xs[2]), 2, B.cuda_stream)
    L.lps_boundary_recv(b, ptr(ys[2]), 2, B.cuda_stream)
    torch.cuda.synchronize()
    for t in range(3):
        assert torch.equal(ys[t], xs[t]), t
    L.lps_boundary_destroy(b)


@pytest.mark.parametrize("d", [2048, 2047])   # 16-byte accesses; odd element count: scalar
def test_f16_pieces_and_combine(L, d):
    rng = np.random.default_rng(14)
    T = 37
    rem = (rng.standard_normal((T, d)) * np.exp(rng.uniform(-6, 6, (T, 1)))).astype(np.float32)
    r16 = torch.zeros((T, d), dtype=torch.int16, device=DEV)
    remd = dev(rem)
    L.lps_f32_to_f16(ptr(remd), ptr(r16), T * d, stream())
    assert np.array_equal(r16.cpu().numpy().view(np.uint16),
                          rem.astype(np.float16).view(np.uint16))
    x0, sh, lo = (rng.standard_normal((T, d)).astype(np.float32) for _ in range(3))
    sr, sm = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    shd, lod = dev(sh), dev(lo)
    for P, alias in ((1, None), (8, None), (8, "bo"), (8, "x"), (3, None), (37, None)):
        x = dev(x0)
        bo = torch.full((T, d), float("nan"), device=DEV)      # poisoned, as a reused buffer
        out = {"bo": bo, "x": x, None: torch.full((T, d), float("nan"), device=DEV)}[alias]
        torch.cuda.synchronize()
        L.lps_moe_combine(ptr(out), ptr(x), ptr(shd), ptr(lod), ptr(r16), ptr(bo), T, d, P,
                          sr.cuda_stream, sm.cuda_stream)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    with pytest.raises(L.LpsError):      # bo may not be an input that is read after it
        L.lps_moe_combine(ptr(out), ptr(x), ptr(shd), ptr(lod), ptr(r16), ptr(lod), T, d, 8,
                          sr.cuda_stream, sm.cuda_stream)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    r32 = f16_pieces_to_f32(rem, 8)
    ref = x0.astype(np.float64) + ((sh.astype(np.float64) + lo) + r32)
    assert np.max(np.abs(outs[0] - ref)) <= 4 * np.spacing(np.abs(ref).max().astype(np.float32))


@pytest.mark.parametrize("d,E", [(2048, 64), (4096, 96)])
def test_moe_route_parity(L, d, E):
    """Router logits (one expert per wave, many workgroups) then one wave per token
    selects: indices equal the oracle's except at certified near ties, at the
    workload's shape and at wider rows with more experts than one wave holds."""
    cfg = synth.MoEConfig("route", n_layers=1, d=d, n_experts=E, top_k=8, ff=16 if d > 2048 else 64,
                          prefill_T=300, steps=0)
    m = synth.make_moe(cfg)
    Lw = m["layers"][0]
    t = {k: dev(Lw[k]) for k in ("g_ffn", "w_r", "w_gu_e", "w_d_e", "w_gu_s", "w_d_s")}
    desc = L.MoEDesc()
    desc.d, desc.n_experts, desc.top_k, desc.ff, desc.remote_from, desc.eps = d, E, 8, cfg.ff, E // 2, cfg.eps
    for k in ("g_ffn", "w_r", "w_gu_e", "w_d_e", "w_gu_s", "w_d_s"):
        setattr(desc, k, ptr(t[k]))
    X = m["x_prefill"]
    T = X.shape[0]
    sb = L.lps_moe_route_scratch_bytes(C.byref(desc), T)
    sc = torch.zeros(sb, dtype=torch.uint8, device=DEV)
    idx = torch.zeros((T, 8), dtype=torch.int32, device=DEV)
    w = torch.zeros((T, 8), dtype=torch.float32, device=DEV)
    Xd = dev(X)
    L.lps_moe_route(C.byref(desc), ptr(Xd), T, ptr(idx), ptr(w), ptr(sc), sb, stream())
    gi, gw = idx.cpu().numpy(), w.cpu().numpy()
    h = rmsnorm(X.astype(np.float64), Lw["g_ffn"], cfg.eps)
    r = h @ onum.bf16_to_f64(Lw["w_r"]).T
    oi, ow = top_k(softmax(r), 8)
    err_r = 2 * (d / 64 + 24) * 2.0 ** -24 * (np.abs(h) @ np.abs(onum.bf16_to_f64(Lw["w_r"])).T)
    near = 0
    for i in range(T):
        if np.array_equal(gi[i], oi[i]):
            assert np.max(np.abs(gw[i] - ow[i])) <= 1e-5
            continue
        # certified near tie: the oracle's order differs only where two logits
        # are closer than twice the bound on the GPU's logit error
        srt = np.sort(r[i])[::-1]
        gaps = np.abs(np.diff(srt[:9]))
        assert gaps.min() <= 2 * err_r[i].max(), (i, gi[i], oi[i])
        near += 1
    assert near <= 3
    # the selection on the GPU's own router logits (left in the scratch, [T, E]
    # f32) is exact: the oracle's top-k of the softmax of the same logits, ties to
    # the lower id, every row, no exceptions; the weights to f32 rounding
    glog = sc[:T * E * 4].view(torch.float32).reshape(T, E).cpu().numpy().astype(np.float64)
    ei, ew = top_k(softmax(glog), 8)
    assert np.array_equal(gi, ei)
    assert np.max(np.abs(gw - ew)) <= 2e-6
    # identical logits in a row: the lowest ids win (the tie rule), also on the GPU
    desc2 = L.MoEDesc()
    ctypes_fields = [f for f, _ in L.MoEDesc._fields_]
    for f in ctypes_fields:
        setattr(desc2, f, getattr(desc, f))
    wz = torch.zeros_like(t["w_r"])                      # a zero router: every logit 0
    desc2.w_r = ptr(wz)
    L.lps_moe_route(C.byref(desc2), ptr(Xd), 4, ptr(idx), ptr(w), ptr(sc), sb, stream())
    assert np.array_equal(idx.cpu().numpy()[:4], np.tile(np.arange(8, dtype=np.int32), (4, 1)))
    assert np.allclose(w.cpu().numpy()[:4], 1 / 8, rtol=0, atol=1e-7)


@pytest.mark.parametrize("d,E,k,ff", [(2048, 64, 8, 1024), (512, 32, 4, 200), (512, 24, 15, 2048),
                                      (256, 16, 4, 2304)])
def test_moe_layer_down_and_combine_equal_slot_gemvs_and_ordered_sum(L, d, E, k, ff):
    """The MoE decode layer's down projections and ordered combine (one launch for
    rows of up to 256 chunks, two above): x' equals, bit for bit, lps_gemv on every
    slot's down matrix with that slot's SwiGLU row (the layer's own selection,
    weights and SwiGLU rows, read from its scratch) followed by the combine done
    on the host in f32 in its order: terms w_j z_j in ascending expert id within
    each half, y = (shared + local) + f32(f16(remote)), x + y.  Ragged rows (ff =
    200: 25 chunks), 16 slots in one workgroup, and the two-launch form (ff = 2304)."""
    cfg = synth.MoEConfig("dc", n_layers=1, d=d, n_experts=E, top_k=k, ff=ff, remote_from=E // 2,
                          prefill_T=0, steps=1)
    m = synth.make_moe(cfg)
    Lw = m["layers"][0]
    t = {n: dev(Lw[n]) for n in ("g_ffn", "w_r", "w_gu_e", "w_d_e", "w_gu_s", "w_d_s")}
    desc = L.MoEDesc()
    desc.d, desc.n_experts, desc.top_k, desc.ff, desc.remote_from, desc.eps = d, E, k, ff, E // 2, cfg.eps
    for n in ("g_ffn", "w_r", "w_gu_e", "w_d_e", "w_gu_s", "w_d_s"):
        setattr(desc, n, ptr(t[n]))
    sb = L.lps_moe_layer_scratch_bytes(C.byref(desc))
    sc = torch.zeros(sb, dtype=torch.uint8, device=DEV)
    x0 = m["x_in"][0]
    x = dev(x0)
    L.lps_moe_layer_decode(C.byref(desc), ptr(x), ptr(sc), sb, stream())
    torch.cuda.synchronize()
    got = x.cpu().numpy()
    # the layer's scratch: ids [16 int32], weights, logits [E], SwiGLU rows [(k+1), ff]
    a256 = lambda n: (n + 255) // 256 * 256
    o_w = a256(16 * 4)
    o_m = o_w + a256(k * 4) + a256(E * 4)
    ids = sc[:4 * k].view(torch.int32).cpu().numpy()
    wts = sc[o_w:o_w + 4 * k].view(torch.float32).cpu().numpy()
    mrows = sc[o_m:o_m + 4 * (k + 1) * ff].view(torch.float32).reshape(k + 1, ff)
    assert len(set(ids.tolist())) == k and ids.min() >= 0 and ids.max() < E
    z = []
    for j in range(k + 1):
        wj = t["w_d_e"][int(ids[j])] if j < k else t["w_d_s"]
        zj = torch.zeros(d, dtype=torch.float32, device=DEV)
        L.lps_gemv(L.LPS_BF16, ptr(wj), None, d, ff, ptr(mrows[j].contiguous()), None, 0.0, ptr(zj),
                   L.LPS_EPI_STORE, stream())
        z.append(zj)
    torch.cuda.synchronize()
    z = np.stack([zj.cpu().numpy() for zj in z])
    order = sorted(range(k), key=lambda j: (int(ids[j]), j))
    f32 = np.float32
    want = np.empty(d, np.float32)
    for r in range(d):
        local, remote = f32(0), f32(0)
        for j in order:
            term = f32(wts[j]) * f32(z[j, r])
            if ids[j] < E // 2:
                local = f32(local + term)
            else:
                remote = f32(remote + term)
        r32 = f32(np.float16(remote))
        y = f32(f32(z[k, r] + local) + r32)
        want[r] = f32(f32(x0[r]) + y)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
