"""Plain float64 decoder forward over contiguous layer stages.

Test infrastructure only.  The block is the plain pre-norm decoder the pages
name the pieces of: RMSNorm, a fused QKV projection whose q heads read kv head
h // (nq / nkv) (TP3 zero-padded dummy heads plan, Implementation status and
Geometry), rotary position embedding, attention over the layer's own cache,
the output projection into the residual, RMSNorm again and a gated MLP whose
fused gate/up matrix holds the gate rows and then the up rows (ninfer "Layer
pipeline stages", Tensor parallelism: status).  The hidden state is stored
as f32 between sublayers and is the only tensor that crosses a stage boundary
(memra ``pp`` module docs, header: ownership across a boundary); the embedding
belongs to stage 0 and the final norm + LM head to the last stage.

Readings where the pages are silent: no biases, no QK norm, no attention
output gate; RMSNorm y = x / sqrt(mean(x^2) + eps) * g; RoPE rotates the pairs
(i, i + hd/2) of every q and k head by p * base^(-2i/hd) at the 0-based
position p; attention is causal over rows 0..p after row p is written, scaled
by 1/sqrt(hd); silu(z) = z / (1 + e^-z); the argmax takes the first maximum,
and a step whose logits hold a NaN has none: its id is vocab, which the next
embedding turns into a NaN row (a poisoned step stays poisoned).

Chunked prefill (memra ``pp`` module docs, functions on the prime split; ninfer
pipeline stages, What is not covered yet: a prefill chunk runs through the
stages in turn): a chunk of T prompt rows goes through each layer as whole-chunk
matrix products; its K and V rows are stored first and each row attends
causally.  Where the pages leave the precision open, the operands the matrix
cores take are rounded to bf16 (the normed rows, the attention output, the
SwiGLU output), everything else is as in decode: attention takes q and its
softmax weights exact, as the decode step does.  With those roundings off the
matrix form reproduces the decode steps exactly (pinned in the tests).
"""
from __future__ import annotations

import math

import numpy as np

from .numerics import (to_f32, round_cache, widen_cache, widen_weight, bf16_to_f64,
                       f32_to_bf16_bits)
from .plan import stage_plan


def rmsnorm(x, g, eps):
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


def rope(u, p, base):
    """u [n_heads, hd] -> rotated copy (rotate-half pairs (i, i + hd/2))."""
    u = np.asarray(u, dtype=np.float64)
    hd = u.shape[-1]
    half = hd // 2
    theta = np.power(float(base), -2.0 * np.arange(half, dtype=np.float64) / hd)
    a = float(p) * theta
    c, s = np.cos(a), np.sin(a)
    lo, hi = u[..., :half], u[..., half:]
    return np.concatenate([lo * c - hi * s, lo * s + hi * c], axis=-1)


def attend(q, K, V):
    """GQA decode attention. q [nq, hd]; K, V [nkv, n, hd] (rows 0..n-1 visible)."""
    nq, hd = q.shape
    nkv = K.shape[0]
    G = nq // nkv
    o = np.empty_like(q, dtype=np.float64)
    for h in range(nq):
        g = h // G
        s = (K[g] @ q[h]) / math.sqrt(hd)
        w = np.exp(s - s.max())
        w /= w.sum()
        o[h] = w @ V[g]
    return o


def silu(z):
    return z / (1.0 + np.exp(-z))


def bf16_act(x64):
    """An activation as a matrix-core operand: f64 -> f32 -> bf16 (nearest even),
    returned widened to f64."""
    return bf16_to_f64(f32_to_bf16_bits(to_f32(x64)))


def causal_attend(Q, K, V, p0):
    """Causal attention over a chunk in matrix form.  Q [T, nq, hd] (rows at
    positions p0 .. p0+T-1); K, V [nkv, p0+T, hd].  Row t sees cache rows
    0 .. p0+t: S = Q K^T / sqrt(hd) with the rows past p0+t masked out, a row
    softmax, O = P V.  Returns O [T, nq, hd].

    q and the softmax weights are not rounding points: the chunk's attention is
    the plain definition, as in the decode step (the cached K and V rows carry
    the cache dtype's rounding)."""
    T, nq, hd = Q.shape
    nkv, n, _ = K.shape
    G = nq // nkv
    visible = np.arange(n)[None, :] <= (p0 + np.arange(T))[:, None]     # [T, n]
    O = np.empty((T, nq, hd), dtype=np.float64)
    for h in range(nq):
        g = h // G
        S = (Q[:, h, :] @ K[g].T) / math.sqrt(hd)
        S = np.where(visible, S, -np.inf)
        W = np.exp(S - S.max(axis=1, keepdims=True))
        O[:, h, :] = (W @ V[g]) / W.sum(axis=1, keepdims=True)
    return O


def matvec_grouped(W, h, group=32):
    """y = W h summed over K in ascending groups of 32 columns (the MXFP4 scale
    groups): each group's 32 products are summed, then the group sums are
    accumulated left to right (a cumulative sum is strictly sequential), so
    zero groups appended at the end of K leave y unchanged."""
    N, K = W.shape
    Wg = W.reshape(N, K // group, group)
    hg = np.asarray(h, dtype=np.float64).reshape(K // group, group)
    part = (Wg * hg).sum(axis=2)                 # [N, K/32]
    return np.cumsum(part, axis=1)[:, -1]


_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        import os
        from concurrent.futures import ThreadPoolExecutor
        _POOL = ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0)))))
    return _POOL


class Decoder:
    """One model, its per-layer KV caches and the staged walk.

    model: a dict from ``synth`` (cfg, layers[...], optional embed / g_out /
    w_lm / k_prefix / v_prefix).  weight_cache=True keeps widened f64 copies."""

    def __init__(self, model: dict, weight_cache: bool = True):
        self.m = model
        self.cfg = model["cfg"]
        self._wc = {} if weight_cache else None
        self.counters = {"stage_walks": 0, "boundary_crossings": 0}
        self.reset()

    # ---- state -----------------------------------------------------------
    def reset(self):
        c = self.cfg
        self.K, self.V = [], []
        sdt = np.float32 if c.kvdtype == "f32" else np.uint16
        for L in self.m["layers"]:
            K = np.zeros((c.nkv, c.ctx_max, c.hd), dtype=sdt)
            V = np.zeros_like(K)
            if c.prefix:
                K[:, :c.prefix] = L["k_prefix"]
                V[:, :c.prefix] = L["v_prefix"]
            self.K.append(K)
            self.V.append(V)

    def W(self, l, name):
        key = (l, name)
        if self._wc is not None and key in self._wc:
            return self._wc[key]
        src = self.m["layers"][l][name] if l >= 0 else self.m[name]
        w = widen_weight(src, self.cfg.wdtype)
        if self._wc is not None:
            self._wc[key] = w
        return w

    def mv(self, l, name, h):
        if self.cfg.wdtype == "mxfp4" and self._wc is None:
            return self._mv_mxfp4_rows(l, name, h)
        W = self.W(l, name)
        if self.cfg.wdtype == "mxfp4":
            return matvec_grouped(W, h)
        return W @ h

    def _mv_mxfp4_rows(self, l, name, h, rows=1024):
        """Same result as matvec_grouped(widen(W), h) (every row is computed
        alone); rows are widened a block at a time on a thread pool so the whole
        f64 matrix never exists at once."""
        codes, scales = self.m["layers"][l][name] if l >= 0 else self.m[name]
        N = codes.shape[0]
        y = np.empty(N, dtype=np.float64)

        def block(i):
            lo, hi = i * rows, min(N, (i + 1) * rows)
            y[lo:hi] = matvec_grouped(widen_weight((codes[lo:hi], scales[lo:hi]), "mxfp4"), h)

        list(_pool().map(block, range((N + rows - 1) // rows)))
        return y

    # ---- one layer ---------------------------------------------------------
    def layer(self, l, x32, p):
        c = self.cfg
        L = self.m["layers"][l]
        nq, nkv, hd = c.nq, c.nkv, c.hd
        x = np.asarray(x32, dtype=np.float32).astype(np.float64)
        h = rmsnorm(x, L["g_attn"], c.eps)
        qkv = self.mv(l, "w_qkv", h)
        q = rope(qkv[:nq * hd].reshape(nq, hd), p, c.rope_base)
        k = rope(qkv[nq * hd:(nq + nkv) * hd].reshape(nkv, hd), p, c.rope_base)
        v = qkv[(nq + nkv) * hd:].reshape(nkv, hd)
        self.K[l][:, p] = round_cache(k, c.kvdtype)
        self.V[l][:, p] = round_cache(v, c.kvdtype)
        Kc = widen_cache(self.K[l][:, :p + 1], c.kvdtype)
        Vc = widen_cache(self.V[l][:, :p + 1], c.kvdtype)
        o = attend(q, Kc, Vc).reshape(-1)
        x = to_f32(x + self.mv(l, "w_o", o)).astype(np.float64)
        h2 = rmsnorm(x, L["g_ffn"], c.eps)
        gu = self.mv(l, "w_gu", h2)
        mm = silu(gu[:c.ff]) * gu[c.ff:]
        return to_f32(x + self.mv(l, "w_d", mm))

    # ---- a prefill chunk (matrix form) -----------------------------------------
    def layer_prefill(self, l, X32, p0, act=bf16_act):
        """One layer over a chunk of T prompt rows at positions p0 .. p0+T-1,
        written as the whole-chunk matrix products.  The chunk's K and V rows
        are rotated and stored first; each row then attends causally.  `act`
        rounds the operands the matrix cores take in prefill: the normed rows,
        the attention output and the SwiGLU output (bf16); the residual stays
        f32 between sublayers, every sum is f64.  act=None keeps them exact,
        which must reproduce the decode steps row by row.  Attention itself
        takes q and the softmax weights exact (causal_attend)."""
        act = act or (lambda a: a)
        c = self.cfg
        L = self.m["layers"][l]
        nq, nkv, hd = c.nq, c.nkv, c.hd
        X = np.asarray(X32, dtype=np.float32).astype(np.float64)
        T = X.shape[0]
        H = act(rmsnorm(X, L["g_attn"], c.eps))
        QKV = H @ self.W(l, "w_qkv").T                                   # [T, N]
        Q = np.stack([rope(QKV[t, :nq * hd].reshape(nq, hd), p0 + t, c.rope_base)
                      for t in range(T)])
        Kn = np.stack([rope(QKV[t, nq * hd:(nq + nkv) * hd].reshape(nkv, hd), p0 + t,
                            c.rope_base) for t in range(T)])
        Vn = QKV[:, (nq + nkv) * hd:].reshape(T, nkv, hd)
        self.K[l][:, p0:p0 + T] = round_cache(Kn.transpose(1, 0, 2), c.kvdtype)
        self.V[l][:, p0:p0 + T] = round_cache(Vn.transpose(1, 0, 2), c.kvdtype)
        Kc = widen_cache(self.K[l][:, :p0 + T], c.kvdtype)
        Vc = widen_cache(self.V[l][:, :p0 + T], c.kvdtype)
        O = causal_attend(Q, Kc, Vc, p0).reshape(T, nq * hd)
        X = to_f32(X + act(O) @ self.W(l, "w_o").T).astype(np.float64)
        H2 = act(rmsnorm(X, L["g_ffn"], c.eps))
        GU = H2 @ self.W(l, "w_gu").T
        M = act(silu(GU[:, :c.ff]) * GU[:, c.ff:])
        return to_f32(X + M @ self.W(l, "w_d").T)

    def prefill(self, ids, p0=None, fence=None, act=bf16_act):
        """A chunk of prompt ids through every stage from position p0 (default:
        just after the cache prefix): embedding rows, each stage's layers over
        the whole chunk, the [T, d] f32 hidden through a slot between stages,
        then the head on the last row.  Returns (last logits, argmax, hidden
        rows [T, d] of the last stage)."""
        c = self.cfg
        p = c.prefix if p0 is None else p0
        if fence is None:
            fence = stage_plan(c.n_layers, 1)
        n = len(fence) - 1
        X = np.stack([self.embed(t) for t in ids])
        for s in range(n):
            for l in range(fence[s], fence[s + 1]):
                X = self.layer_prefill(l, X, p, act)
            self.counters["stage_walks"] += 1
            if s < n - 1:
                X = X.copy()
                self.counters["boundary_crossings"] += 1
        logits, a = self.head(X[-1])
        return logits, a, X

    # ---- stages, embedding, head --------------------------------------------
    def embed(self, tok):
        """The embedding row of an id; an id outside the table has no row: a NaN
        row stands for it, so a poisoned step stays poisoned."""
        if not 0 <= int(tok) < self.cfg.vocab:
            return np.full(self.cfg.d, np.nan, dtype=np.float32)
        return to_f32(widen_weight(self.m["embed"][int(tok)], self.cfg.wdtype))

    def head(self, x32):
        """Logits and the first maximum; logits holding a NaN have no maximum and
        give the id vocab (outside the table)."""
        hf = rmsnorm(np.asarray(x32, np.float32).astype(np.float64), self.m["g_out"], self.cfg.eps)
        logits = self.mv(-1, "w_lm", hf)
        if np.isnan(logits).any():
            return logits, self.cfg.vocab
        return logits, int(np.argmax(logits))

    def walk(self, x32, p, fence=None):
        """All stages in order; after every stage but the last the hidden goes
        through an f32 boundary slot (a copy of what is already f32)."""
        c = self.cfg
        if fence is None:
            fence = stage_plan(c.n_layers, 1)
        n = len(fence) - 1
        x = np.asarray(x32, dtype=np.float32)
        for s in range(n):
            for l in range(fence[s], fence[s + 1]):
                x = self.layer(l, x, p)
            self.counters["stage_walks"] += 1
            if s < n - 1:
                slot = np.empty(c.d, dtype=np.float32)
                slot[:] = x
                x = slot.copy()
                self.counters["boundary_crossings"] += 1
        return x

    def step(self, inp, p, fence=None):
        """One decode step at position p.  inp: a token id (models with a
        vocabulary) or an f32 hidden row.  Returns (logits, argmax) or the
        output hidden."""
        if self.cfg.vocab:
            x = self.embed(inp)
            return self.head(self.walk(x, p, fence))
        return self.walk(inp, p, fence)

    def greedy(self, prompt, n_steps, p0=None, fence=None, feed=None):
        """Feed the prompt ids one per step from position p0 (default: just
        after the cache prefix), then n_steps greedy steps that each feed the
        previous step's argmax.  feed: a full list of ids to feed instead
        (teacher forcing: the oracle follows another decoder's tokens).
        Returns (fed ids, argmax per step, logits per step)."""
        c = self.cfg
        p = c.prefix if p0 is None else p0
        P = len(prompt)
        total = P + n_steps if feed is None else len(feed)
        fed, am, out = [], [], []
        for i in range(total):
            if feed is not None:
                t = int(feed[i])
            else:
                t = int(prompt[i]) if i < P else am[-1]
            logits, a = self.step(t, p + i, fence)
            fed.append(t)
            am.append(a)
            out.append(logits)
        return fed, am, out
