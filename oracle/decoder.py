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
by 1/sqrt(hd); silu(z) = z / (1 + e^-z); the argmax takes the first maximum.
"""
from __future__ import annotations

import math

import numpy as np

from .numerics import (to_f32, round_cache, widen_cache, widen_weight)
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

    # ---- stages, embedding, head --------------------------------------------
    def embed(self, tok):
        return to_f32(widen_weight(self.m["embed"][int(tok)], self.cfg.wdtype))

    def head(self, x32):
        hf = rmsnorm(np.asarray(x32, np.float32).astype(np.float64), self.m["g_out"], self.cfg.eps)
        logits = self.mv(-1, "w_lm", hf)
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
