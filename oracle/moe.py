"""Plain float64 MoE FFN layer: router, top-k, experts, fixed-order sums and
the FP16 per-token sums moved in pieces.

Test infrastructure only.  Follows strata PR #3648 ("--peer-device host
route ... in 8 pieces"): one half of the experts returns its per-token sums
as FP16; those sums may be moved and converted piece by piece; the FP16->FP32
conversion is exact and the combine keeps the order of its additions, so any
piece split gives the one-piece result bit for bit (Problem and result;
Approach: sums, the combine kernel, piece bounds).  The combine may be given
an output that is one of its inputs (Approach: the combine kernel reads each
element before writing it).

Readings where the page is silent:
  router     logits r = W_r h; pi = softmax(r) over all experts; the top k by
             pi with ties to the lower expert id, listed by descending pi;
             weights pi_j / sum of the selected pi
  experts    e_j(h) = W_d,j (silu(W_g,j h) * W_u,j h); one shared expert of the
             same shape, ungated, always added
  halves     experts with id < remote_from are summed in f32 ("local"); the
             others form the FP16-returned half ("remote"); inside each half
             the weighted terms are added in ascending expert id
  combine    y = (shared + local) + f32(f16(remote)); x <- f32(x + y)
  pieces     piece p of P covers token rows [floor(pT/P), floor((p+1)T/P))
  prefill    the grouped-GEMM inputs (the normed rows and the SwiGLU output)
             are rounded to bf16 before each expert matrix product; the
             router reads the unrounded rows, as at decode
"""
from __future__ import annotations

import numpy as np

from .decoder import rmsnorm, silu
from .numerics import bf16_to_f64, to_f32, f16_round, f32_to_bf16_bits


def softmax(r):
    r = np.asarray(r, dtype=np.float64)
    z = np.exp(r - r.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def top_k(pi, k):
    """[T, E] -> (idx [T, k] int32 by descending pi, ties to the lower id,
    weights [T, k] = pi_sel / sum pi_sel)."""
    pi = np.asarray(pi, dtype=np.float64)
    order = np.argsort(-pi, axis=-1, kind="stable")[:, :k]
    sel = np.take_along_axis(pi, order, axis=-1)
    return order.astype(np.int32), sel / sel.sum(axis=-1, keepdims=True)


def bf16_round(x):
    return bf16_to_f64(f32_to_bf16_bits(to_f32(x)))


def expert(h, w_gu, w_d, ff, prefill=False):
    """h [T, d] f64 -> [T, d] f64 for one expert (bf16 weight bits)."""
    Wgu = bf16_to_f64(w_gu)
    gu = h @ Wgu.T
    m = silu(gu[:, :ff]) * gu[:, ff:]
    if prefill:
        m = bf16_round(m)
    return m @ bf16_to_f64(w_d).T


def piece_bounds(T, P):
    return [(p * T // P, (p + 1) * T // P) for p in range(P)]


def f16_pieces_to_f32(remote32, P, out=None):
    """Round the remote sums to f16 and widen them back, one piece of rows at a
    time, into a preallocated f32 buffer."""
    remote32 = np.asarray(remote32, dtype=np.float32)
    T = remote32.shape[0]
    if out is None:
        out = np.empty_like(remote32)
    for lo, hi in piece_bounds(T, P):
        out[lo:hi] = f16_round(remote32[lo:hi]).astype(np.float32)
    return out


def combine(x32, shared32, local32, r32, out=None):
    """out = f32(x + ((shared + local) + r32)) elementwise, f64 inside; ``out``
    may be the same array as ``local32`` or ``r32`` (every element is read
    before it is written)."""
    y = (np.asarray(shared32, np.float64) + np.asarray(local32, np.float64)) \
        + np.asarray(r32, np.float64)
    res = to_f32(np.asarray(x32, np.float64) + y)
    if out is None:
        return res
    out[...] = res
    return out


def moe_layer(x32, L, cfg, prefill=False, n_pieces=1, forced_idx=None, trace=None):
    """x32 [T, d] f32 -> [T, d] f32.  forced_idx: routing to use instead of the
    oracle's own top-k (near-tie adoption).  trace: dict that receives the
    router logits, idx, weights and the three partial sums."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    T = x.shape[0]
    ff, E, k = cfg.ff, cfg.n_experts, cfg.top_k
    h = rmsnorm(x, L["g_ffn"], cfg.eps)
    r = h @ bf16_to_f64(L["w_r"]).T               # the router reads the unrounded rows
    if prefill:
        h = bf16_round(h)
    pi = softmax(r)
    idx, w = top_k(pi, k)
    if forced_idx is not None:
        idx = np.asarray(forced_idx, dtype=np.int32)
        sel = np.take_along_axis(pi, idx.astype(np.int64), axis=-1)
        w = sel / sel.sum(axis=-1, keepdims=True)
    shared = expert(h, L["w_gu_s"], L["w_d_s"], ff, prefill)
    local = np.zeros_like(x)
    remote = np.zeros_like(x)
    for e in range(E):                              # ascending expert id
        rows, slot = np.nonzero(idx == e)
        if rows.size == 0:
            continue
        contrib = w[rows, slot][:, None] * expert(h[rows], L["w_gu_e"][e], L["w_d_e"][e], ff, prefill)
        if e < cfg.remote_from:
            local[rows] += contrib
        else:
            remote[rows] += contrib
    r32 = f16_pieces_to_f32(to_f32(remote), n_pieces)
    out = combine(to_f32(x), to_f32(shared), to_f32(local), r32)
    if trace is not None:
        trace.update(logits=r, idx=idx, w=w, shared=shared, local=local, remote=remote, r32=r32)
    return out


class MoEStack:
    """The MoE FFN layer stack (no attention, no head): x <- x + MoE(RMSNorm(x))."""

    def __init__(self, model):
        self.m = model
        self.cfg = model["cfg"]

    def forward(self, x32, prefill=False, n_pieces=1, forced=None, traces=None):
        x = np.asarray(x32, dtype=np.float32)
        squeeze = x.ndim == 1
        if squeeze:
            x = x[None]
        for l, L in enumerate(self.m["layers"]):
            tr = {} if traces is not None else None
            x = moe_layer(x, L, self.cfg, prefill=prefill, n_pieces=n_pieces,
                          forced_idx=None if forced is None else forced[l], trace=tr)
            if traces is not None:
                traces.append(tr)
        return x[0] if squeeze else x
