"""Decode driver over liblps: device buffers and streams from PyTorch, every
step of the path in the library's kernels.

memra-engine `pp` module docs (header): the trunk is cut into N stages with a
stream each; N-1 boundary runtimes with two persistent slots and
ev_tx / ev_rx events carry the [n_embd] f32 hidden; the embedding lives with
stage 0, the final norm and LM head with the last stage; a step's logits stay
on the device and drain through a dedicated readback stream while later
steps keep being enqueued (struct PendingLogits).  ninfer "Multi-GPU: layer
pipeline stages" (What it is and is not): repeating one device id runs the
whole staged path on a single card, which is what this driver does: every
stage is a stream on the same GPU.

Nothing here computes: this module allocates, uploads, picks pointers and
calls the C entry points in order.  There is no CPU fallback; without the
built library or a GPU, construction fails.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import numpy as np
import torch

from . import _lib as lps
from . import layout


def _need_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("liblps needs a ROCm GPU (gfx950); none is visible")
    lps.load()


def to_dev(a: np.ndarray, device) -> torch.Tensor:
    """Upload a numpy array unchanged (uint16 bf16 bits travel as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device, non_blocking=False)


def ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def sp(stream) -> int:
    """hipStream_t of a torch stream, as an int for ctypes."""
    return stream.cuda_stream


def _weight(w, device):
    if isinstance(w, tuple):  # MXFP4 (codes, scales)
        return to_dev(w[0], device), to_dev(w[1], device)
    return to_dev(w, device), None


def _row_bytes(wdtype: str, k: int) -> int:
    """Bytes of one weight row of length k (MXFP4: k/2 codes + k/32 scales)."""
    return {"f32": 4 * k, "bf16": 2 * k, "mxfp4": k // 2 + k // 32}[wdtype]


def memory_balanced_fence(n_layers, d, nq, nkv, hd, ff, vocab, wdtype, kvdtype, n_stages,
                          free_bytes, page_tokens=16, stage_overhead=0, max_groups=1 << 30):
    """Split for devices with free_bytes[s] each, by lps_stage_solve (ninfer
    "Multi-GPU: layer pipeline stages", How it works: the most KV page groups
    every stage can hold, then the least-full stage).  A layer's fixed bytes are
    its weights and norm gains; its KV bytes per page group are K and V rows of
    page_tokens positions.  The embedding counts on stage 0 and the final norm
    and LM head on the last stage (where this path runs them), plus
    stage_overhead on every stage.  Returns (fence, page groups)."""
    layer_w = ((nq + 2 * nkv) * hd * _row_bytes(wdtype, d) + d * _row_bytes(wdtype, nq * hd)
               + 2 * ff * _row_bytes(wdtype, d) + d * _row_bytes(wdtype, ff) + 2 * d * 4)
    kv = 2 * nkv * hd * page_tokens * (4 if kvdtype == "f32" else 2)
    emb = vocab * _row_bytes("bf16" if wdtype == "mxfp4" else wdtype, d)
    over = [stage_overhead] * n_stages
    over[0] += emb
    over[-1] += emb + d * 4
    return lps.stage_solve(list(free_bytes), over, [layer_w] * n_layers, [kv] * n_layers,
                           n_stages, max_groups)


def mark_schedule(total, ring, mark_every):
    """The replay loop's marks: marked(i) says whether a pending follows replay i
    (every mark_every-th and the last; mark_every is capped at ring - 1 so that
    the mark covering step i is launched before step i + ring reuses its row), and
    cover(i) is the first marked step at or after i, whose pending the drain of
    step i waits for."""
    m = max(1, min(mark_every, ring - 1))

    def marked(i):
        return i % m == m - 1 or i == total - 1

    def cover(i):
        return min(i + (m - 1 - i % m), total - 1)

    return marked, cover


def _hop(b, src, dst, step, producer, consumer):
    """One boundary crossing: the send and the receive, or on the same-stream seam
    the single-kernel hop."""
    if producer is consumer:
        lps.lps_boundary_hop(b, src, dst, step, sp(producer))
    else:
        lps.lps_boundary_send(b, src, step, sp(producer))
        lps.lps_boundary_recv(b, dst, step, sp(consumer))


@dataclass
class StepResult:
    fed: list
    argmax: list
    logits: list


class DeviceDecoder:
    """A synth decoder model (dense f32/bf16 or MXFP4) resident on one GPU,
    walked as N stages on N streams of that GPU."""

    def __init__(self, model: dict, fence=None, device="cuda:0", ring: int = 4,
                 streams: str = "per-stage"):
        _need_gpu()
        self.cfg = cfg = model["cfg"]
        self.device = torch.device(device)
        self.ring = ring
        dev = self.device
        wdt = lps.DTYPES[cfg.wdtype]
        kvdt = lps.DTYPES[cfg.kvdtype]
        self.layers = []
        descs = (lps.LayerDesc * cfg.n_layers)()
        # cache rows: bf16 caches are stored in 16-row tiles (layout.py) and need
        # the row count to be a multiple of 16
        self.ctx_rows = ctx = (cfg.ctx_max + 15) // 16 * 16
        self.tiled = cfg.kvdtype == "bf16"
        # cos / sin of every cache position, read by the device-position walk
        self.rope_cs = to_dev(lps.rope_table(cfg.hd, cfg.rope_base, ctx), dev)
        kv_torch = torch.float32 if cfg.kvdtype == "f32" else torch.int16
        for l, L in enumerate(model["layers"]):
            t = {}
            t["g_attn"] = to_dev(L["g_attn"], dev)
            t["g_ffn"] = to_dev(L["g_ffn"], dev)
            for n in ("w_qkv", "w_o", "w_gu", "w_d"):
                t[n], t["s" + n[1:]] = _weight(L[n], dev)
            if self.tiled:
                kshape = (cfg.nkv, ctx // 16, cfg.hd // 8, 16, 8)
                vshape = (cfg.nkv, ctx // 16, cfg.hd, 16)
            else:
                kshape = vshape = (cfg.nkv, ctx, cfg.hd)
            t["k"] = torch.zeros(kshape, dtype=kv_torch, device=dev)
            t["v"] = torch.zeros(vshape, dtype=kv_torch, device=dev)
            if cfg.prefix:
                t["k_prefix"] = to_dev(L["k_prefix"], dev)
                t["v_prefix"] = to_dev(L["v_prefix"], dev)
            self.layers.append(t)
            d = descs[l]
            d.d, d.nq, d.nkv, d.hd, d.ff = cfg.d, cfg.nq, cfg.nkv, cfg.hd, cfg.ff
            d.wdtype, d.kvdtype, d.ctx_max = wdt, kvdt, ctx
            d.eps, d.rope_base = cfg.eps, cfg.rope_base
            d.g_attn, d.g_ffn = ptr(t["g_attn"]), ptr(t["g_ffn"])
            d.w_qkv, d.s_qkv = ptr(t["w_qkv"]), ptr(t["s_qkv"])
            d.w_o, d.s_o = ptr(t["w_o"]), ptr(t["s_o"])
            d.w_gu, d.s_gu = ptr(t["w_gu"]), ptr(t["s_gu"])
            d.w_d, d.s_d = ptr(t["w_d"]), ptr(t["s_d"])
            d.k_cache, d.v_cache = ptr(t["k"]), ptr(t["v"])
            d.rope_cs = ptr(self.rope_cs)
        self.descs = descs
        h = C.c_void_p()
        lps.lps_model_create(descs, cfg.n_layers, C.byref(h))
        self.model = h
        self.scratch_bytes = lps.lps_model_scratch_bytes(h)
        self.head = None
        if cfg.vocab:
            self.embed = to_dev(model["embed"], dev)
            self.g_out = to_dev(model["g_out"], dev)
            self.w_lm = to_dev(model["w_lm"], dev)
            hd = lps.HeadDesc()
            hd.d, hd.vocab, hd.wdtype, hd.eps = cfg.d, cfg.vocab, wdt, cfg.eps
            hd.g_out, hd.w_lm = ptr(self.g_out), ptr(self.w_lm)
            self.head = hd
            self.head_scratch = torch.zeros(lps.lps_head_scratch_bytes(C.byref(hd)),
                                            dtype=torch.uint8, device=dev)
            self.logits_ring = torch.zeros((ring, cfg.vocab), dtype=torch.float32, device=dev)
            self.tok_ring = torch.zeros(ring, dtype=torch.int32, device=dev)
            self.host_logits = torch.zeros((ring, cfg.vocab), dtype=torch.float32).pin_memory()
            self.host_tok = torch.zeros(ring, dtype=torch.int32).pin_memory()
            # the graph mode's next input id, this step's argmax and logits
            self.g_tok = torch.zeros(1, dtype=torch.int32, device=dev)
            self.g_logits = torch.zeros(cfg.vocab, dtype=torch.float32, device=dev)
        # device step state of the graph mode: [pos, step, flags]
        self.g_state = torch.zeros(4, dtype=torch.int32, device=dev)
        self.readback = torch.cuda.Stream(device=dev)
        self._streams_mode = streams
        self.reset()
        self.set_fence(fence)

    # ---- stage plan / stage runtime ----------------------------------------------
    def set_fence(self, fence=None):
        cfg = self.cfg
        if fence is None:
            fence = lps.stage_plan(cfg.n_layers, 1)
        fence = list(fence)
        # the library validates the cuts; the ends must be 0 and n_layers
        plan = lps.stage_plan(cfg.n_layers, len(fence) - 1, fence[1:-1]) if len(fence) >= 2 else None
        if plan != fence:
            raise lps.LpsError(lps.LPS_EINVAL, f"fence {fence} is not a plan of {cfg.n_layers} layers")
        self.fence = fence
        self.n_stages = n = len(fence) - 1
        self._fence_c = lps.i32_array(fence)
        dev = self.device
        if self._streams_mode == "single":
            s = torch.cuda.Stream(device=dev)
            self.streams = [s] * n
        else:
            self.streams = [torch.cuda.Stream(device=dev) for _ in range(n)]
        self.x = [torch.zeros(cfg.d, dtype=torch.float32, device=dev) for _ in range(n)]
        self.scratch = [torch.zeros(self.scratch_bytes, dtype=torch.uint8, device=dev)
                        for _ in range(n)]
        self._close_boundaries()
        self.slots, self.bounds = [], []
        for _ in range(n - 1):
            s0 = torch.full((cfg.d,), float("nan"), dtype=torch.float32, device=dev)
            s1 = torch.full((cfg.d,), float("nan"), dtype=torch.float32, device=dev)
            b = C.c_void_p()
            lps.lps_boundary_create(cfg.d, ptr(s0), ptr(s1), C.byref(b))
            self.slots.append((s0, s1))
            self.bounds.append(b)
        self.step_no = 0   # boundary step counter (monotone across runs)
        torch.cuda.synchronize(dev)

    def _close_boundaries(self):
        for b in getattr(self, "bounds", []) + getattr(self, "_pf_bounds", []):
            lps.lps_boundary_destroy(b)
        self.bounds = []
        self._pf_bounds = []
        self._pf_key = None

    def reset(self):
        """Restore every cache to its seeded prefix (rows past it are rewritten
        before they are read)."""
        for t in self.layers:
            if "k_prefix" in t:
                P = t["k_prefix"].shape[1]
                if self.tiled:
                    # whole tiles: rows P .. P16 - 1 get zeros (written before read)
                    P16 = (P + 15) // 16 * 16
                    for name, to_tiles in (("k", layout.k_to_tiles), ("v", layout.v_to_tiles)):
                        src = t[name + "_prefix"]
                        rows = torch.zeros((src.shape[0], P16, src.shape[2]), dtype=src.dtype,
                                           device=self.device)
                        rows[:, :P].copy_(src)
                        t[name][:, :P16 // 16].copy_(to_tiles(rows))
                else:
                    t["k"][:, :P].copy_(t["k_prefix"])
                    t["v"][:, :P].copy_(t["v_prefix"])
        torch.cuda.synchronize(self.device)

    def close(self):
        torch.cuda.synchronize(self.device)
        self._close_boundaries()
        if getattr(self, "model", None):
            lps.lps_model_destroy(self.model)
            self.model = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- one step ------------------------------------------------------------------
    def _walk(self, pos):
        """Enqueue all stages of one step; stage 0's input is already in x[0]."""
        n, st = self.n_stages, self.streams
        t = self.step_no
        for s in range(n):
            if s > 0:
                _hop(self.bounds[s - 1], ptr(self.x[s - 1]), ptr(self.x[s]), t, st[s - 1], st[s])
            lps.lps_stage_forward(self.model, self._fence_c, n, s, ptr(self.x[s]), pos,
                                  ptr(self.scratch[s]), self.scratch_bytes, sp(st[s]))
        self.step_no += 1

    def run_tokens(self, prompt, n_steps=0, feed=None, p0=None) -> StepResult:
        """Feed the prompt ids one per step from position p0 (default: right after
        the cache prefix), then n_steps greedy steps whose token is the device
        argmax of the step before (it never visits the host).  feed: a full id
        list to feed instead (teacher forcing).  Logits drain through the
        readback ring; the host runs up to `ring` steps ahead of the GPU."""
        cfg = self.cfg
        assert self.head is not None, "model has no vocabulary"
        p = cfg.prefix if p0 is None else p0
        ids = list(prompt) if feed is None else list(feed)
        P = len(ids)
        total = P + (0 if feed is not None else n_steps)
        assert p + total <= cfg.ctx_max, "cache too short for this run"
        dev = self.device
        feed_dev = torch.tensor(ids + [0], dtype=torch.int32, device=dev)
        torch.cuda.synchronize(dev)
        st0, stl = self.streams[0], self.streams[-1]
        done = [torch.cuda.Event() for _ in range(self.ring)]
        pend = [None] * self.ring
        out_logits, out_tok = [None] * total, [None] * total
        R = self.ring

        def drain(i):
            lps.lps_pending_wait(pend[i % R])
            pend[i % R] = None
            out_logits[i] = self.host_logits[i % R].numpy().copy()
            out_tok[i] = int(self.host_tok[i % R])

        for i in range(total):
            if i >= R:
                drain(i - R)
            if i < P:
                tok_ptr = ptr(feed_dev) + 4 * i
            else:
                tok_ptr = ptr(self.tok_ring) + 4 * ((i - 1) % R)
                if stl is not st0:
                    st0.wait_event(done[(i - 1) % R])
            lps.lps_embed(ptr(self.embed), lps.DTYPES[cfg.wdtype], cfg.vocab, cfg.d, tok_ptr,
                          ptr(self.x[0]), sp(st0))
            self._walk(p + i)
            k = i % R
            lps.lps_head_forward(C.byref(self.head), ptr(self.x[-1]), ptr(self.logits_ring[k]),
                                 ptr(self.tok_ring) + 4 * k, ptr(self.head_scratch),
                                 self.head_scratch.numel(), sp(stl))
            if stl is not st0:
                done[k].record(stl)
            h = C.c_void_p()
            lps.lps_logits_defer(ptr(self.logits_ring[k]), ptr(self.tok_ring) + 4 * k, cfg.vocab,
                                 sp(stl), sp(self.readback), ptr(self.host_logits[k]),
                                 ptr(self.host_tok) + 4 * k, C.byref(h))
            pend[k] = h
        for i in range(max(0, total - R), total):
            drain(i)
        fed = ids[:P] + [out_tok[i - 1] for i in range(P, total)]
        return StepResult(fed=fed, argmax=out_tok, logits=out_logits)

    # ---- chunked prefill through the stages ----------------------------------------
    def _prefill_buffers(self, T):
        """Per-stage [T, d] hidden rows and prefill scratch, and boundaries whose
        slots carry a whole chunk; rebuilt when the chunk size or fence changes."""
        key = (T, tuple(self.fence))
        if getattr(self, "_pf_key", None) == key:
            return
        cfg, dev, n = self.cfg, self.device, self.n_stages
        for b in getattr(self, "_pf_bounds", []):
            lps.lps_boundary_destroy(b)
        self._pf_x = [torch.zeros((T, cfg.d), dtype=torch.float32, device=dev) for _ in range(n)]
        nb = lps.lps_prefill_scratch_bytes(self.model, T)
        self._pf_scratch = [torch.zeros(nb, dtype=torch.uint8, device=dev) for _ in range(n)]
        self._pf_slots, self._pf_bounds = [], []
        for _ in range(n - 1):
            s0 = torch.zeros((T, cfg.d), dtype=torch.float32, device=dev)
            s1 = torch.zeros_like(s0)
            b = C.c_void_p()
            lps.lps_boundary_create(T * cfg.d, ptr(s0), ptr(s1), C.byref(b))
            self._pf_slots.append((s0, s1))
            self._pf_bounds.append(b)
        self._pf_step = 0
        self._pf_key = key
        torch.cuda.synchronize(dev)

    def prefill(self, ids, chunk=None, p0=None, hidden=True):
        """Feed the prompt ids as chunks of `chunk` rows (default: all at once)
        from position p0 (default: right after the cache prefix), each chunk
        through every stage in turn (a [T, d] f32 block per boundary), then the
        head on the prompt's last row.  Returns (logits, argmax, last stage's
        hidden rows of the last chunk, or None with hidden=False)."""
        cfg = self.cfg
        assert self.head is not None, "model has no vocabulary"
        ids = list(ids)
        p = cfg.prefix if p0 is None else p0
        chunk = len(ids) if chunk is None else chunk
        assert ids and p + len(ids) <= cfg.ctx_max, "cache too short for this prompt"
        self._prefill_buffers(chunk)
        dev, n, st = self.device, self.n_stages, self.streams
        tok_dev = torch.tensor(ids, dtype=torch.int32, device=dev)
        torch.cuda.synchronize(dev)
        T = 0
        for c0 in range(0, len(ids), chunk):
            T = min(chunk, len(ids) - c0)
            lps.lps_embed_rows(ptr(self.embed), lps.DTYPES[cfg.wdtype], cfg.vocab, cfg.d,
                               ptr(tok_dev) + 4 * c0, T, ptr(self._pf_x[0]), sp(st[0]))
            k = self._pf_step
            for s in range(n):
                if s > 0:
                    lps.lps_boundary_send(self._pf_bounds[s - 1], ptr(self._pf_x[s - 1]), k,
                                          sp(st[s - 1]))
                    lps.lps_boundary_recv(self._pf_bounds[s - 1], ptr(self._pf_x[s]), k, sp(st[s]))
                lps.lps_stage_prefill(self.model, self._fence_c, n, s, ptr(self._pf_x[s]), T, p,
                                      ptr(self._pf_scratch[s]), self._pf_scratch[s].numel(),
                                      sp(st[s]))
            self._pf_step += 1
            p += T
        last = ptr(self._pf_x[-1]) + 4 * cfg.d * (T - 1)
        lps.lps_head_forward(C.byref(self.head), last, ptr(self.logits_ring[0]),
                             ptr(self.tok_ring), ptr(self.head_scratch),
                             self.head_scratch.numel(), sp(st[-1]))
        torch.cuda.synchronize(dev)
        X = self._pf_x[-1][:T].cpu().numpy().copy() if hidden else None
        return self.logits_ring[0].cpu().numpy().copy(), int(self.tok_ring[0]), X

    # ---- the whole pass as one graph --------------------------------------------
    def _walk_dpos(self):
        """Enqueue all stages of one step, the position read from g_state[0].  On
        one stream each boundary hop is folded into the producing stage's last
        launch (lps_stage_forward_dpos_hop)."""
        n, st = self.n_stages, self.streams
        t = self.step_no
        pos_dev = ptr(self.g_state)
        for s in range(n):
            if s + 1 < n and st[s] is st[s + 1]:
                lps.lps_stage_forward_dpos_hop(self.model, self._fence_c, n, s, ptr(self.x[s]),
                                               pos_dev, ptr(self.scratch[s]), self.scratch_bytes,
                                               self.bounds[s], ptr(self.x[s + 1]), t, sp(st[s]))
                continue
            lps.lps_stage_forward_dpos(self.model, self._fence_c, n, s, ptr(self.x[s]), pos_dev,
                                       ptr(self.scratch[s]), self.scratch_bytes, sp(st[s]))
            if s + 1 < n:
                _hop(self.bounds[s], ptr(self.x[s]), ptr(self.x[s + 1]), t, st[s], st[s + 1])
        self.step_no += 1

    def capture_step(self, feed_dev, n_feed, tok_hist, logits_hist, hist_cap, ring=None):
        """Capture one decode step (every stage and boundary, then the head and the
        token chain in lps_step_finish, which also writes the next step's input row
        into x[0]) into a graph on stage 0's stream; the other stage streams fork
        into it through the boundary events and are joined back at the end.  The
        run seeds x[0] before the first replay.  ring: an optional lps.HostRing the
        step's kernels write its logits and id into.  Returns the graph handle
        (lps_graph_destroy frees it)."""
        cfg = self.cfg
        st0, stl = self.streams[0], self.streams[-1]
        torch.cuda.synchronize(self.device)
        lps.lps_graph_begin(sp(st0))
        g = C.c_void_p()
        try:
            self._walk_dpos()
            lps.lps_step_finish(C.byref(self.head), ptr(self.x[-1]), ptr(self.g_logits),
                                ptr(self.g_state), cfg.ctx_max, feed_dev, n_feed, tok_hist,
                                logits_hist, hist_cap, ptr(self.embed), lps.DTYPES[cfg.wdtype],
                                ptr(self.x[0]), ptr(self.g_tok),
                                C.byref(ring) if ring is not None else None,
                                ptr(self.head_scratch), self.head_scratch.numel(), sp(stl))
        finally:
            join = (C.c_void_p * len(self.streams))(*[sp(s) for s in self.streams])
            lps.lps_graph_end(sp(st0), join, len(self.streams), C.byref(g))
        return g

    def run_tokens_graph(self, prompt, n_steps=0, feed=None, p0=None, logits=True,
                         timer=None, mark_every=3) -> StepResult:
        """run_tokens with the whole step captured once and replayed: the
        position, the step and the next input id live on the device and are
        advanced by the graph itself, so the host only launches replays.  The
        step's own kernels store its argmax (and, with logits=True, its logits)
        into row t % ring of the pinned host ring; a pending marks every
        mark_every-th replay and the last (lps_pending_mark: each mark costs the
        stream a system-scope fence), and the host drains step t - ring, waiting
        for the first mark at or after it, while later replays run.  (A copy on
        the readback stream would make that stream wait for every step, which
        costs the replays ~45 us per step.)  timer: an optional callable run
        around the replays and their readback (for the bench)."""
        cfg = self.cfg
        assert self.head is not None, "model has no vocabulary"
        p = cfg.prefix if p0 is None else p0
        ids = list(prompt) if feed is None else list(feed)
        P = len(ids)
        total = P + (0 if feed is not None else n_steps)
        assert P >= 1 and p + total <= cfg.ctx_max, "cache too short for this run"
        dev = self.device
        feed_dev = torch.tensor(ids, dtype=torch.int32, device=dev)
        tok_hist = torch.zeros(total, dtype=torch.int32, device=dev)
        R = self.ring
        ring = lps.HostRing()
        ring.logits = ptr(self.host_logits) if logits else None
        ring.tok, ring.slots = ptr(self.host_tok), R
        self.g_state.copy_(torch.tensor([p, 0, 0, 0], dtype=torch.int32))
        self.g_tok.fill_(ids[0])
        g = self.capture_step(ptr(feed_dev), P, ptr(tok_hist), None, total, ring)
        pend = [None] * R
        toks, lg = [None] * total, [None] * total
        marked, cover = mark_schedule(total, R, mark_every)

        def drain(i):
            j = cover(i)                    # the first marked step at or after i
            if pend[j % R] is not None:
                lps.lps_pending_wait(pend[j % R])
                pend[j % R] = None
            toks[i] = int(self.host_tok[i % R])
            if logits:
                lg[i] = self.host_logits[i % R].numpy().copy()

        try:
            st0 = self.streams[0]
            # the first step's input row; every replay writes the next one
            lps.lps_embed(ptr(self.embed), lps.DTYPES[cfg.wdtype], cfg.vocab, cfg.d,
                          ptr(self.g_tok), ptr(self.x[0]), sp(st0))
            torch.cuda.synchronize(dev)
            if timer is not None:
                timer(True)
            for i in range(total):
                if i >= R:
                    drain(i - R)             # frees host ring slot i % R
                lps.lps_graph_launch(g, sp(st0))
                if marked(i):
                    h = C.c_void_p()
                    lps.lps_pending_mark(sp(st0), C.byref(h))
                    pend[i % R] = h
            for i in range(max(0, total - R), total):
                drain(i)
            if timer is not None:
                timer(False)
        finally:
            torch.cuda.synchronize(dev)
            lps.lps_graph_destroy(g)
        state = self.g_state.cpu().tolist()
        assert state[1] == total, state
        fed = ids[:P] + [toks[i - 1] for i in range(P, total)]
        return StepResult(fed=fed, argmax=toks, logits=lg)

    def run_hidden_graph(self, xs: np.ndarray, p0=None, timer=None) -> np.ndarray:
        """run_hidden with the whole step captured once and replayed: the input row
        of step s (xs[s]) is copied in and the last stage's hidden copied out at the
        device step, and the position advances on the device.  timer: an optional
        callable run around the replays (for the bench)."""
        cfg = self.cfg
        p = cfg.prefix if p0 is None else p0
        T = xs.shape[0]
        assert T >= 1 and p + T <= cfg.ctx_max
        dev = self.device
        xin = to_dev(np.ascontiguousarray(xs, dtype=np.float32), dev)
        out = torch.zeros((T, cfg.d), dtype=torch.float32, device=dev)
        self.g_state.copy_(torch.tensor([p, 0, 0, 0], dtype=torch.int32))
        st0, stl = self.streams[0], self.streams[-1]
        torch.cuda.synchronize(dev)
        lps.lps_graph_begin(sp(st0))
        g = C.c_void_p()
        try:
            lps.lps_row_at_step(ptr(self.g_state), ptr(xin), cfg.d, ptr(self.x[0]), 0, cfg.d, T,
                                sp(st0))
            self._walk_dpos()
            lps.lps_row_at_step(ptr(self.g_state), ptr(self.x[-1]), 0, ptr(out), cfg.d, cfg.d, T,
                                sp(stl))
            lps.lps_step_advance(ptr(self.g_state), cfg.ctx_max, None, None, None, 0, None, 0,
                                 None, 0, None, sp(stl))
        finally:
            join = (C.c_void_p * len(self.streams))(*[sp(x) for x in self.streams])
            lps.lps_graph_end(sp(st0), join, len(self.streams), C.byref(g))
        try:
            torch.cuda.synchronize(dev)
            if timer is not None:
                timer(True)
            for _ in range(T):
                lps.lps_graph_launch(g, sp(st0))
            torch.cuda.synchronize(dev)
            if timer is not None:
                timer(False)
        finally:
            torch.cuda.synchronize(dev)
            lps.lps_graph_destroy(g)
        assert self.g_state.cpu().tolist()[1] == T
        return out.cpu().numpy()

    def run_hidden(self, xs: np.ndarray, p0=None) -> np.ndarray:
        """Models without a vocabulary: step t feeds the f32 row xs[t] at position
        p0 + t and returns the last stage's hidden rows [steps, d]."""
        cfg = self.cfg
        p = cfg.prefix if p0 is None else p0
        T = xs.shape[0]
        assert p + T <= cfg.ctx_max
        dev = self.device
        xin = to_dev(np.ascontiguousarray(xs, dtype=np.float32), dev)
        out = torch.zeros((T, cfg.d), dtype=torch.float32, device=dev)
        torch.cuda.synchronize(dev)
        st0, stl = self.streams[0], self.streams[-1]
        for t in range(T):
            lps.lps_copy_f32(ptr(xin) + 4 * cfg.d * t, ptr(self.x[0]), cfg.d, sp(st0))
            self._walk(p + t)
            lps.lps_copy_f32(ptr(self.x[-1]), ptr(out) + 4 * cfg.d * t, cfg.d, sp(stl))
        torch.cuda.synchronize(dev)
        return out.cpu().numpy()


class DeviceMoEStack:
    """A synth MoE FFN stack resident on one GPU, walked as N stages on N streams:
    every layer is an FFN-only block (nq 0) whose FFN is the MoE of its lps_moe_desc;
    the stages and boundaries are those of the dense decoder (lps_stage_forward,
    lps_boundary_send / recv).  Decode takes one row per step; prefill takes a
    chunk of rows through each stage's layers (the grouped-GEMM path) with a
    [T, d] block per boundary."""

    def __init__(self, model: dict, fence=None, device="cuda:0", streams: str = "per-stage"):
        _need_gpu()
        self.cfg = cfg = model["cfg"]
        self.device = dev = torch.device(device)
        self.layers, self.descs = [], []
        for L in model["layers"]:
            t = {k: to_dev(L[k], dev) for k in ("g_ffn", "w_r", "w_gu_e", "w_d_e", "w_gu_s", "w_d_s")}
            d = lps.MoEDesc()
            d.d, d.n_experts, d.top_k, d.ff = cfg.d, cfg.n_experts, cfg.top_k, cfg.ff
            d.remote_from, d.eps = cfg.remote_from, cfg.eps
            d.g_ffn, d.w_r = ptr(t["g_ffn"]), ptr(t["w_r"])
            d.w_gu_e, d.w_d_e = ptr(t["w_gu_e"]), ptr(t["w_d_e"])
            d.w_gu_s, d.w_d_s = ptr(t["w_gu_s"]), ptr(t["w_d_s"])
            self.layers.append(t)
            self.descs.append(d)
        ld = (lps.LayerDesc * cfg.n_layers)()
        for l, d in enumerate(self.descs):
            ld[l].d, ld[l].nq, ld[l].wdtype, ld[l].eps = cfg.d, 0, lps.LPS_BF16, cfg.eps
            ld[l].ffn_kind, ld[l].moe = lps.LPS_FFN_MOE, C.addressof(d)
        h = C.c_void_p()
        lps.lps_model_create(ld, cfg.n_layers, C.byref(h))
        self.model = h
        self.scratch_bytes = lps.lps_model_scratch_bytes(h)
        self.stream = torch.cuda.Stream(device=dev)     # the unstaged prefill's main stream
        self.g_state = torch.zeros(4, dtype=torch.int32, device=dev)   # [pos, step, flags]
        self._streams_mode = streams
        self.bounds, self._pf_bounds = [], []
        self._pf_scratch = None
        self.set_fence(fence)

    def set_fence(self, fence=None):
        cfg, dev = self.cfg, self.device
        fence = list(fence) if fence is not None else lps.stage_plan(cfg.n_layers, 1)
        if lps.stage_plan(cfg.n_layers, len(fence) - 1, fence[1:-1]) != fence:
            raise lps.LpsError(lps.LPS_EINVAL, f"fence {fence} is not a plan of {cfg.n_layers} layers")
        self.fence, self.n_stages = fence, len(fence) - 1
        n = self.n_stages
        self._fence_c = lps.i32_array(fence)
        if self._streams_mode == "single":
            self.streams = [torch.cuda.Stream(device=dev)] * n
        else:
            self.streams = [torch.cuda.Stream(device=dev) for _ in range(n)]
        self.x = [torch.zeros(cfg.d, dtype=torch.float32, device=dev) for _ in range(n)]
        self.scratch = [torch.zeros(self.scratch_bytes, dtype=torch.uint8, device=dev)
                        for _ in range(n)]
        self._close_boundaries()
        self.slots = []
        for _ in range(n - 1):
            s0 = torch.full((cfg.d,), float("nan"), dtype=torch.float32, device=dev)
            s1 = torch.full((cfg.d,), float("nan"), dtype=torch.float32, device=dev)
            b = C.c_void_p()
            lps.lps_boundary_create(cfg.d, ptr(s0), ptr(s1), C.byref(b))
            self.slots.append((s0, s1))
            self.bounds.append(b)
        self.step_no = 0
        torch.cuda.synchronize(dev)

    def _close_boundaries(self):
        for b in self.bounds + self._pf_bounds:
            lps.lps_boundary_destroy(b)
        self.bounds, self._pf_bounds, self._pf_key = [], [], None

    def close(self):
        torch.cuda.synchronize(self.device)
        self._close_boundaries()
        if getattr(self, "model", None):
            lps.lps_model_destroy(self.model)
            self.model = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _walk(self):
        n, st, t = self.n_stages, self.streams, self.step_no
        for s in range(n):
            if s > 0:
                _hop(self.bounds[s - 1], ptr(self.x[s - 1]), ptr(self.x[s]), t, st[s - 1], st[s])
            lps.lps_stage_forward(self.model, self._fence_c, n, s, ptr(self.x[s]), 0,
                                  ptr(self.scratch[s]), self.scratch_bytes, sp(st[s]))
        self.step_no += 1

    def decode(self, xs: np.ndarray) -> np.ndarray:
        """Step t feeds the f32 row xs[t] and returns the last stage's rows [steps, d]."""
        cfg, dev = self.cfg, self.device
        xin = to_dev(np.ascontiguousarray(xs, dtype=np.float32), dev)
        out = torch.zeros_like(xin)
        torch.cuda.synchronize(dev)
        st0, stl = self.streams[0], self.streams[-1]
        for t in range(xs.shape[0]):
            lps.lps_copy_f32(ptr(xin) + 4 * cfg.d * t, ptr(self.x[0]), cfg.d, sp(st0))
            self._walk()
            lps.lps_copy_f32(ptr(self.x[-1]), ptr(out) + 4 * cfg.d * t, cfg.d, sp(stl))
        torch.cuda.synchronize(dev)
        return out.cpu().numpy()

    def decode_graph(self, xs: np.ndarray, timer=None) -> np.ndarray:
        """decode with the whole step (row in, every stage and boundary, row out,
        step advance) captured once and replayed once per row."""
        cfg, dev = self.cfg, self.device
        T = xs.shape[0]
        xin = to_dev(np.ascontiguousarray(xs, dtype=np.float32), dev)
        out = torch.zeros_like(xin)
        self.g_state.zero_()
        st0, stl = self.streams[0], self.streams[-1]
        torch.cuda.synchronize(dev)
        lps.lps_graph_begin(sp(st0))
        g = C.c_void_p()
        try:
            lps.lps_row_at_step(ptr(self.g_state), ptr(xin), cfg.d, ptr(self.x[0]), 0, cfg.d, T,
                                sp(st0))
            self._walk()
            lps.lps_row_at_step(ptr(self.g_state), ptr(self.x[-1]), 0, ptr(out), cfg.d, cfg.d, T,
                                sp(stl))
            lps.lps_step_advance(ptr(self.g_state), 1 << 30, None, None, None, 0, None, 0, None, 0,
                                 None, sp(stl))
        finally:
            join = (C.c_void_p * len(self.streams))(*[sp(x) for x in self.streams])
            lps.lps_graph_end(sp(st0), join, len(self.streams), C.byref(g))
        try:
            torch.cuda.synchronize(dev)
            if timer is not None:
                timer(True)
            for _ in range(T):
                lps.lps_graph_launch(g, sp(st0))
            torch.cuda.synchronize(dev)
            if timer is not None:
                timer(False)
        finally:
            torch.cuda.synchronize(dev)
            lps.lps_graph_destroy(g)
        assert self.g_state.cpu().tolist()[1] == T
        return out.cpu().numpy()

    def _prefill_scratch(self, T):
        sb = lps.lps_moe_prefill_scratch_bytes(C.byref(self.descs[0]), T)
        if self._pf_scratch is None or self._pf_scratch.numel() < sb:
            self._pf_scratch = torch.empty(sb, dtype=torch.uint8, device=self.device)

    def prefill(self, X: np.ndarray, n_pieces: int = 8, remote_stream=None) -> np.ndarray:
        """All layers over a chunk of T rows (the grouped-GEMM path), stage by stage
        with a [T, d] block through each boundary; returns the output rows [T, d]."""
        cfg, dev, n = self.cfg, self.device, self.n_stages
        T = X.shape[0]
        xs = [to_dev(np.ascontiguousarray(X, dtype=np.float32), dev)]
        xs += [torch.empty((T, cfg.d), dtype=torch.float32, device=dev) for _ in range(n - 1)]
        self._prefill_scratch(T)
        if n == 1:
            rs = remote_stream or torch.cuda.Stream(device=dev)
            torch.cuda.synchronize(dev)
            self.prefill_dev(xs[0], T, n_pieces, rs)
            torch.cuda.synchronize(dev)
            return xs[0].cpu().numpy()
        key = (T, tuple(self.fence))
        if self._pf_key != key:
            for b in self._pf_bounds:
                lps.lps_boundary_destroy(b)
            self._pf_bounds, self._pf_slots = [], []
            for _ in range(n - 1):
                s0 = torch.empty((T, cfg.d), dtype=torch.float32, device=dev)
                s1 = torch.empty_like(s0)
                b = C.c_void_p()
                lps.lps_boundary_create(T * cfg.d, ptr(s0), ptr(s1), C.byref(b))
                self._pf_slots.append((s0, s1))
                self._pf_bounds.append(b)
            self._pf_key, self._pf_step = key, 0
        # one scratch serves every stage: the stages run one after the other here
        rs = remote_stream or torch.cuda.Stream(device=dev)
        st = self.streams
        torch.cuda.synchronize(dev)
        k = self._pf_step
        for s in range(n):
            if s > 0:
                lps.lps_boundary_send(self._pf_bounds[s - 1], ptr(xs[s - 1]), k, sp(st[s - 1]))
                lps.lps_boundary_recv(self._pf_bounds[s - 1], ptr(xs[s]), k, sp(st[s]))
            for l in range(self.fence[s], self.fence[s + 1]):
                lps.lps_moe_prefill(C.byref(self.descs[l]), ptr(xs[s]), T, n_pieces,
                                    ptr(self._pf_scratch), self._pf_scratch.numel(), sp(st[s]),
                                    sp(rs))
            torch.cuda.synchronize(dev)   # the shared scratch is free for the next stage
        self._pf_step += 1
        return xs[-1].cpu().numpy()

    def prefill_dev(self, x, T, n_pieces, remote_stream):
        """Enqueue every layer over device rows x [T, d] (in place) on self.stream."""
        for d in self.descs:
            lps.lps_moe_prefill(C.byref(d), ptr(x), T, n_pieces, ptr(self._pf_scratch),
                                self._pf_scratch.numel(), sp(self.stream), sp(remote_stream))
