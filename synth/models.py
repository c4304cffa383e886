"""Workload shapes and seeded model/input builders.

Every builder returns plain numpy arrays in the storage format the decode
path consumes:
  'f32'   float32 arrays
  'bf16'  uint16 arrays of bf16 bit patterns (RNE of an f32 N(0, std^2) draw)
  'mxfp4' (codes u8 [N, K/2], scales u8 [N, K/32]) pairs, OCP MX v1.0
Norm gains are 1.0 (the workloads state only the matrix distribution).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

from .gen import normal_f32, uniform_ints, bf16_bits, mxfp4_encode


@dataclass(frozen=True)
class DecoderConfig:
    name: str
    n_layers: int
    d: int
    nq: int
    nkv: int
    hd: int
    ff: int
    vocab: int            # 0: no embedding table and no head (hidden in, hidden out)
    wdtype: str           # 'f32' | 'bf16' | 'mxfp4'
    kvdtype: str          # 'f32' | 'bf16'
    eps: float = 1e-6
    rope_base: float = 10000.0
    prefix: int = 0       # seeded KV rows already present in every layer's cache
    prompt: int = 0       # prompt token count (vocab > 0)
    steps: int = 0        # decode steps after the prompt / prefix
    std: float = 0.02
    seed: int = 0
    # zero-padded dummy geometry (real counts; equal to the padded ones when unpadded)
    nq_real: int = 0
    nkv_real: int = 0
    ff_real: int = 0

    @property
    def ctx_max(self) -> int:
        return self.prefix + self.prompt + self.steps

    @property
    def qkv_rows(self) -> int:
        return (self.nq + 2 * self.nkv) * self.hd

    def real(self) -> "DecoderConfig":
        """The unpadded model that a padded config stands for."""
        if not self.nq_real:
            return self
        return replace(self, name=self.name + "-unpadded", nq=self.nq_real, nkv=self.nkv_real,
                       ff=self.ff_real, nq_real=0, nkv_real=0, ff_real=0)


@dataclass(frozen=True)
class MoEConfig:
    name: str
    n_layers: int = 4
    d: int = 2048
    n_experts: int = 64
    top_k: int = 8
    ff: int = 1024
    remote_from: int = 32     # experts >= this id form the FP16-summed half
    n_pieces: int = 8
    prefill_T: int = 16384
    steps: int = 128
    eps: float = 1e-6
    std: float = 0.02
    router_std: float = 0.0   # 0 -> 1/sqrt(d): router logits ~N(0,1) on RMS-1 rows
    seed: int = 0

    @property
    def rstd(self) -> float:
        return self.router_std or 1.0 / np.sqrt(self.d)


# ---- the workloads -------------------------------------------------------
TINY = DecoderConfig("tiny-f32", n_layers=4, d=256, nq=4, nkv=2, hd=64, ff=704, vocab=1024,
                     wdtype="f32", kvdtype="f32", prompt=8, steps=16)
TINY_N4 = replace(TINY, name="tiny-f32-ctx96", prompt=32, steps=64)
DENSE8B = DecoderConfig("dense-8b-slice", n_layers=8, d=4096, nq=32, nkv=8, hd=128, ff=14336,
                        vocab=32000, wdtype="bf16", kvdtype="bf16", prefix=4096, prompt=1, steps=127)
MOE = MoEConfig("moe-64x8")
PAD = DecoderConfig("pad-mxfp4", n_layers=4, d=5120, nq=36, nkv=6, hd=256, ff=17472, vocab=0,
                    wdtype="mxfp4", kvdtype="bf16", prefix=8192, steps=32,
                    nq_real=24, nkv_real=4, ff_real=17408)


def _w(cfg, name, shape, std=None):
    a = normal_f32(cfg.seed, f"{cfg.name}/{name}", shape, cfg.std if std is None else std)
    if cfg.wdtype == "f32":
        return a
    if cfg.wdtype == "bf16":
        return bf16_bits(a)
    raise ValueError(cfg.wdtype)


def _kv(cfg, name, shape):
    a = normal_f32(cfg.seed, f"{cfg.name}/{name}", shape, 1.0)
    return a if cfg.kvdtype == "f32" else bf16_bits(a)


def make_tiny(cfg: DecoderConfig = TINY) -> dict:
    return make_dense(cfg)


def make_dense(cfg: DecoderConfig = DENSE8B) -> dict:
    """Dense decoder (f32 or bf16 weights): embedding, layers, final norm, LM head,
    optional seeded KV prefix, prompt ids."""
    assert cfg.wdtype in ("f32", "bf16")
    d, hd = cfg.d, cfg.hd
    m = {"cfg": cfg, "layers": []}
    if cfg.vocab:
        m["embed"] = _w(cfg, "embed", (cfg.vocab, d))
        m["g_out"] = np.ones(d, np.float32)
        m["w_lm"] = _w(cfg, "lm_head", (cfg.vocab, d))
    for l in range(cfg.n_layers):
        L = {
            "g_attn": np.ones(d, np.float32),
            "w_qkv": _w(cfg, f"l{l}/qkv", (cfg.qkv_rows, d)),
            "w_o": _w(cfg, f"l{l}/o", (d, cfg.nq * hd)),
            "g_ffn": np.ones(d, np.float32),
            "w_gu": _w(cfg, f"l{l}/gate_up", (2 * cfg.ff, d)),   # gate rows, then up rows
            "w_d": _w(cfg, f"l{l}/down", (d, cfg.ff)),
        }
        if cfg.prefix:
            L["k_prefix"] = _kv(cfg, f"l{l}/k_prefix", (cfg.nkv, cfg.prefix, hd))
            L["v_prefix"] = _kv(cfg, f"l{l}/v_prefix", (cfg.nkv, cfg.prefix, hd))
        m["layers"].append(L)
    if cfg.vocab and cfg.prompt:
        m["prompt"] = uniform_ints(cfg.seed, f"{cfg.name}/prompt", cfg.prompt, cfg.vocab)
    if not cfg.vocab and cfg.steps:
        m["x_in"] = normal_f32(cfg.seed, f"{cfg.name}/x_in", (cfg.steps, d), 1.0)
    return m


def _mx(cfg, name, shape):
    return mxfp4_encode(normal_f32(cfg.seed, f"{cfg.name}/{name}", shape, cfg.std))


def _pad_rows(cs, n_zero_rows, at_rows=None):
    """Append (or insert before row index at_rows) zero e2m1 rows with 2^0 scales."""
    codes, scales = cs
    zc = np.zeros((n_zero_rows, codes.shape[1]), np.uint8)
    zs = np.full((n_zero_rows, scales.shape[1]), 0x7F, np.uint8)
    return np.concatenate([codes, zc]), np.concatenate([scales, zs])


def _pad_cols(cs, n_zero_k):
    codes, scales = cs
    assert n_zero_k % 32 == 0
    zc = np.zeros((codes.shape[0], n_zero_k // 2), np.uint8)
    zs = np.full((codes.shape[0], n_zero_k // 32), 0x7F, np.uint8)
    return np.concatenate([codes, zc], axis=1), np.concatenate([scales, zs], axis=1)


def make_pad_pair(cfg: DecoderConfig = PAD):
    """(padded, unpadded) models sharing one draw of the real weights."""
    return make_pad(cfg, padded=True, _both=True)


def make_pad(cfg: DecoderConfig = PAD, padded: bool = True, _both: bool = False):
    """MXFP4 decoder whose real part is shared by the padded and the unpadded
    model.  Padded: dummy q/kv heads and FFN rows/columns appended at the end of
    every padded axis (codes 0x00, scales 0x7F = 2^0)."""
    assert cfg.wdtype == "mxfp4" and cfg.nq_real
    real = cfg.real()
    d, hd = cfg.d, cfg.hd
    out_cfg = cfg if padded else real
    m = {"cfg": out_cfg, "layers": []}
    um = {"cfg": real, "layers": []}
    dq, dkv, dff = cfg.nq - real.nq, cfg.nkv - real.nkv, cfg.ff - real.ff
    for l in range(cfg.n_layers):
        wq = _mx(cfg, f"l{l}/q", (real.nq * hd, d))
        wk = _mx(cfg, f"l{l}/k", (real.nkv * hd, d))
        wv = _mx(cfg, f"l{l}/v", (real.nkv * hd, d))
        wo = _mx(cfg, f"l{l}/o", (d, real.nq * hd))
        wg = _mx(cfg, f"l{l}/gate", (real.ff, d))
        wu = _mx(cfg, f"l{l}/up", (real.ff, d))
        wd = _mx(cfg, f"l{l}/down", (d, real.ff))
        kp = bf16_bits(normal_f32(cfg.seed, f"{cfg.name}/l{l}/k_prefix", (real.nkv, cfg.prefix, hd)))
        vp = bf16_bits(normal_f32(cfg.seed, f"{cfg.name}/l{l}/v_prefix", (real.nkv, cfg.prefix, hd)))
        cat = lambda *ts: (np.concatenate([t[0] for t in ts]), np.concatenate([t[1] for t in ts]))
        if _both:
            um["layers"].append({
                "g_attn": np.ones(d, np.float32), "w_qkv": cat(wq, wk, wv), "w_o": wo,
                "g_ffn": np.ones(d, np.float32), "w_gu": cat(wg, wu), "w_d": wd,
                "k_prefix": kp, "v_prefix": vp,
            })
        if padded:
            wq, wk, wv = _pad_rows(wq, dq * hd), _pad_rows(wk, dkv * hd), _pad_rows(wv, dkv * hd)
            wo = _pad_cols(wo, dq * hd)
            wg, wu = _pad_rows(wg, dff), _pad_rows(wu, dff)
            wd = _pad_cols(wd, dff)
            z = np.zeros((dkv, cfg.prefix, hd), np.uint16)
            kp, vp = np.concatenate([kp, z]), np.concatenate([vp, z])
        m["layers"].append({
            "g_attn": np.ones(d, np.float32),
            "w_qkv": cat(wq, wk, wv),
            "w_o": wo,
            "g_ffn": np.ones(d, np.float32),
            "w_gu": cat(wg, wu),
            "w_d": wd,
            "k_prefix": kp,
            "v_prefix": vp,
        })
    m["x_in"] = normal_f32(cfg.seed, f"{cfg.name}/x_in", (cfg.steps, d), 1.0)
    if _both:
        um["x_in"] = m["x_in"]
        return m, um
    return m


def make_moe(cfg: MoEConfig = MOE, prefill: bool = True, decode: bool = True) -> dict:
    """MoE FFN stack: per layer a norm gain, router [E, d], E routed experts and one
    shared expert (gate/up [2ff, d] with gate rows first, down [d, ff]), all bf16."""
    d, E, ff = cfg.d, cfg.n_experts, cfg.ff
    m = {"cfg": cfg, "layers": []}

    def w(name, shape, std):
        return bf16_bits(normal_f32(cfg.seed, f"{cfg.name}/{name}", shape, std))

    for l in range(cfg.n_layers):
        m["layers"].append({
            "g_ffn": np.ones(d, np.float32),
            "w_r": w(f"l{l}/router", (E, d), cfg.rstd),
            "w_gu_e": w(f"l{l}/experts_gate_up", (E, 2 * ff, d), cfg.std),
            "w_d_e": w(f"l{l}/experts_down", (E, d, ff), cfg.std),
            "w_gu_s": w(f"l{l}/shared_gate_up", (2 * ff, d), cfg.std),
            "w_d_s": w(f"l{l}/shared_down", (d, ff), cfg.std),
        })
    if prefill and cfg.prefill_T:
        m["x_prefill"] = normal_f32(cfg.seed, f"{cfg.name}/x_prefill", (cfg.prefill_T, d), 1.0)
    if decode and cfg.steps:
        m["x_in"] = normal_f32(cfg.seed, f"{cfg.name}/x_in", (cfg.steps, d), 1.0)
    return m
