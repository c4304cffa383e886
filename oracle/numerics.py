"""Operand widening and the storage roundings of the decode path (float64).

Test infrastructure only.  Formats:
  bf16   upper 16 bits of an IEEE binary32 pattern
  f16    IEEE binary16 (numpy float16), round to nearest even
  MXFP4  OCP Microscaling v1.0: FP4 E2M1 elements (1 sign bit, 2 exponent bits
         with bias 1, 1 mantissa bit; no Inf/NaN) and one E8M0 scale per 32
         elements (value 2^(s-127); 0xFF is NaN).  Layout from the TP3
         zero-padded dummy heads plan (Weight-padding design): packed weight
         bytes [N, K/2] with two e2m1 codes per byte and an e8m0 scale array
         [N, K/32]; padding fills 0x00 (two +0 codes) and 0x7F (2^0).
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_f32(x) -> np.ndarray:
    """Round to binary32 (the storage of the residual stream and f32 caches)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(x32) -> np.ndarray:
    """binary32 -> bf16 bits, round to nearest, ties to even (finite inputs)."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def round_cache(x64, kvdtype: str):
    """A K/V row as the cache stores it: f32, or f64 -> f32 -> bf16 (RNE)."""
    x32 = to_f32(x64)
    if kvdtype == "f32":
        return x32
    if kvdtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(kvdtype)


def widen_cache(stored, kvdtype: str) -> np.ndarray:
    if kvdtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    return bf16_to_f64(stored)


def f16_round(x32) -> np.ndarray:
    """binary32 -> binary16, round to nearest even (numpy's IEEE conversion)."""
    return np.asarray(x32, dtype=np.float32).astype(np.float16)


# E2M1 element value of codes 0..15: sign in bit 3; magnitude from exponent
# bits [2:1] (bias 1) and mantissa bit 0; exponent 0 is the subnormal range.
def e2m1_value(code: int) -> float:
    s = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        return s * 0.5 * m                      # 0 or 0.5 (subnormal: 2^(1-1) * m/2)
    return s * (2.0 ** (e - 1)) * (1.0 + 0.5 * m)


E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e8m0_value(s) -> np.ndarray:
    s = np.asarray(s, dtype=np.int64)
    v = np.ldexp(1.0, s - 127)
    return np.where(s == 255, np.nan, v)


# element pair (low nibble, high nibble) of every byte value
_PAIR = np.stack([E2M1[np.arange(256) & 0x0F], E2M1[np.arange(256) >> 4]], axis=1)


def mxfp4_to_f64(codes, scales) -> np.ndarray:
    """codes u8 [N, K/2], scales u8 [N, K/32] -> f64 [N, K].

    Byte b of a row holds element 2b in its low nibble, 2b+1 in its high one."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, Kh = codes.shape
    K = 2 * Kh
    el = _PAIR[codes].reshape(N, K)                # [N, K/2, 2] -> elements 2b, 2b+1
    sc = e8m0_value(scales)                        # [N, K/32]
    el = el.reshape(N, K // 32, 32)
    el *= sc[..., None]
    return el.reshape(N, K)


def widen_weight(w, wdtype: str) -> np.ndarray:
    if wdtype == "f32":
        return np.asarray(w, dtype=np.float32).astype(np.float64)
    if wdtype == "bf16":
        return bf16_to_f64(w)
    if wdtype == "mxfp4":
        return mxfp4_to_f64(*w)
    raise ValueError(wdtype)
