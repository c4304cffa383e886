"""Chunked, thread-parallel seeded draws and the storage encoders."""
from __future__ import annotations

import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22          # elements per independently seeded chunk
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        n = min(16, len(os.sched_getaffinity(0)))
        _POOL = ThreadPoolExecutor(max(1, n))
    return _POOL


def _stream(seed: int, name: str, chunk: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(zlib.crc32(name.encode()), chunk))
    return np.random.Generator(np.random.PCG64(ss))


def normal_f32(seed: int, name: str, shape, std: float = 1.0) -> np.ndarray:
    """f32 array ~ N(0, std^2) of the given shape, chunk-seeded by name."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = _stream(seed, name, c)
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if std != 1.0:
            out[lo:hi] *= np.float32(std)

    list(_pool().map(fill, range(nchunks)))
    return out.reshape(shape)


def uniform_ints(seed: int, name: str, n: int, high: int) -> np.ndarray:
    """n int32 ids uniform in [0, high)."""
    g = _stream(seed, name, 0)
    return g.integers(0, high, size=n, dtype=np.int64).astype(np.int32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """f32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Inputs here are finite draws; NaN/Inf handling is not needed."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    flat = a.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    n = flat.size
    nchunks = (n + CHUNK - 1) // CHUNK

    def conv(c):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        u = flat[lo:hi].view(np.uint32)
        out[lo:hi] = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
                      >> np.uint32(16)).astype(np.uint16)

    list(_pool().map(conv, range(nchunks)))
    return out.reshape(a.shape)


# e2m1 magnitudes in code order 0..7 (OCP MX v1.0, FP4 E2M1: 1 sign, 2 exponent,
# 1 mantissa bit, bias 1; codes 0b000/0b001 are zero and the subnormal 0.5).
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
# decision points between adjacent magnitudes, with the tie going to the even code
_E2M1_MID = (_E2M1_GRID[1:] + _E2M1_GRID[:-1]) / 2


def _encode_rows(w: np.ndarray):
    """w [R, K] f32 (K % 32 == 0) -> codes u8 [R, K/2], scales u8 [R, K/32]."""
    R, K = w.shape
    g = w.astype(np.float64).reshape(R, K // 32, 32)
    amax = np.abs(g).max(axis=2)
    # shared exponent: floor(log2(amax)) - emax(e2m1)=2; all-zero groups get 2^0
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, 0)
    e = np.clip(e, -127, 127).astype(np.int64)
    scale = np.ldexp(1.0, e)[..., None]
    v = g / scale
    mag = np.abs(v)
    # side="left": a magnitude exactly at a midpoint gets the lower code ...
    code = np.searchsorted(_E2M1_MID, mag, side="left")
    # ... and round-half-to-even moves it up when that lower code is odd
    at_mid = mag == _E2M1_MID[np.minimum(code, 6)]
    code = np.where(at_mid & (code % 2 == 1), code + 1, code)   # > 5.0 saturates to code 7 (6.0)
    sign = (v < 0) & (code > 0)
    nib = (code | (sign.astype(np.int64) << 3)).astype(np.uint8).reshape(R, K)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = (e + 127).astype(np.uint8)
    return packed, scales


def mxfp4_encode(w: np.ndarray, rows_per_task: int = 512):
    """Quantise f32 rows to MXFP4 (OCP MX v1.0): returns (codes, scales).

    codes u8 [N, K/2]: byte b of a row holds element 2b in its low nibble and
    element 2b+1 in its high nibble.  scales u8 [N, K/32]: e8m0 biased
    exponent (value 2^(s-127)) for elements [32j, 32j+32)."""
    N, K = w.shape
    assert K % 32 == 0
    codes = np.empty((N, K // 2), dtype=np.uint8)
    scales = np.empty((N, K // 32), dtype=np.uint8)

    def task(i):
        lo, hi = i * rows_per_task, min(N, (i + 1) * rows_per_task)
        codes[lo:hi], scales[lo:hi] = _encode_rows(w[lo:hi])

    list(_pool().map(task, range((N + rows_per_task - 1) // rows_per_task)))
    return codes, scales
