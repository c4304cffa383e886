"""Pins of oracle.numerics against independent converters and the MX spec table."""
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle.numerics import (bf16_to_f64, f32_to_bf16_bits, f16_round, E2M1, e8m0_value,
                             mxfp4_to_f64, round_cache)

GOLD = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_spec.txt")


def _spec():
    codes, scales = {}, {}
    for line in open(GOLD):
        line = line.split("#")[0].strip()
        if not line:
            continue
        p = line.split()
        if p[0] == "e8m0":
            scales[int(p[1])] = float(p[2])
        else:
            codes[int(p[0])] = float(p[1])
    return codes, scales


def _f32_cases(n=20000):
    rng = np.random.default_rng(7)
    a = (rng.standard_normal(n) * np.exp(rng.uniform(-20, 20, n))).astype(np.float32)
    # exact ties at bf16 precision: low 16 bits = 0x8000, both parities of bit 16
    u = rng.integers(0, 1 << 31, n // 4, dtype=np.uint64).astype(np.uint32)
    u = (u & np.uint32(0x7F7F0000)) | np.uint32(0x8000)
    return np.concatenate([a, u.view(np.float32), -u.view(np.float32),
                           np.array([0.0, -0.0, 1.0, 65504.0], np.float32)])


def test_bf16_rounding_matches_torch():
    x = _f32_cases()
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_widening_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]                    # finite patterns
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_to_f64(bits), ref)


def test_f16_rounding_matches_torch():
    x = _f32_cases()
    x = x[np.abs(x) < 65000]
    ours = f16_round(x)
    ref = torch.from_numpy(x).half().numpy()
    assert np.array_equal(ours.view(np.uint16), ref.view(np.uint16))
    # widening back is exact
    assert np.array_equal(ours.astype(np.float32).astype(np.float16).view(np.uint16),
                          ours.view(np.uint16))


def test_e2m1_table_is_the_spec():
    codes, _ = _spec()
    for c, v in codes.items():
        assert E2M1[c] == v and math.copysign(1, E2M1[c]) == math.copysign(1, v), c


def test_e8m0_values_are_the_spec():
    _, scales = _spec()
    for s, v in scales.items():
        got = float(e8m0_value(s))
        if math.isnan(v):
            assert math.isnan(got)
        else:
            assert got == v


def test_mxfp4_nibble_order_and_group_scale():
    # row of 64 elements: byte 0 = 0x21 -> element 0 code 1 (0.5), element 1 code 2 (1.0);
    # second group scaled by 2^3
    codes = np.zeros((1, 32), np.uint8)
    codes[0, 0] = 0x21
    codes[0, 16] = 0xF7            # element 32 -> code 7 (6.0), element 33 -> code 15 (-6.0)
    scales = np.array([[127, 130]], np.uint8)
    w = mxfp4_to_f64(codes, scales)
    assert w[0, 0] == 0.5 and w[0, 1] == 1.0 and w[0, 32] == 48.0 and w[0, 33] == -48.0
    assert np.count_nonzero(w) == 4


def test_generator_encoder_round_trips_through_oracle_decoder():
    """synth's MXFP4 encoder and the oracle's decoder are written separately:
    values already on the grid survive exactly; others land within half a grid
    step of the group scale."""
    rng = np.random.default_rng(3)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    vals = rng.choice(grid, size=(8, 256)) * rng.choice([-1, 1], size=(8, 256))
    vals[:, ::32] = 6.0                       # pin every group's amax so its exponent is 0+e
    e = rng.integers(-10, 10, size=(8, 8))
    w = (vals.reshape(8, 8, 32) * np.ldexp(1.0, e)[..., None]).reshape(8, 256).astype(np.float32)
    c, s = synth.mxfp4_encode(w)
    assert np.array_equal(mxfp4_to_f64(c, s), w.astype(np.float64))
    x = (rng.standard_normal((16, 512)) * 0.02).astype(np.float32)
    c, s = synth.mxfp4_encode(x)
    d = mxfp4_to_f64(c, s)
    sc = e8m0_value(s).repeat(32, axis=1)
    # the shared exponent puts |x| / scale in [0, 8): below 6 the grid spacing is
    # at most 2 (error <= 1 scale), above 6 the value saturates to 6 (error < 2)
    r = np.abs(x) / sc
    assert np.all(r < 8)
    assert np.all(np.abs(d - x) <= np.where(r <= 6, 1.0, 2.0) * sc)
    assert np.all(np.abs(d) <= 6 * sc)


def test_round_cache():
    v = np.array([1.0 + 2 ** -9, -3.25, 1e-3])
    assert np.array_equal(round_cache(v, "f32"), v.astype(np.float32))
    b = round_cache(v, "bf16")
    assert b.dtype == np.uint16
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(b, ref.view(np.uint16))
