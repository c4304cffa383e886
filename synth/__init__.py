"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module only *makes* inputs: random weights, caches, prompts and hidden
vectors at the shapes of the staged-decode workloads.  It holds none of the
decode arithmetic (no norm, projection, attention, routing or combine): the
oracle and the HIP path each implement those on their own.  Weight storage
formats are produced here because they are how the inputs are handed over:
bf16 bit patterns (round-to-nearest-even of an f32 draw) and MXFP4 blocks
(OCP Microscaling v1.0: e2m1 element codes, one e8m0 exponent per 32 values).

Determinism: every tensor is drawn in fixed-size chunks, each from its own
PCG64 stream keyed by (seed, crc32(tensor name), chunk index), so the values
do not depend on the thread count used to draw them.
"""
from .gen import (  # noqa: F401
    normal_f32, uniform_ints, bf16_bits, mxfp4_encode, CHUNK,
)
from .models import (  # noqa: F401
    DecoderConfig, MoEConfig,
    make_tiny, make_dense, make_moe, make_pad, make_pad_pair,
    TINY, TINY_N4, DENSE8B, MOE, PAD,
)
