"""CPU float64 oracle for the staged single-token decode path.

TEST INFRASTRUCTURE.  Only the tests, the smoke check of the package entry
and the benchmark's CPU-baseline leg import this package.  The product path
(the HIP library and its Python binding) never imports, links or runs it, and
this package imports nothing from the product path: the two share only the
seeded input arrays made by ``synth``.

What it computes is the plain definition of the decode forward that the
pages' staged runtime must reproduce bit for bit: the stages, boundary slots,
FP16 pieces and deferred readback change scheduling, not arithmetic (memra
``pp`` module docs, header: the deferred arm moves when work runs, not what
it computes; strata PR #3648, Approach: exact FP16->FP32 conversion with the
additions in their order).  Everything is evaluated in float64 over the stored operands; the
rounding points are the storage formats the path itself uses: f32 for the
residual stream, the cache dtype for K/V rows, f16 for the remote MoE partial
sums, bf16 for the inputs of the prefill grouped GEMM.

Modules
  plan      stage fence, even split / explicit cuts / per-stage counts, stage_of
  numerics  widening of bf16 / f16 / MXFP4 (e2m1 + e8m0) operands, storage roundings
  decoder   RMSNorm, RoPE, GQA attention, SwiGLU, dense/MXFP4 layer, head, staged walk,
            chunked prefill in matrix form (causal mask, bf16 matrix-core operands)
  moe       router softmax + top-k, experts, fixed-order local/remote sums, FP16 pieces

Pins (each checked by a CPU test against something other than this code):
  plan      closed form and brute force over every cut set (exact)
  numerics  bf16/f16 against torch's and numpy's own converters; the OCP MX
            v1.0 e2m1 value table and the e8m0 special values (exact)
  decoder   RMSNorm / RoPE / attention special cases and brute force on tiny
            shapes; the prefill matrix form (exact operands) equals the decode
            steps, chunk and stage splits change nothing, and a planted
            off-by-one mask is caught; bf16 operand rounding against torch;
            every prefill rounding point (normed rows, attention output,
            normed rows, SwiGLU output) and the gate/up order by closed forms
            on hand-built layers, each with a planted removal that fails;
            staged == unstaged bit for bit; padded == unpadded bit
            for bit; a one-token closed form of a whole layer
  moe       top-k against exhaustive subset search; FP16 pieces == one piece
            and aliased == separate combine, bit for bit; a whole layer (router,
            experts' gate/up order, the prefill bf16 rounding points, the f16
            remote sum) by closed forms on a hand-built layer, with planted
            removals of each rounding point
Absolute logits of a whole model have no printed worked example on the pages:
they are pinned only through the rows above (parity unpinned beyond that).
"""
