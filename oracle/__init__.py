"""CPU oracle for group-wise weight-quantized GEMV / GEMM / grouped MoE GEMM.

TEST INFRASTRUCTURE ONLY.  This package is imported by the tests, by the
smoke check and by the CPU-baseline leg of the benchmark, and by nothing
else: the GPU library never calls it, links it or falls back to it.  It
shares no code with the HIP path; the two meet only in the seeded input
generators of the ``synth`` package.

What it computes, and where that is defined
-------------------------------------------
BaseRT (native-Metal LLM inference on Apple Silicon), §3.3 "kernel fusion
and specialization": every matmul kernel, GEMV for decode (M=1) and GEMM for
prefill (M>1), folds dequantization into its inner loop instead of writing
dequantized weights to memory.  The fused kernel therefore computes exactly
(up to the order of floating-point rounding) what the plain two-step
definition computes: first dequantize every weight, then multiply.  This
oracle is that plain definition, in float64:

    W_hat[n, k] = s[n, g] * q[n, k] + b[n, g],   g = k // group_size
    y[m, n]     = sum_k x[m, k] * W_hat[n, k]

The quantizer and the bit packing are an encoding, not a closed form; they
follow the format fixed for the workloads (asymmetric min/max per group of
64 along K, fp16 scale and bias, codes packed little-endian along K: 8
nibbles per uint32 for 4-bit, 4 bytes per uint32 for 8-bit).  The pages
name widths from 2 to 8 bits (BaseRT §3.3 and §4.1: Q2, Q3, Q4, Q5, Q6,
Q8) without giving a layout; every width here uses the same little-endian
bit stream.  Scale groups of 32, 64 or 128 codes are supported.  The 16-bit
format (unquantized fp16 weights, §4.1 FP16) is the plain matmul with each
weight at its exact fp16 value (hmatmul_f64); bf16 weights enter it through
their fp16 rounding (bf16_to_f16_bits).  Around the grouped products
of a mixture-of-experts FFN block: the SwiGLU input of the down projection,
silu(gate) * up per pair (moe_swiglu_f64), and the routing-weighted sum of
each token's pair rows (moe_combine_f64).

Pins (all in the CPU test-suite): hand-worked packed words and quantizer
cases, exhaustive pack/unpack round trips, brute-force code enumeration and
exact rational dot products on 4x64 matrices, closed forms (one-hot and
all-ones activations, integer codes with unit scale), quantizer error
bounds, fp16/fp32 rounding checked against exact rational rounding, and
routing invariants.  No function here is "parity unpinned".
"""
from .qmm_oracle import (  # noqa: F401
    f16_bits, f16_value, quantize, pack, unpack, dequant_f64, round_to_f32,
    round_to_f16_bits, matmul_f64, qmatmul_f64, hmatmul_f64, grouped_f64, route,
    packed_words_per_row, silu_f64, moe_swiglu_f64, moe_combine_f64, bf16_to_f16_bits,
)
