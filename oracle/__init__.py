"""CPU oracle for rollout-guided FP4 fake quantization (TRACE).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute anything in this package: only the test suite, the smoke check and the
benchmark's CPU-baseline leg use it. The oracle shares no code with the HIP
library (no kernels, headers, tables or helpers); the two meet only through the
seeded inputs of the ``synthetic`` package, which holds no quantization
arithmetic.

The oracle is plain and slow on purpose: NumPy float32 where the formats fix
binary32 arithmetic (the NVFP4 global scale is FP32, the decoded outputs are
bf16), exact integer arithmetic for codes, and float64 (or exact rationals in
the tests) for the discrepancy sums. Each function cites the passage of the
paper it follows:

    "TRACE: Rollout-Guided Quantization-Aware Training for FP4 Reinforcement
    Learning of MoE Language Models" (arXiv 2610.07767), reader-view page.

Where the paper is silent or its equations were lost in extraction, the
function states the reading it takes.

Modules:
    formats  bf16, FP4 E2M1, FP8 E4M3 and E8M0 encodings
    fp4      the method: scales, RTN, guidance encode/decode, guided rounding,
             discrepancy sums
    sizes    the guidance-size arithmetic of §3.2 and §4.2
    record   the page gather that collects a request's records

Pins (tests marked ``not gpu``) tie every function here to something other
than itself: values the paper prints, library casts (torch bf16 / float8),
closed forms, invariants and brute force on small inputs.
"""

from . import formats, fp4, sizes  # noqa: F401
