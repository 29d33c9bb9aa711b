"""CPU oracle for the grouped expert MLP — TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 numpy definition of what the routed, grouped SwiGLU expert
MLP computes, forward and backward, in BF16 and in MXFP8.  Only the tests, the
smoke check and the CPU-baseline leg of the benchmark may import it; the library
never does, and it imports nothing from the library (it shares no code, tables or
helpers with the HIP path).

Sources followed (titles of the pages this is written from):
  [P1] "NVIDIA Shows an Efficient MoE Training Path for Biological Foundation
       Models" — sections "Grouped experts instead of a Python loop",
       "Memory and quantization overhead".
  [P2] "BioNeMo recipe 2.21x throughput ..." — sections "Fragmented Expert Kernels",
       "Memory Pressure From Long Sequences", "Quantization Overhead".
  [P4] ai4snews report on the BioNeMo MoE recipe — paragraphs on GroupedLinear,
       on FP8/MXFP8 and on the Sequential fusion.
  [OCP] OCP Microscaling Formats (MX) v1.0 specification — E4M3 element format,
       E8M0 shared scale, the scale-selection and conversion rules (external; the
       pages fix only one scale per 32 consecutive values).

Modules:
  oracle.mx     — E4M3 / E8M0 encode-decode, block quantization (row / column, column
                  with 32-row blocks restarting at segment starts) and FP8 with one
                  scale per tensor.
  oracle.route  — top-k routing, split_sizes, group offsets, stable permutation,
                  and the router backward (d_logits from d_prob).
  oracle.mlp    — per-token (O-slow) and grouped (O-grouped) forward, backward,
                  and the MXFP8 pipeline stages fed with given quantized operands.
  oracle.metrics— relative Frobenius error.

Every function is pinned by tests in tests/test_oracle_*.py (brute force, closed
forms, invariants, finite differences); none is "parity unpinned".
"""
