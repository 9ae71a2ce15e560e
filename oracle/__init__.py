"""Oracle for fused exact attention (forward and backward) -- TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 CPU implementations of what the GPU path computes.  Nothing
in the product (the ``exact_attention_75_amd`` package, its C-ABI library or its
kernels) imports, links or calls anything here; only the tests, the smoke check
and the CPU-baseline leg of the benchmark do.  The oracle shares no code, no
tables and no constants with the GPU path.

Modules
  attention  the definition softmax(scale * Q K^T + mask) V with a per-row
             natural-log LSE, the full score matrix materialised per head;
             the same over a sub-range of the keys (the partial state of one
             key split) and the combine formula that merges such partials;
             the backward (dQ, dK, dV, with an optional LSE gradient) by the
             chain rule through that definition
  fp8        OCP E4M3 encode/decode, per-128-row block quantisation, the
             Sylvester Hadamard matrix and the signed rotation

Parity status: every function here is pinned by tests that run without a GPU
(closed forms, invariants, library routines, brute force); none is
"parity unpinned".
"""
from . import attention, fp8  # noqa: F401
