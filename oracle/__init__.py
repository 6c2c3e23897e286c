"""CPU fp64 oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE.  Only `tests/`, `__graft_entry__.smoke()` and the `cpu_baseline` leg of
`bench.py` may import or call anything in this package.  The product path (the HIP library
and its Python binding) never imports it, and this package never imports the product.

Contents
  attention.py  the plain definition, materialising S and P per (batch, head) in fp64:
                forward (O, LSE) and backward (dQ, dK, dV) by differentiation of that
                definition; row-chunked so that long sequences fit host memory.
  online.py     the pages' tiled loop with the online-softmax update, in fp64, used by the
                tests as an independent witness that the re-association is exact.
  mx.py         MX-FP8 (E4M3 elements, power-of-two scales per 32 elements) quantisation from
                the OCP Microscaling Formats specification, for the FP8 forward's inputs; the
                FP8 forward's reference is forward_head on the dequantised inputs, and its
                tolerance attention.p_rounding_bound (the rounding of P to E4M3).

Page keys used in citations:
  [P1] "How FlashAttention Bypasses the GPU Memory Bottleneck to Enable Long-Context AI" (factlen.com)
  [P2] "FlashAttention: how a memory trick unlocked today's giant AI models" (khetwal.com)
  [P3] "How FlashAttention Eliminates Transformer Memory Bottlenecks" (Galileo blog)

Parity status: every function here is pinned by `tests/test_oracle.py` (brute force on tiny
inputs, closed forms, invariants of softmax attention, central finite differences for the
backward, and agreement with the tiled online-softmax loop) and `tests/test_oracle_mx.py` (the
E4M3 code table, nearest-even rounding by brute force over every code, the shared-exponent
rule; p_rounding_bound against worst-signed perturbations and actual E4M3 rounding of P).  No function is parity-unpinned.
"""
from .attention import (  # noqa: F401
    MASK_BLOCK,
    visible,
    probabilities,
    forward_head,
    forward,
    backward_head,
    backward,
    s_matrix_bytes,
    p_rounding_bound,
)
from .online import tiled_forward_head  # noqa: F401
from . import mx  # noqa: F401
