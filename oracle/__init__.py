"""CPU oracle for the PASA forward pass: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg import this
package.  The product path never does.

"Online Pseudo-average Shifting Attention (PASA) for Robust Low-precision LLM
Inference", Abstract: PASA is mathematically equivalent to attention, so the
oracle is plain softmax attention in binary64 (see ``oracle.c`` for the
definition it evaluates).
"""
from .oracle import attn_fp64, combine_fp64, num_threads, load  # noqa: F401
