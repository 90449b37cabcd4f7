"""CPU oracle for the quantized MoE expert layer -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct NumPy implementation of what the layer
computes, in float64 wherever a value is not a stored narrow format.  Only the
tests, the smoke check and the benchmark's CPU-baseline leg may import it; the
product path (the HIP library and its Python binding) never does, and this
package imports nothing from the product path.

Modules:
  formats -- OCP FP8 E4M3, bfloat16 and INT4 storage formats (encode/decode/pack)
  layer   -- routing, per-token FP8 quantization, permutation, grouped GEMMs,
             SiLU gating, combine, shared experts and the whole layer

Pinning: every function here is checked by ``tests/test_oracle_*.py`` against
something other than itself (library casts, brute force, closed forms,
hand-derived examples of the pages' stated rules).  Functions with no such pin
say "parity unpinned" in their docstring.
"""
from . import formats, layer  # noqa: F401
