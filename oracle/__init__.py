"""Float64 CPU oracle for the FP8 MoE feed-forward step.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The HIP library never calls it, and it shares no code, table, constant generator or
helper with the HIP library: every number here is derived from the definitions of
the operations, written out plainly and evaluated in float64.

What it computes (the pages name the pieces but print no formulas):

* FP8 weights and activations for the GEMMs and the MoE part of the model
  (Blackwell 1,000 TPS/user blog, zh translation, lead list and the paragraph on
  FP8 data types for GEMM, MoE and attention).
* The FC13 GEMM (gate and up projections side by side) with SwiGLU fused onto it,
  and a quantize step in front of the next GEMM (same page, section
  "CUDA kernel optimisation and fusion", item "operator fusion").
* A mixture-of-experts layer: one shared expert that every token uses plus one
  routed expert per token (top-1).  The pages only name "MoE"; the top-1 plus
  shared structure, the sigmoid gate and the OCP e4m3 format are readings of them,
  the plainest that the rest of the pages support.

Modules:

* ``oracle.fp8``   -- OCP e4m3 decode/encode and bf16 conversions.
* ``oracle.ffn``   -- quantise, route, FC13+SwiGLU, re-quantise, FC2, combine.
* ``oracle.loops`` -- a second, loop-only version of the whole step for tiny
  inputs, written with different algorithms (linear search encoder, Fraction
  based bf16 rounding), used to pin ``oracle.ffn``.

Every function in ``oracle.fp8`` and ``oracle.ffn`` is pinned by a ``-m "not gpu"``
test in ``tests/test_oracle_*.py`` against something other than itself: the
torch e4m3 and bf16 casts, IEEE float32 division, integer arithmetic, closed forms
worked out by hand, algebraic invariants, or the loop-only version.
"""

from . import fp8, ffn, loops  # noqa: F401
