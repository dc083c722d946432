"""CPU oracle for the fused weight-gradient + optimizer step (FORGE).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything in this package: only the tests, the package smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library.

What it computes (FORGE explainer pages, gist.science, "FORGE: Fused
On-Register Gradient Elimination for Memory-Efficient LLM Training"):

* Technical Summary section 1 "The Problem": the standard two-phase schedule
  that first forms the full weight gradient and then runs the optimizer.
* Technical Summary section 2 "Core Mechanism" and "Precision and Fidelity":
  the tile schedule reaches exactly the two-phase result for element-wise
  optimizers, up to the floating-point order of the sum over tokens.  So the
  oracle is the plain two-phase definition in float64: dW = dY^T X from the
  exact values of the stored inputs, one element-wise optimizer step in
  float64, then the storage roundings (fp32 cast, stochastic rounding of the
  bf16 weight, block-64 int8 moments).
* Technical Summary section 3 "Key Contributions" names the eight optimizers.

Modules:
  philox      Philox4x64-10 counter-based generator (Salmon et al., SC'11).
  numerics    bf16 / e4m3 decoding, bf16 stochastic and nearest rounding,
              block-64 int8 moment codec (linear absmax map).
  dynmap      the dynamic 8-bit map for block-64 moments (comparison format).
  optimizers  per-step scalars and the eight element-wise update rules.
  wgrad       dW, dX, and the full and tiled step schedules.

Every function is pinned by tests under tests/ (marked "not gpu") against
library routines, closed forms, brute force and invariants.
"""
from . import philox, numerics, dynmap, optimizers, wgrad  # noqa: F401
