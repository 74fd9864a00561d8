"""CPU oracle for the native 4-bit MoE expert layer (NVFP4 forward, MXFP8 backward).

TEST INFRASTRUCTURE ONLY. This package is the slow, plain, obviously-correct
definition of every result the HIP library computes. It exists so that the GPU
path can be checked against it; it is never part of the product path. Only the
test suite, the smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg
of ``bench.py`` may import it. It shares no code with the HIP library and does
not import it.

Sources ("End-to-End 4-Bit Training", Thinking Machines, as summarised on the
pages under the reference; cited by page title and section):

* "Inkling 2 Small uses four-bit training ..." (ai-primer), section
  "Block scales and per-token activations": NVFP4 = 4-bit values, one 8-bit
  E4M3 scale per block of 16, 4.5 bits/value; an FP32 outer scale per expert
  (weights) and per token (activations); MXFP8 costs 8.25 bits/value.
* same page, section "Stochastic rounding across transposes": dequantize the
  saved forward weights/activations, transpose in higher precision,
  re-quantize to MXFP8 with stochastic rounding, run MXFP8 gradient matmuls;
  worked example 4.5 -> 4 (p=0.75) / 6 (p=0.25).
* same page, section "NVFP4 forward, MXFP8 backward".
* "Thinking Machines Lab ... 4-bit precision" (aibuzzwire), section
  "Why Fewer Bits Means Faster Training": round-to-nearest illustration
  3.2 -> 3 with error 0.2.

Everything the pages leave open (rounding modes, scale formulas, the random
number mapping, layouts) is a stated reading; each function's docstring says
which.

Parity status: every function here is pinned by tests under ``tests/``
(``test_oracle_*.py``) against closed forms, brute force, the pages' worked
examples or independent library routines. Philox4x32-10 is pinned against the
rocRAND source header's host implementation and known-answer vectors.
"""

from . import formats, philox, nvfp4, mxfp8, permute, gemm, ffn, nvfp4_bwd  # noqa: F401

__all__ = ["formats", "philox", "nvfp4", "mxfp8", "permute", "gemm", "ffn", "nvfp4_bwd"]
