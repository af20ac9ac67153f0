"""Plain, slow, float64 CPU oracle for the ReaDy state-reader path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
package: only the tests, the smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code with the HIP library or its Python binding.

Pages cited (by title):
  * "ReaDy: Recurrent States as Dynamic Context for Speculative Drafting in
    Hybrid Linear Attention Large Language Models" -- the arXiv 2610.20503v1
    text (cited as "arXiv text", with its section / equation / appendix).
  * The Chinese summary of the same paper on paper.rainbus.top (cited as
    "rainbus summary", with its section heading).
  * The Korean summary on onedev.kr (cited as "onedev summary").

Modules:
  reader   -- steps 1-5 of the state reader (gather, state preparation, shared
              projection, per-position query/readout, packing + bottleneck
              MLP + residual), plus fp64 helpers for bf16 decoding/rounding.
  gdn      -- the Gated DeltaNet recurrence in float64, the Proposition 1
              query-span split and the Proposition 2 unrolled identity, and
              the state-vs-KV footprint count.
"""
from . import reader, gdn  # noqa: F401
