"""CPU oracle for speculative-sampling verification.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the bench's
CPU-baseline leg import this package.  The GPU library never calls it, links it
or falls back to it, and it shares no code with the GPU library.

Pages cited in this package:
  [FI]  intuitivepapers.ai, "Fast Inference from Transformers via Speculative Decoding"
  [SD]  nonconvexcard course page, "Speculative Decoding"
  [LH]  lihaoran.work article on speculative decoding (sections "Three candidates
        explain the acceptance rule", "What does 'unchanged output' mean?",
        "Fix the benchmark conditions first")
  [DB]  deval-blog, "Speculative decoding"
  [NZ]  nazmi.tech, "Speculative decoding and self-speculative decoding"

Modules:
  verify  -- fp64 NumPy sampler: softmax, overlap, ratio test, accepted prefix,
             residual or bonus row, inverse-CDF sample, argmax mode.
  exact   -- exact-rational (fractions.Fraction) statements of the single-step
             mass identity, the overlap, and the expected-yield formula.
  lmhead  -- fp64 LM-head product for the fused LM-head workload.
  kvcache -- the KV-cache crop after a verification step, as plain slicing
             (contiguous and paged caches).

Parity status: every function here is pinned by a CPU test against values the
pages print, closed forms, library routines or brute force.  None is marked
"parity unpinned".
"""

from . import exact, kvcache, lmhead, verify  # noqa: F401
