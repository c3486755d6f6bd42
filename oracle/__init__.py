"""Plain, slow, fp64 CPU oracle for the parallel transformer block with
sliding-window attention and for the LAMB optimizer step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
anything in this package: only the test suite, the smoke check and the bench's
CPU-baseline leg use it.  It shares no code with the HIP library.

Sources (pages, by title and section):
  * "MegaScale study guide" (ai-yanyi-papers, paper arXiv:2402.15627), chapter 2
    section 2.2 (paper section 3.1), table of the three algorithmic changes:
    the PTB row (the parallel block formula), the SWA row (each token sees a
    fixed window w) and the LAMB row (layer-wise adaptive trust ratio, You et
    al. 2020); section 2.1 (paper section 2): MFU and the 6N FLOPs/token
    estimate; section 2.5 (paper section 6.1), Table 1: the 175B/530B shapes.

Modules:
  ptb   -- LayerNorm, SWA, GeLU, the block forward and its backward
  lamb  -- one LAMB step over a list of parameter tensors
  flops -- FLOP counts and the MFU arithmetic

Every function is pinned by tests that do not retype it (see tests/test_oracle_*):
closed forms, invariants, brute force on tiny inputs, library special cases and
finite differences.  No function here is "parity unpinned".
"""
from . import flops, lamb, ptb  # noqa: F401
