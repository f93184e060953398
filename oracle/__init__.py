"""CPU oracle for the batch-invariant token-logprob path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this package.  The product path (``invariant_gemm_token_amd``) never imports,
links or calls it, and this package imports nothing from the product path.

Contents (all in ``oracle.reference``):

* fp64 definitions of what the path computes: the exact contraction, the
  max-shifted log-softmax, the sampled-token logprob and the MoE combine;
* float32 emulators of the two places where the method fixes a rounding
  order that a test can check bit for bit: the fixed binary tree over
  leaves and the ascending-expert-id FP32 combine.

Parity status of each function is stated in its docstring.  The rounding
inside one leaf (the matrix-core instruction's own summation) and the
hardware exp2/log2 are not modelled: those results are checked within the
stated tolerances only ("parity unpinned" beyond the tolerance).
"""

from .reference import *  # noqa: F401,F403
