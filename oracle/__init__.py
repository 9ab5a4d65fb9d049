"""fp64 CPU oracle for training-free block-sparse attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this package.  The product path (the HIP library and its
Python binding) never calls it, and this package never imports the product
package: the two share no code, no headers, no tables.  The only common
dependency is ``workloads`` (seeded random inputs, no method arithmetic).

What is computed, and where on the pages it comes from:

* ``attention``  -- scaled dot-product attention and the restricted softmax
  (SparseAttn article, section 3.1), removed-mass identity and bound (3.2),
  spatio-temporal teaching masks and pair counts (3.3), the local causal
  window and block-pair masks and ledger ("Local Sliding and Sparse
  Attention", Steps 2 and 4), the causal access patterns and their ledger
  ("Attention Access Pattern Benchmark", Steps 2 and 4).
* ``layout``     -- token reorders: [t,h,w]-window reorder with the first frame
  kept in front and text moved last (MindIE-SD "sparse" page, rf_v2) and the
  Hilbert-curve order (SpargeAttn notes, section 2.5), written from Skilling's
  published transform; permute / unpermute (SparseAttn article, section 3.4).
* ``predict``    -- block statistics and the block-mask predictor (SpargeAttn
  notes, section 2.2), with sink, window and keep-floor forcing.
* ``flash``      -- attention restricted to a block CSR, with the optional
  PV-skip emulation in the online-softmax recurrence (SpargeAttn notes,
  sections 2.1 and 2.3).
* ``numerics``   -- exact bf16 upcast and float32 -> bf16 round-to-nearest-even.
* ``quant``      -- per-block 8-bit (OCP FP8 E4M3) quantization of the QK
  operands with one dequantization scale per block (SpargeAttn notes,
  section 2.4), written from the format's definition.
* ``admissible`` -- which mask rows the predictor's reading admits when a
  decision lies within rounding of its threshold (used by the parity checks).

Every function is pinned by a ``-m "not gpu"`` test against values printed on
the pages, closed forms, brute force or textbook special cases.  The quality
of the predicted mask against dense attention (relative L1, MSE) is reported
but **parity unpinned**: the pages' quality figures come from real models.
"""

from . import admissible, attention, flash, layout, numerics, predict, quant  # noqa: F401
