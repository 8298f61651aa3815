"""CPU oracle for the NVFP4 dense-MoE router path.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, exact reference
that the HIP library is checked against. Only the test suite, the smoke
entry point and the benchmark's CPU-baseline leg may import it; the product
path (the C-ABI library and its Python binding) never does, and this package
never imports the product. It shares no code, tables or constants with the
HIP sources.

Sources (the three pages are commit messages of the nvfp4-megamoe-kernel
repository; they are cited by commit and by the paragraph a fact sits in):

* commit 04cf8ca8, ``dsv4/layers/router.py`` -- the runtime global-scale fix
  (gsa from the activation's own max magnitude, E4M3 block-scale ceiling 448,
  the bound on x/gsa), the NVFP4 gate paths and the fused-router dispatch.
* commit e0f60b9f, ``dsv4/kernels/router/__init__.py`` -- the working path:
  gate GEMM then a single-pass six-step activation/top-k epilogue.
* commit df05289d, ``dsv4/layers/grouped_linear.py`` -- device-only global
  scale, no host syncs, caller-owned pre-allocated buffers, the grouped
  layer's flattened quantization and device-side group offsets.

Facts the pages leave open are fixed by the NVFP4 format (16-element blocks
along the contraction axis, E4M3 block scales, E2M1 elements, one fp32
per-tensor scale) and by the router epilogue this path implements (sigmoid
score, selection bias, top-k, gather of unbiased scores, renormalization,
routed scale).

Parity status per function:

* ``formats``: pinned (format tables brute-forced against exact rationals).
* ``quant_ref``: pinned (closed forms, hand-worked examples, exhaustive
  bf16 sweep, scalar exact-rational twin).
* ``router_ref``: pinned (hand cases, zero-input and zero-bias reductions,
  brute-force subsets, exact-rational logits).
* ``check``: pinned by mutation tests (planted mistakes must be caught).
* ``lmhead_ref``: pinned (one-hot hand case with a tie, brute force over
  rows, mutation tests of its checker); its logits are router_ref's.
* ``grouped_ref``: pinned (hand cases with per-group weight scales and a
  shared activation scale set by another group, offsets closed form, exact
  rational brute force on tiny groups, empty groups).

Two conventions are not fixed by the pages and are parity unpinned by them:
the nibble order of packed codes (even element in the low nibble) and the
code of -0 and of negatives that round to zero (sign kept: 0x8). The tests
pin the oracle to these stated conventions.
"""

from . import formats, quant_ref, router_ref, check, lmhead_ref, grouped_ref  # noqa: F401
