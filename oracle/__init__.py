"""Float64 CPU oracle for row-wise ICL attention -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plainly written reference against which the HIP
path is checked.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path (the
C-ABI library and its Python binding) never imports, links or calls it, and
the two share no code: only the seeded input generator
(``long_context_tabular_amd.inputs``, which holds no arithmetic of the method)
feeds both.

Contents
--------
``numerics``  exact fp16 / fp32 / OCP e4m3 rounding helpers.
``icl``       the method: shared-length LogScale / GatedLogScale query scaling
              ("Fuse shared-length query scaling during inference", Problem
              identified and Solution), context-derived per-head FP8 e4m3
              quantisation ("[FP8 3/4] Integrate FP8 attention and caching into
              TabICLv2", introduction), and non-causal row-wise attention of
              context rows and of query rows against the context K/V (same
              page, walkthrough: one shared projection, then PyTorch's
              scaled dot-product attention).

Every function cites the passage it follows.  Where the pages leave a step
open, the reading taken is stated in the function's docstring.
"""
from . import numerics, icl  # noqa: F401
