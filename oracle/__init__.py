"""Plain, slow, float64 CPU oracle for routed block-sparse attention over a
Gilbert-ordered KV history.

This package is TEST INFRASTRUCTURE.  Only the test suite, the package smoke
check and the CPU-baseline leg of the benchmark may import it.  The product
path (the HIP library and its Python binding) never imports, calls or links
anything here, and this package imports nothing from the product path.

What it computes, and where the pages say so:

* ``gilbert``   -- the generalized-Hilbert ("Gilbert") token order of one 3-D
  latent chunk [Velox: Spatial Memory Makes World Models Efficient -- Key
  Contributions 3; Methodology, Step 6] [Light Interaction -- abstract,
  "3D block sparse attention"].
* ``layout``    -- raster <-> Gilbert head-major block-padded layouts.
* ``route``     -- mean-pooled block importance, soft geometric fusion with
  unbiased fallback, and top-K route materialisation [Velox -- Key
  Contributions 1-2; Methodology, Steps 4-5].
* ``attention`` -- attention restricted to the routed KV blocks, and the
  dense special case [Velox -- Methodology, Step 6; Main Findings].

Every function works in float64 on exactly-converted inputs (bf16 and fp32
values are representable exactly in float64).  Attention is computed with a
two-pass softmax, and top-K with a full sort, i.e. the plain definitions,
not the streaming forms the GPU uses.
"""

from . import gilbert, layout, route, attention, numerics  # noqa: F401

__all__ = ["gilbert", "layout", "route", "attention", "numerics"]
