"""Plain fp64 CPU oracle for one GPU's share of the Q-KV assignment matrix.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
Python binding) may import, call or execute anything in this package.  Only the
tests, the smoke check and the CPU-baseline leg of the bench use it.  It shares
no code, tables or helpers with the HIP path; the only common module is
``synthetic`` (seeded input draws, no attention arithmetic).

Sources (cited by title and section; the pages are the authority):

* [Mesh]  "Mesh-Attention: A New Communication-Efficient Distributed Attention
  with Improved Data Locality" (arXiv 2512.20968).
* [CHARM+] "CHARM+: Cross-Hardware Attention with Re-Merge Multistream
  Mechanism" (arXiv 2611.05906v1).
* [Ring]  "Ring Attention and Context Parallelism: How Long-Context LLMs Are
  Trained Across GPUs" (blog post).

Modules:

* ``attention`` - the forward tile (partial O and LSE), the LSE merge, the
  tile backward and the add-reduce of partial gradients, each written as the
  plain definition in float64.
* ``layout``   - token positions (contiguous, zigzag, striped), the assignment
  matrix with basic tiling and KV partition rotation, footprints, groups, and
  tile classification by brute-force enumeration.

Every function is pinned by a ``-m "not gpu"`` test against something other than
itself (brute force, closed forms, invariants, values printed on the pages).
No function here is "parity unpinned".
"""

from .attention import attn_tile, merge, attn_tile_bwd, attn_bwd_multi, reduce_add  # noqa: F401
from . import layout  # noqa: F401
