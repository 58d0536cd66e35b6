"""CPU oracle for the KDA chunked prefill.

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's CPU
baseline leg may import this package. The product path (the HIP library and
its Python binding) never imports, links or runs anything here, and this
package never imports the product.

Contents
  kda_ref_fwd  -- fp64 token-by-token recurrence (C, OpenMP over (sequence, head));
                  the plain definition of what the method computes.
  gdn_ref_fwd  -- the same recurrence with one scalar gate per (token, head)
                  (Gated DeltaNet, the scalar-gate method KDA refines).
  chunk_ref    -- fp64 chunk algebra (numpy): per-chunk log-gate scan, the
                  beta-weighted gated K K^T, its unit-lower-triangular inverse,
                  W, U, the per-chunk states and corrections, and the output.
                  It is the chunked evaluation of the same recurrence, exact up
                  to rounding order, and is pinned against the recurrence.
"""
from .ref import gdn_ref_fwd, kda_ref_fwd, threads, load  # noqa: F401
