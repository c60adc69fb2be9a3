"""Plain fp64 CPU oracle for F4 paged attention with YaRN rope.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, links or runs this
package; only the tests, the smoke check in ``__graft_entry__`` and the CPU
baseline leg of ``bench.py`` may use it.  It shares no code, table or helper
with the HIP path: it is written from the pages' description of the method and
the layout spec below, in numpy float64, as slowly and plainly as that takes.

Modules
-------
yarn       static YaRN frequency table and mscale (mistral.rs PR #2375,
           "Changes by area" item 1; ignis context-and-speculation page,
           ``--model-rope-scaling`` row) and the NEOX rotation.
f4         the symmetric 4-bit block quantiser ``(nibble - 8) * scale``
           (mistral.rs PR #2375, "Changes by area" item 2 and "Known
           limitations") and the cache's physical byte layout.
attention  paged gather, exact softmax decode attention, partial states and
           their log-sum-exp fold (FreeToken issue #568, "Proposed solution"
           item 2), and causal chunked prefill.
fp8        the 8-bit prefill (ignis context-and-speculation page,
           ``--model-prefill-attention`` row: Q.K^T in INT8, P.V in E4M3) as a
           model of its rounding steps, E4M3 rounding and the INT8 quantisers.

Every function here is pinned by ``tests/test_oracle_*.py`` against values
the pages print, closed forms, invariants or brute force.  The one result with
no such pin is the end-to-end equivalence of F4 attention to unquantised
attention: parity unpinned (the pages say it was never measured).
"""
from . import yarn, f4, attention, fp8  # noqa: F401
