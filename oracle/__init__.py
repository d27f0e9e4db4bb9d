"""Plain CPU oracle for the DDTree draft-tree hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, table or
helper with the HIP library; the only thing both sides see is the seeded
input generator module, which holds none of the method's arithmetic.

Every function is the slow, obviously correct definition written out in
numpy and Python (fp64 for floating point unless the decision being made is
one the device takes in fp32, which is then mirrored in fp32 and says so).
Sources are the five web pages on DDTree; each function cites the page and
the section, figure or proposition it follows.

Modules
-------
softmax_topk  per-position log-softmax and top-K ranking
tree          prefix scores, the order on prefixes, the top-B set
              (brute force, sort-and-expand, best-first heap), tree arrays
              and the ancestor-or-self mask
attention     ancestor-only tree attention (naive, fp64)
commit        target argmax, greedy accept walk and KV-cache compaction
budget        cost-aware node budget from the pop-order scores
              (Proposition 1's expected acceptance per budget)
sampling      temperature > 0: Philox4x32-10 uniforms, Gumbel-max target
              sample per node (the walk then runs on the samples)

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against values the pages print, closed forms, theorems checked by
exhaustive enumeration, or textbook/library reductions.
"""
from . import attention, budget, commit, sampling, softmax_topk, tree  # noqa: F401
