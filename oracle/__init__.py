"""Plain, slow, fp64 CPU oracle for head-classified segmented paged attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import anything here.  The product
path (``long_context_serving_amd`` and its HIP library) never imports it and
shares no code, header, helper or table with it; the only thing both sides
use is the seeded input generator ``long_context_serving_amd.workloads``,
which holds none of the method's arithmetic.

Modules:
  attention  masked softmax attention with per-head causal/window visibility
  segments   which tokens a head's segment must store
  ledger     closed-form visible-pair, FLOP and byte counts
  rope       query-side rotary relocation by a per-head position offset
  merge      head-decomposition merge: per-(row, head) select or log-sum-exp merge
  fork       token-level model of copy-on-write forks of per-head segments
  router     attention-mass token scores and their top-k (sparse-FFN routing)
"""
