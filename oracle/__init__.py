"""Float64 CPU oracle for one context-parallel rank's share of causal attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
anything in this package: only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg use it.  It shares no code with the HIP library
(no kernels, headers, helpers, tables or pre/post-processing); the only module both
sides use is ``workloads``, which draws seeded inputs and contains no attention
arithmetic.

What it computes is the plain definition, written out slowly and in float64:

* ``partition``: the zigzag chunk pair of a rank, its per-document (packed THD)
  form and the striped (interleaved) split, as direct loops over chunks / documents
  / tokens.
* ``attention``: masked softmax attention per query block (scores, row max, exp,
  sum, weighted V), the associative log-sum-exp merge, the streaming (m, l, a)
  update in the order the pages write it, and the softmax-Jacobian backward (also
  evaluated for a chosen subset of key rows).
* ``rope``: rotary position embedding at the positions a rank keeps (global
  positions, or positions inside each packed document).

Every function cites the page passage it follows.  The pins that tie it to
something other than itself live in ``tests/test_oracle_*.py``.  Parity status of
each function is listed in its docstring; the one passage whose numbers were lost
from the pages (the two-owner worked tables of the teaching page) is "parity
unpinned" and is not used.
"""
from .partition import zigzag_indices, striped_indices, thd_indices, thd_doc_ids  # noqa: F401
from .attention import (visible_mask, attention_fwd, merge, stream_fwd,  # noqa: F401
                        attention_bwd, attention_bwd_keys, MASK_NONE, MASK_CAUSAL,
                        MASK_CAUSAL_DOC)
from .rope import apply_rope, thd_positions  # noqa: F401
