"""Float64 CPU oracle for exact ring-ordered attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
or run anything in this package.  The product path (the HIP library and its
Python binding) never imports it, and this package imports nothing from the
product path: the two share no code.  Inputs for both come from the separate
``synthetic`` module, which holds random draws only.

Contents:

* :mod:`oracle.layout` -- token layouts (contiguous, striped, zig-zag), the
  ring order of KV chunks, causal classification of chunk pairs and
  visible-pair counts, all derived from explicit position arrays.
* :mod:`oracle.attention` -- the plain definition of exact softmax attention,
  an independent chunked (m, l, o) loop in ring order, the single-chunk state
  update, finalize, and the log-sum-exp merge of two partials.
* :mod:`oracle.backward` -- the gradients dq, dk, dv of exact attention by
  the steps of the pages' backward listing, and the same steps taken in ring
  order with P recomputed from the forward's log-sum-exp.

Every function states the passage of the source pages it follows.  Pins
(checks against things other than the oracle itself) live in
``tests/test_oracle_*.py``.  Nothing here is parity-unpinned.
"""
from . import attention, backward, layout  # noqa: F401
