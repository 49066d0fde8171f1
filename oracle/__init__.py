"""CPU oracle for the Ulysses sequence-parallel hot path — TEST INFRASTRUCTURE.

A plain, slow, obviously correct NumPy (float64) statement of what the hot
path computes, written from the pages' description of the method:

  * ``ranges``   — balanced contiguous token / head ranges and the head-chunk
                   plan;
  * ``relayout`` — the sequence-sharded <-> head-sharded relayouts on either
                   side of the all-to-all (whole head groups, or one head
                   chunk per phase of the two-phase exchange), as explicit
                   index loops, and the model-boundary scatter / gather;
  * ``attention`` — direct two-pass softmax(sigma * Q K^T) V per head, a
                   pure-Python brute force for tiny inputs, and a process-pool
                   driver over host cores;
  * ``ulysses``  — the composition pack -> per-head-group attention -> unpack,
                   head-chunked passes, and the two-phase exchange (pack ->
                   attention -> unpack once per head chunk);
  * ``ring``     — the log-sum-exp merge of attention over key blocks and the
                   Ulysses+Ring composition on a U x R grid, whole or in
                   head-chunk phases.

Only the test suite, the smoke check in ``__graft_entry__`` and the CPU
baseline leg of ``bench.py`` may import this package. The product path (the
HIP library and its Python binding) never imports, calls or links it, and
this package imports nothing from the product path. The two share only the
seeded input generator, which holds none of the method's arithmetic.

Every function is pinned by tests that do not re-use its own formula: printed
splits, library routines (``numpy.array_split``, PyTorch's CPU
``scaled_dot_product_attention``), closed forms, invariants and brute force.
"""
from . import attention, ranges, relayout, ring, ulysses  # noqa: F401
